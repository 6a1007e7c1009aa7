// dQ of the causal GQA flash-attention backward for one head chunk
// (gfx950, d = 128); the chain rule and the split into a key-stationary
// dK/dV kernel and this query-stationary dQ kernel are described in
// flash_bwd.hip.  A workgroup owns 128 queries of one q head (4 waves x 32
// queries) and walks the key tiles up to the diagonal like the forward
// kernel: S^T = K Q^T and dP^T = V dO^T give each lane one query (its LSE
// and D are per-lane scalars), dS^T feeds dQ^T = K^T dS^T as a B operand from
// registers, and K^T is the transpose read of the same K tile; K/V tiles are
// double-buffered, two workgroups per CU.  The epilogue scales dQ, applies
// the inverse RoPE in registers and writes bf16.
//
// This file is compiled with the max-ILP machine scheduler (see the build
// script): for this kernel it measured 2.5% faster than the default, while
// the dK/dV kernel measured 3% slower with it, hence the separate file.
#include "kernels.h"

namespace upipe {
namespace {

constexpr int QBM = 128;       // queries per dq workgroup
constexpr int QBN = 64;        // keys per dq step

// K and V tiles double-buffered in distinct fields (the key loop is unrolled
// by two): every LDS address is a per-lane base plus an immediate.
struct __attribute__((aligned(16))) DqSmem {
  uint16_t K0[QBN * 128], V0[QBN * 128];
  uint16_t K1[QBN * 128], V1[QBN * 128];
};

__global__ __launch_bounds__(256, 2) void flash_bwd_dq_kernel(BwdArgs a) {
  __shared__ DqSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;

  const int nqt = (int)(a.Lp / QBM);
  const int head = blockIdx.x % a.nh;
  const int qt = nqt - 1 - (int)(blockIdx.x / a.nh);
  const int q0 = qt * QBM;
  if (q0 >= a.L) return;
  const int L = (int)a.L;
  const int kvh = (a.q_head0 + head) / a.group - a.kv_head0;
  const uint16_t* qp = a.q + (int64_t)head * a.Lp * 128;
  const uint16_t* dop = a.dO + (int64_t)head * a.Lp * 128;
  const uint16_t* kp = a.k + (int64_t)kvh * a.Lp * 128;
  const uint16_t* vp = a.v + (int64_t)kvh * a.Lp * 128;

  const int r0 = q0 + 32 * wave;
  const int my_q = r0 + l32;

  // Q and dO of this lane's query as B operands (column = query, k = d)
  u32x4 qreg[8], doreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qreg[ks] = *reinterpret_cast<const u32x4*>(qp + (int64_t)my_q * 128 + ks * 16 + g * 8);
    doreg[ks] = *reinterpret_cast<const u32x4*>(dop + (int64_t)my_q * 128 + ks * 16 + g * 8);
  }
  const float nlse2 = a.lse2[(int64_t)head * a.Lp + my_q];  // -LSE, base 2
  const float ndval = a.dvec[(int64_t)head * a.Lp + my_q];  // -D
  // the lane's -D and -LSE in all 16 registers: the starting values of each
  // dP^T and S^T chain (the first MFMA reads them as its C operand), so
  // dP - D and S - LSE cost no vector instruction per element
  f32x16 nd16, nl16;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    nd16[r] = ndval;
    nl16[r] = nlse2;
  }

  const int kv_end = (q0 + QBM < L) ? q0 + QBM : L;
  const int n_kt = (kv_end + QBN - 1) / QBN;

  // per-lane element offsets, fixed for the whole loop
  //  K/V rows (A operands of S^T and dP^T): row kb*32 + l32, chunk 2ks + g
  // (held for step 0 only: the swizzle XORs a row's chunk index with a
  // per-row constant, so step ks sits at koff0 ^ (ks << 4) and column block
  // db of the transpose reads at offt0 ^ (db << 5), one v_xor per read;
  // the registers go to the -LSE tuple)
  const int koff0 = tile_off(l32, g);
  //  K^T (A operand of dQ^T, see tile_read_t): column block db, rows
  //  4g + (lane%16)/4 and +8; 16 st more rows are an immediate
  int offt0[2];
  {
    const int sl = lane & 15, grp2 = (lane >> 4) & 1;
    const int rr = 4 * g + (sl >> 2);
    const int col = 16 * grp2 + 4 * (sl & 3);
    offt0[0] = tile_off(rr, col >> 3) + (col & 7);
    offt0[1] = tile_off(rr + 8, col >> 3) + (col & 7);
  }
  //  tile copies: wave w moves rows 16w .. 16w+15 of the K and V tiles
  uint32_t tdma[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + (lane >> 4);
    tdma[i] = (uint32_t)(row * 128 + (((lane & 15) ^ swz(row)) << 3));
  }
  auto load = [&](int kt, uint16_t* Kd, uint16_t* Vd) {
    const uint16_t* ksrc = kp + (int64_t)kt * QBN * 128;
    const uint16_t* vsrc = vp + (int64_t)kt * QBN * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16_untracked(ksrc + tdma[i], lds_addr(Kd + (wave * 4 + i) * 512));
      dma16_untracked(vsrc + tdma[i], lds_addr(Vd + (wave * 4 + i) * 512));
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};

  auto step = [&](int kt, const uint16_t* Kt, const uint16_t* Vt) {
    const int kstart = kt * QBN;
    if (kstart > r0 + 31) return;  // every key of the tile is in this wave's future
    // S^T = K Q^T, dP^T = V dO^T: element (key kb*32+acc_row(r,g), query my_q)
    f32x16 sv[2], dp[2];
    // the S/dP MFMAs issue at raised wave priority, the rest at the default
    // (measured: the dQ MFMAs at raised priority too is slower)
    int ko = koff0;
    asm volatile("" : "+v"(ko));  // keeps the XORed offsets out of registers
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sv[kb] = nl16;
      dp[kb] = nd16;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sv[kb] = mfma32(*reinterpret_cast<const u32x4*>(Kt + (ko ^ (ks << 4)) + kb * 4096), qreg[ks], sv[kb]);
        dp[kb] = mfma32(*reinterpret_cast<const u32x4*>(Vt + (ko ^ (ks << 4)) + kb * 4096), doreg[ks], dp[kb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (kstart + QBN - 1 > r0) {  // the tile reaches past this wave's first query
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kstart + kb * 32 + acc_row(r, g) > my_q) sv[kb][r] = -__builtin_inff();
    }
    u32x4 pS[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(sv[kb][r]);
        ds[r] = p * dp[kb][r];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          pS[kb * 2 + h][t] = pack_bf16x2(ds[8 * h + 2 * t], ds[8 * h + 2 * t + 1]);
    }
    int ot0 = offt0[0], ot1 = offt0[1];
    asm volatile("" : "+v"(ot0), "+v"(ot1));
    // dQ^T += K^T dS^T; B slot t of step st is key 16*st + 8*(t/4) + 4*g + t%4
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 lo = lds_read_tr16(Kt + (ot0 ^ (db << 5)) + st * 2048);
        const u32x2 hi = lds_read_tr16(Kt + (ot1 ^ (db << 5)) + st * 2048);
        acc[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pS[st], acc[db]);
      }
    // K^T transpose reads kept six (three MFMAs) ahead, then two per MFMA
    // (measured 0.9% faster than the compiler's order; eight ahead 0.5%,
    // four ahead no gain)
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 13; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  };

  load(0, sm.K0, sm.V0);
  lds_dma_wait();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    if (kt + 1 < n_kt) load(kt + 1, sm.K1, sm.V1);
    step(kt, sm.K0, sm.V0);
    lds_dma_wait();
    __syncthreads();
    if (kt + 1 >= n_kt) break;
    if (kt + 2 < n_kt) load(kt + 2, sm.K0, sm.V0);
    step(kt + 1, sm.K1, sm.V1);
    lds_dma_wait();
    __syncthreads();
  }

  if (my_q >= L) return;
  // element (d = db*32 + acc_row(r,g), query my_q): scale, inverse RoPE, bf16
  uint16_t* orow = a.dq_out + (int64_t)my_q * a.dq_ld + (int64_t)head * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d = db * 32 + j4 * 8 + g * 4;
      float r4[4];
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        float cs, sn;
        rope_cos_sin(a.rope, my_q, (d >> 1) + pi, cs, sn);
        float e = acc[db][4 * j4 + 2 * pi] * a.scale, o = acc[db][4 * j4 + 2 * pi + 1] * a.scale;
        r4[2 * pi] = e * cs + o * sn;
        r4[2 * pi + 1] = -e * sn + o * cs;
      }
      u32x2 w = {pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3])};
      *reinterpret_cast<u32x2*>(orow + d) = w;
    }
}

}  // namespace

hipError_t launch_flash_bwd_dq(const BwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / QBM) * a.nh));
  hipLaunchKernelGGL(flash_bwd_dq_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace upipe
