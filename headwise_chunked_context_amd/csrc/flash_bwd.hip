// Causal GQA flash-attention backward for one head chunk (gfx950, d = 128).
//
// Chain rule of exact softmax attention (FlashAttention, Builds-on list of
// "Untied Ulysses: Memory-Efficient Context Parallelism via Headwise
// Chunking"): with P recomputed from the saved log-sum-exp,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = dS K / sqrt(d),
//   dK = dS^T Q / sqrt(d),      D_i = dO_i . O_i
// (q arrives multiplied by log2(e)/sqrt(d), so the score MFMAs give base-2
// exponents, and dK divides that factor out again).
//
// Two kernels, so that no gradient needs atomics:
//  * dkdv: a workgroup owns 128 keys of one KV head (8 waves, two per SIMD:
//    four 32-key blocks x two 32-query halves of every tile) and walks every
//    q head of that KV group in the chunk and every 64-query tile at or
//    below the diagonal, accumulating dK/dV of the group in fp32 registers;
//    each wave holds its 32 K and V rows in registers for the whole walk;
//    the two halves' partial sums meet in LDS once, at the end.  Scores are
//    computed S = Q K^T so each lane owns ONE key: the S/dP accumulators
//    feed dV^T = dO^T P and dK^T = Q^T dS as MFMA B operands straight from
//    registers, with the dO^T / Q^T operands read from the row-major tiles
//    by the LDS transpose read.  Query tiles are walked from the END of the
//    sequence towards the diagonal (all of the group's heads per tile), so
//    workgroups that run together stream the same Q/dO tiles in the same
//    order and share them in L2.  The next tile arrives by asynchronous
//    global->LDS loads issued before the current tile's MFMAs.
//  * dq (flash_bwd_dq.hip): a workgroup owns 128 queries of one q head
//    (4 waves x 32 queries) and walks the key tiles up to the diagonal like
//    the forward kernel (two workgroups per CU, double-buffered K/V tiles):
//    S^T = K Q^T and dP^T = V dO^T give each lane ONE query (its LSE and D
//    are per-lane scalars), dS^T feeds dQ^T = K^T dS^T as a B operand from
//    registers and K^T is the transpose read of the same K tile.  The
//    epilogue scales dQ, applies the inverse RoPE in registers and writes
//    bf16.
// All tiles are [rows][128] in the XOR-swizzled layout of common.h.
// dQ costs a second evaluation of S and dP (+4 d flops per score pair over
// the 10 of one fused kernel) in exchange for no fp32 read-modify-write
// traffic to memory.
#include "kernels.h"

namespace upipe {
namespace {

constexpr int BNK = 128;       // keys per dkdv workgroup
constexpr int BMQ = 64;        // queries per dkdv step
constexpr int DKDV_THREADS = 512;

// The query tiles are double-buffered in distinct fields (the step loop is
// unrolled by two), so every LDS address is a per-lane base plus an
// immediate and reads of one buffer are visibly independent of the copy in
// flight into the other.  The per-step buffers come first: LDS immediates
// reach 64 KB.  The workgroup's K and V rows, loaded once, come last.
struct __attribute__((aligned(16))) DkdvSmem {
  float L0[BMQ], L1[BMQ];           // -LSE of the tile's rows (base 2)
  float E0[BMQ], E1[BMQ];           // -D = -(dO . O) of the tile's rows
  uint16_t Q0[BMQ * 128], Q1[BMQ * 128];
  uint16_t O0[BMQ * 128], O1[BMQ * 128];  // dO tiles
  uint16_t K[BNK * 128];
  uint16_t V[BNK * 128];
};

// 8 waves: wave w owns keys k0 + 32*(w%4) .. +32 and, of every 64-query
// tile, the queries 32*(w/4) .. +32.  The two waves sharing a key block
// hold partial dK/dV that are summed through LDS once at the end.
__global__ __launch_bounds__(DKDV_THREADS) void flash_bwd_dkdv_kernel(BwdArgs a) {
  __shared__ DkdvSmem sm;
  float* const L0 = sm.L0;
  float* const L1 = sm.L1;
  float* const E0 = sm.E0;
  float* const E1 = sm.E1;
  uint16_t* const Q0 = sm.Q0;
  uint16_t* const Q1 = sm.Q1;
  uint16_t* const O0 = sm.O0;
  uint16_t* const O1 = sm.O1;
  uint16_t* const Ks = sm.K;
  uint16_t* const Vs = sm.V;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kwave = wave & 3, qh = wave >> 2;
  const int g = lane >> 5, l32 = lane & 31;

  const int kv = blockIdx.x % a.nkv;
  const int ktile = blockIdx.x / a.nkv;
  const int k0 = ktile * BNK;
  if (k0 >= a.L) return;
  const int L = (int)a.L;
  const int kw0 = k0 + 32 * kwave;
  const int my_key = kw0 + l32;

  const uint16_t* kp = a.k + ((int64_t)kv * a.Lp + k0) * 128;
  const uint16_t* vp = a.v + ((int64_t)kv * a.Lp + k0) * 128;

  // K and V rows of the workgroup -> LDS (swizzled), 4 KB per wave each
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = wave * 4 + i;
    const int row = 4 * n + (lane >> 4);
    const uint32_t off = (uint32_t)(row * 128 + (((lane & 15) ^ swz(row)) << 3));
    dma16_untracked(kp + off, lds_addr(Ks + n * 512));
    dma16_untracked(vp + off, lds_addr(Vs + n * 512));
  }

  // per-lane element offsets.  Each is held for k step / column block 0
  // only: the swizzle XORs chunk c of a row with swz(row) < 16, so the
  // other steps' offsets are that one XOR a constant, rebuilt per step with
  // one v_xor each; holding all of them would take 14 more registers, which
  // the K rows need (below).
  //  row-per-lane operands: Q/dO rows 32*qh + l32, chunk 2ks + g: ks is
  //  chunk bits 1-3, element-offset bits 4-6, so offset(ks) = offq0 ^ (ks << 4);
  //  the K/V rows 32*kwave + l32 sit a uniform distance dko further (same
  //  swizzle)
  const int offq0 = tile_off(32 * qh + l32, g);
  const int dko_init = (kwave - qh) * 32 * 128;
  //  transposed operands dO^T / Q^T (see tile_read_t): column block db,
  //  rows 32*qh + 4g + (lane%16)/4 and +8; db is chunk bits 2-3, element-
  //  offset bits 5-6, so offset(db) = offt0 ^ (db << 5); 16h more rows are
  //  an immediate
  int offt0[2];
  {
    const int sl = lane & 15, grp2 = (lane >> 4) & 1;
    const int r0 = 32 * qh + 4 * g + (sl >> 2);
    const int col = 16 * grp2 + 4 * (sl & 3);
    offt0[0] = tile_off(r0, col >> 3) + (col & 7);
    offt0[1] = tile_off(r0 + 8, col >> 3) + (col & 7);
  }
  //  per-row scalars of the lane's queries 32*qh + 8*r4 + 4g + i
  const int offl = 32 * qh + 4 * g;
  //  query tile copy: wave w moves rows 8w .. 8w+7 of the Q and dO tiles
  uint32_t qdma[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * wave + 4 * i + (lane >> 4);
    qdma[i] = (uint32_t)(row * 128 + (((lane & 15) ^ swz(row)) << 3));
  }

  f32x16 acc_dk[4], acc_dv[4];
  u32x4 vreg[8], kreg[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc_dk[i] = f32x16{};
    acc_dv[i] = f32x16{};
  }

  const int gkv = a.kv_head0 + kv;
  int j0 = gkv * a.group - a.q_head0;
  int j1 = j0 + a.group;
  if (j0 < 0) j0 = 0;
  if (j1 > a.nh) j1 = a.nh;
  const int qs_lo = k0 / BMQ;                 // first tile that sees these keys
  const int qs_hi = (L + BMQ - 1) / BMQ;      // one past the last tile
  const int nsteps = (qs_hi - qs_lo) * (j1 - j0);

  // Steps walk the query tiles from the end of the sequence backwards, all
  // heads of the group per tile, so workgroups that run at the same time
  // read the same Q/dO tiles in the same order (shared in L2) until each
  // reaches its own diagonal.  (j, qt) is the step being loaded.
  int ld_j = j0, ld_qt = qs_hi - 1;
  auto load_next = [&](uint16_t* Qd, uint16_t* Od, float* Ld, float* Ed) {
    const int64_t base = (int64_t)ld_j * a.Lp + ld_qt * BMQ;
    const uint16_t* qsrc = a.q + base * 128;
    const uint16_t* osrc = a.dO + base * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      dma16_untracked(qsrc + qdma[i], lds_addr(Qd + (wave * 2 + i) * 512));
      dma16_untracked(osrc + qdma[i], lds_addr(Od + (wave * 2 + i) * 512));
    }
    if (wave == 0) dma4_untracked(a.lse2 + base + lane, lds_addr(Ld));
    if (wave == 1) dma4_untracked(a.dvec + base + lane, lds_addr(Ed));
    if (++ld_j == j1) {
      ld_j = j0;
      --ld_qt;
    }
  };

  auto step = [&](int qt, const uint16_t* Qt, const uint16_t* Ot, const float* Lt, const float* Et) {
    const int q0 = qt * BMQ;
    const int qw0 = q0 + 32 * qh;            // this wave's first query
    if (qw0 + 31 < kw0) return;              // every score is masked
    const bool need_mask = (qw0 < kw0 + 32) || (qw0 + 32 > L);
    // S = Q K^T and dP - D = dO V^T - D: element (query 32*qh +
    // acc_row(r,g), key my_key), q carrying the scale so that S is in base-2
    // units; the dP accumulator starts from the tile's -D rows, so dS below
    // is one multiply per element.  (Starting S from the -LSE rows as well
    // saves the add below but delays the first MFMA behind four more reads:
    // measured 1.2% slower, and 0.8% with K in registers.)  The empty asm
    // keeps the compiler from hoisting the eight XORed offsets out of the
    // loop into registers.
    int oq = offq0;
    asm volatile("" : "+v"(oq));
    f32x16 sv = f32x16{}, dp;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 e4 = *reinterpret_cast<const f32x4*>(Et + offl + 8 * r4);
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[r4 * 4 + i] = e4[i];
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sv = mfma32(*reinterpret_cast<const u32x4*>(Qt + (oq ^ (ks << 4))), kreg[ks], sv);
      dp = mfma32(*reinterpret_cast<const u32x4*>(Ot + (oq ^ (ks << 4))), vreg[ks], dp);
    }
    // the -D rows and two k steps (four reads) ahead, then two per two
    // MFMAs (three or four steps ahead no longer fit the registers)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (need_mask) {  // key after the query, or a padding query row
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + 32 * qh + acc_row(r, g);
        if (my_key > qrow || qrow >= L) sv[r] = -__builtin_inff();
      }
    }
    u32x4 pP[2], pS[2];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 nl4 = *reinterpret_cast<const f32x4*>(Lt + offl + 8 * r4);  // -LSE
      float pv[4], dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r4 * 4 + i;
        pv[i] = __builtin_amdgcn_exp2f(sv[r] + nl4[i]);
        dsv[i] = pv[i] * dp[r];
      }
      // registers r4*4 .. +3 are B slots 4*(r4%2) .. +3 of step r4/2
      pP[r4 >> 1][2 * (r4 & 1)] = pack_bf16x2(pv[0], pv[1]);
      pP[r4 >> 1][2 * (r4 & 1) + 1] = pack_bf16x2(pv[2], pv[3]);
      pS[r4 >> 1][2 * (r4 & 1)] = pack_bf16x2(dsv[0], dsv[1]);
      pS[r4 >> 1][2 * (r4 & 1) + 1] = pack_bf16x2(dsv[2], dsv[3]);
    }
    // the dV/dK MFMAs issue at raised wave priority (the other wave of the
    // SIMD then gets the VALU slots for its P/dS work)
    __builtin_amdgcn_s_setprio(1);
    int ot0 = offt0[0], ot1 = offt0[1];
    asm volatile("" : "+v"(ot0), "+v"(ot1));
    // dV^T += dO^T P, dK^T += Q^T dS over this wave's 32 queries; B slot t
    // of step h is query 32*qh + 16*h + 8*(t/4) + 4*g + t%4
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const u32x2 o_lo = lds_read_tr16(Ot + (ot0 ^ (db << 5)) + h * 2048);
        const u32x2 o_hi = lds_read_tr16(Ot + (ot1 ^ (db << 5)) + h * 2048);
        acc_dv[db] = mfma32(u32x4{o_lo[0], o_lo[1], o_hi[0], o_hi[1]}, pP[h], acc_dv[db]);
        const u32x2 q_lo = lds_read_tr16(Qt + (ot0 ^ (db << 5)) + h * 2048);
        const u32x2 q_hi = lds_read_tr16(Qt + (ot1 ^ (db << 5)) + h * 2048);
        acc_dk[db] = mfma32(u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}, pS[h], acc_dk[db]);
      }
    // transpose reads kept eight (four MFMAs) ahead, then two per MFMA:
    // measured 1% faster than the compiler's order (LLVM's generic LDS/MFMA
    // interleave here was 4% slower)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  if (nsteps > 0) load_next(Q0, O0, L0, E0);
  lds_dma_wait();
  __syncthreads();
  // the wave's 32 K and 32 V rows, the B operands of S = Q K^T and
  // dP = dO V^T, held in registers for the whole loop (64 VGPRs): each step
  // then reads only Q, dO and their transposes from LDS (32 of 40 KB per
  // wave with K read from LDS: measured 1.6-1.8% faster per launch)
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint32_t a = lds_addr(Ks) + 2 * (dko_init + (offq0 ^ (ks << 4)));
    kreg[ks] = lds_load16(a, 0);
    vreg[ks] = lds_load16(a, BNK * 128 * 2);
  }
  int qt = qs_hi - 1, hj = j0;  // step being computed: tile qt, head hj
  auto advance = [&]() {
    if (++hj == j1) {
      hj = j0;
      --qt;
    }
  };
  for (int s = 0; s < nsteps; s += 2) {
    if (s + 1 < nsteps) load_next(Q1, O1, L1, E1);  // lands during this step's MFMAs
    step(qt, Q0, O0, L0, E0);
    advance();
    lds_dma_wait();
    __syncthreads();
    if (s + 1 >= nsteps) break;
    if (s + 2 < nsteps) load_next(Q0, O0, L0, E0);
    step(qt, Q1, O1, L1, E1);
    advance();
    lds_dma_wait();
    __syncthreads();
  }
  (void)hj;

  // ---- sum the two query halves' partial dK/dV (waves w and w+4), half
  // of one accumulator set per pass through the K rows' LDS
  float* red = reinterpret_cast<float*>(sm.K);
  float* mine = red + (kwave * 32) * 64 + lane;   // [kwave][reg][lane]
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    f32x16* acc = (pass < 2 ? acc_dk : acc_dv) + 2 * (pass & 1);
    __syncthreads();
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64] = acc[db][r];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] += mine[(db * 16 + r) * 64];
    }
  }
  if (qh == 1) return;

  // ---- epilogue: element (d = db*32 + acc_row(r,g), key my_key)
  if (my_key >= L) return;
  float* dka = a.dk_acc + ((int64_t)kv * a.Lp + my_key) * 128;
  float* dva = a.dv_acc + ((int64_t)kv * a.Lp + my_key) * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int d = db * 32 + j4 * 8 + g * 4;
      f32x4 kk, vv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kk[i] = acc_dk[db][4 * j4 + i] * a.dk_scale;
        vv[i] = acc_dv[db][4 * j4 + i];
      }
      if (!a.kv_first) {
        kk += *reinterpret_cast<const f32x4*>(dka + d);
        vv += *reinterpret_cast<const f32x4*>(dva + d);
      }
      if (!a.kv_last) {
        *reinterpret_cast<f32x4*>(dka + d) = kk;
        *reinterpret_cast<f32x4*>(dva + d) = vv;
        continue;
      }
      // inverse RoPE on pairs (d, d+1) and (d+2, d+3)
      f32x4 kr;
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        float cs, sn;
        rope_cos_sin(a.rope, my_key, (d >> 1) + pi, cs, sn);
        float e = kk[2 * pi], o = kk[2 * pi + 1];
        kr[2 * pi] = e * cs + o * sn;
        kr[2 * pi + 1] = -e * sn + o * cs;
      }
      u32x2 wk = {pack_bf16x2(kr[0], kr[1]), pack_bf16x2(kr[2], kr[3])};
      u32x2 wv = {pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
      *reinterpret_cast<u32x2*>(a.dk_out + (int64_t)my_key * a.out_ld + (int64_t)kv * 128 + d) = wk;
      *reinterpret_cast<u32x2*>(a.dv_out + (int64_t)my_key * a.out_ld + (int64_t)kv * 128 + d) = wv;
    }
}

}  // namespace

hipError_t launch_flash_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / BNK) * a.nkv));
  hipLaunchKernelGGL(flash_bwd_dkdv_kernel, grid, dim3(DKDV_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace upipe
