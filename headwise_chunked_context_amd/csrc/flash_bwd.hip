// Causal GQA flash-attention backward for one head chunk (gfx950, d = 128).
//
// Chain rule of exact softmax attention (FlashAttention, Builds-on list of
// "Untied Ulysses: Memory-Efficient Context Parallelism via Headwise
// Chunking"): with P recomputed from the saved log-sum-exp,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = dS K / sqrt(d),
//   dK = dS^T Q / sqrt(d),      D_i = dO_i . O_i.
//
// Two kernels, so that no gradient needs atomics:
//  * dkdv: a workgroup owns 128 keys of one KV head (8 waves, two per SIMD:
//    four 32-key blocks x two 32-query halves of every tile) and walks every
//    q head of that KV group in the chunk and every 64-query tile at or
//    below the diagonal, accumulating dK/dV of the group in fp32 registers;
//    the two halves' partial sums meet in LDS once, at the end.  Scores are
//    computed S = Q K^T so each lane owns ONE key: the S/dP accumulators
//    feed dV^T = dO^T P and dK^T = Q^T dS as MFMA B operands straight from
//    registers, with the dO^T / Q^T operands read from the row-major tiles
//    by the LDS transpose read.  Query tiles are walked from the END of the
//    sequence towards the diagonal (all of the group's heads per tile), so
//    workgroups that run together stream the same Q/dO tiles in the same
//    order and share them in L2.  The next tile arrives by asynchronous
//    global->LDS loads issued before the current tile's MFMAs.
//  * dq: a workgroup owns 128 queries of one q head (4 waves x 32 queries)
//    and walks the key tiles up to the diagonal like the forward kernel
//    (two workgroups per CU, single-buffered K/V tiles):
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

struct __attribute__((aligned(16))) DkdvSmem {
  uint16_t K[BNK * 128];        // the workgroup's K and V rows, loaded once
  uint16_t V[BNK * 128];
  uint16_t Q[2][BMQ * 128];     // double-buffered query tiles
  uint16_t dO[2][BMQ * 128];
  float lse2[2][BMQ];
  float dvec[2][BMQ];
};
// the epilogue reuses the same LDS for the cross-wave reduction
constexpr int kRedFloats = 4 * 64 * 64;
static_assert(sizeof(DkdvSmem) >= kRedFloats * sizeof(float), "reduction buffer");

// 8 waves: wave w owns keys k0 + 32*(w%4) .. +32 and, of every 64-query
// tile, the queries 32*(w/4) .. +32.  The two waves sharing a key block
// hold partial dK/dV that are summed through LDS once at the end.
__global__ __launch_bounds__(DKDV_THREADS) void flash_bwd_dkdv_kernel(BwdArgs a) {
  __shared__ DkdvSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kwave = wave & 3, qh = wave >> 2;
  const int g = lane >> 5, l32 = lane & 31;

  const int kv = blockIdx.x % a.nkv;
  const int ktile = blockIdx.x / a.nkv;
  const int64_t k0 = (int64_t)ktile * BNK;
  if (k0 >= a.L) return;
  const int64_t kw0 = k0 + 32 * kwave;
  const int64_t my_key = kw0 + l32;

  const uint16_t* kp = a.k + (int64_t)kv * a.Lp * 128;
  const uint16_t* vp = a.v + (int64_t)kv * a.Lp * 128;

  // K and V rows of the workgroup into LDS: B operands (column = key,
  // k = d) of S = Q K^T and dP = dO V^T, read back per step
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + DKDV_THREADS * i;
    *reinterpret_cast<u32x4*>(&sm.K[tile_off(c >> 4, c & 15)]) =
        *reinterpret_cast<const u32x4*>(kp + (k0 + (c >> 4)) * 128 + (c & 15) * 8);
    *reinterpret_cast<u32x4*>(&sm.V[tile_off(c >> 4, c & 15)]) =
        *reinterpret_cast<const u32x4*>(vp + (k0 + (c >> 4)) * 128 + (c & 15) * 8);
  }

  f32x16 acc_dk[4], acc_dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc_dk[i] = f32x16{};
    acc_dv[i] = f32x16{};
  }

  const float c = a.scale_log2;
  const int gkv = a.kv_head0 + kv;
  int j0 = gkv * a.group - a.q_head0;
  int j1 = j0 + a.group;
  if (j0 < 0) j0 = 0;
  if (j1 > a.nh) j1 = a.nh;
  const int qs_lo = (int)(k0 / BMQ);                 // first tile that sees these keys
  const int qs_hi = (int)((a.L + BMQ - 1) / BMQ);    // one past the last tile
  const int steps_per_head = qs_hi - qs_lo;
  const int nsteps = steps_per_head * (j1 - j0);

  // step s -> (query tile qs, head j): tiles walked from the end backwards,
  // all heads of the group per tile, so workgroups that run at the same
  // time read the same Q/dO tiles in the same order (shared in L2) until
  // each reaches its own diagonal
  const int nheads = j1 - j0;
  auto step_head = [&](int s) { return j0 + s % nheads; };
  auto step_tile = [&](int s) { return qs_hi - 1 - s / nheads; };

  // the tiles of step s arrive in buffer s % 2 by asynchronous DMA
  auto load_step = [&](int s, int buf) {
    const int j = step_head(s);
    const int64_t q0 = (int64_t)step_tile(s) * BMQ;
    tile_dma<BMQ, 8>(sm.Q[buf], a.q + ((int64_t)j * a.Lp + q0) * 128, wave, lane);
    tile_dma<BMQ, 8>(sm.dO[buf], a.dO + ((int64_t)j * a.Lp + q0) * 128, wave, lane);
    if (wave == 0) vec64_dma(sm.lse2[buf], a.lse2 + (int64_t)j * a.Lp + q0, lane);
    if (wave == 1) vec64_dma(sm.dvec[buf], a.dvec + (int64_t)j * a.Lp + q0, lane);
  };

  if (nsteps > 0) load_step(0, 0);
  lds_dma_wait();
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const int64_t q0 = (int64_t)step_tile(s) * BMQ;
    if (s + 1 < nsteps) load_step(s + 1, cur ^ 1);  // lands during this step's MFMAs

    const int64_t qw0 = q0 + 32 * qh;        // this wave's first query
    if (qw0 + 31 >= kw0) {                   // else every score is masked
      const bool need_mask = (qw0 < kw0 + 32) || (qw0 + 32 > a.L);
      const uint16_t* Qt = sm.Q[cur];
      const uint16_t* dOt = sm.dO[cur];
      // S = Q K^T and dP = dO V^T: element (query 32*qh + acc_row(r,g), key my_key)
      f32x16 sv = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sv = mfma32(tile_read_row(Qt, 32 * qh + l32, 2 * ks + g),
                    tile_read_row(sm.K, 32 * kwave + l32, 2 * ks + g), sv);
        dp = mfma32(tile_read_row(dOt, 32 * qh + l32, 2 * ks + g),
                    tile_read_row(sm.V, 32 * kwave + l32, 2 * ks + g), dp);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi = 32 * qh + r4 * 8 + g * 4;
        f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[cur][qi]);
        f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dvec[cur][qi]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r4 * 4 + i;
          float p = __builtin_amdgcn_exp2f(fmaf(sv[r], c, -l4[i]));
          if (need_mask) {
            const int64_t qrow = q0 + qi + i;
            if (my_key > qrow || qrow >= a.L) p = 0.f;
          }
          pv[r] = p;
          dsv[r] = p * (dp[r] - d4[i]);
        }
      }
      u32x4 pP[2], pS[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          pP[h][t] = pack_bf16x2(pv[8 * h + 2 * t], pv[8 * h + 2 * t + 1]);
          pS[h][t] = pack_bf16x2(dsv[8 * h + 2 * t], dsv[8 * h + 2 * t + 1]);
        }
      // dV^T += dO^T P, dK^T += Q^T dS over this wave's 32 queries; B slot t
      // of step h is query 32*qh + 16*h + 8*(t/4) + 4*g + t%4
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          acc_dv[db] = mfma32(tile_read_t(dOt, 32 * qh + 16 * h, db * 32, lane), pP[h], acc_dv[db]);
          acc_dk[db] = mfma32(tile_read_t(Qt, 32 * qh + 16 * h, db * 32, lane), pS[h], acc_dk[db]);
        }
    }
    lds_dma_wait();
    __syncthreads();
  }

  // ---- sum the two query halves' partial dK/dV (waves w and w+4)
  float* red = reinterpret_cast<float*>(&sm);
  float* mine = red + (kwave * 64) * 64 + lane;   // [kwave][reg][lane]
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? acc_dk : acc_dv;
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(db * 16 + r) * 64] = acc[db][r];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] += mine[(db * 16 + r) * 64];
    }
    __syncthreads();
  }
  if (qh == 1) return;

  // ---- epilogue: element (d = db*32 + acc_row(r,g), key my_key)
  if (my_key >= a.L) return;
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
        kk[i] = acc_dk[db][4 * j4 + i] * a.scale;
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
      *reinterpret_cast<u32x2*>(a.dk_out + my_key * a.out_ld + (int64_t)kv * 128 + d) = wk;
      *reinterpret_cast<u32x2*>(a.dv_out + my_key * a.out_ld + (int64_t)kv * 128 + d) = wv;
    }
}

// ------------------------------------------------------------------ dQ
constexpr int QBM = 128;       // queries per dq workgroup
constexpr int QBN = 64;        // keys per dq step

struct __attribute__((aligned(16))) DqSmem {
  uint16_t K[QBN * 128];
  uint16_t V[QBN * 128];
};

__global__ __launch_bounds__(256, 2) void flash_bwd_dq_kernel(BwdArgs a) {
  __shared__ DqSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  const int nqt = (int)(a.Lp / QBM);
  const int head = blockIdx.x % a.nh;
  const int qt = nqt - 1 - (int)(blockIdx.x / a.nh);
  const int64_t q0 = (int64_t)qt * QBM;
  if (q0 >= a.L) return;
  const int kvh = (a.q_head0 + head) / a.group - a.kv_head0;
  const uint16_t* qp = a.q + (int64_t)head * a.Lp * 128;
  const uint16_t* dop = a.dO + (int64_t)head * a.Lp * 128;
  const uint16_t* kp = a.k + (int64_t)kvh * a.Lp * 128;
  const uint16_t* vp = a.v + (int64_t)kvh * a.Lp * 128;

  const int64_t r0 = q0 + 32 * wave;
  const int64_t my_q = r0 + l32;

  // Q and dO of this lane's query as B operands (column = query, k = d)
  u32x4 qreg[8], doreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qreg[ks] = *reinterpret_cast<const u32x4*>(qp + my_q * 128 + ks * 16 + g * 8);
    doreg[ks] = *reinterpret_cast<const u32x4*>(dop + my_q * 128 + ks * 16 + g * 8);
  }
  const float lse2 = a.lse2[(int64_t)head * a.Lp + my_q];
  const float dval = a.dvec[(int64_t)head * a.Lp + my_q];

  const int64_t kv_end = (q0 + QBM < a.L) ? q0 + QBM : a.L;
  const int n_kt = (int)((kv_end + QBN - 1) / QBN);

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  const float c = a.scale_log2;

  // single-buffered K/V tiles: with two workgroups per CU the other
  // workgroup's MFMAs cover this one's loads
  for (int kt = 0; kt < n_kt; ++kt) {
    {
      TileCopy<QBN> pk, pv;
      pk.load(kp + (int64_t)kt * QBN * 128, tid);
      pv.load(vp + (int64_t)kt * QBN * 128, tid);
      __syncthreads();  // previous tile's reads are done
      pk.store(sm.K, tid);
      pv.store(sm.V, tid);
      __syncthreads();
    }
    const int64_t kstart = (int64_t)kt * QBN;
    if (kstart <= r0 + 31) {
      const bool need_mask = kstart + QBN - 1 > r0;
      // S^T = K Q^T, dP^T = V dO^T: element (key kb*32+acc_row(r,g), query my_q)
      f32x16 sv[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sv[kb] = f32x16{};
        dp[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          sv[kb] = mfma32(tile_read_row(sm.K, kb * 32 + l32, 2 * ks + g), qreg[ks], sv[kb]);
          dp[kb] = mfma32(tile_read_row(sm.V, kb * 32 + l32, 2 * ks + g), doreg[ks], dp[kb]);
        }
      }
      u32x4 pS[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], c, -lse2));
          if (need_mask && kstart + kb * 32 + acc_row(r, g) > my_q) p = 0.f;
          ds[r] = p * (dp[kb][r] - dval);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            pS[kb * 2 + h][t] = pack_bf16x2(ds[8 * h + 2 * t], ds[8 * h + 2 * t + 1]);
      }
      // dQ^T += K^T dS^T; B slot t of step st is key 16*st + 8*(t/4) + 4*g + t%4
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = mfma32(tile_read_t(sm.K, st * 16, db * 32, lane), pS[st], acc[db]);
      }
    }
  }

  if (my_q >= a.L) return;
  // element (d = db*32 + acc_row(r,g), query my_q): scale, inverse RoPE, bf16
  uint16_t* orow = a.dq_out + my_q * a.dq_ld + (int64_t)head * 128;
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

hipError_t launch_flash_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / BNK) * a.nkv));
  hipLaunchKernelGGL(flash_bwd_dkdv_kernel, grid, dim3(DKDV_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_flash_bwd_dq(const BwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / QBM) * a.nh));
  hipLaunchKernelGGL(flash_bwd_dq_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace upipe
