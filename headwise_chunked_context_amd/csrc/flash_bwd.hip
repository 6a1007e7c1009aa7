// Causal GQA flash-attention backward for one head chunk (gfx950, d = 128).
//
// Chain rule of exact softmax attention (FlashAttention, Builds-on list of
// "Untied Ulysses: Memory-Efficient Context Parallelism via Headwise
// Chunking"): with P recomputed from the saved log-sum-exp,
//   dV += P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = dS K / sqrt(d),
//   dK += dS^T Q / sqrt(d),     D_i = dO_i . O_i.
//
// Layout choices for CDNA4:
//  * a workgroup owns 128 keys of one KV head (4 waves x 32 keys) and walks
//    every q head of that KV group inside the chunk and every 64-query tile
//    at or below the diagonal, so dK/dV of the group accumulate in registers
//    (fp32) across the group's heads with no atomics;
//  * scores are computed S = Q K^T so each lane owns ONE key: the S/dP
//    accumulators feed dV^T = dO^T P and dK^T = Q^T dS as MFMA B operands
//    straight from registers, with dO^T/Q^T read from d-major copies;
//  * dQ = dS K is a cross-wave contraction over the workgroup's 128 keys:
//    dS goes through LDS once and each wave adds a 64x32 slab of dQ into an
//    fp32 accumulator with hardware float atomics;
//  * at the last chunk of a KV group the epilogue scales dK, applies the
//    inverse RoPE in registers and writes bf16; when a group spans several
//    chunks the partial dK/dV live in fp32 workspace between chunks.
#include "kernels.h"

namespace upipe {
namespace {

constexpr int BNK = 128;       // keys per workgroup
constexpr int BMQ = 64;        // queries per step
constexpr int RP = 128 + 8;    // row-major [*, 128] tile pitch (bf16)
constexpr int TP = BMQ + 8;    // d-major [128][64] tile pitch (bf16)
constexpr int SP = BNK + 8;    // dS [64][128] pitch (bf16)

struct __attribute__((aligned(16))) BwdSmem {
  uint16_t Q[BMQ * RP];
  uint16_t dO[BMQ * RP];
  uint16_t QT[128 * TP];
  uint16_t dOT[128 * TP];
  uint16_t dS[BMQ * SP];
  uint16_t KT[128 * SP];
  float lse2[BMQ];
  float dvec[BMQ];
};

__global__ __launch_bounds__(256) void flash_bwd_kernel(BwdArgs a) {
  __shared__ BwdSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  const int kv = blockIdx.x % a.nkv;
  const int ktile = blockIdx.x / a.nkv;
  const int64_t k0 = (int64_t)ktile * BNK;
  if (k0 >= a.L) return;
  const int64_t kw0 = k0 + 32 * wave;
  const int64_t my_key = kw0 + l32;

  const uint16_t* kp = a.k + (int64_t)kv * a.Lp * 128;
  const uint16_t* vp = a.v + (int64_t)kv * a.Lp * 128;
  const uint16_t* ktp = a.kt + (int64_t)kv * a.Lp * 128;

  // K and V of this lane's key as B operands (column = key, k = d)
  u32x4 kreg[8], vreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kreg[ks] = *reinterpret_cast<const u32x4*>(kp + my_key * 128 + ks * 16 + g * 8);
    vreg[ks] = *reinterpret_cast<const u32x4*>(vp + my_key * 128 + ks * 16 + g * 8);
  }
  // K^T of the workgroup's 128 keys for the dQ contraction
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int c = tid + 256 * i;
    int dd = c >> 4, cc = c & 15;
    *reinterpret_cast<u32x4*>(&sm.KT[dd * SP + cc * 8]) =
        *reinterpret_cast<const u32x4*>(ktp + (int64_t)dd * a.Lp + k0 + cc * 8);
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
  const int qs0 = (int)(k0 / BMQ);
  const int qs1 = (int)((a.L + BMQ - 1) / BMQ);

  for (int j = j0; j < j1; ++j) {
    const uint16_t* qp = a.q + (int64_t)j * a.Lp * 128;
    const uint16_t* qtp = a.qt + (int64_t)j * a.Lp * 128;
    const uint16_t* dop = a.dO + (int64_t)j * a.Lp * 128;
    const uint16_t* dotp = a.dOt + (int64_t)j * a.Lp * 128;
    const float* lsep = a.lse2 + (int64_t)j * a.Lp;
    const float* dvp = a.dvec + (int64_t)j * a.Lp;
    float* dqp = a.dq_acc + (int64_t)j * a.Lp * 128;

    for (int qs = qs0; qs < qs1; ++qs) {
      const int64_t q0 = (int64_t)qs * BMQ;
      __syncthreads();  // previous step's LDS reads are done
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int c2 = tid + 256 * i;
        int row = c2 >> 4, cc = c2 & 15;
        *reinterpret_cast<u32x4*>(&sm.Q[row * RP + cc * 8]) =
            *reinterpret_cast<const u32x4*>(qp + (q0 + row) * 128 + cc * 8);
        *reinterpret_cast<u32x4*>(&sm.dO[row * RP + cc * 8]) =
            *reinterpret_cast<const u32x4*>(dop + (q0 + row) * 128 + cc * 8);
        int dd = c2 >> 3, tc = c2 & 7;
        *reinterpret_cast<u32x4*>(&sm.QT[dd * TP + tc * 8]) =
            *reinterpret_cast<const u32x4*>(qtp + (int64_t)dd * a.Lp + q0 + tc * 8);
        *reinterpret_cast<u32x4*>(&sm.dOT[dd * TP + tc * 8]) =
            *reinterpret_cast<const u32x4*>(dotp + (int64_t)dd * a.Lp + q0 + tc * 8);
      }
      if (tid < BMQ) sm.lse2[tid] = lsep[q0 + tid];
      else if (tid < 2 * BMQ) sm.dvec[tid - BMQ] = dvp[q0 + tid - BMQ];
      __syncthreads();

      const bool need_mask = (q0 < k0 + BNK) || (q0 + BMQ > a.L);
      // S = Q K^T and dP = dO V^T: element (query qb*32+acc_row(r,g), key my_key)
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = f32x16{};
        dp[qb] = f32x16{};
        const uint16_t* qb_base = &sm.Q[(qb * 32 + l32) * RP + g * 8];
        const uint16_t* db_base = &sm.dO[(qb * 32 + l32) * RP + g * 8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          s[qb] = mfma32(*reinterpret_cast<const u32x4*>(qb_base + ks * 16), kreg[ks], s[qb]);
          dp[qb] = mfma32(*reinterpret_cast<const u32x4*>(db_base + ks * 16), vreg[ks], dp[qb]);
        }
      }
      u32x4 pP[4], pS[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float pv[16], dsv[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int qi = qb * 32 + r4 * 8 + g * 4;
          f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[qi]);
          f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dvec[qi]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = r4 * 4 + i;
            float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -l4[i]));
            if (need_mask) {
              const int64_t qrow = q0 + qi + i;
              if (my_key > qrow || qrow >= a.L) p = 0.f;
            }
            pv[r] = p;
            dsv[r] = p * (dp[qb][r] - d4[i]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            pP[qb * 2 + h][t] = pack_bf16x2(pv[8 * h + 2 * t], pv[8 * h + 2 * t + 1]);
            pS[qb * 2 + h][t] = pack_bf16x2(dsv[8 * h + 2 * t], dsv[8 * h + 2 * t + 1]);
          }
        }
        // dS to LDS, query-major with keys contiguous, for the dQ contraction
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          uint32_t w = pS[qb * 2 + (r >> 3)][(r & 7) >> 1];
          uint16_t hbits = (r & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
          sm.dS[(qb * 32 + acc_row(r, g)) * SP + 32 * wave + l32] = hbits;
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS; B slot t of step st is query
      // 16*st + 8*(t/4) + 4*g + t%4
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const uint16_t* ob = &sm.dOT[(db * 32 + l32) * TP + st * 16 + g * 4];
          const uint16_t* qtb = &sm.QT[(db * 32 + l32) * TP + st * 16 + g * 4];
          u32x2 olo = *reinterpret_cast<const u32x2*>(ob);
          u32x2 ohi = *reinterpret_cast<const u32x2*>(ob + 8);
          u32x2 qlo = *reinterpret_cast<const u32x2*>(qtb);
          u32x2 qhi = *reinterpret_cast<const u32x2*>(qtb + 8);
          acc_dv[db] = mfma32(u32x4{olo[0], olo[1], ohi[0], ohi[1]}, pP[st], acc_dv[db]);
          acc_dk[db] = mfma32(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, pS[st], acc_dk[db]);
        }
      }
      __syncthreads();  // dS complete
      // dQ[:, 32*wave .. +32] += dS (64 x 128 keys) K (128 keys x 32 d)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 dq = f32x16{};
        const uint16_t* sb = &sm.dS[(qb * 32 + l32) * SP + g * 8];
        const uint16_t* kb = &sm.KT[(32 * wave + l32) * SP + g * 8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          dq = mfma32(*reinterpret_cast<const u32x4*>(sb + ks * 16),
                      *reinterpret_cast<const u32x4*>(kb + ks * 16), dq);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t qrow = q0 + qb * 32 + acc_row(r, g);
          atomicAdd(dqp + qrow * 128 + 32 * wave + l32, dq[r]);
        }
      }
    }
  }

  // ---- epilogue: element (d = db*32 + acc_row(r,g), key my_key)
  if (my_key >= a.L) return;
  float* dka = a.dk_acc ? a.dk_acc + ((int64_t)kv * a.Lp + my_key) * 128 : nullptr;
  float* dva = a.dv_acc ? a.dv_acc + ((int64_t)kv * a.Lp + my_key) * 128 : nullptr;
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

}  // namespace

hipError_t launch_flash_bwd(const BwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / BNK) * a.nkv));
  hipLaunchKernelGGL(flash_bwd_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace upipe
