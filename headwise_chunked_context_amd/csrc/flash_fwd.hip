// Causal GQA flash-attention forward for one head chunk (gfx950, d = 128).
//
// Exact softmax attention evaluated tile by tile with a running maximum and
// sum (FlashAttention, cited in the Builds-on list of "Untied Ulysses:
// Memory-Efficient Context Parallelism via Headwise Chunking"); the chunk
// loop that calls it is the headwise schedule of "Untied Ulysses Pushes
// Llama-3-8B Training to 5 Million Tokens" (Untied Ulysses section).
//
// Layout choices for CDNA4:
//  * a workgroup is 4 waves x 32 query rows = 128 queries of one q head;
//    key/value tiles of 64 keys are staged in LDS (double-buffered, loads
//    for tile t+1 issued before the MFMAs of tile t); registers are capped
//    so that two workgroups share a CU (2 waves per SIMD), letting one
//    wave's softmax run while the other's MFMAs do;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns ONE query and 16 keys of
//    a 32-key block, so the row max/sum need one cross-half exchange
//    (lane ^ 32) and the output rescale is a per-lane scalar;
//  * the P^T accumulator registers feed the O^T = V^T P^T MFMA directly as
//    its B operand (no LDS round trip); the V^T operand is read from the
//    row-major V tile with the LDS transpose read (ds_read_b64_tr_b16), in
//    the key order of the accumulator layout;
//  * K and V tiles use the XOR-swizzled 256-byte-row layout (no padding, no
//    bank conflicts for either read pattern);
//  * P and V enter O = P V as fp16 (v_mfma_f32_32x32x16_f16, same rate as
//    bf16): P lies in [0, 1] and fp16's 10-bit mantissa keeps the forward
//    output inside its error budget where bf16's 7 bits do not;
//  * the softmax runs in base 2 with the 1/sqrt(d) scale folded into one FMA;
//    the running maximum is raised lazily (only when a score exceeds it by
//    more than 2^8), which removes the per-tile rescale of O;
//  * workgroups are issued heaviest (last query tile) first, and consecutive
//    workgroups take different heads of the chunk so the heads sharing a KV
//    group spread over the XCDs while each XCD streams one head's K/V.
#include "kernels.h"

namespace upipe {
namespace {

constexpr int BM = 128;       // queries per workgroup
constexpr int BN = 64;        // keys per step

__global__ __launch_bounds__(256, 2) void flash_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * 128];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BN * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;

  const int nqt = (int)(a.Lp / BM);
  const int head = blockIdx.x % a.nh;
  const int qt = nqt - 1 - (int)(blockIdx.x / a.nh);
  const int64_t q0 = (int64_t)qt * BM;
  if (q0 >= a.L) return;  // whole tile is padding
  const int kvh = (a.q_head0 + head) / a.group - a.kv_head0;
  const uint16_t* qp = a.q + (int64_t)head * a.Lp * 128;
  const uint16_t* kp = a.k + (int64_t)kvh * a.Lp * 128;
  const uint16_t* vp = a.v + (int64_t)kvh * a.Lp * 128;

  const int64_t r0 = q0 + 32 * wave;  // first query row of this wave
  const int64_t my_q = r0 + l32;

  // Q as the B operand of S^T = K Q^T: lane holds query my_q, d = 16ks+8g..+7
  u32x4 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qreg[ks] = *reinterpret_cast<const u32x4*>(qp + my_q * 128 + ks * 16 + g * 8);

  const int64_t kv_end = (q0 + BM < a.L) ? q0 + BM : a.L;
  const int n_kt = (int)((kv_end + BN - 1) / BN);

  TileCopy<BN> pk, pv;
  auto load_kv = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BN;
    pk.load(kp + k0 * 128, tid);
    pv.load(vp + k0 * 128, tid);
  };
  auto store_kv = [&](int buf) {
    pk.store(Ks[buf], tid);
    pv.store(Vs[buf], tid);
  };

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = a.scale_log2;

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < n_kt) load_kv(kt + 1);
    const int64_t kstart = (int64_t)kt * BN;
    if (kstart <= r0 + 31) {  // otherwise every key of the tile is in this wave's future
      const bool need_mask = kstart + BN - 1 > r0;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
          s[kb] = mfma32(tile_read_row(Ks[cur], kb * 32 + l32, 2 * ks + g), qreg[ks], s[kb]);
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            int64_t key = kstart + kb * 32 + acc_row(r, g);
            if (key > my_q) s[kb][r] = -__builtin_inff();
          }
      }
      // running maximum, raised lazily: only when some row's new score
      // exceeds it by more than 2^8 in the exponent (wave-uniform), so the
      // 64-register rescale of O runs a few times per row instead of every
      // tile; in between P <= 256, well inside fp16 and fp32
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[0][r], s[0][r + 1]));
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[1][r], s[1][r + 1]));
      mx = half_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx * c > fmaf(m_run, c, 8.f))) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc_o[db] *= alpha;
        m_run = m_new;
      }
      const float mc = m_run * c;
      float rsum = 0.f;
      u32x4 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mc));
          rsum += p[r];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          pb[kb * 2 + h][0] = pack_f16x2(p[8 * h + 0], p[8 * h + 1]);
          pb[kb * 2 + h][1] = pack_f16x2(p[8 * h + 2], p[8 * h + 3]);
          pb[kb * 2 + h][2] = pack_f16x2(p[8 * h + 4], p[8 * h + 5]);
          pb[kb * 2 + h][3] = pack_f16x2(p[8 * h + 6], p[8 * h + 7]);
        }
      }
      l_run += rsum;
      // O^T += V^T P^T; B slot t of step st is key 16*st + 8*(t/4) + 4*g + t%4
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc_o[db] = mfma32_f16(tile_read_t(Vs[cur], st * 16, db * 32, lane), pb[st], acc_o[db]);
      }
    }
    if (kt + 1 < n_kt) store_kv(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = half_sum(l_run);
  if (my_q >= a.L) return;
  const float inv = 1.f / l_tot;
  const int hg = a.q_head0 + head;
  uint16_t* orow = a.o + my_q * a.o_ld + (int64_t)hg * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int d = db * 32 + j * 8 + g * 4;
      u32x2 w = {pack_bf16x2(acc_o[db][4 * j] * inv, acc_o[db][4 * j + 1] * inv),
                 pack_bf16x2(acc_o[db][4 * j + 2] * inv, acc_o[db][4 * j + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d) = w;
    }
  if (g == 0) a.lse[(int64_t)hg * a.L + my_q] = (m_run * c + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_flash_fwd(const FwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / BM) * a.nh));
  hipLaunchKernelGGL(flash_fwd_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace upipe
