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
//    key tiles of 64 keys are staged in LDS, double-buffered, by
//    asynchronous global->LDS loads issued one tile ahead; registers are
//    capped so that two workgroups share a CU (2 waves per SIMD), letting
//    one wave's softmax run while the other's MFMAs do;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then owns ONE query and 16 keys of
//    a 32-key block, so the row max/sum need one cross-half exchange
//    (lane ^ 32) and the output rescale is a per-lane scalar;
//  * the P^T accumulator registers feed the O^T = V^T P^T MFMA directly as
//    its B operand (no LDS round trip).  The V^T operand is a row-per-lane
//    16-byte read because the prep pass stores V already transposed, in
//    64-key tiles whose keys follow the accumulator's key order (see
//    prep.hip), as the exact image the LDS tile takes;
//  * K tiles use the XOR-swizzled 256-byte-row layout, V^T tiles a 128-byte
//    row variant: no padding, no bank conflicts;
//  * P and V enter O = P V as fp16 (v_mfma_f32_32x32x16_f16, same rate as
//    bf16): P lies in [0, 2^8] and fp16's 10-bit mantissa keeps the forward
//    output inside its error budget where bf16's 7 bits do not.  The row
//    sum is taken from the same fp16 P by v_dot2_f32_f16, so numerator and
//    denominator see identical probabilities;
//  * the softmax runs in base 2: q arrives multiplied by log2(e)/sqrt(d), so
//    the score MFMAs produce base-2 exponents directly, and their chains
//    start from -(running maximum), so they produce the exponents of P
//    themselves; the running maximum is raised lazily (only when a score
//    exceeds it by more than 2^8), which removes the per-tile rescale of O;
//  * the two LDS buffers are distinct arrays and the key loop is unrolled
//    by two, so every LDS address is a per-lane base plus an immediate and
//    the compiler can see that reads of one buffer never alias the copy in
//    flight into the other;
//  * workgroups are issued heaviest (last query tile) first, and consecutive
//    workgroups take different heads of the chunk so the heads sharing a KV
//    group spread over the XCDs while each XCD streams one head's K/V.
#include "kernels.h"

namespace upipe {
namespace {

constexpr int BM = 128;       // queries per workgroup
constexpr int BN = 64;        // keys per step

// max(x, x of lane ^ 32) by the lane-swap VALU instruction (no LDS round
// trip): one copy of x gets its upper half from the other's lower half and
// vice versa, so the two results hold the two halves in either order
__device__ __forceinline__ float half_max_swap(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// FROM_LSE: the backward's recompute of O from the forward's saved LSE.  The
// probabilities P = exp2(s - LSE2) are final at once, so the running
// maximum, its rescale and the row sum drop out and O needs no division;
// nothing but O is written.
template <bool FROM_LSE>
__global__ __launch_bounds__(256, 2) void flash_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t K0[BN * 128];
  __shared__ __attribute__((aligned(16))) uint16_t K1[BN * 128];
  __shared__ __attribute__((aligned(16))) uint16_t V0[128 * BN];
  __shared__ __attribute__((aligned(16))) uint16_t V1[128 * BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;

  const int nqt = (int)(a.Lp / BM);
  const int head = blockIdx.x % a.nh;
  const int qt = nqt - 1 - (int)(blockIdx.x / a.nh);
  const int q0 = qt * BM;
  if (q0 >= a.L) return;  // whole tile is padding
  const int L = (int)a.L;
  const int kvh = (a.q_head0 + head) / a.group - a.kv_head0;
  const uint16_t* qp = a.q + (int64_t)head * a.Lp * 128;
  const uint16_t* kp = a.k + (int64_t)kvh * a.Lp * 128;
  const uint16_t* vp = a.v + (int64_t)kvh * a.Lp * 128;

  const int r0 = q0 + 32 * wave;  // first query row of this wave
  const int my_q = r0 + l32;

  // Q as the B operand of S^T = K Q^T: lane holds query my_q, d = 16ks+8g..+7
  u32x4 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qreg[ks] = *reinterpret_cast<const u32x4*>(qp + (int64_t)my_q * 128 + ks * 16 + g * 8);

  const int kv_end = (q0 + BM < L) ? q0 + BM : L;
  const int n_kt = (kv_end + BN - 1) / BN;

  // per-lane element offsets, fixed for the whole loop (the swizzles XOR a
  // row's chunk index with a per-row constant, so step ks (st) sits at the
  // step-0 offset XOR ks << 4 (st << 4))
  //  K reads (A operand of S^T): row kb*32 + l32, chunk 2ks + g
  const int koff0 = tile_off(l32, g);
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = koff0 ^ (ks << 4);
  //  V^T reads (A operand of O^T): row db*32 + l32, chunk 2st + g
  const int voff0 = l32 * 64 + ((g ^ ((l32 >> 1) & 7)) << 3);
  int voff[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) voff[st] = voff0 ^ (st << 4);
  //  K tile copy: wave w moves rows 16w .. 16w+15, four 1 KB pieces
  uint32_t kdma[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + (lane >> 4);
    kdma[i] = (uint32_t)(row * 128 + (((lane & 15) ^ swz(row)) << 3));
  }

  // K tile kt -> LDS (swizzled on the way); V^T tile kt -> LDS as is
  auto dma_k = [&](int kt, uint16_t* Kd) {
    const uint16_t* src = kp + (int64_t)kt * BN * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_untracked(src + kdma[i], lds_addr(Kd + (wave * 4 + i) * 512));
  };
  auto dma_v = [&](int kt, uint16_t* Vd) {
    const uint16_t* src = vp + (int64_t)kt * BN * 128 + wave * 2048 + lane * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_untracked(src + i * 512, lds_addr(Vd + (wave * 4 + i) * 512));
  };

  f32x16 acc_o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc_o[i] = f32x16{};
  // the running maximum in base-2 units, as the scores; from the saved LSE
  // (base 2) when it is given (padding rows: 0, their O is not stored)
  float m_run = -__builtin_inff();
  if (FROM_LSE) m_run = my_q < L ? a.lse_in[(int64_t)(a.q_head0 + head) * L + my_q] * kLog2e : 0.f;
  // -m_run in all 16 registers: the starting value (C operand) of the next
  // tile's score chains, so the scores come out as s - m_run and the
  // exponentials need no subtraction; sref is the maximum the held scores
  // are relative to (tile 0 is computed from 0 before m_run exists)
  f32x16 nm16;
#pragma unroll
  for (int r = 0; r < 16; ++r) nm16[r] = -m_run;
  float sref = FROM_LSE ? m_run : 0.f;
  float l_run = 0.f;
  const f16x2 ones = {(_Float16)1.f, (_Float16)1.f};

  // S^T of one key tile: element (key kb*32 + acc_row(r,g), query my_q)
  auto scores = [&](const uint16_t* Kc, f32x16* s, bool from_zero) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (from_zero)
        s[kb] = f32x16{};
      else
        s[kb] = nm16;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[kb] = mfma32(*reinterpret_cast<const u32x4*>(Kc + koff[ks] + kb * 4096), qreg[ks], s[kb]);
    }
  };

  // Software pipeline over key tiles: iteration t holds the scores of tile
  // t (computed one iteration earlier) and, in one straight-line block,
  // issues the score MFMAs of tile t+1 alongside the softmax VALU work of
  // tile t and then its O^T += V^T P^T MFMAs, so matrix and vector units
  // work at the same time within a wave.  K and V^T have their own buffer
  // pairs: during iteration t the K buffer holds tile t+1 and the V^T
  // buffer tile t, while the copies of K tile t+2 and V^T tile t+1 fill the
  // other two.
  f32x16 sc[2];
  auto iteration = [&](int kt, const uint16_t* Knext, const uint16_t* Vc) {
    const int kstart = kt * BN;
    if (kstart > r0 + 31) return;  // this and every later tile lie in the wave's future
    if (kstart + BN - 1 > r0) {    // the tile reaches past this wave's first query
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kstart + kb * 32 + acc_row(r, g) > my_q) sc[kb][r] = -__builtin_inff();
    }
    // running maximum, raised lazily: only when some row's new score
    // exceeds it by more than 2^8 in the exponent (wave-uniform), so the
    // 64-register rescale of O runs a few times per row instead of every
    // tile; in between P <= 256, well inside fp16 and fp32
    if constexpr (!FROM_LSE) {
      float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sc[0][r]), sc[0][r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sc[1][r]), sc[1][r + 1]);
      mx = half_max_swap(mx) + sref;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc_o[db] *= alpha;
        // the held scores move to the new reference (0 for lanes whose
        // maximum stays), and so do the next tile's chains
        const float d = m_new - sref;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[kb][r] -= d;
#pragma unroll
        for (int r = 0; r < 16; ++r) nm16[r] = -m_new;
        m_run = m_new;
        sref = m_new;
      }
    }
    // scores of the next tile (unused past the last tile or the diagonal;
    // the buffer then holds stale but finite-or-ignored data)
    f32x16 sn[2];
    // this block (the next tile's score MFMAs interleaved with this tile's
    // exponentials) issues at raised wave priority and the PV MFMAs below
    // at the default: measured 2.5% faster than raising the PV MFMAs
    // instead, 6% faster than raising both
    __builtin_amdgcn_s_setprio(1);
    scores(Knext, sn, false);
    // LLVM's MFMA / exponential interleave strategy for this block (the
    // next tile's score MFMAs with this tile's exponentials): measured 1%
    // faster than the default schedule; the simpler variant (3) was slower
    // (with the scores starting from -m_run: default 1.8%, variant 1 0.6%
    // slower)
    __builtin_amdgcn_iglp_opt(2);
    // P in fp16, packed in pairs as the B operand; the row sum is taken
    // from each fp16 pair before it goes into the operand vector
    u32x4 pb[4];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(sc[kb][r]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x2 pair = {pr[8 * h + 2 * t], pr[8 * h + 2 * t + 1]};
          const f16x2 hp = __builtin_convertvector(pair, f16x2);
          if (FROM_LSE)
            ;  // no row sum: P is already normalised
          else if (t & 1)
            ls1 = __builtin_amdgcn_fdot2(hp, ones, ls1, false);
          else
            ls0 = __builtin_amdgcn_fdot2(hp, ones, ls0, false);
          pb[kb * 2 + h][t] = __builtin_bit_cast(uint32_t, hp);
        }
    }
    l_run += ls0 + ls1;
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T; B slot t of step st is key 16*st + 8*(t/4) + 4*g + t%4,
    // the order in which the V^T tile stores the keys of each 16-key step
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc_o[db] = mfma32_f16(*reinterpret_cast<const u32x4*>(Vc + voff[st] + db * 2048), pb[st], acc_o[db]);
    // V^T reads kept four MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    sc[0] = sn[0];
    sc[1] = sn[1];
  };

  dma_k(0, K0);
  dma_v(0, V0);
  if (n_kt > 1) dma_k(1, K1);
  lds_dma_wait();
  __syncthreads();
  scores(K0, sc, !FROM_LSE);   // tile 0 is visible to every wave
  __syncthreads();  // K0 is refilled below
  for (int kt = 0; kt < n_kt; kt += 2) {
    // K1 = tile kt+1, V0 = tile kt
    if (kt + 2 < n_kt) dma_k(kt + 2, K0);
    if (kt + 1 < n_kt) dma_v(kt + 1, V1);
    iteration(kt, K1, V0);
    lds_dma_wait();
    __syncthreads();
    if (kt + 1 >= n_kt) break;
    // K0 = tile kt+2, V1 = tile kt+1
    if (kt + 3 < n_kt) dma_k(kt + 3, K1);
    if (kt + 2 < n_kt) dma_v(kt + 2, V0);
    iteration(kt + 1, K0, V1);
    lds_dma_wait();
    __syncthreads();
  }

  const float l_tot = FROM_LSE ? 1.f : half_sum(l_run);
  if (my_q >= L) return;
  const float inv = FROM_LSE ? 1.f : 1.f / l_tot;  // (with the LSE, P sums to 1)
  const int hg = a.q_head0 - a.o_head0 + head;
  uint16_t* orow = a.o + (int64_t)my_q * a.o_ld + (int64_t)hg * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int d = db * 32 + j * 8 + g * 4;
      u32x2 w = {pack_bf16x2(acc_o[db][4 * j] * inv, acc_o[db][4 * j + 1] * inv),
                 pack_bf16x2(acc_o[db][4 * j + 2] * inv, acc_o[db][4 * j + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d) = w;
    }
  if (!FROM_LSE && g == 0)
    a.lse[(int64_t)hg * a.L + my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_flash_fwd(const FwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / BM) * a.nh));
  hipLaunchKernelGGL(flash_fwd_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_flash_fwd_lse(const FwdArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.Lp / BM) * a.nh));
  hipLaunchKernelGGL(flash_fwd_kernel<true>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace upipe
