// bf16 MFMA GEMM for the layer's projections (gfx950).
//
// One kernel template covers the three operand layouts the layer needs:
//   NT  x . W_rows^T, O . W_o^T       (both operands k-contiguous)
//   NN  dy . W_o[:, cols], dqkv . W   (B n-contiguous)
//   TN  dy^T . O, dqkv^T . x          (both m/n-contiguous; K = L, split-K)
// Workgroup tile 256 x 256, k step 64, on 512 threads: 8 waves, two per
// SIMD, each owning 128 x 64 of C as 8 x 4 blocks of
// v_mfma_f32_16x16x32_bf16 (fp32 accumulators, 128 registers; the 16x16
// shape moves half the accumulator data per FLOP of the 32x32x16 one, which
// measured on par here: the GEMMs run near 2 GHz, below the power limit
// that binds the attention kernels).  (One wave
// per SIMD with 128 x 128 each halves the LDS reads per MFMA but measured
// slower, with and without software-pipelined operand reads.)
// Operand tiles go straight from global memory to LDS by asynchronous
// global->LDS copies into two LDS stages of 64 KB.  Each wave holds one k
// half of operand fragments in registers while it reads the next, and the
// one barrier per step sits between the two halves' MFMAs: the copy of step
// t+2 is issued there and lands within a step, and the MFMAs after the
// barrier start from registers (3% less GEMM time for NT/NN, and 3% more
// once TN's transpose-read addresses, XORed from one base per operand,
// left it the registers for the second set of fragments).  (A k step of 32
// with four stages measured 4% slower: twice the barriers and operand-read
// latency bubbles per MFMA.)  The copies stage the tiles as they lie in
// memory, no transposing stores:
//  * a k-contiguous operand is [256 rows][64 k] with 128-byte rows and the
//    16-byte chunk index XORed with (row / 2) % 8, so 16 lanes reading 16
//    rows at one k offset hit 16 different bank groups;
//  * an m/n-contiguous operand is [64 k][256] kept as two [64][128] halves in
//    the swizzled 256-byte-row layout of common.h and read with the LDS
//    transpose read (ds_read_b64_tr_b16), which hands each lane eight
//    consecutive k of one column.
// Rows past M or N are read clamped (their products land in rows or columns
// of C that are not stored); k rows past the end of a split are zeroed in
// LDS after they land, so clamped reads never reach a stored result.
#include <stdint.h>

#include "kernels.h"

namespace upipe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int WM = 2, WN = 4;               // waves along M and N
constexpr int NT = 64 * WM * WN;            // threads
constexpr int MB = BM / WM / 16;            // 16x16 blocks per wave along M
constexpr int NB = BN / WN / 16;            // ... along N
constexpr int STAGES = BK == 32 ? 4 : 2;   // 128 KB of LDS either way
static_assert(WM == 2, "the bf16 epilogue stages one 128-row half of C per wave row");
constexpr int TILE = 256 * BK;              // elements of one operand tile
constexpr int HALF = 128 * BK;              // one [BK][128] half of an m/n-major tile
constexpr int CHUNKS = BK / 8;              // 16-byte chunks per k-major row
constexpr int ROWS_PER_KB = 512 / BK;       // k-major rows per 1 KB copy block
constexpr int STAGE = 2 * TILE;             // A and B tiles of one k step
static_assert((2 * HALF) % 256 == 0 && (2 * TILE) % 256 == 0 && (2 * STAGE) % 256 == 0,
              "tile bases keep the low 8 LDS address bits clear");

// k-major tile: rows of BK elements, the 16-byte chunk index XORed so that
// 16 lanes reading 16 consecutive rows at one chunk hit distinct banks
// (64-byte rows: by (row / 4) % 4; 128-byte rows: by (row / 2) % 8)
__device__ __forceinline__ int kmaj_swz(int row) {
  return BK == 32 ? (row >> 2) & 3 : (row >> 1) & 7;
}
__device__ __forceinline__ int kmaj_off(int row, int chunk) {
  return row * BK + ((chunk ^ kmaj_swz(row)) << 3);
}

// 16x16x32 operand from an m/n-major tile (k down the rows, m/n along the
// columns; the swizzled 256-byte-row layout of common.h): lane l gets
// column m0 + l % 16 and rows k0 + 8*(l/16) .. +7.  Two transpose reads: in
// each 16-lane group, lane p addresses row k0 + 8*(l/16) + p/4 (+4) and the
// four columns m0 + 4*(p%4) .., so lane i receives column m0 + i.
// The addresses keep two registers per operand instead of two per column
// block.  In the swizzled layout the byte
// address of (row r, column 16j + 4(s%4)) is r*256 + 8*(s%2) + 16*(c ^ swz(r))
// with c = 2j + (s%4)/2; j only enters through bits 5..7, so for a tile at a
// 256-byte aligned address, column block j's address is block 0's XOR (j << 5).
// tr16_base gives block 0's addresses of the lo (k0 + 8*(l/16) + p/4) and hi
// (+4) rows; 32 more k rows are +8192 bytes (the swizzle repeats every 16 rows).
__device__ __forceinline__ u32x2 tr16_base(uint32_t tile, int lane) {
  const int s = lane & 15;
  const int c0 = (s & 3) >> 1, half = 4 * (s & 1);
  const int r0 = 8 * (lane >> 4) + (s >> 2);
  return u32x2{tile + 2u * (uint32_t)(tile_off(r0, c0) + half),
               tile + 2u * (uint32_t)(tile_off(r0 + 4, c0) + half)};
}
__device__ __forceinline__ u32x2 lds_tr16_at(uint32_t addr) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2, v);
}
// column block j at k rows 32*ks .. of a tile whose block-0 addresses are b
__device__ __forceinline__ u32x4 tr16_read(u32x2 b, int j, int ks) {
  const u32x2 lo = lds_tr16_at((b[0] ^ (uint32_t)(j << 5)) + 8192u * ks);
  const u32x2 hi = lds_tr16_at((b[1] ^ (uint32_t)(j << 5)) + 8192u * ks);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

__device__ __forceinline__ int64_t seg_map(const RowSegments& s, int idx) {
  if (s.count == 0) return idx;
  int start = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i < s.count && idx < s.end[i]) return s.row0[i] + (idx - start);
    if (i < s.count) start = s.end[i];
  }
  return s.row0[0] + idx;  // unreachable for valid maps
}

// Maximum and sum over the 32 lanes of each half-wave by VALU lane exchanges
// (DPP within 4, 8 and 16 lanes, then the swap of 16-lane rows) instead of
// LDS permutes with their round trips.  Every lane ends with the same value
// (each step combines two equal-sized partial results; fp addition is
// commutative), so the result is reproducible.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <bool MAX>
__device__ __forceinline__ float half_wave_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]: lane ^ 1
  x = op(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]: lane ^ 2
  x = op(x, dpp_mov<0x141>(x));  // row_half_mirror: the other quad of 8 lanes
  x = op(x, dpp_mov<0x140>(x));  // row_mirror: the other 8 of 16 lanes
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 0<->1, 2<->3
  return op(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// s_waitcnt vmcnt(n), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
  // 256-byte aligned: the transpose-read addresses below rely on it
  __shared__ __attribute__((aligned(256))) uint16_t smem[STAGES * STAGE];  // 128 KB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave -> (wm, wn): the waves of a workgroup are dealt to the CU's four
  // SIMDs round-robin (wave w on SIMD w % 4), so the two waves of a SIMD take
  // columns from different halves of the tile (wn < 2 and wn >= 2): when a
  // tile is only partly inside N (N % 256 == 128) every SIMD keeps one busy
  // wave instead of two SIMDs keeping two
  static_assert(WM == 2 && WN == 4, "wave mapping below");
  const int wm = (wave >> 1) & 1, wn = (wave & 1) + 2 * (wave >> 2);

  // XCD-aware tile order: the dispatcher deals workgroups to the 8 XCDs
  // round-robin, so workgroup i runs on XCD i % 8.  Renumber so that each
  // XCD receives one contiguous range of tiles: the workgroups
  // an XCD runs together then share A row panels and B k-slices in its L2
  // instead of every XCD fetching every panel.  The grid is one-dimensional
  // (gx * gy * splits workgroups), so no per-dimension grid limit applies.
  const int gx = (p.N + BN - 1) / BN, gy = (p.M + BM - 1) / BM;
  const int total = gridDim.x;
  const int id = blockIdx.x;
  const int q8 = total >> 3, r8 = total & 7, xcd = id & 7, local = id >> 3;
  const int tile = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + local;
  // Within a split, tiles go in bands of GM rows, down the band's rows
  // first: the ~32 tiles one XCD runs at a time then span GM row panels of
  // A and 32 / GM column panels of B, so each panel fetched into the XCD's
  // L2 serves several tiles (bands of 4 measured 0.3-0.6% faster than 8 on
  // the layer's and the MLP's GEMMs; 2 and 16 slower).
  constexpr int GM = 4;
  const int t = tile % (gx * gy);
  const int m_first = (t / (GM * gx)) * GM;
  const int gm = min(gy - m_first, GM);
  const int u = t % (GM * gx);
  const int n0 = (u / gm) * BN;
  const int m0 = (m_first + u % gm) * BM;
  const int kbeg = (tile / (gx * gy)) * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // ---- copy plan: each wave moves CPW consecutive 1 KB blocks of
  // the A tile and of the B tile; per lane a source pointer (k = 0 of the
  // split) and, for m/n-major operands, its k row within the tile
  constexpr int CPW = (TILE / 512) / (WM * WN);  // 1 KB blocks per operand tile, per wave
  const uint16_t* asrc[CPW];
  const uint16_t* bsrc[CPW];
  int arow[CPW], brow[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int n = CPW * wave + i;
    if (A_K) {  // ROWS_PER_KB rows of 2 BK bytes per block
      const int row = ROWS_PER_KB * n + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ kmaj_swz(row);
      const int m = min(m0 + row, (p.rows_valid > 0 ? p.rows_valid : p.M) - 1);
      asrc[i] = p.A + (int64_t)m * p.lda + kbeg + c * 8;
      arow[i] = 0;
    } else {    // 4 k rows x 256 bytes of one 128-column half per block
      const int half = n / (BK / 4), row = 4 * (n % (BK / 4)) + (lane >> 4);
      const int c = (lane & 15) ^ swz(row);
      const int col = min(m0 + half * 128 + c * 8, p.M - 8);
      asrc[i] = p.A + (int64_t)kbeg * p.lda + col;
      arow[i] = row;
    }
    if (B_K) {
      const int row = ROWS_PER_KB * n + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ kmaj_swz(row);
      const int nn = min(n0 + row, p.N - 1);
      bsrc[i] = p.B + seg_map(p.bseg, nn) * p.ldb + kbeg + c * 8;
      brow[i] = 0;
    } else {
      const int half = n / (BK / 4), row = 4 * (n % (BK / 4)) + (lane >> 4);
      const int c = (lane & 15) ^ swz(row);
      const int col = min(n0 + half * 128 + c * 8, p.N - 8);
      bsrc[i] = p.B + col;  // rows come from the segment map per k step
      brow[i] = row;
    }
  }
  // issue the copies of k step kt into stage kt % STAGES
  auto issue = [&](int kt) {
    const int k0 = kt * BK;  // relative to kbeg
    uint16_t* st = smem + (kt % STAGES) * STAGE;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int n = CPW * wave + i;
      const uint16_t* a;
      if (A_K) {
        a = asrc[i] + k0;
      } else {
        const int k = min(kbeg + k0 + arow[i], kend - 1) - kbeg;
        a = asrc[i] + (int64_t)k * p.lda;
      }
      dma16_untracked(a, lds_addr(st + n * 512));
      const uint16_t* b;
      if (B_K) {
        b = bsrc[i] + k0;
      } else {
        // a BK-row k step never crosses a segment (segments are multiples of
        // 128): one uniform segment lookup per step, rows clamped only in a
        // split's last, partial step
        const int kb0 = kbeg + k0;
        const int64_t row = kb0 + BK <= kend ? seg_map(p.bseg, kb0) + brow[i]
                                             : seg_map(p.bseg, min(kb0 + brow[i], kend - 1));
        b = bsrc[i] + row * p.ldb;
      }
      dma16_untracked(b, lds_addr(st + TILE + n * 512));
    }
  };

  // per-lane LDS element offsets of the MFMA operands within a stage
  //  (16x16x32 operands: row l % 16 of a 16-row block, k chunk 4ks + l/16;
  //  16 rows further keep the swizzle, so blocks are an immediate apart)
  const int l16 = lane & 15, q4 = lane >> 4;
  int aoff[BK / 32], boff[BK / 32];
#pragma unroll
  for (int ks = 0; ks < BK / 32; ++ks) {
    aoff[ks] = A_K ? kmaj_off(wm * (BM / WM) + l16, 4 * ks + q4) : 0;
    boff[ks] = B_K ? kmaj_off(wn * (BN / WN) + l16, 4 * ks + q4) : 0;
  }

  const bool active = m0 + wm * (BM / WM) < p.M && n0 + wn * (BN / WN) < p.N;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The two k halves of a step are read into separate registers, and the
  // barrier sits between the halves' MFMAs instead of in front of a step's
  // first reads:
  //   [MFMAs of half 0 | reads of half 1]  wait, barrier, copy of kt+2
  //   [MFMAs of half 1 | reads of half 0 of step kt+1]
  // At the barrier every wave has all of step kt in registers (its stage
  // may be refilled) and step kt+1 has landed, so the MFMAs after the
  // barrier start from registers while the next step's first reads are in
  // flight.
  static_assert(STAGES == 2 && BK == 64, "two stages of two k halves");
  constexpr int RD = (A_K ? MB : 2 * MB) + (B_K ? NB : 2 * NB);  // LDS reads per k half
  // one read per MFMA from the half's start, so the last read lands well
  // before the next half needs it (measured 0.5-2% less GEMM time than
  // spreading the reads over the half: MLP tiles, layer GEMMs)
  constexpr int MPR = 1;                                          // MFMAs per read
  static_assert(MPR >= 1, "interleave");
  u32x4 a0[MB], b0[NB], a1[MB], b1[NB];
  // block-0 transpose-read addresses of stage 0 (m/n-major operands)
  const u32x2 atr = tr16_base(lds_addr(smem) + 2u * (uint32_t)(wm * HALF), lane);
  const u32x2 btr = tr16_base(lds_addr(smem) + 2u * (uint32_t)(TILE + (wn >> 1) * HALF), lane);
  auto frags = [&](int stage, int ks, u32x4* af, u32x4* bf) __attribute__((always_inline)) {
    const uint16_t* at = smem + stage * STAGE;
    const uint16_t* bt = at + TILE;
    const uint32_t so = 2u * (uint32_t)(stage * STAGE);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (B_K)
        bf[nb] = *reinterpret_cast<const u32x4*>(bt + boff[ks] + nb * 16 * BK);
      else
        bf[nb] = tr16_read(u32x2{btr[0] + so, btr[1] + so}, 4 * (wn & 1) + nb, ks);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (A_K)
        af[mb] = *reinterpret_cast<const u32x4*>(at + aoff[ks] + mb * 16 * BK);
      else
        af[mb] = tr16_read(u32x2{atr[0] + so, atr[1] + so}, mb, ks);
    }
  };
  auto mfmas = [&](const u32x4* af, const u32x4* bf) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma16(af[mb], bf[nb], acc[mb][nb]);
  };
  // MFMAs of one half with the RD reads of the other between them
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MB * NB - RD * MPR, 0);
  };
  // An m/n-major A read k rows past the end of the split clamped: once step
  // kt has landed, its rows past the end are zeroed (a uniform branch taken
  // by every wave, active or not, with the barrier that publishes the zeros)
  auto zero_tail = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kbeg + kt * BK;
    if (A_K || k0 + BK <= kend) return;
    uint16_t* st = smem + (kt & 1) * STAGE;
    const int valid = kend - k0;
    for (int c = tid; c < BK * 32; c += NT) {
      const int row = c >> 5;
      if (row >= valid)
        *reinterpret_cast<u32x4*>(st + (c & 16 ? HALF : 0) + row * 128 + (c & 15) * 8) = u32x4{0, 0, 0, 0};
    }
    __syncthreads();
  };

  // (the launcher sizes the grid so every split has at least one k step;
  // the guard keeps an empty one from copying past its end regardless)
  if (nk > 0) issue(0);
  wait_vmcnt<0>();
  __syncthreads();
  zero_tail(0);
  if (nk > 1) issue(1);
  if (active) {
    frags(0, 0, a0, b0);
    for (int kt = 0; kt < nk; ++kt) {
      frags(kt & 1, 1, a1, b1);
      mfmas(a0, b0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);  // the wait below stays after the half's MFMAs
      // this wave's reads of the stage have returned; the copies of step
      // kt+1 (the only ones in flight) have landed
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      if (kt + 1 < nk) wait_vmcnt<0>();
      __syncthreads();
      if (kt + 1 < nk) zero_tail(kt + 1);
      if (kt + 2 < nk) issue(kt + 2);  // into the stage just released
      // (after the last step these reads are unused: the stage they read
      // is a valid one that nothing writes any more)
      // the half after the barrier issues at raised wave priority
      // (measured 0.6% less GEMM time; raising the first half: no change)
      __builtin_amdgcn_s_setprio(1);
      frags((kt + 1) & 1, 0, a0, b0);
      mfmas(a1, b1);
      interleave();
      __builtin_amdgcn_s_setprio(0);
    }
  } else {
    // a wave whose rows or columns all lie outside C skips its reads and
    // MFMAs (their results would not be stored), not the copies and barriers
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) wait_vmcnt<0>();
      __syncthreads();
      if (kt + 1 < nk) zero_tail(kt + 1);
      if (kt + 2 < nk) issue(kt + 2);
    }
  }
  __syncthreads();  // the epilogue reuses the stages

  if (EPI == EPI_STORE_F32 || EPI == EPI_ADD_F32) {
    // fp32 [M][N]: each split stores its partial tile into its own [M][N]
    // slice (summed in split order afterwards), or a single split, which
    // owns its elements, adds its tile.  Staged through LDS one 128-row
    // half at a time (128 KB, the two operand stages), so every lane moves
    // 16 bytes of one row and a wave covers whole 1 KB row segments.
    float* C = reinterpret_cast<float*>(p.C) +
               (EPI == EPI_STORE_F32 ? (int64_t)(tile / (gx * gy)) * p.M * p.N : 0);
    float* Cs = reinterpret_cast<float*>(smem);
    constexpr int FIT = 128 * (BN / 4) / NT;  // 16-byte chunks per thread per half
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Cs[(mb * 16 + 4 * q4 + r) * BN + wn * (BN / WN) + nb * 16 + l16] = acc[mb][nb][r];
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < FIT; ++it) {
        const int c = tid + NT * it;
        const int r = c >> 6, cc = c & 63;
        const int m = m0 + half * 128 + r, n = n0 + cc * 4;
        if (m < p.M && n < p.N) {
          f32x4 v = *reinterpret_cast<const f32x4*>(Cs + r * BN + cc * 4);
          f32x4* dst = reinterpret_cast<f32x4*>(C + (int64_t)m * p.N + n);
          if (EPI == EPI_ADD_F32) v += *dst;
          *dst = v;
        }
      }
      __syncthreads();
    }
    return;
  }
  if (EPI == EPI_ATOMIC_F32) {
    // fp32 accumulator [M][N]: split-K partial tiles meet by atomic adds
    float* C = reinterpret_cast<float*>(p.C);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = n0 + wn * (BN / WN) + nb * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * (BM / WM) + mb * 16 + 4 * q4 + r;
          if (m < p.M && n < p.N) {
            atomicAdd(C + (int64_t)m * p.N + n, acc[mb][nb][r]);
          }
        }
      }
    return;
  }

  // bf16 epilogue through LDS (128 rows at a time) so every store is a
  // 16-byte row chunk
  float* Cs = reinterpret_cast<float*>(smem);
  uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // accumulate: the old values of this half's C rows are requested first,
    // all eight at once, so their latency overlaps the LDS staging below
    constexpr int EIT = 128 * (BN / 8) / NT;  // 16-byte chunks per thread per half
    u32x4 old[EIT];
    if (EPI == EPI_ACCUM_BF16) {
#pragma unroll
      for (int it = 0; it < EIT; ++it) {
        const int c = tid + NT * it;
        const int m = m0 + half * 128 + (c >> 5), n = n0 + (c & 31) * 8;
        old[it] = (m < p.M && n < p.N)
                      ? *reinterpret_cast<const u32x4*>(C + (int64_t)m * p.ldc + n)
                      : u32x4{0, 0, 0, 0};
      }
    }
    if (wm == half) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Cs[(mb * 16 + 4 * q4 + r) * BN + wn * (BN / WN) + nb * 16 + l16] = acc[mb][nb][r];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < EIT; ++it) {
      const int c = tid + NT * it;
      const int r = c >> 5, cc = c & 31;
      const int m = m0 + half * 128 + r;
      const int n = n0 + cc * 8;
      if (EPI == EPI_CE_STATS) {
        // the 32 lanes of a half-wave hold one row's 256 columns, 8 each:
        // its maximum and sum of 2^(y - max), y = logit log2 e, over the
        // tile's columns inside N (every lane takes part in the exchanges)
        const float* src = Cs + r * BN + cc * 8;
        const bool row_ok = m < p.M;
        float y[8], mx = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          y[i] = row_ok && n + i < p.N ? src[i] * kLog2e : -__builtin_inff();
          mx = fmaxf(mx, y[i]);
        }
        mx = half_wave_reduce<true>(mx);
        float sum = 0.f;
        if (mx != -__builtin_inff()) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sum += __builtin_amdgcn_exp2f(y[i] - mx);
        }
        sum = half_wave_reduce<false>(sum);
        if (row_ok) {
          if (cc == 0) {
            const int nct = (p.N + BN - 1) / BN;
            *reinterpret_cast<f32x2*>(p.ce_stats + ((int64_t)m * nct + n0 / BN) * 2) = f32x2{mx, sum};
          }
          const int t = p.ce_targets[p.ce_row0 + m];
          if (t >= n && t < n + 8 && t < p.N) p.ce_tlogit[m] = src[t - n];
          if (p.ce_logits16 && n < p.N) {
            // the fused forward-backward keeps the logits in fp16 (finite
            // values beyond +-65504 saturate) for its dlogits pass
            u32x4 h16;
#pragma unroll
            for (int i = 0; i < 4; ++i) h16[i] = pack_f16x2_sat(src[2 * i], src[2 * i + 1]);
            *reinterpret_cast<u32x4*>(p.ce_logits16 + (int64_t)m * p.N + n) = h16;
          }
        }
        continue;
      }
      if (EPI == EPI_CE_GRAD) {
        // dlogits = (exp(logit - lse) - [n == target]) * scale, 0 for an
        // ignored row, NaN for a target outside [0, N)
        if (m < p.M && n < p.N) {
          const float* src = Cs + r * BN + cc * 8;
          const int64_t row = p.ce_row0 + m;
          const int t = p.ce_targets[row];
          float v[8];
          if (t == p.ce_ignore) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
          } else {
            const float l2 = p.ce_lse[row] * kLog2e, sc = *p.ce_scale;
            const bool in_range = t >= 0 && t < p.N;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              float e = __builtin_amdgcn_exp2f(fmaf(src[i], kLog2e, -l2));
              if (n + i == t) e -= 1.f;
              v[i] = in_range ? e * sc : quiet_nan();
            }
          }
          u32x4 out;
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
          *reinterpret_cast<u32x4*>(C + (int64_t)m * p.ldc + n) = out;
        }
        continue;
      }
      const bool head_major = EPI == EPI_STORE_BF16 && n < p.hm_end;
      const int rows = head_major || p.rows_valid <= 0 ? p.M : p.rows_valid;
      if (m < rows && n < p.N) {
        const float* src = Cs + r * BN + cc * 8;
        f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
        u32x4* dst = reinterpret_cast<u32x4*>(
            !head_major ? C + (int64_t)m * p.ldc + n
            : n < p.hm_split ? p.hm_q + (int64_t)(n >> 7) * p.hm_stride + (int64_t)m * 128 + (n & 127)
                             : p.hm_k + (int64_t)((n - p.hm_split) >> 7) * p.hm_stride + (int64_t)m * 128 +
                                   ((n - p.hm_split) & 127));
        if (EPI == EPI_STORE_BF16 && n < p.rope_cols) {
          // RoPE in fp32 on the four pairs of this 8-column chunk, position m
          float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const int pair0 = (n & 127) >> 1;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float cs, sn;
            rope_cos_sin(p.rope, m, pair0 + j, cs, sn);
            float e = v[2 * j], o = v[2 * j + 1];
            v[2 * j] = e * cs - o * sn;
            v[2 * j + 1] = e * sn + o * cs;
          }
          lo = f32x4{v[0], v[1], v[2], v[3]};
          hi = f32x4{v[4], v[5], v[6], v[7]};
        }
        if (EPI == EPI_STORE_BF16 && head_major && n < p.hm_split) {
          lo *= p.hm_q_scale;
          hi *= p.hm_q_scale;
        }
        if (EPI == EPI_ACCUM_BF16) {
          const u32x4 o = old[it];
          lo[0] += bf16_lo(o[0]); lo[1] += bf16_hi(o[0]);
          lo[2] += bf16_lo(o[1]); lo[3] += bf16_hi(o[1]);
          hi[0] += bf16_lo(o[2]); hi[1] += bf16_hi(o[2]);
          hi[2] += bf16_lo(o[3]); hi[3] += bf16_hi(o[3]);
        }
        u32x4 out;
        if (EPI == EPI_STORE_BF16 && p.f16_from > 0 && n >= p.f16_from) {
          out[0] = pack_f16x2_sat(lo[0], lo[1]);
          out[1] = pack_f16x2_sat(lo[2], lo[3]);
          out[2] = pack_f16x2_sat(hi[0], hi[1]);
          out[3] = pack_f16x2_sat(hi[2], hi[3]);
        } else {
          out[0] = pack_bf16x2(lo[0], lo[1]);
          out[1] = pack_bf16x2(lo[2], lo[3]);
          out[2] = pack_bf16x2(hi[0], hi[1]);
          out[3] = pack_bf16x2(hi[2], hi[3]);
        }
        *dst = out;
      }
    }
    __syncthreads();
  }
}

// fp32 accumulator [M][N] -> bf16 dst rows dst[map(m)*ld + n]; clears acc.
__global__ __launch_bounds__(256) void acc_to_bf16_kernel(float* acc, int M, int N, uint16_t* dst,
                                                          int64_t ld, RowSegments rows) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 8-wide chunk each
  int64_t chunks = (int64_t)M * (N / 8);
  if (idx >= chunks) return;
  int m = (int)(idx / (N / 8));
  int n = (int)(idx % (N / 8)) * 8;
  float* src = acc + (int64_t)m * N + n;
  f32x4 a = *reinterpret_cast<const f32x4*>(src);
  f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
  *reinterpret_cast<f32x4*>(src) = f32x4{0, 0, 0, 0};
  *reinterpret_cast<f32x4*>(src + 4) = f32x4{0, 0, 0, 0};
  u32x4 out;
  out[0] = pack_bf16x2(a[0], a[1]);
  out[1] = pack_bf16x2(a[2], a[3]);
  out[2] = pack_bf16x2(b[0], b[1]);
  out[3] = pack_bf16x2(b[2], b[3]);
  int64_t row = seg_map(rows, m);
  *reinterpret_cast<u32x4*>(dst + row * ld + n) = out;
}

// dst[m][n] (bf16) = sum over s of slices[s][m][n] (fp32), added in slice
// order, so the result does not depend on which split finished first
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* slices, int nslices, int M,
                                                         int N, uint16_t* dst, int64_t ld) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 8-wide chunk each
  const int64_t chunks = (int64_t)M * (N / 8);
  if (idx >= chunks) return;
  const int m = (int)(idx / (N / 8));
  const int n = (int)(idx % (N / 8)) * 8;
  f32x4 a = f32x4{0, 0, 0, 0}, b = f32x4{0, 0, 0, 0};
  for (int sl = 0; sl < nslices; ++sl) {
    const float* src = slices + (int64_t)sl * M * N + (int64_t)m * N + n;
    a += *reinterpret_cast<const f32x4*>(src);
    b += *reinterpret_cast<const f32x4*>(src + 4);
  }
  u32x4 out;
  out[0] = pack_bf16x2(a[0], a[1]);
  out[1] = pack_bf16x2(a[2], a[3]);
  out[2] = pack_bf16x2(b[0], b[1]);
  out[3] = pack_bf16x2(b[2], b[3]);
  *reinterpret_cast<u32x4*>(dst + (int64_t)m * ld + n) = out;
}

}  // namespace

hipError_t launch_sum_slices(const float* slices, int nslices, int M, int N, uint16_t* dst,
                             int64_t ld, hipStream_t s) {
  const int64_t chunks = (int64_t)M * (N / 8);
  dim3 grid((unsigned)((chunks + 255) / 256));
  hipLaunchKernelGGL(sum_slices_kernel, grid, dim3(256), 0, s, slices, nslices, M, N, dst, ld);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmLayout layout, GemmEpilogue epi, const GemmArgs& a, hipStream_t s) {
  // k steps of BK must not read past a k-contiguous row, nor splits overlap;
  // only the atomic epilogue may combine several splits
  if (a.k_per_split % BK != 0 || (layout != GEMM_TN && a.K % BK != 0)) return hipErrorInvalidValue;
  if (epi != EPI_ATOMIC_F32 && epi != EPI_STORE_F32 && a.k_per_split < a.K) return hipErrorInvalidValue;
  dim3 grid((unsigned)(((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM) *
                       ((a.K + a.k_per_split - 1) / a.k_per_split)));
  dim3 block(NT);
#define UPIPE_GEMM_CASE(AK, BK_, E) hipLaunchKernelGGL((gemm_kernel<AK, BK_, E>), grid, block, 0, s, a)
  switch (layout) {
    case GEMM_NT:
      if (epi == EPI_STORE_BF16) UPIPE_GEMM_CASE(true, true, EPI_STORE_BF16);
      else if (epi == EPI_ACCUM_BF16) UPIPE_GEMM_CASE(true, true, EPI_ACCUM_BF16);
      else if (epi == EPI_ATOMIC_F32) UPIPE_GEMM_CASE(true, true, EPI_ATOMIC_F32);
      else if (epi == EPI_STORE_F32) UPIPE_GEMM_CASE(true, true, EPI_STORE_F32);
      else if (epi == EPI_CE_STATS) UPIPE_GEMM_CASE(true, true, EPI_CE_STATS);
      else if (epi == EPI_CE_GRAD) UPIPE_GEMM_CASE(true, true, EPI_CE_GRAD);
      else return hipErrorInvalidValue;
      break;
    case GEMM_NN:
      if (epi == EPI_STORE_BF16) UPIPE_GEMM_CASE(true, false, EPI_STORE_BF16);
      else if (epi == EPI_ACCUM_BF16) UPIPE_GEMM_CASE(true, false, EPI_ACCUM_BF16);
      else if (epi == EPI_ATOMIC_F32) UPIPE_GEMM_CASE(true, false, EPI_ATOMIC_F32);
      else if (epi == EPI_STORE_F32) UPIPE_GEMM_CASE(true, false, EPI_STORE_F32);
      else return hipErrorInvalidValue;
      break;
    case GEMM_TN:
      if (epi == EPI_ATOMIC_F32) UPIPE_GEMM_CASE(false, false, EPI_ATOMIC_F32);
      else if (epi == EPI_STORE_F32) UPIPE_GEMM_CASE(false, false, EPI_STORE_F32);
      else if (epi == EPI_ADD_F32) UPIPE_GEMM_CASE(false, false, EPI_ADD_F32);
      else return hipErrorInvalidValue;
      break;
  }
#undef UPIPE_GEMM_CASE
  return hipGetLastError();
}

// Split-K factor of a weight-gradient GEMM (reduction over K = L rows).  The
// 256 x 256 workgroups run one per CU, so with s splits the GEMM takes about
// ceil(tiles*s / 256) rounds of ceil(L / (64 s)) k steps each, plus its
// epilogue over the M x N output: with several splits every split adds its
// partial tile by fp32 atomics (about 1.2 TB/s, measured), with one split a
// plain store or read-modify-write (about five times faster).  In units of a
// round's k step (~2 us at the GEMMs' rate), an atomic pass over M x N
// elements costs about M N / 600000, a plain one M N / 3000000 (for the
// attention layer's weight gradients, M N ~ 4-6 million, that is 7-10 k
// steps per split).  Each split keeps at least 512 rows.
int gemm_reduction_splits(int64_t L, int M, int N) {
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t elems = (int64_t)M * N;
  int max_s = (int)((L + 511) / 512);
  if (max_s > 32) max_s = 32;
  if (max_s < 1) max_s = 1;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int sp = 1; sp <= max_s; ++sp) {
    const int64_t rounds = (tiles * sp + 255) / 256;
    const int64_t steps = (L + 64LL * sp - 1) / (64LL * sp);
    const int64_t epilogue = sp > 1 ? sp * elems / 600000 : elems / 3000000;
    const int64_t cost = rounds * steps + epilogue;
    if (cost < best_cost) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

int gemm_k_per_split(int64_t L, int splits) {
  const int64_t k = (L + splits - 1) / splits;
  return (int)((k + BK - 1) / BK * BK);
}

hipError_t launch_acc_to_bf16(float* acc, int M, int N, uint16_t* dst, int64_t ld_dst,
                              const RowSegments& rows, hipStream_t s) {
  int64_t chunks = (int64_t)M * (N / 8);
  dim3 grid((unsigned)((chunks + 255) / 256));
  hipLaunchKernelGGL(acc_to_bf16_kernel, grid, dim3(256), 0, s, acc, M, N, dst, ld_dst, rows);
  return hipGetLastError();
}

}  // namespace upipe
