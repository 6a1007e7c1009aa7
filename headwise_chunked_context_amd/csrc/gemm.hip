// bf16 MFMA GEMM for the layer's projections (gfx950).
//
// One kernel template covers the three operand layouts the layer needs:
//   NT  x . W_rows^T, O . W_o^T       (both operands k-contiguous)
//   NN  dy . W_o[:, cols], dqkv . W   (B n-contiguous)
//   TN  dy^T . O, dqkv^T . x          (both m/n-contiguous; K = L, split-K)
// Workgroup tile 256 x 256 x 64 on 512 threads: 8 waves, two per SIMD, each
// owning 128 x 64 of C as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (fp32
// accumulators, 128 registers).  Operand tiles are staged in LDS as they lie
// in memory -- no transposing stores:
//  * a k-contiguous operand is [256 rows][64 k] with 128-byte rows and the
//    16-byte chunk index XORed with (row / 2) % 8, so 16 lanes reading 16
//    rows at one k offset hit 16 different bank groups;
//  * an m/n-contiguous operand is [64 k][256] kept as two [64][128] halves in
//    the swizzled 256-byte-row layout of common.h and read with the LDS
//    transpose read (ds_read_b64_tr_b16), which hands each lane eight
//    consecutive k of one column.
// Global loads for k step t+1 are issued before the MFMAs of step t
// (register double buffering, two LDS buffers, one barrier per step).
#include "kernels.h"

namespace upipe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 512;                     // threads
constexpr int TILE = 256 * BK;              // elements of one operand tile
constexpr int HALF = 128 * BK;              // one [64][128] half of an m/n-major tile

__device__ __forceinline__ int kmaj_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}
__device__ __forceinline__ int mnmaj_off(int k, int chunk32) {
  return (chunk32 >> 4) * HALF + tile_off(k, chunk32 & 15);
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

template <bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(NT) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];  // 128 KB
  auto As = [&](int b) { return smem + 2 * b * TILE; };
  auto Bs = [&](int b) { return smem + (2 * b + 1) * TILE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int g = lane >> 5, l32 = lane & 31;

  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int kbeg = blockIdx.z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // ---- per-thread source pointers of the k-contiguous operands
  const uint16_t* a_rows[4];
  bool a_ok[4];
  const uint16_t* b_rows[4];
  bool b_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NT * i;
    const int r = c >> 3, ch = c & 7;
    if (A_K) {
      const int m = m0 + r;
      a_ok[i] = m < p.M;
      a_rows[i] = p.A + (int64_t)(a_ok[i] ? m : 0) * p.lda + ch * 8;
    }
    if (B_K) {
      const int n = n0 + r;
      b_ok[i] = n < p.N;
      b_rows[i] = p.B + seg_map(p.bseg, b_ok[i] ? n : 0) * p.ldb + ch * 8;
    }
  }

  u32x4 ra[4], rb[4];
  auto load_tiles = [&](int kt) {
    const int k0 = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NT * i;
      if (A_K) {
        ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4*>(a_rows[i] + k0) : u32x4{0, 0, 0, 0};
      } else {
        const int k = k0 + (c >> 5), col = m0 + (c & 31) * 8;
        ra[i] = (k < kend && col < p.M)
                    ? *reinterpret_cast<const u32x4*>(p.A + (int64_t)k * p.lda + col)
                    : u32x4{0, 0, 0, 0};
      }
      if (B_K) {
        rb[i] = b_ok[i] ? *reinterpret_cast<const u32x4*>(b_rows[i] + k0) : u32x4{0, 0, 0, 0};
      } else {
        // a 64-row k tile never crosses a segment (segments are multiples of 128)
        const int k = k0 + (c >> 5), col = n0 + (c & 31) * 8;
        rb[i] = (k < kend && col < p.N)
                    ? *reinterpret_cast<const u32x4*>(p.B + (seg_map(p.bseg, k0) + (c >> 5)) * p.ldb + col)
                    : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + NT * i;
      const int aofs = A_K ? kmaj_off(c >> 3, c & 7) : mnmaj_off(c >> 5, c & 31);
      *reinterpret_cast<u32x4*>(As(buf) + aofs) = ra[i];
      const int bofs = B_K ? kmaj_off(c >> 3, c & 7) : mnmaj_off(c >> 5, c & 31);
      *reinterpret_cast<u32x4*>(Bs(buf) + bofs) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
    const uint16_t* at = As(cur);
    const uint16_t* bt = Bs(cur);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 a[4], b[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = wm * 128 + mb * 32;
        if (A_K)
          a[mb] = *reinterpret_cast<const u32x4*>(at + kmaj_off(row + l32, 2 * ks + g));
        else
          a[mb] = tile_read_t_nat(at + wm * HALF, ks * 16, mb * 32, lane);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = wn * 64 + nb * 32;
        if (B_K)
          b[nb] = *reinterpret_cast<const u32x4*>(bt + kmaj_off(col + l32, 2 * ks + g));
        else
          b[nb] = tile_read_t_nat(bt + (col >> 7) * HALF, ks * 16, col & 127, lane);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(a[mb], b[nb], acc[mb][nb]);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  if (EPI == EPI_ATOMIC_F32) {
    // split-K: every split adds its partial tile into one fp32 accumulator
    float* C = reinterpret_cast<float*>(p.C);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = n0 + wn * 64 + nb * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 128 + mb * 32 + acc_row(r, g);
          if (m < p.M && n < p.N) atomicAdd(C + (int64_t)m * p.N + n, acc[mb][nb][r]);
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
    if (wm == half) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            Cs[(mb * 32 + acc_row(r, g)) * BN + wn * 64 + nb * 32 + l32] = acc[mb][nb][r];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = tid + NT * it;
      const int r = c >> 5, cc = c & 31;
      const int m = m0 + half * 128 + r;
      const int n = n0 + cc * 8;
      if (m < p.M && n < p.N) {
        const float* src = Cs + r * BN + cc * 8;
        f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
        u32x4* dst = reinterpret_cast<u32x4*>(C + (int64_t)m * p.ldc + n);
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
        if (EPI == EPI_ACCUM_BF16) {
          u32x4 old = *dst;
          lo[0] += bf16_lo(old[0]); lo[1] += bf16_hi(old[0]);
          lo[2] += bf16_lo(old[1]); lo[3] += bf16_hi(old[1]);
          hi[0] += bf16_lo(old[2]); hi[1] += bf16_hi(old[2]);
          hi[2] += bf16_lo(old[3]); hi[3] += bf16_hi(old[3]);
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

}  // namespace

hipError_t launch_gemm(GemmLayout layout, GemmEpilogue epi, const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, (a.K + a.k_per_split - 1) / a.k_per_split);
  dim3 block(NT);
#define UPIPE_GEMM_CASE(AK, BK_, E) hipLaunchKernelGGL((gemm_kernel<AK, BK_, E>), grid, block, 0, s, a)
  switch (layout) {
    case GEMM_NT:
      if (epi == EPI_STORE_BF16) UPIPE_GEMM_CASE(true, true, EPI_STORE_BF16);
      else if (epi == EPI_ACCUM_BF16) UPIPE_GEMM_CASE(true, true, EPI_ACCUM_BF16);
      else return hipErrorInvalidValue;
      break;
    case GEMM_NN:
      if (epi == EPI_STORE_BF16) UPIPE_GEMM_CASE(true, false, EPI_STORE_BF16);
      else if (epi == EPI_ACCUM_BF16) UPIPE_GEMM_CASE(true, false, EPI_ACCUM_BF16);
      else return hipErrorInvalidValue;
      break;
    case GEMM_TN:
      if (epi == EPI_ATOMIC_F32) UPIPE_GEMM_CASE(false, false, EPI_ATOMIC_F32);
      else return hipErrorInvalidValue;
      break;
  }
#undef UPIPE_GEMM_CASE
  return hipGetLastError();
}

hipError_t launch_acc_to_bf16(float* acc, int M, int N, uint16_t* dst, int64_t ld_dst,
                              const RowSegments& rows, hipStream_t s) {
  int64_t chunks = (int64_t)M * (N / 8);
  dim3 grid((unsigned)((chunks + 255) / 256));
  hipLaunchKernelGGL(acc_to_bf16_kernel, grid, dim3(256), 0, s, acc, M, N, dst, ld_dst, rows);
  return hipGetLastError();
}

}  // namespace upipe
