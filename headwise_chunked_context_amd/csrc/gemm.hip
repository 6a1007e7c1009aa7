// bf16 MFMA GEMM for the layer's projections (gfx950).
//
// One kernel template covers the three operand layouts the layer needs:
//   NT  y-like:  x[L,D] . W_rows^T            (both operands k-contiguous)
//   NN  dO, dx:  dy[L,D] . W[:, cols]         (B n-contiguous)
//   TN  dW:      dy^T . O, dqkv^T . x         (both m/n-contiguous; K = L)
// Tiles are 128x128x64 on 256 threads (four waves in a 2x2 grid, 64x64 per
// wave as 2x2 blocks of v_mfma_f32_32x32x16_bf16).  Operand tiles are staged
// through LDS as [row][k] with a 16-byte row pad; m/n-contiguous operands are
// transposed on the way in (each thread reads four k rows of eight elements
// and writes eight 4-element k runs).  Global loads for tile k+1 are issued
// before the MFMAs of tile k (register double buffering, two LDS buffers,
// one barrier per k step).
#include "kernels.h"

namespace upipe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_PITCH = BK + 8;           // bf16 elements per LDS row
constexpr int TILE_ELEMS = 128 * LDS_PITCH; // one operand tile
constexpr int C_PITCH = BN + 4;             // fp32 epilogue staging pitch

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

__device__ __forceinline__ void store_kmajor_tile(uint16_t* lds, const u32x4 v[4], int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int c = tid + 256 * i;
    int r = c >> 3, kc = c & 7;
    *reinterpret_cast<u32x4*>(lds + r * LDS_PITCH + kc * 8) = v[i];
  }
}

// v[i] holds eight consecutive r at k = 4*kg + i; write 4-k runs per r.
__device__ __forceinline__ void store_mnmajor_tile(uint16_t* lds, const u32x4 v[4], int tid) {
  int rg = tid & 15, kg = tid >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // pairs of r: (2j, 2j+1)
    uint32_t w0 = v[0][j], w1 = v[1][j], w2 = v[2][j], w3 = v[3][j];
    // element r=2j is the low half of each word, r=2j+1 the high half
    u32x2 lo, hi;
    lo[0] = (w0 & 0xffffu) | (w1 << 16);
    lo[1] = (w2 & 0xffffu) | (w3 << 16);
    hi[0] = (w0 >> 16) | (w1 & 0xffff0000u);
    hi[1] = (w2 >> 16) | (w3 & 0xffff0000u);
    *reinterpret_cast<u32x2*>(lds + (8 * rg + 2 * j) * LDS_PITCH + 4 * kg) = lo;
    *reinterpret_cast<u32x2*>(lds + (8 * rg + 2 * j + 1) * LDS_PITCH + 4 * kg) = hi;
  }
}

template <bool A_K, bool B_K, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE_ELEMS];
  // buffer b: A tile at smem + 2b*TILE_ELEMS, B tile right after it
  auto As = [&](int b) { return smem + 2 * b * TILE_ELEMS; };
  auto Bs = [&](int b) { return smem + (2 * b + 1) * TILE_ELEMS; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;

  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int kbeg = blockIdx.z * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // ---- per-thread source pointers
  const uint16_t* a_rows[4];
  bool a_ok[4];
  const uint16_t* b_rows[4];
  if (A_K) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = (tid + 256 * i) >> 3, kc = (tid + 256 * i) & 7;
      int m = m0 + r;
      a_ok[i] = m < p.M;
      a_rows[i] = p.A + (int64_t)(a_ok[i] ? m : 0) * p.lda + kc * 8;
    }
  }
  int64_t b_row_base = 0;
  if (B_K) {
    b_row_base = seg_map(p.bseg, n0);  // a 128-wide n tile never crosses a segment
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = (tid + 256 * i) >> 3, kc = (tid + 256 * i) & 7;
      b_rows[i] = p.B + (b_row_base + r) * p.ldb + kc * 8;
    }
  }
  const int rg = tid & 15, kg = tid >> 4;

  u32x4 ra[4], rb[4];
  auto load_tiles = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    if (A_K) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ra[i] = a_ok[i] ? *reinterpret_cast<const u32x4*>(a_rows[i] + k0) : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int k = k0 + 4 * kg + i;
        ra[i] = (k < kend) ? *reinterpret_cast<const u32x4*>(p.A + (int64_t)k * p.lda + m0 + 8 * rg)
                           : u32x4{0, 0, 0, 0};
      }
    }
    if (B_K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const u32x4*>(b_rows[i] + k0);
    } else {
      // a 64-wide k tile never crosses a segment (segments are multiples of 128)
      const int64_t krow = seg_map(p.bseg, k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int k = k0 + 4 * kg + i;
        rb[i] = (k < kend) ? *reinterpret_cast<const u32x4*>(p.B + (krow + 4 * kg + i) * p.ldb + n0 + 8 * rg)
                           : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tiles = [&](int buf) {
    if (A_K) store_kmajor_tile(As(buf), ra, tid); else store_mnmajor_tile(As(buf), ra, tid);
    if (B_K) store_kmajor_tile(Bs(buf), rb, tid); else store_mnmajor_tile(Bs(buf), rb, tid);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
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
    const uint16_t* a_base = As(cur) + (wm * 64 + l32) * LDS_PITCH + 8 * g;
    const uint16_t* b_base = Bs(cur) + (wn * 64 + l32) * LDS_PITCH + 8 * g;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 a0 = *reinterpret_cast<const u32x4*>(a_base + ks * 16);
      u32x4 a1 = *reinterpret_cast<const u32x4*>(a_base + 32 * LDS_PITCH + ks * 16);
      u32x4 b0 = *reinterpret_cast<const u32x4*>(b_base + ks * 16);
      u32x4 b1 = *reinterpret_cast<const u32x4*>(b_base + 32 * LDS_PITCH + ks * 16);
      acc[0][0] = mfma32(a0, b0, acc[0][0]);
      acc[0][1] = mfma32(a0, b1, acc[0][1]);
      acc[1][0] = mfma32(a1, b0, acc[1][0]);
      acc[1][1] = mfma32(a1, b1, acc[1][1]);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  if (EPI == EPI_ATOMIC_F32) {
    // split-K: every split adds its partial tile into one fp32 accumulator
    float* C = reinterpret_cast<float*>(p.C);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int m = m0 + wm * 64 + i * 32 + acc_row(r, g);
          int n = n0 + wn * 64 + j * 32 + l32;
          if (m < p.M) atomicAdd(C + (int64_t)m * p.N + n, acc[i][j][r]);
        }
    return;
  }

  // bf16 epilogue through LDS so every store is a 16-byte row chunk.
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        Cs[(wm * 64 + i * 32 + acc_row(r, g)) * C_PITCH + wn * 64 + j * 32 + l32] = acc[i][j][r];
  __syncthreads();
  uint16_t* C = reinterpret_cast<uint16_t*>(p.C);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    int c = tid + 256 * it;
    int r = c >> 4, cc = c & 15;
    int m = m0 + r;
    if (m >= p.M) continue;
    const float* src = Cs + r * C_PITCH + cc * 8;
    f32x4 lo = *reinterpret_cast<const f32x4*>(src);
    f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
    u32x4* dst = reinterpret_cast<u32x4*>(C + (int64_t)m * p.ldc + n0 + cc * 8);
    if (EPI == EPI_STORE_BF16 && n0 + cc * 8 < p.rope_cols) {
      // RoPE in fp32 on the four pairs of this 8-column chunk, position m
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int pair0 = ((n0 + cc * 8) & 127) >> 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float c, s;
        rope_cos_sin(p.rope, m, pair0 + j, c, s);
        float e = v[2 * j], o = v[2 * j + 1];
        v[2 * j] = e * c - o * s;
        v[2 * j + 1] = e * s + o * c;
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
    if (EPI == EPI_STORE_BF16 && p.f16_from > 0 && n0 + cc * 8 >= p.f16_from) {
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
  dim3 grid(a.N / BN, (a.M + BM - 1) / BM, (a.K + a.k_per_split - 1) / a.k_per_split);
  dim3 block(256);
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
