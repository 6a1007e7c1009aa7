// C ABI of the sequence-tiled SwiGLU MLP (include/upipe_mlp.h): argument
// checks, workspace planning, the tile loop, and the activation kernels.
//
// The MLP is the gated one of "GLU Variants Improve Transformer" (Builds-on
// list of "Untied Ulysses: Memory-Efficient Context Parallelism via
// Headwise Chunking"); tiling it along the sequence is the Arctic Long
// Sequence Training step of the memory progression in "Untied Ulysses
// Pushes Llama-3-8B Training to 5 Million Tokens".  Per tile of T rows the
// projections run on the layer's bf16 MFMA GEMM (gemm.hip):
//   forward   gu = x_t [W_gate; W_up]^T  (NT, [T, 2F])
//             a  = silu(h) * u            (swiglu_fwd_kernel, [T, F])
//             y_t = a W_down^T            (NT)
//   backward  gu = x_t [W_gate; W_up]^T  (recomputed)
//             da = dy_t W_down            (NN, [T, F])
//             dh, du (into gu), a (into da)  (swiglu_bwd_kernel)
//             dx_t = [dh | du] [W_gate; W_up]  (NN)
//             dW_gate_up += [dh | du]^T x_t,  dW_down += dy_t^T a
//                                          (TN, fp32 atomics into
//                                           accumulators the size of the
//                                           weights, converted once at the end)
// The activation kernels are HBM-bound elementwise passes: 16-byte vector
// loads and stores of eight bf16 values per thread.
#include <math.h>
#include <string.h>

#include "../../include/upipe_mlp.h"
#include "kernels.h"

using namespace upipe;

namespace {

constexpr int64_t kMaxL = int64_t(1) << 24;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// silu(h) = h * s and silu'(h) = s (1 + h (1 - s)), s = 1 / (1 + exp(-h));
// exp(-h) overflows to +inf for very negative h, which gives s = 0.
__device__ __forceinline__ float sigmoid_f(float h) {
  return 1.f / (1.f + __builtin_amdgcn_exp2f(-h * kLog2e));
}

// a[r][f] = silu(gu[r][f]) * gu[r][F + f]
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t* gu, uint16_t* a,
                                                         int64_t rows, int F) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 8-wide chunk each
  const int cpr = F / 8;
  if (idx >= rows * cpr) return;
  const int64_t r = idx / cpr;
  const int f = (int)(idx % cpr) * 8;
  const u32x4 hv = *reinterpret_cast<const u32x4*>(gu + r * 2 * F + f);
  const u32x4 uv = *reinterpret_cast<const u32x4*>(gu + r * 2 * F + F + f);
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float h0 = bf16_lo(hv[j]), h1 = bf16_hi(hv[j]);
    const float a0 = h0 * sigmoid_f(h0) * bf16_lo(uv[j]);
    const float a1 = h1 * sigmoid_f(h1) * bf16_hi(uv[j]);
    out[j] = pack_bf16x2(a0, a1);
  }
  *reinterpret_cast<u32x4*>(a + r * F + f) = out;
}

// In place: gu = [h | u] -> [dh | du] and ad = da -> a, with
//   du = da * silu(h),  dh = da * u * silu'(h),  a = silu(h) * u
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(uint16_t* gu, uint16_t* ad, int64_t rows,
                                                         int F) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = F / 8;
  if (idx >= rows * cpr) return;
  const int64_t r = idx / cpr;
  const int f = (int)(idx % cpr) * 8;
  uint16_t* hp = gu + r * 2 * F + f;
  uint16_t* up = hp + F;
  uint16_t* ap = ad + r * F + f;
  const u32x4 hv = *reinterpret_cast<const u32x4*>(hp);
  const u32x4 uv = *reinterpret_cast<const u32x4*>(up);
  const u32x4 dv = *reinterpret_cast<const u32x4*>(ap);
  u32x4 dh, du, av;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float h[2] = {bf16_lo(hv[j]), bf16_hi(hv[j])};
    float u[2] = {bf16_lo(uv[j]), bf16_hi(uv[j])};
    float da[2] = {bf16_lo(dv[j]), bf16_hi(dv[j])};
    float o_dh[2], o_du[2], o_a[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float s = sigmoid_f(h[e]);
      const float sl = h[e] * s;
      o_a[e] = sl * u[e];
      o_du[e] = da[e] * sl;
      o_dh[e] = da[e] * u[e] * (s * (1.f + h[e] * (1.f - s)));
    }
    dh[j] = pack_bf16x2(o_dh[0], o_dh[1]);
    du[j] = pack_bf16x2(o_du[0], o_du[1]);
    av[j] = pack_bf16x2(o_a[0], o_a[1]);
  }
  *reinterpret_cast<u32x4*>(hp) = dh;
  *reinterpret_cast<u32x4*>(up) = du;
  *reinterpret_cast<u32x4*>(ap) = av;
}

struct MlpShape {
  int64_t L;
  int D, F, T;  // T = rows per tile (at most L)
};

int check_mlp_shape(int64_t L, int32_t hidden, int32_t ffn, int32_t tile_rows, MlpShape* s) {
  if (L < 1 || hidden < 1 || ffn < 1 || tile_rows < 1) return UPIPE_EINVAL;
  if (L > kMaxL || hidden % 128 != 0 || ffn % 128 != 0) return UPIPE_EUNSUPPORTED;
  if ((int64_t)hidden * ffn >= (int64_t(1) << 33)) return UPIPE_EUNSUPPORTED;
  s->L = L;
  s->D = hidden;
  s->F = ffn;
  s->T = (int)(tile_rows < L ? tile_rows : L);
  // launch grids stay below 2^32 work-items: GEMMs of 256 x 256 tiles on 512
  // threads (the weight-gradient GEMMs with up to 32 splits), the activation
  // kernels one thread per 8 elements
  const int64_t lim = (int64_t)UINT32_MAX;
  const int64_t mt = (s->T + 255) / 256;
  const int64_t wide = 2 * (int64_t)ffn > hidden ? 2 * (int64_t)ffn : hidden;
  if (mt * ((wide + 255) / 256) * 512 > lim ||
      ((2 * (int64_t)ffn + 255) / 256) * ((hidden + 255) / 256) * 32 * 512 > lim ||
      (int64_t)s->T * ffn / 8 + 255 > lim)
    return UPIPE_EUNSUPPORTED;
  return UPIPE_OK;
}

// A GEMM whose output is hidden wide ([T, hidden]: the down projection and
// dx) has only ceil(T/256) * ceil(hidden/256) workgroups of 256 x 256; below
// one per CU its reduction is split so the chip fills, each split storing
// its fp32 partial result into its own [T, hidden] slice, and the slices are
// summed in split order into the bf16 output (the same bits every run).
constexpr int kCUs = 256;
int out_splits(const MlpShape& s, int K) {
  const int64_t tiles = (int64_t)((s.T + 255) / 256) * ((s.D + 255) / 256);
  if (tiles >= kCUs) return 1;
  int sp = (int)((kCUs + tiles - 1) / tiles);
  const int max_sp = K / 512;  // each split keeps at least 8 k steps
  if (sp > max_sp) sp = max_sp;
  return sp < 1 ? 1 : sp;
}

struct MlpPlan {
  size_t gu;        // [T][2F] bf16: h | u, then dh | du
  size_t ad;        // [T][F] bf16: a (forward), da then a (backward)
  size_t acc_out;   // [splits][T][D] fp32: the split hidden-wide GEMM's partial results
  size_t acc_gu;    // [2F][D] fp32 dW_gate_up accumulator (backward)
  size_t acc_down;  // [D][F] fp32 dW_down accumulator (backward)
  size_t total;
};

MlpPlan make_mlp_plan(const MlpShape& s, int pass) {
  MlpPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = (size_t)s.T, D = (size_t)s.D, F = (size_t)s.F;
  p.gu = take(T * 2 * F * 2);
  p.ad = take(T * F * 2);
  const int K = pass == UPIPE_PASS_BWD ? 2 * s.F : s.F;
  const int sp = out_splits(s, K);
  p.acc_out = sp > 1 ? take((size_t)sp * T * D * 4) : (size_t)-1;
  if (pass == UPIPE_PASS_BWD) {
    p.acc_gu = take(2 * F * D * 4);
    p.acc_down = take(D * F * 4);
  } else {
    p.acc_gu = p.acc_down = (size_t)-1;
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return off == (size_t)-1 ? nullptr : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_ws(const MlpShape& s, int pass, void* ws, size_t ws_bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0 ||
      ws_bytes < make_mlp_plan(s, pass).total)
    return UPIPE_EWORKSPACE;
  return UPIPE_OK;
}

#define UPIPE_TRY(expr)                     \
  do {                                      \
    const hipError_t upipe_e_ = (expr);     \
    if (upipe_e_ != hipSuccess) {           \
      note_hip_error(upipe_e_);             \
      return UPIPE_EHIP;                    \
    }                                       \
  } while (0)

GemmArgs gemm_args(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C,
                   int64_t ldc, int M, int N, int K) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.k_per_split = K;
  return g;
}

hipError_t launch_swiglu(bool bwd, uint16_t* gu, uint16_t* ad, int64_t rows, int F,
                         hipStream_t st) {
  const int64_t chunks = rows * (F / 8);
  dim3 grid((unsigned)((chunks + 255) / 256));
  if (bwd)
    hipLaunchKernelGGL(swiglu_bwd_kernel, grid, dim3(256), 0, st, gu, ad, rows, F);
  else
    hipLaunchKernelGGL(swiglu_fwd_kernel, grid, dim3(256), 0, st, gu, ad, rows, F);
  return hipGetLastError();
}

// hidden-wide GEMM of one tile, out[rows][D] = A B (layout NT or NN, K the
// reduction): one split stores bf16 directly; several store fp32 slices that
// are then summed in order into out
hipError_t launch_out(GemmLayout layout, const uint16_t* A, int64_t lda, const uint16_t* B,
                      int64_t ldb, uint16_t* out, int rows, int D, int K, int splits, float* acc,
                      hipStream_t st) {
  if (splits <= 1)
    return launch_gemm(layout, EPI_STORE_BF16, gemm_args(A, lda, B, ldb, out, D, rows, D, K), st);
  GemmArgs g = gemm_args(A, lda, B, ldb, acc, 0, rows, D, K);
  g.k_per_split = gemm_k_per_split(K, splits);
  const int used = (K + g.k_per_split - 1) / g.k_per_split;  // splits the GEMM launches
  hipError_t e = launch_gemm(layout, EPI_STORE_F32, g, st);
  if (e != hipSuccess) return e;
  return launch_sum_slices(acc, used, rows, D, out, D, st);
}

// weight-gradient GEMM of one tile: acc[M][N] (+)= A^T B over `rows` rows
hipError_t launch_dw(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* acc,
                     int M, int N, int rows, bool first, hipStream_t st) {
  GemmArgs g = gemm_args(A, lda, B, ldb, acc, 0, M, N, rows);
  const int splits = gemm_reduction_splits(rows, M, N);
  g.k_per_split = gemm_k_per_split(rows, splits);
  const GemmEpilogue epi = splits > 1 ? EPI_ATOMIC_F32 : (first ? EPI_STORE_F32 : EPI_ADD_F32);
  return launch_gemm(GEMM_TN, epi, g, st);
}

// debug mode: the tile's intermediates are NaN-filled before the tile
hipError_t debug_fill_tile(uint16_t* gu, uint16_t* ad, const MlpShape& s, hipStream_t st) {
  if (!g_debug_fill) return hipSuccess;
  const hipError_t e = launch_fill(gu, (size_t)s.T * 2 * s.F * 2, 0xFFFFFFFFu, st);
  if (e != hipSuccess) return e;
  return launch_fill(ad, (size_t)s.T * s.F * 2, 0xFFFFFFFFu, st);
}

}  // namespace

extern "C" {

int upipe_mlp_workspace_bytes(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t tile_rows,
                              int32_t pass, size_t* bytes) {
  if (!bytes || (pass != UPIPE_PASS_FWD && pass != UPIPE_PASS_BWD)) return UPIPE_EINVAL;
  MlpShape s;
  const int rc = check_mlp_shape(seq_len, hidden, ffn, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  *bytes = make_mlp_plan(s, pass).total;
  return UPIPE_OK;
}

int upipe_mlp_choose_tile(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t pass,
                          size_t budget_bytes, int32_t* tile_rows, size_t* bytes) {
  if (!tile_rows || !bytes || (pass != UPIPE_PASS_FWD && pass != UPIPE_PASS_BWD)) return UPIPE_EINVAL;
  MlpShape s;
  int rc = check_mlp_shape(seq_len, hidden, ffn, 1, &s);
  if (rc != UPIPE_OK) return rc;
  // candidates: multiples of 256 rows and the whole sequence; fewer, longer
  // tiles run faster, so the largest that fits wins (the size is not
  // monotone in the tile where the split buffers of short tiles appear)
  int64_t best = 0;
  size_t best_bytes = 0;
  for (int64_t t = 256; t < seq_len + 256; t += 256) {
    const int64_t tt = t < seq_len ? t : seq_len;
    MlpShape c;
    if (check_mlp_shape(seq_len, hidden, ffn, (int32_t)tt, &c) != UPIPE_OK) continue;
    const size_t b = make_mlp_plan(c, pass).total;
    if (b <= budget_bytes && tt > best) {
      best = tt;
      best_bytes = b;
    }
  }
  if (best == 0) return UPIPE_EWORKSPACE;
  *tile_rows = (int32_t)best;
  *bytes = best_bytes;
  return UPIPE_OK;
}

int upipe_mlp_fwd(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t tile_rows,
                  const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                  uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
  MlpShape s;
  int rc = check_mlp_shape(seq_len, hidden, ffn, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  if (!x || !w_gate_up || !w_down || !y) return UPIPE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y))
    return UPIPE_EINVAL;
  rc = check_ws(s, UPIPE_PASS_FWD, workspace, workspace_bytes);
  if (rc != UPIPE_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const MlpPlan p = make_mlp_plan(s, UPIPE_PASS_FWD);
  uint16_t* gu = at<uint16_t>(workspace, p.gu);
  uint16_t* ad = at<uint16_t>(workspace, p.ad);
  float* acc_out = at<float>(workspace, p.acc_out);
  const int D = s.D, F = s.F;
  const int splits = acc_out ? out_splits(s, F) : 1;
  for (int64_t t0 = 0; t0 < s.L; t0 += s.T) {
    const int rows = (int)(s.L - t0 < s.T ? s.L - t0 : s.T);
    const uint16_t* xt = x + t0 * D;
    UPIPE_TRY(debug_fill_tile(gu, ad, s, st));
    UPIPE_TRY(launch_gemm(GEMM_NT, EPI_STORE_BF16,
                          gemm_args(xt, D, w_gate_up, D, gu, 2 * F, rows, 2 * F, D), st));
    UPIPE_TRY(launch_swiglu(false, gu, ad, rows, F, st));
    UPIPE_TRY(launch_out(GEMM_NT, ad, F, w_down, F, y + t0 * D, rows, D, F, splits, acc_out, st));
  }
  return UPIPE_OK;
}

int upipe_mlp_bwd(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t tile_rows,
                  const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                  const uint16_t* dy, uint16_t* dx, uint16_t* dw_gate_up, uint16_t* dw_down,
                  void* workspace, size_t workspace_bytes, void* stream) {
  MlpShape s;
  int rc = check_mlp_shape(seq_len, hidden, ffn, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  if (!x || !w_gate_up || !w_down || !dy || !dx || !dw_gate_up || !dw_down) return UPIPE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(dw_gate_up) || !aligned16(dw_down))
    return UPIPE_EINVAL;
  rc = check_ws(s, UPIPE_PASS_BWD, workspace, workspace_bytes);
  if (rc != UPIPE_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const MlpPlan p = make_mlp_plan(s, UPIPE_PASS_BWD);
  uint16_t* gu = at<uint16_t>(workspace, p.gu);
  uint16_t* ad = at<uint16_t>(workspace, p.ad);
  float* acc_gu = at<float>(workspace, p.acc_gu);
  float* acc_down = at<float>(workspace, p.acc_down);
  float* acc_out = at<float>(workspace, p.acc_out);
  const int D = s.D, F = s.F;
  const int splits = acc_out ? out_splits(s, 2 * F) : 1;
  // the accumulators start at zero only if some tile's reduction is split
  // (the first tile of a one-split reduction stores instead)
  if (gemm_reduction_splits(s.T, 2 * F, D) > 1 || gemm_reduction_splits(s.T, D, F) > 1 ||
      gemm_reduction_splits(s.L % s.T ? s.L % s.T : s.T, 2 * F, D) > 1 ||
      gemm_reduction_splits(s.L % s.T ? s.L % s.T : s.T, D, F) > 1) {
    UPIPE_TRY(launch_zero(acc_gu, (size_t)2 * F * D * 4, st));
    UPIPE_TRY(launch_zero(acc_down, (size_t)D * F * 4, st));
  }
  for (int64_t t0 = 0; t0 < s.L; t0 += s.T) {
    const int rows = (int)(s.L - t0 < s.T ? s.L - t0 : s.T);
    const uint16_t* xt = x + t0 * D;
    const uint16_t* dyt = dy + t0 * D;
    UPIPE_TRY(debug_fill_tile(gu, ad, s, st));
    // recompute h | u, then da = dy_t W_down
    UPIPE_TRY(launch_gemm(GEMM_NT, EPI_STORE_BF16,
                          gemm_args(xt, D, w_gate_up, D, gu, 2 * F, rows, 2 * F, D), st));
    UPIPE_TRY(launch_gemm(GEMM_NN, EPI_STORE_BF16,
                          gemm_args(dyt, D, w_down, F, ad, F, rows, F, D), st));
    UPIPE_TRY(launch_swiglu(true, gu, ad, rows, F, st));
    // dx_t = [dh | du] [W_gate; W_up]
    UPIPE_TRY(launch_out(GEMM_NN, gu, 2 * F, w_gate_up, D, dx + t0 * D, rows, D, 2 * F, splits,
                         acc_out, st));
    // dW_gate_up += [dh | du]^T x_t ;  dW_down += dy_t^T a.  A tile's GEMM
    // whose reduction is one split owns every accumulator element: the first
    // tile stores, later ones add, both with plain stores (the tiles run in
    // order on one stream); split reductions add with atomics into the
    // accumulators cleared above
    UPIPE_TRY(launch_dw(gu, 2 * F, xt, D, acc_gu, 2 * F, D, rows, t0 == 0, st));
    UPIPE_TRY(launch_dw(dyt, D, ad, F, acc_down, D, F, rows, t0 == 0, st));
  }
  RowSegments ident;
  memset(&ident, 0, sizeof(ident));
  UPIPE_TRY(launch_acc_to_bf16(acc_gu, 2 * F, D, dw_gate_up, D, ident, st));
  UPIPE_TRY(launch_acc_to_bf16(acc_down, D, F, dw_down, F, ident, st));
  return UPIPE_OK;
}

}  // extern "C"
