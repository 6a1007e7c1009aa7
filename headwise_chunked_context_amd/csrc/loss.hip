// C ABI of the sequence-tiled language-model loss (include/upipe_loss.h):
// argument checks, workspace planning, the tile loop, and the row kernels.
//
// The loss is the mean cross-entropy of next-token training over the
// vocabulary projection of the final hidden states; computing it a tile of
// positions at a time is the Arctic Long Sequence Training step of the
// memory progression in "Untied Ulysses Pushes Llama-3-8B Training to 5
// Million Tokens" (losses and MLPs need not allocate sequence-wide buffers).
// Per tile of T rows, on the layer's bf16 MFMA GEMM (gemm.hip):
//   forward   logits = h_t W^T, kept in registers: the GEMM's epilogue
//             (EPI_CE_STATS) reduces each row over each 256-column tile to
//             (max, sum 2^(y - max)) and picks out the target's logit
//             lse_r, loss_r per row from those pairs   (ce_combine_kernel)
//             loss = sum of loss_r / count     (ce_reduce_kernel, fixed order)
//   backward  logits = h_t W^T recomputed, and the epilogue (EPI_CE_GRAD)
//             stores dlogits = (exp(logits - lse) - onehot) * dloss / count
//             in bf16
//             dh_t = dlogits W                 (NN; short tiles split the
//                                               vocabulary reduction into fp32
//                                               slices summed in order)
//             dW += dlogits^T h_t              (TN, one split: the first tile
//                                               stores, later tiles add; fp32
//                                               accumulator the size of W)
// No fp32 logits are ever stored: the forward keeps 8 bytes per row and
// 256-column tile, the backward one bf16 [T, V] tile; the forward hands the
// backward the per-row log-sum-exp (4 bytes per position).
#include <math.h>
#include <string.h>

#include "../../include/upipe_loss.h"
#include "kernels.h"

using namespace upipe;

namespace {

constexpr int64_t kMaxL = int64_t(1) << 24;
constexpr size_t kAlign = 256;
constexpr int kCUs = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// (m, s) summarises a set of values y (base-2 logits, y = x log2 e) as its
// maximum m and s = sum 2^(y - m); two summaries combine exactly.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -__builtin_inff()) return;  // both empty
  s = s * __builtin_amdgcn_exp2f(m - mm) + s2 * __builtin_amdgcn_exp2f(m2 - mm);
  m = mm;
}

// One workgroup per row of the tile: the row's log-sum-exp from the
// (max, sum) pairs of its 256-column tiles, and its loss lse - logit[target]
// (0 for an ignored row, NaN for a target outside the vocabulary).
__global__ __launch_bounds__(256) void ce_combine_kernel(const float* stats, int nct,
                                                         const float* tlogit, int V,
                                                         const int32_t* targets, int64_t row0,
                                                         int ignore_index, float* lse,
                                                         float* loss_rows) {
  __shared__ float sm_m[4], sm_s[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x;
  float m = -__builtin_inff(), s = 0.f;
  for (int j = tid; j < nct; j += 256) {
    const f32x2 ms = *reinterpret_cast<const f32x2*>(stats + (r * nct + j) * 2);
    lse_combine(m, s, ms[0], ms[1]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_combine(m, s, m2, s2);
  }
  if (lane == 0) {
    sm_m[wave] = m;
    sm_s[wave] = s;
  }
  __syncthreads();
  if (tid != 0) return;
  m = sm_m[0];
  s = sm_s[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_combine(m, s, sm_m[w], sm_s[w]);
  const float l = (m + __builtin_amdgcn_logf(s)) * kLn2;  // v_log_f32 is base 2
  const int64_t row = row0 + r;
  const int t = targets[row];
  float loss = 0.f;
  if (t != ignore_index) loss = (t >= 0 && t < V) ? l - tlogit[r] : quiet_nan();
  lse[row] = l;
  loss_rows[row] = loss;
}

// Rows that count (target != ignore_index), and either the mean of their
// loss (loss != nullptr) or the backward's scale dloss / count, on one
// workgroup: every thread sums a fixed stride of rows in fp64 and the
// partial sums meet in a fixed order, so the result has the same bits on
// every run.  No row counts: loss 0, scale 0.
__global__ __launch_bounds__(1024) void ce_reduce_kernel(const float* loss_rows,
                                                         const int32_t* targets, int64_t L,
                                                         int ignore_index, float dloss,
                                                         float* loss, float* scale) {
  __shared__ double sm_sum[16];
  __shared__ long long sm_cnt[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double sum = 0.0;
  long long cnt = 0;
  for (int64_t r = tid; r < L; r += 1024) {
    if (targets[r] == ignore_index) continue;
    ++cnt;
    if (loss) sum += (double)loss_rows[r];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sum += __shfl_xor(sum, off);
    cnt += __shfl_xor(cnt, off);
  }
  if (lane == 0) {
    sm_sum[wave] = sum;
    sm_cnt[wave] = cnt;
  }
  __syncthreads();
  if (tid != 0) return;
  sum = 0.0;
  cnt = 0;
  for (int w = 0; w < 16; ++w) {
    sum += sm_sum[w];
    cnt += sm_cnt[w];
  }
  if (loss) *loss = cnt > 0 ? (float)(sum / (double)cnt) : 0.f;
  if (scale) *scale = cnt > 0 ? (float)((double)dloss / (double)cnt) : 0.f;
}

// In place, fp16 logits -> bf16 dlogits = (exp(logit - lse_r) - [j == t_r])
// * scale (0 for an ignored row, NaN for a target outside the vocabulary);
// one thread per 8 consecutive vocabulary entries of a row, each reading and
// writing only its own 16 bytes.
__global__ __launch_bounds__(256) void ce_grad_f16_kernel(uint16_t* buf, int V,
                                                          const int32_t* targets, int64_t row0,
                                                          int rows, const float* lse,
                                                          const float* scale, int ignore_index) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = V / 8;
  if (idx >= (int64_t)rows * cpr) return;
  const int64_t r = idx / cpr;
  const int j = (int)(idx % cpr) * 8;
  const int64_t row = row0 + r;
  const int t = targets[row];
  u32x4* p = reinterpret_cast<u32x4*>(buf + r * V + j);
  float v[8];
  if (t == ignore_index) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  } else {
    const u32x4 x = *p;
    const float l2 = lse[row] * kLog2e, sc = *scale;
    const bool in_range = t >= 0 && t < V;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float lg = (i & 1) ? f16_hi(x[i >> 1]) : f16_lo(x[i >> 1]);
      float e = __builtin_amdgcn_exp2f(fmaf(lg, kLog2e, -l2));
      if (j + i == t) e -= 1.f;
      v[i] = in_range ? e * sc : quiet_nan();
    }
  }
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *p = out;
}

struct LossShape {
  int64_t L;
  int D, V, T;  // T = rows per tile (at most L)
};

int check_loss_shape(int64_t L, int32_t hidden, int32_t vocab, int32_t tile_rows, LossShape* s) {
  if (L < 1 || hidden < 1 || vocab < 1 || tile_rows < 1) return UPIPE_EINVAL;
  if (L > kMaxL || hidden % 128 != 0 || vocab % 128 != 0) return UPIPE_EUNSUPPORTED;
  if ((int64_t)hidden * vocab >= (int64_t(1) << 33)) return UPIPE_EUNSUPPORTED;
  s->L = L;
  s->D = hidden;
  s->V = vocab;
  s->T = (int)(tile_rows < L ? tile_rows : L);
  // launch grids stay below 2^32 work-items: GEMMs of 256 x 256 tiles on 512
  // threads (the dh GEMM with up to 256 splits), the gradient rows one thread
  // per 8 entries
  const int64_t lim = (int64_t)UINT32_MAX;
  const int64_t mt = (s->T + 255) / 256;
  if (mt * ((vocab + 255) / 256) * 512 > lim || mt * ((hidden + 255) / 256) * 256 * 512 > lim ||
      ((int64_t)vocab + 255) / 256 * ((hidden + 255) / 256) * 512 > lim ||
      (int64_t)s->T * (vocab / 8) + 255 > lim)
    return UPIPE_EUNSUPPORTED;
  return UPIPE_OK;
}

// splits of the dh GEMM ([T, hidden] output, reduction over the vocabulary):
// enough 256 x 256 workgroups to fill the chip, each split at least 8 k steps
int dh_splits(const LossShape& s) {
  const int64_t tiles = (int64_t)((s.T + 255) / 256) * ((s.D + 255) / 256);
  if (tiles >= kCUs) return 1;
  int sp = (int)((kCUs + tiles - 1) / tiles);
  const int max_sp = s.V / 512;
  if (sp > max_sp) sp = max_sp;
  return sp < 1 ? 1 : sp;
}

struct LossPlan {
  size_t stats;      // [T][ceil(V/256)] (max, sum) fp32 pairs (forward)
  size_t tlogit;     // [T] fp32 target logits (forward)
  size_t loss_rows;  // [L] fp32 per-row loss (forward)
  size_t dlogits;    // [T][V] bf16 (backward)
  size_t dh_acc;     // [splits][T][D] fp32 partial dh (backward, split only)
  size_t dw_acc;     // [V][D] fp32 dW accumulator (backward)
  size_t scale;      // one fp32: dloss / count (backward)
  size_t total;
};

int col_tiles(const LossShape& s) { return (s.V + 255) / 256; }

LossPlan make_loss_plan(const LossShape& s, int pass) {
  LossPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = (size_t)s.T, D = (size_t)s.D, V = (size_t)s.V;
  const size_t none = (size_t)-1;
  if (pass == UPIPE_PASS_FWD_BWD) {
    // forward statistics and per-row loss, and the backward's buffers; the
    // [T][V] tile holds fp16 logits, then (in place) bf16 dlogits
    p.stats = take(T * (size_t)col_tiles(s) * 8);
    p.tlogit = take(T * 4);
    p.loss_rows = take((size_t)s.L * 4);
    p.dlogits = take(T * V * 2);
    const int sp = dh_splits(s);
    p.dh_acc = sp > 1 ? take((size_t)sp * T * D * 4) : none;
    p.dw_acc = take(V * D * 4);
    p.scale = take(4);
  } else if (pass == UPIPE_PASS_BWD) {
    p.stats = p.tlogit = p.loss_rows = none;
    p.dlogits = take(T * V * 2);
    const int sp = dh_splits(s);
    p.dh_acc = sp > 1 ? take((size_t)sp * T * D * 4) : none;
    p.dw_acc = take(V * D * 4);
    p.scale = take(4);
  } else {
    p.dlogits = p.dh_acc = p.dw_acc = p.scale = none;
    p.stats = take(T * (size_t)col_tiles(s) * 8);
    p.tlogit = take(T * 4);
    p.loss_rows = take((size_t)s.L * 4);
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return off == (size_t)-1 ? nullptr : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_ws(const LossShape& s, int pass, void* ws, size_t ws_bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0 ||
      ws_bytes < make_loss_plan(s, pass).total)
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

// logits of one tile, h_t W^T, reduced in the GEMM's epilogue: forward
// statistics (EPI_CE_STATS) or the backward's bf16 dlogits (EPI_CE_GRAD)
GemmArgs logits_args(const uint16_t* ht, const uint16_t* w, int rows, const LossShape& s,
                     const int32_t* targets, int ignore_index, int64_t row0) {
  GemmArgs g = gemm_args(ht, s.D, w, s.D, nullptr, s.V, rows, s.V, s.D);
  g.ce_targets = targets;
  g.ce_ignore = ignore_index;
  g.ce_row0 = row0;
  return g;
}

// the weight-side products of one tile's bf16 dlogits [rows][V]:
//   dh_t = dlogits W   (NN; one split stores bf16, several store fp32
//                       slices summed in split order)
//   dW  += dlogits^T h_t  (TN, one split: the first tile stores, later ones
//                       add with plain stores; the tiles run in order on one
//                       stream)
hipError_t grads_of_tile(const uint16_t* dlogits, const uint16_t* ht, const uint16_t* w,
                         uint16_t* dh_t, float* dh_acc, float* dw_acc, int rows, int splits,
                         const LossShape& s, bool first, hipStream_t st) {
  const int D = s.D, V = s.V;
  hipError_t e;
  if (splits <= 1) {
    e = launch_gemm(GEMM_NN, EPI_STORE_BF16, gemm_args(dlogits, V, w, D, dh_t, D, rows, D, V), st);
  } else {
    GemmArgs g = gemm_args(dlogits, V, w, D, dh_acc, 0, rows, D, V);
    g.k_per_split = gemm_k_per_split(V, splits);
    const int used = (V + g.k_per_split - 1) / g.k_per_split;
    e = launch_gemm(GEMM_NN, EPI_STORE_F32, g, st);
    if (e == hipSuccess) e = launch_sum_slices(dh_acc, used, rows, D, dh_t, D, st);
  }
  if (e != hipSuccess) return e;
  GemmArgs g = gemm_args(dlogits, V, ht, D, dw_acc, 0, V, D, rows);
  g.k_per_split = gemm_k_per_split(rows, 1);
  return launch_gemm(GEMM_TN, first ? EPI_STORE_F32 : EPI_ADD_F32, g, st);
}

// debug mode: the tile's buffers are NaN-filled before the tile
hipError_t debug_fill(void* p, size_t bytes, hipStream_t st) {
  if (!g_debug_fill || !p) return hipSuccess;
  return launch_fill(p, bytes, 0xFFFFFFFFu, st);
}

}  // namespace

extern "C" {

int upipe_loss_workspace_bytes(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                               int32_t pass, size_t* bytes) {
  if (!bytes || (pass != UPIPE_PASS_FWD && pass != UPIPE_PASS_BWD && pass != UPIPE_PASS_FWD_BWD))
    return UPIPE_EINVAL;
  LossShape s;
  const int rc = check_loss_shape(seq_len, hidden, vocab, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  *bytes = make_loss_plan(s, pass).total;
  return UPIPE_OK;
}

int upipe_loss_choose_tile(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t pass,
                           size_t budget_bytes, int32_t* tile_rows, size_t* bytes) {
  if (!tile_rows || !bytes ||
      (pass != UPIPE_PASS_FWD && pass != UPIPE_PASS_BWD && pass != UPIPE_PASS_FWD_BWD))
    return UPIPE_EINVAL;
  LossShape s;
  int rc = check_loss_shape(seq_len, hidden, vocab, 1, &s);
  if (rc != UPIPE_OK) return rc;
  // candidates: multiples of 256 rows and the whole sequence; the largest
  // that fits wins (the size is not monotone in the tile where the split
  // buffers of short tiles appear)
  int64_t best = 0;
  size_t best_bytes = 0;
  for (int64_t t = 256; t < seq_len + 256; t += 256) {
    const int64_t tt = t < seq_len ? t : seq_len;
    LossShape c;
    if (check_loss_shape(seq_len, hidden, vocab, (int32_t)tt, &c) != UPIPE_OK) continue;
    const size_t b = make_loss_plan(c, pass).total;
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

int upipe_loss_fwd(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                   const uint16_t* h, const uint16_t* w, const int32_t* targets,
                   int32_t ignore_index, float* loss, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  LossShape s;
  int rc = check_loss_shape(seq_len, hidden, vocab, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  if (!h || !w || !targets || !loss || !lse) return UPIPE_EINVAL;
  if (!aligned16(h) || !aligned16(w) || !aligned4(targets) || !aligned4(loss) || !aligned4(lse))
    return UPIPE_EINVAL;
  rc = check_ws(s, UPIPE_PASS_FWD, workspace, workspace_bytes);
  if (rc != UPIPE_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const LossPlan p = make_loss_plan(s, UPIPE_PASS_FWD);
  float* stats = at<float>(workspace, p.stats);
  float* tlogit = at<float>(workspace, p.tlogit);
  float* loss_rows = at<float>(workspace, p.loss_rows);
  const int nct = col_tiles(s);
  for (int64_t t0 = 0; t0 < s.L; t0 += s.T) {
    const int rows = (int)(s.L - t0 < s.T ? s.L - t0 : s.T);
    UPIPE_TRY(debug_fill(stats, (size_t)s.T * nct * 8, st));
    UPIPE_TRY(debug_fill(tlogit, (size_t)s.T * 4, st));
    GemmArgs g = logits_args(h + t0 * s.D, w, rows, s, targets, ignore_index, t0);
    g.ce_stats = stats;
    g.ce_tlogit = tlogit;
    UPIPE_TRY(launch_gemm(GEMM_NT, EPI_CE_STATS, g, st));
    hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)rows), dim3(256), 0, st, stats, nct,
                       tlogit, s.V, targets, t0, ignore_index, lse, loss_rows);
    UPIPE_TRY(hipGetLastError());
  }
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(1024), 0, st, loss_rows, targets, s.L,
                     ignore_index, 0.f, loss, (float*)nullptr);
  UPIPE_TRY(hipGetLastError());
  return UPIPE_OK;
}

int upipe_loss_bwd(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                   const uint16_t* h, const uint16_t* w, const int32_t* targets,
                   int32_t ignore_index, const float* lse, float dloss, uint16_t* dh,
                   uint16_t* dw, void* workspace, size_t workspace_bytes, void* stream) {
  LossShape s;
  int rc = check_loss_shape(seq_len, hidden, vocab, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  if (!h || !w || !targets || !lse || !dh || !dw) return UPIPE_EINVAL;
  if (!aligned16(h) || !aligned16(w) || !aligned4(targets) || !aligned4(lse) || !aligned16(dh) ||
      !aligned16(dw))
    return UPIPE_EINVAL;
  rc = check_ws(s, UPIPE_PASS_BWD, workspace, workspace_bytes);
  if (rc != UPIPE_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const LossPlan p = make_loss_plan(s, UPIPE_PASS_BWD);
  uint16_t* dlogits = at<uint16_t>(workspace, p.dlogits);
  float* dh_acc = at<float>(workspace, p.dh_acc);
  float* dw_acc = at<float>(workspace, p.dw_acc);
  float* scale = at<float>(workspace, p.scale);
  const int D = s.D, V = s.V;
  const int splits = dh_acc ? dh_splits(s) : 1;
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(1024), 0, st, (const float*)nullptr, targets,
                     s.L, ignore_index, dloss, (float*)nullptr, scale);
  UPIPE_TRY(hipGetLastError());
  for (int64_t t0 = 0; t0 < s.L; t0 += s.T) {
    const int rows = (int)(s.L - t0 < s.T ? s.L - t0 : s.T);
    const uint16_t* ht = h + t0 * D;
    UPIPE_TRY(debug_fill(dlogits, (size_t)s.T * V * 2, st));
    GemmArgs gl = logits_args(ht, w, rows, s, targets, ignore_index, t0);
    gl.C = dlogits;
    gl.ce_lse = lse;
    gl.ce_scale = scale;
    UPIPE_TRY(launch_gemm(GEMM_NT, EPI_CE_GRAD, gl, st));
    UPIPE_TRY(grads_of_tile(dlogits, ht, w, dh + t0 * D, dh_acc, dw_acc, rows, splits, s, t0 == 0, st));
  }
  RowSegments ident;
  memset(&ident, 0, sizeof(ident));
  UPIPE_TRY(launch_acc_to_bf16(dw_acc, V, D, dw, D, ident, st));
  return UPIPE_OK;
}

int upipe_loss_fwd_bwd(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                       const uint16_t* h, const uint16_t* w, const int32_t* targets,
                       int32_t ignore_index, float dloss, float* loss, float* lse, uint16_t* dh,
                       uint16_t* dw, void* workspace, size_t workspace_bytes, void* stream) {
  LossShape s;
  int rc = check_loss_shape(seq_len, hidden, vocab, tile_rows, &s);
  if (rc != UPIPE_OK) return rc;
  if (!h || !w || !targets || !loss || !lse || !dh || !dw) return UPIPE_EINVAL;
  if (!aligned16(h) || !aligned16(w) || !aligned4(targets) || !aligned4(loss) || !aligned4(lse) ||
      !aligned16(dh) || !aligned16(dw))
    return UPIPE_EINVAL;
  rc = check_ws(s, UPIPE_PASS_FWD_BWD, workspace, workspace_bytes);
  if (rc != UPIPE_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const LossPlan p = make_loss_plan(s, UPIPE_PASS_FWD_BWD);
  float* stats = at<float>(workspace, p.stats);
  float* tlogit = at<float>(workspace, p.tlogit);
  float* loss_rows = at<float>(workspace, p.loss_rows);
  uint16_t* dlogits = at<uint16_t>(workspace, p.dlogits);
  float* dh_acc = at<float>(workspace, p.dh_acc);
  float* dw_acc = at<float>(workspace, p.dw_acc);
  float* scale = at<float>(workspace, p.scale);
  const int D = s.D, V = s.V, nct = col_tiles(s);
  const int splits = dh_acc ? dh_splits(s) : 1;
  // the count of counted rows (hence dloss / count) depends on the targets
  // only, so the gradients of each tile follow its forward at once
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(1024), 0, st, (const float*)nullptr, targets,
                     s.L, ignore_index, dloss, (float*)nullptr, scale);
  UPIPE_TRY(hipGetLastError());
  for (int64_t t0 = 0; t0 < s.L; t0 += s.T) {
    const int rows = (int)(s.L - t0 < s.T ? s.L - t0 : s.T);
    const uint16_t* ht = h + t0 * D;
    UPIPE_TRY(debug_fill(stats, (size_t)s.T * nct * 8, st));
    UPIPE_TRY(debug_fill(tlogit, (size_t)s.T * 4, st));
    UPIPE_TRY(debug_fill(dlogits, (size_t)s.T * V * 2, st));
    // logits once: row statistics, target logits and fp16 logits
    GemmArgs g = logits_args(ht, w, rows, s, targets, ignore_index, t0);
    g.ce_stats = stats;
    g.ce_tlogit = tlogit;
    g.ce_logits16 = dlogits;
    UPIPE_TRY(launch_gemm(GEMM_NT, EPI_CE_STATS, g, st));
    hipLaunchKernelGGL(ce_combine_kernel, dim3((unsigned)rows), dim3(256), 0, st, stats, nct,
                       tlogit, V, targets, t0, ignore_index, lse, loss_rows);
    UPIPE_TRY(hipGetLastError());
    const int64_t chunks = (int64_t)rows * (V / 8);
    hipLaunchKernelGGL(ce_grad_f16_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st,
                       dlogits, V, targets, t0, rows, lse, scale, ignore_index);
    UPIPE_TRY(hipGetLastError());
    UPIPE_TRY(grads_of_tile(dlogits, ht, w, dh + t0 * D, dh_acc, dw_acc, rows, splits, s, t0 == 0, st));
  }
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(1024), 0, st, loss_rows, targets, s.L,
                     ignore_index, 0.f, loss, (float*)nullptr);
  UPIPE_TRY(hipGetLastError());
  RowSegments ident;
  memset(&ident, 0, sizeof(ident));
  UPIPE_TRY(launch_acc_to_bf16(dw_acc, V, D, dw, D, ident, st));
  return UPIPE_OK;
}

}  // extern "C"
