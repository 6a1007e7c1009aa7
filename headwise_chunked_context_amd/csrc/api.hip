// C ABI of the headwise-chunked causal GQA attention layer: argument checks,
// workspace planning and the chunk scheduler (host side, one HIP stream).
//
// The schedule is the method's: one head chunk at a time, the chunk's rows of
// W_qkv project its q (and k/v when a KV group is first touched), attention
// runs and the per-head output is stored as the chunk's partial result; the
// next chunk reuses the same workspace buffers
// ("Untied Ulysses Pushes Llama-3-8B Training to 5 Million Tokens", Untied
// Ulysses section).  A KV group stays resident in the workspace while any of
// its query heads is being processed (grouped-query tailoring, same section).
#include <math.h>
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "../../include/upipe_attn.h"
#include "kernels.h"

using namespace upipe;

namespace upipe {
bool g_debug_fill = false;

thread_local hipError_t t_last_hip_error = hipSuccess;
void note_hip_error(hipError_t e) { t_last_hip_error = e; }
}

namespace {

constexpr int64_t kMaxL = int64_t(1) << 24;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t round_up64(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Factor the rotated q is stored with: log2(e) / sqrt(d), the softmax scale
// and the change to base 2, so that q . k is the score in base-2 units
float q_prescale(int d) { return kLog2e / sqrtf((float)d); }

struct Shape {
  int64_t L, Lp;
  int D, Hq, Hkv, d, hc, G, kc;  // kc = KV heads a chunk touches
  bool proj;
};

int check_shape(int64_t L, int32_t hidden, int32_t n_q, int32_t n_kv, int32_t head_dim,
                int32_t hc, Shape* s) {
  if (L < 1 || hidden < 0 || n_q < 1 || n_kv < 1 || head_dim < 1 || hc < 1) return UPIPE_EINVAL;
  if (n_q % n_kv != 0) return UPIPE_EINVAL;
  if (head_dim != 128) return UPIPE_EUNSUPPORTED;
  if (hidden % 128 != 0) return UPIPE_EUNSUPPORTED;
  if (L > kMaxL) return UPIPE_EUNSUPPORTED;
  const int G = n_q / n_kv;
  if (n_q % hc != 0) return UPIPE_ECHUNK;
  if (!(hc % G == 0 || G % hc == 0)) return UPIPE_ECHUNK;
  s->L = L;
  s->Lp = round_up64(L, 256);
  s->D = hidden;
  s->Hq = n_q;
  s->Hkv = n_kv;
  s->d = head_dim;
  s->hc = hc;
  s->G = G;
  s->kc = hc >= G ? hc / G : 1;
  s->proj = hidden > 0;
  // every launch must stay below 2^32 work-items (the dispatch packet's
  // grid size is 32-bit): attention grids are Lp/128 workgroups per head
  // (256 threads, 512 for dK/dV per KV head); the sequence-long GEMMs are
  // 256 x 256 tiles of 512 threads, the weight-gradient GEMMs at most 32
  // splits of them
  const int64_t lim = (int64_t)UINT32_MAX;
  const int64_t width = (int64_t)(hc + 2 * s->kc) * head_dim;
  const int64_t wide = width > hidden ? width : hidden;
  const int64_t mt = (s->Lp + 255) / 256;
  if ((s->Lp / 128) * hc * 256 > lim || (s->Lp / 128) * s->kc * 512 > lim ||
      mt * ((wide + 255) / 256) * 512 > lim ||
      ((int64_t)(hidden + 255) / 256) * ((width + 255) / 256) * 32 * 512 > lim)
    return UPIPE_EUNSUPPORTED;
  return UPIPE_OK;
}

// Workspace layout.  Every buffer that grows with the sequence is either
// per q head of ONE chunk (hc) or per KV head a chunk touches (kc): the size
// is affine in hc and independent of Hq.
struct Plan {
  size_t staging;              // [L][(hc+2kc)d] bf16 GEMM output / gradient staging
  size_t q_rm;                 // [hc][Lp][d] bf16, rotated
  size_t k_rm, v_rm;           // [kc][Lp][d] bf16 (k rotated; v fp16 in the forward)
  size_t q_rm2, k_rm2, v_rm2;  // the same, second slot (forward and backward pipeline)
  size_t staging2, do_rm2, lse2_2, dvec2, dw_acc2;  // second slot (backward pipeline)
  size_t do_rm;                // [hc][Lp][d] bf16 (bwd)
  size_t lse2, dvec;           // [hc][Lp] fp32 (bwd)
  size_t dk_acc, dv_acc;       // [kc][Lp][d] fp32 (bwd, only when a group spans chunks)
  size_t dw_acc;               // fp32 weight-gradient accumulator (bwd, projection mode)
  size_t o_c;                  // [L][hc d] bf16 recomputed attention output (bwd recompute)
  size_t v_t;                  // [kc][Lp][d] fp16 transposed V tiles (bwd recompute)
  size_t total;
};

Plan make_plan(const Shape& s, int pass) {
  Plan p;
  memset(&p, 0, sizeof(p));
  const size_t Lp = (size_t)s.Lp, d = (size_t)s.d, hc = (size_t)s.hc, kc = (size_t)s.kc;
  const size_t width = (hc + 2 * kc) * d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t head_bf16 = Lp * d * 2;
  const size_t no = (size_t)-1;
  p.staging = s.proj ? take((size_t)s.L * width * 2) : no;
  p.q_rm = take(hc * head_bf16);
  p.k_rm = take(kc * head_bf16);
  p.v_rm = take(kc * head_bf16);
  if (pass == UPIPE_PASS_FWD_PIPELINED || pass == UPIPE_PASS_BWD_PIPELINED) {
    // the next chunk's q/k/v are prepared while this chunk's attention runs
    p.q_rm2 = take(hc * head_bf16);
    p.k_rm2 = take(kc * head_bf16);
    p.v_rm2 = take(kc * head_bf16);
  } else {
    p.q_rm2 = p.k_rm2 = p.v_rm2 = no;
  }
  p.o_c = p.v_t = no;
  p.staging2 = p.do_rm2 = p.lse2_2 = p.dvec2 = p.dw_acc2 = no;
  if (pass == UPIPE_PASS_BWD_PIPELINED) {
    // the rest of the next chunk's slot: its staging block, dO, LSE2 and D
    // rows and its weight-gradient accumulator
    p.staging2 = s.proj ? take((size_t)s.L * width * 2) : no;
    p.do_rm2 = take(hc * head_bf16);
    p.lse2_2 = take(hc * Lp * 4);
    p.dvec2 = take(hc * Lp * 4);
    p.dw_acc2 = s.proj ? take(width * (size_t)s.D * 4) : no;
  }
  if (pass == UPIPE_PASS_BWD || pass == UPIPE_PASS_BWD_RECOMPUTE || pass == UPIPE_PASS_BWD_PIPELINED) {
    p.do_rm = take(hc * head_bf16);
    p.lse2 = take(hc * Lp * 4);
    p.dvec = take(hc * Lp * 4);
    // cross-chunk dK/dV accumulators (used while a KV group spans chunks;
    // always reserved so the size stays affine in the chunk)
    p.dk_acc = take(kc * Lp * d * 4);
    p.dv_acc = take(kc * Lp * d * 4);
    // fp32 split-K accumulator of the weight gradients: dW_o[:, cols(c)] is
    // [D][hc d], dW_qkv[rows(c)] is [(hc+2kc) d][D]
    p.dw_acc = s.proj ? take(width * (size_t)s.D * 4) : no;
    if (pass == UPIPE_PASS_BWD_RECOMPUTE) {
      // the chunk's attention output, recomputed (its LSE goes to lse2,
      // which prep_dout rewrites afterwards), and the forward's V tiles,
      // which persist while a KV group spans chunks
      p.o_c = take((size_t)s.L * hc * d * 2);
      p.v_t = take(kc * head_bf16);
    }
  } else {
    p.do_rm = p.lse2 = p.dvec = p.dk_acc = p.dv_acc = p.dw_acc = no;
  }
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return off == (size_t)-1 ? nullptr : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

RopeTable make_rope(double theta, int d) {
  RopeTable t;
  for (int i = 0; i < d / 2; ++i)
    t.rev_per_pos[i] = pow(theta, -2.0 * i / d) / (2.0 * M_PI);
  return t;
}

int check_common(const Shape& s, double theta, const void* x, const void* w_qkv, const void* w_o,
                 void* ws, size_t ws_bytes, int pass) {
  if (!(theta > 0.0) || !isfinite(theta)) return UPIPE_EINVAL;
  if (!x) return UPIPE_EINVAL;
  if (s.proj != (w_qkv != nullptr) || s.proj != (w_o != nullptr)) return UPIPE_EINVAL;
  if (!aligned16(x) || (w_qkv && !aligned16(w_qkv)) || (w_o && !aligned16(w_o))) return UPIPE_EINVAL;
  Plan p = make_plan(s, pass);
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0 || ws_bytes < p.total)
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

// ---- optional per-kernel-class timing (see upipe_profile_enable)
constexpr int kKinds = 8;
static_assert(UPIPE_PROFILE_ALL == (1 << kKinds) - 1, "one mask bit per kernel class");
struct Profiler {
  int mask = 0;  // bit k: launches of kernel class k are bracketed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[kKinds];
  std::vector<hipEvent_t> pool;
};
Profiler g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <typename F>
hipError_t timed(int kind, hipStream_t st, F&& launch) {
  if (!((g_prof.mask >> kind) & 1)) return launch();
  hipEvent_t a = prof_event(), b = prof_event();
  auto give_back = [&]() {  // events of a failed bracket return to the pool
    if (a) g_prof.pool.push_back(a);
    if (b) g_prof.pool.push_back(b);
  };
  if (!a || !b) {
    give_back();
    return hipErrorOutOfMemory;
  }
  if (hipEventRecord(a, st) != hipSuccess) {
    give_back();
    return hipErrorUnknown;
  }
  hipError_t e = launch();
  if (hipEventRecord(b, st) != hipSuccess) {
    give_back();
    return hipErrorUnknown;
  }
  g_prof.rec[kind].push_back({a, b});
  return e;
}

#define UPIPE_LAUNCH(kind, expr) UPIPE_TRY(timed((kind), st, [&]() { return (expr); }))

// ---- two-slot pipeline: a second stream per device.  While chunk c's
// attention runs on the caller's stream, chunk c+1's projection and layout
// pass run on this one into the other slot of q/k/v buffers; events order
// the slot hand-over in both directions.  The stream and its events are
// created on a device's first pipelined call and kept for the process.
constexpr int kMaxDevices = 64;
struct Side {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t ready[2] = {nullptr, nullptr};  // slot's q/k/v prepared
  hipEvent_t done[2] = {nullptr, nullptr};   // slot's attention finished
};
Side g_side[kMaxDevices];
std::mutex g_side_mu;
bool g_pipeline = false;

// debug mode: NaN-fill (0xFF bytes) a buffer on the stream that will write it
hipError_t debug_fill(void* p, size_t bytes, hipStream_t st) {
  if (!g_debug_fill || !p) return hipSuccess;
  return timed(UPIPE_KERNEL_FINALIZE, st, [&]() { return launch_fill(p, bytes, 0xFFFFFFFFu, st); });
}

int side_stream(Side** out) {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    note_hip_error(ge != hipSuccess ? ge : hipErrorInvalidDevice);
    return UPIPE_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_side_mu);
  Side& sd = g_side[dev];
  if (!sd.stream) {
    // created into a local copy and published only when everything exists,
    // so a failed attempt leaves nothing behind and the next call retries
    Side fresh;
    hipEvent_t* evs[5] = {&fresh.fork, &fresh.ready[0], &fresh.ready[1], &fresh.done[0],
                          &fresh.done[1]};
    hipError_t err = hipSuccess;
    for (hipEvent_t* e : evs)
      if (err == hipSuccess) err = hipEventCreateWithFlags(e, hipEventDisableTiming);
    if (err == hipSuccess) err = hipStreamCreateWithFlags(&fresh.stream, hipStreamNonBlocking);
    if (err != hipSuccess) {
      for (hipEvent_t* e : evs)
        if (*e) (void)hipEventDestroy(*e);
      if (fresh.stream) (void)hipStreamDestroy(fresh.stream);
      note_hip_error(err);
      return UPIPE_EHIP;
    }
    sd = fresh;
  }
  *out = &sd;
  return UPIPE_OK;
}

struct Chunk {
  int h0;        // first q head
  int g0;        // first KV group touched
  int nkv;       // KV groups touched (kc)
  bool kv_first; // the chunk starts its KV groups (project / prepare K, V)
  bool kv_last;  // the chunk finishes its KV groups
};

Chunk chunk_info(const Shape& s, int c) {
  Chunk ch;
  ch.h0 = c * s.hc;
  ch.g0 = ch.h0 / s.G;
  ch.nkv = s.kc;
  ch.kv_first = (ch.h0 % s.G) == 0;
  ch.kv_last = ((ch.h0 + s.hc) % s.G) == 0;
  return ch;
}

// Project the chunk's q (and k, v when it starts a group).  q and k leave
// the GEMM rotated and head-major, straight in q_rm / k_rm ([head][Lp][d],
// all Lp rows: the padding rows L .. Lp-1 repeat x's last row, rotated at
// their own positions, finite values that every attention kernel masks); v
// goes to staging[L][hc*d | kc*d | kc*d] at its columns, for the layout
// pass.
int project_chunk(const Shape& s, const Chunk& ch, const uint16_t* x, const uint16_t* w_qkv,
                  uint16_t* staging, uint16_t* q_rm, uint16_t* k_rm, const RopeTable& rope,
                  hipStream_t st) {
  const int d = s.d;
  const int width = (s.hc + 2 * s.kc) * d;
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = x;
  g.lda = s.D;
  g.B = w_qkv;
  g.ldb = s.D;
  g.bseg.count = ch.kv_first ? 3 : 1;
  g.bseg.end[0] = s.hc * d;
  g.bseg.row0[0] = (int64_t)ch.h0 * d;
  g.bseg.end[1] = (s.hc + s.kc) * d;
  g.bseg.row0[1] = (int64_t)(s.Hq + ch.g0) * d;
  g.bseg.end[2] = width;
  g.bseg.row0[2] = (int64_t)(s.Hq + s.Hkv + ch.g0) * d;
  g.C = staging;
  g.ldc = width;
  g.M = (int)s.Lp;
  g.rows_valid = (int)s.L;
  g.N = ch.kv_first ? width : s.hc * d;
  g.K = s.D;
  g.k_per_split = s.D;
  g.hm_q = q_rm;
  g.hm_k = k_rm;
  g.hm_split = s.hc * d;
  g.hm_end = ch.kv_first ? (s.hc + s.kc) * d : s.hc * d;
  g.hm_stride = s.Lp * d;
  g.hm_q_scale = q_prescale(d);
  // q and k leave the GEMM already rotated: one bf16 rounding after RoPE;
  // v leaves it as fp16 (the forward's P V product takes fp16 operands)
  g.rope_cols = (s.hc + s.kc) * d;
  g.f16_from = (s.hc + s.kc) * d;
  g.rope = rope;
  UPIPE_LAUNCH(UPIPE_KERNEL_GEMM, launch_gemm(GEMM_NT, EPI_STORE_BF16, g, st));
  return UPIPE_OK;
}

}  // namespace

extern "C" {

int upipe_version(void) { return 100; }

int upipe_pipeline_enable(int on) {
  g_pipeline = on != 0;
  return UPIPE_OK;
}

int upipe_last_hip_error(void) { return (int)t_last_hip_error; }

const char* upipe_last_hip_error_string(void) {
  return t_last_hip_error == hipSuccess ? "no HIP error recorded" : hipGetErrorString(t_last_hip_error);
}

int upipe_debug_enable(int on) {
  g_debug_fill = on != 0;
  return UPIPE_OK;
}

int upipe_profile_enable(int mask) {
  if (mask < 0 || mask > UPIPE_PROFILE_ALL) return UPIPE_EINVAL;
  for (int k = 0; k < kKinds; ++k) {
    for (auto& pr : g_prof.rec[k]) {
      g_prof.pool.push_back(pr.first);
      g_prof.pool.push_back(pr.second);
    }
    g_prof.rec[k].clear();
  }
  g_prof.mask = mask;
  return UPIPE_OK;
}

int upipe_profile_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= kKinds || !total_ms || !launches) return UPIPE_EINVAL;
  double sum = 0.0;
  for (auto& pr : g_prof.rec[kind]) {
    UPIPE_TRY(hipEventSynchronize(pr.second));
    float ms = 0.f;
    UPIPE_TRY(hipEventElapsedTime(&ms, pr.first, pr.second));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)g_prof.rec[kind].size();
  return UPIPE_OK;
}

const char* upipe_strerror(int status) {
  switch (status) {
    case UPIPE_OK: return "ok";
    case UPIPE_EINVAL: return "invalid argument (sizes, head counts, pointers or theta)";
    case UPIPE_EUNSUPPORTED: return "unsupported shape (head_dim must be 128, hidden a multiple of 128, L <= 2^24, launch grids below 2^32 threads)";
    case UPIPE_ECHUNK: return "head_chunk must divide n_q_heads and not split a KV group's query heads";
    case UPIPE_EWORKSPACE: return "workspace missing, not 256-byte aligned, or smaller than upipe_attn_workspace_bytes";
    case UPIPE_EHIP: return "HIP runtime error while launching a kernel";
    case UPIPE_ESCRATCH: return "the shapes need more workspace than the static scratch of upipe_attn_fwd_static holds (256 MiB); use upipe_attn_fwd with a workspace";
    default: return "unknown status";
  }
}

int upipe_attn_workspace_bytes(int64_t seq_len, int32_t hidden, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t head_chunk,
                               int32_t pass, size_t* bytes) {
  if (!bytes || pass < UPIPE_PASS_FWD || pass > UPIPE_PASS_BWD_PIPELINED) return UPIPE_EINVAL;
  Shape s;
  int rc = check_shape(seq_len, hidden, n_q_heads, n_kv_heads, head_dim, head_chunk, &s);
  if (rc != UPIPE_OK) return rc;
  if (pass == UPIPE_PASS_BWD_RECOMPUTE && !s.proj) return UPIPE_EINVAL;
  *bytes = make_plan(s, pass).total;
  return UPIPE_OK;
}

}  // extern "C"

namespace {

// The forward after its argument checks.  `pipelined` selects the two-slot
// schedule (its workspace layout and second stream).
int attn_fwd_run(const Shape& s, double rope_theta, const uint16_t* x, const uint16_t* w_qkv,
                 const uint16_t* w_o, uint16_t* y, uint16_t* o_saved, float* lse, void* workspace,
                 bool pipelined, hipStream_t st) {
  int rc = UPIPE_OK;
  const int pass = pipelined ? UPIPE_PASS_FWD_PIPELINED : UPIPE_PASS_FWD;
  const Plan p = make_plan(s, pass);
  const RopeTable rope = make_rope(rope_theta, s.d);
  const int d = s.d;
  uint16_t* staging = at<uint16_t>(workspace, p.staging);
  uint16_t* q_slot[2] = {at<uint16_t>(workspace, p.q_rm), at<uint16_t>(workspace, p.q_rm2)};
  uint16_t* k_slot[2] = {at<uint16_t>(workspace, p.k_rm), at<uint16_t>(workspace, p.k_rm2)};
  uint16_t* v_slot[2] = {at<uint16_t>(workspace, p.v_rm), at<uint16_t>(workspace, p.v_rm2)};
  const int64_t qkv_ld = (int64_t)(s.Hq + 2 * s.Hkv) * d;
  const int width = (s.hc + 2 * s.kc) * d;
  const int nchunks = s.Hq / s.hc;

  // Chunk c's q uses slot c % 2; a KV group's k/v use the slot after the
  // previous group's.  The projection half of chunk c waits for chunk
  // c - 2's attention (the last reader of its q slot; a KV slot's last
  // reader is at least as early), the attention of chunk c for its
  // projection half.
  Side* side = nullptr;
  hipStream_t sb = st;
  if (pipelined && nchunks > 1) {
    rc = side_stream(&side);
    if (rc != UPIPE_OK) return rc;
    sb = side->stream;
    UPIPE_TRY(hipEventRecord(side->fork, st));
    UPIPE_TRY(hipStreamWaitEvent(sb, side->fork, 0));
  }
  int kslot = 1;
  for (int c = 0; c < nchunks; ++c) {
    const Chunk ch = chunk_info(s, c);
    const int qslot = side ? c & 1 : 0;
    if (ch.kv_first) kslot = side ? kslot ^ 1 : 0;
    uint16_t* q_rm = q_slot[qslot];
    uint16_t* k_rm = k_slot[kslot];
    uint16_t* v_rm = v_slot[kslot];
    if (side && c >= 2) UPIPE_TRY(hipStreamWaitEvent(sb, side->done[qslot], 0));
    {
      const size_t head_bytes = (size_t)s.Lp * d * 2;
      if (staging) UPIPE_TRY(debug_fill(staging, (size_t)s.L * width * 2, sb));
      UPIPE_TRY(debug_fill(q_rm, s.hc * head_bytes, sb));
      if (ch.kv_first) {
        UPIPE_TRY(debug_fill(k_rm, s.kc * head_bytes, sb));
        UPIPE_TRY(debug_fill(v_rm, s.kc * head_bytes, sb));
      }
    }
    // 1. chunked QKV projection (or pick the given q/k/v columns) + RoPE
    PrepArgs pa;
    memset(&pa, 0, sizeof(pa));
    if (s.proj) {
      rc = project_chunk(s, ch, x, w_qkv, staging, q_rm, k_rm, rope, sb);
      if (rc != UPIPE_OK) return rc;
      pa.src_v = staging + (s.hc + s.kc) * d;
      pa.src_ld = width;
      pa.v_only = 1;  // q and k are in place
    } else {
      pa.src_q = x + (int64_t)ch.h0 * d;
      pa.src_k = x + (int64_t)(s.Hq + ch.g0) * d;
      pa.src_v = x + (int64_t)(s.Hq + s.Hkv + ch.g0) * d;
      pa.src_ld = qkv_ld;
    }
    pa.nq = s.hc;
    pa.nkv = ch.kv_first ? s.kc : 0;
    pa.q_rm = q_rm;
    pa.k_rm = k_rm;
    pa.v_rm = v_rm;
    pa.L = s.L;
    pa.Lp = s.Lp;
    pa.rotate = s.proj ? 0 : 1;
    pa.q_scale = q_prescale(d);
    pa.v_src_f16 = s.proj ? 1 : 0;
    pa.v_out_f16 = 1;
    pa.v_tiles = 1;
    if (!pa.v_only || pa.nkv > 0)
      UPIPE_TRY(timed(UPIPE_KERNEL_PREP, sb, [&]() { return launch_prep_qkv(pa, rope, sb); }));
    if (side) {
      UPIPE_TRY(hipEventRecord(side->ready[qslot], sb));
      UPIPE_TRY(hipStreamWaitEvent(st, side->ready[qslot], 0));
    }

    // 2. causal attention of the chunk's heads; stores O and LSE
    FwdArgs fa;
    memset(&fa, 0, sizeof(fa));
    fa.q = q_rm;
    fa.k = k_rm;
    fa.v = v_rm;
    fa.nh = s.hc;
    fa.group = s.G;
    fa.q_head0 = ch.h0;
    fa.kv_head0 = ch.g0;
    fa.o_head0 = 0;
    fa.o = o_saved;
    fa.o_ld = (int64_t)s.Hq * d;
    fa.lse = lse;
    fa.L = s.L;
    fa.Lp = s.Lp;
    UPIPE_LAUNCH(UPIPE_KERNEL_ATTN_FWD, launch_flash_fwd(fa, st));
    if (side) UPIPE_TRY(hipEventRecord(side->done[qslot], st));
  }

  // 3. output projection: y = sum over chunks of O_c W_o[:, cols(c)]^T.  The
  // chunks' partial results are the column blocks of o_saved; the GEMM's K
  // loop walks them chunk after chunk and accumulates in fp32, so y is
  // rounded to bf16 once instead of once per chunk.
  if (s.proj) {
    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.A = o_saved;
    g.lda = (int64_t)s.Hq * d;
    g.B = w_o;
    g.ldb = (int64_t)s.Hq * d;
    g.C = y;
    g.ldc = s.D;
    g.M = (int)s.L;
    g.N = s.D;
    g.K = s.Hq * d;
    g.k_per_split = g.K;
    UPIPE_LAUNCH(UPIPE_KERNEL_GEMM, launch_gemm(GEMM_NT, EPI_STORE_BF16, g, st));
  }
  return UPIPE_OK;
}

int check_fwd_outputs(const Shape& s, const uint16_t* y, const uint16_t* o_saved, const float* lse) {
  if (!o_saved || !lse || s.proj != (y != nullptr)) return UPIPE_EINVAL;
  if (!aligned16(o_saved) || !aligned16(lse) || (y && !aligned16(y))) return UPIPE_EINVAL;
  return UPIPE_OK;
}

// ---- the allocation-free forward's scratch: a static device array that
// stands in for the workspace.  Its host-side name is not a device address:
// the address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that pointer is handed to kernels.
constexpr size_t kScratchBytes = UPIPE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

int scratch_ptr(void** out) {
  int dev = -1;
  UPIPE_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return UPIPE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    UPIPE_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) UPIPE_TRY(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return UPIPE_OK;
}

}  // namespace

extern "C" {

int upipe_attn_choose_chunk(int64_t seq_len, int32_t hidden, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int32_t pass,
                            size_t budget_bytes, int32_t* head_chunk, size_t* bytes) {
  if (!head_chunk || !bytes || pass < UPIPE_PASS_FWD || pass > UPIPE_PASS_BWD_PIPELINED)
    return UPIPE_EINVAL;
  int best = 0, first_rc = UPIPE_ECHUNK;
  size_t best_bytes = 0;
  for (int c = 1; c <= n_q_heads; ++c) {
    size_t b = 0;
    const int rc = upipe_attn_workspace_bytes(seq_len, hidden, n_q_heads, n_kv_heads, head_dim, c,
                                              pass, &b);
    if (rc == UPIPE_ECHUNK) continue;  // not a valid chunk for these head counts
    if (rc != UPIPE_OK) return rc;     // the shapes themselves are refused
    first_rc = UPIPE_OK;
    if (b <= budget_bytes) {           // the workspace grows with the chunk: keep the largest
      best = c;
      best_bytes = b;
    }
  }
  if (first_rc != UPIPE_OK) return first_rc;
  if (best == 0) return UPIPE_EWORKSPACE;
  *head_chunk = best;
  *bytes = best_bytes;
  return UPIPE_OK;
}

int upipe_attn_fwd(int64_t seq_len, int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, double rope_theta, int32_t head_chunk, const uint16_t* x,
                   const uint16_t* w_qkv, const uint16_t* w_o, uint16_t* y, uint16_t* o_saved,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_shape(seq_len, hidden, n_q_heads, n_kv_heads, head_dim, head_chunk, &s);
  if (rc != UPIPE_OK) return rc;
  const bool pipelined = g_pipeline;
  const int pass = pipelined ? UPIPE_PASS_FWD_PIPELINED : UPIPE_PASS_FWD;
  rc = check_common(s, rope_theta, x, w_qkv, w_o, workspace, workspace_bytes, pass);
  if (rc != UPIPE_OK) return rc;
  rc = check_fwd_outputs(s, y, o_saved, lse);
  if (rc != UPIPE_OK) return rc;
  return attn_fwd_run(s, rope_theta, x, w_qkv, w_o, y, o_saved, lse, workspace, pipelined,
                      reinterpret_cast<hipStream_t>(stream));
}

int upipe_attn_fwd_static(int64_t seq_len, int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, double rope_theta, int32_t head_chunk,
                          const uint16_t* x, const uint16_t* w_qkv, const uint16_t* w_o,
                          uint16_t* y, uint16_t* o_saved, float* lse, void* stream) {
  Shape s;
  int rc = check_shape(seq_len, hidden, n_q_heads, n_kv_heads, head_dim, head_chunk, &s);
  if (rc != UPIPE_OK) return rc;
  if (make_plan(s, UPIPE_PASS_FWD).total > kScratchBytes) return UPIPE_ESCRATCH;
  // the scratch stands in for the workspace argument of the checks
  rc = check_common(s, rope_theta, x, w_qkv, w_o, reinterpret_cast<void*>(kAlign), kScratchBytes,
                    UPIPE_PASS_FWD);
  if (rc != UPIPE_OK) return rc;
  rc = check_fwd_outputs(s, y, o_saved, lse);
  if (rc != UPIPE_OK) return rc;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc != UPIPE_OK) return rc;
  // one stream, no profiling events: nothing is created or allocated
  const int mask = g_prof.mask;
  g_prof.mask = 0;
  rc = attn_fwd_run(s, rope_theta, x, w_qkv, w_o, y, o_saved, lse, ws, false,
                    reinterpret_cast<hipStream_t>(stream));
  g_prof.mask = mask;
  return rc;
}

int upipe_attn_bwd(int64_t seq_len, int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, double rope_theta, int32_t head_chunk, const uint16_t* x,
                   const uint16_t* w_qkv, const uint16_t* w_o, const uint16_t* o_saved,
                   const float* lse, const uint16_t* dy, uint16_t* dx, uint16_t* dw_qkv,
                   uint16_t* dw_o, void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_shape(seq_len, hidden, n_q_heads, n_kv_heads, head_dim, head_chunk, &s);
  if (rc != UPIPE_OK) return rc;
  // o_saved == NULL: recompute each chunk's attention output (projection mode)
  const bool recompute = o_saved == nullptr;
  if (recompute && !s.proj) return UPIPE_EINVAL;
  // the two-slot schedule applies to the saved-output backward
  const bool pipelined = g_pipeline && !recompute;
  const int pass = recompute ? UPIPE_PASS_BWD_RECOMPUTE
                             : (pipelined ? UPIPE_PASS_BWD_PIPELINED : UPIPE_PASS_BWD);
  rc = check_common(s, rope_theta, x, w_qkv, w_o, workspace, workspace_bytes, pass);
  if (rc != UPIPE_OK) return rc;
  if (!lse || !dy || !dx) return UPIPE_EINVAL;
  if (s.proj != (dw_qkv != nullptr) || s.proj != (dw_o != nullptr)) return UPIPE_EINVAL;
  if ((o_saved && !aligned16(o_saved)) || !aligned16(lse) || !aligned16(dy) || !aligned16(dx) ||
      (dw_qkv && !aligned16(dw_qkv)) || (dw_o && !aligned16(dw_o)))
    return UPIPE_EINVAL;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Plan p = make_plan(s, pass);
  const RopeTable rope = make_rope(rope_theta, s.d);
  const int d = s.d;
  const int64_t qkv_ld = (int64_t)(s.Hq + 2 * s.Hkv) * d;
  const int width = (s.hc + 2 * s.kc) * d;
  const int nchunks = s.Hq / s.hc;
  // per-chunk buffers, two slots in the pipelined schedule (the second slot
  // of a single-slot plan is the first)
  auto slot2 = [&](size_t a, size_t b) { return b == (size_t)-1 ? a : b; };
  uint16_t* staging[2] = {at<uint16_t>(workspace, p.staging), at<uint16_t>(workspace, slot2(p.staging, p.staging2))};
  uint16_t* q_rm[2] = {at<uint16_t>(workspace, p.q_rm), at<uint16_t>(workspace, slot2(p.q_rm, p.q_rm2))};
  uint16_t* k_rm[2] = {at<uint16_t>(workspace, p.k_rm), at<uint16_t>(workspace, slot2(p.k_rm, p.k_rm2))};
  uint16_t* v_rm[2] = {at<uint16_t>(workspace, p.v_rm), at<uint16_t>(workspace, slot2(p.v_rm, p.v_rm2))};
  uint16_t* do_rm[2] = {at<uint16_t>(workspace, p.do_rm), at<uint16_t>(workspace, slot2(p.do_rm, p.do_rm2))};
  float* lse2[2] = {at<float>(workspace, p.lse2), at<float>(workspace, slot2(p.lse2, p.lse2_2))};
  float* dvec[2] = {at<float>(workspace, p.dvec), at<float>(workspace, slot2(p.dvec, p.dvec2))};
  float* dw_acc[2] = {at<float>(workspace, p.dw_acc), at<float>(workspace, slot2(p.dw_acc, p.dw_acc2))};
  float* dk_acc = at<float>(workspace, p.dk_acc);
  float* dv_acc = at<float>(workspace, p.dv_acc);
  uint16_t* o_c = at<uint16_t>(workspace, p.o_c);
  uint16_t* v_t = at<uint16_t>(workspace, p.v_t);
  const size_t dw_bytes = (size_t)width * s.D * 4;

  // the weight-gradient accumulators start at zero; each conversion pass
  // clears what it consumed
  if (dw_acc[0]) {
    UPIPE_LAUNCH(UPIPE_KERNEL_FINALIZE, launch_zero(dw_acc[0], dw_bytes, st));
    if (dw_acc[1] != dw_acc[0]) UPIPE_LAUNCH(UPIPE_KERNEL_FINALIZE, launch_zero(dw_acc[1], dw_bytes, st));
  }

  // ---- stage 1 of chunk c on stream `sq` (buffers of slot `sl`, KV slot
  // `kl`): recompute the rotated q (k, v at a group start), the attention
  // output in recompute mode, dO, D and the base-2 LSE, and dW_o
  auto stage_prepare = [&](int c, int sl, int kl, hipStream_t sq) -> int {
    const Chunk ch = chunk_info(s, c);
    if (g_debug_fill) {
      const size_t head_bytes = (size_t)s.Lp * d * 2;
      UPIPE_TRY(debug_fill(staging[sl], (size_t)s.L * width * 2, sq));
      UPIPE_TRY(debug_fill(q_rm[sl], s.hc * head_bytes, sq));
      UPIPE_TRY(debug_fill(do_rm[sl], s.hc * head_bytes, sq));
      UPIPE_TRY(debug_fill(lse2[sl], (size_t)s.hc * s.Lp * 4, sq));
      UPIPE_TRY(debug_fill(dvec[sl], (size_t)s.hc * s.Lp * 4, sq));
      UPIPE_TRY(debug_fill(o_c, (size_t)s.L * s.hc * d * 2, sq));
      if (ch.kv_first) {
        UPIPE_TRY(debug_fill(k_rm[kl], s.kc * head_bytes, sq));
        UPIPE_TRY(debug_fill(v_rm[kl], s.kc * head_bytes, sq));
        UPIPE_TRY(debug_fill(v_t, s.kc * head_bytes, sq));
      }
    }
    // 1. recompute the chunk's rotated q (and k, v at a group start)
    PrepArgs pa;
    memset(&pa, 0, sizeof(pa));
    if (s.proj) {
      const int r = project_chunk(s, ch, x, w_qkv, staging[sl], q_rm[sl], k_rm[kl], rope, sq);
      if (r != UPIPE_OK) return r;
      pa.src_v = staging[sl] + (s.hc + s.kc) * d;
      pa.src_ld = width;
      pa.v_only = 1;  // q and k are in place
    } else {
      pa.src_q = x + (int64_t)ch.h0 * d;
      pa.src_k = x + (int64_t)(s.Hq + ch.g0) * d;
      pa.src_v = x + (int64_t)(s.Hq + s.Hkv + ch.g0) * d;
      pa.src_ld = qkv_ld;
    }
    pa.nq = s.hc;
    pa.nkv = ch.kv_first ? s.kc : 0;
    pa.q_rm = q_rm[sl];
    pa.k_rm = k_rm[kl];
    pa.v_rm = v_rm[kl];
    pa.L = s.L;
    pa.Lp = s.Lp;
    pa.rotate = s.proj ? 0 : 1;
    pa.q_scale = q_prescale(d);
    pa.v_src_f16 = s.proj ? 1 : 0;
    pa.v_out_f16 = 0;
    if (!pa.v_only || pa.nkv > 0)
      UPIPE_TRY(timed(UPIPE_KERNEL_PREP, sq, [&]() { return launch_prep_qkv(pa, rope, sq); }));

    // 1b. full recompute: the chunk's attention output again, into o_c, in
    // one pass from the same q, k and (fp16 tile) v and the saved LSE
    // (P = exp(S - LSE) is final at once: no running maximum or row sum)
    if (recompute) {
      if (ch.kv_first) {
        PrepArgs pv = pa;
        pv.v_only = 1;
        pv.v_rm = v_t;
        pv.v_out_f16 = 1;
        pv.v_tiles = 1;
        UPIPE_TRY(timed(UPIPE_KERNEL_PREP, sq, [&]() { return launch_prep_qkv(pv, rope, sq); }));
      }
      FwdArgs fa;
      memset(&fa, 0, sizeof(fa));
      fa.q = q_rm[sl];
      fa.k = k_rm[kl];
      fa.v = v_t;
      fa.nh = s.hc;
      fa.group = s.G;
      fa.q_head0 = ch.h0;
      fa.kv_head0 = ch.g0;
      fa.o_head0 = ch.h0;
      fa.o = o_c;
      fa.o_ld = (int64_t)s.hc * d;
      fa.lse = nullptr;  // not written from the LSE
      fa.lse_in = lse;
      fa.L = s.L;
      fa.Lp = s.Lp;
      UPIPE_TRY(timed(UPIPE_KERNEL_ATTN_FWD, sq, [&]() { return launch_flash_fwd_lse(fa, sq); }));
    }
    const uint16_t* o_chunk = recompute ? o_c : o_saved + (int64_t)ch.h0 * d;
    const int64_t o_chunk_ld = recompute ? (int64_t)s.hc * d : (int64_t)s.Hq * d;

    // 2. dO of the chunk's heads (dy W_o[:, cols] or the given dO) and dW_o
    PrepDoutArgs pd;
    pd.o = o_chunk;
    pd.o_ld = o_chunk_ld;
    pd.lse = lse + (int64_t)ch.h0 * s.L;
    pd.nh = s.hc;
    pd.do_rm = do_rm[sl];
    pd.lse2 = lse2[sl];
    pd.dvec = dvec[sl];
    pd.L = s.L;
    pd.Lp = s.Lp;
    if (s.proj) {
      GemmArgs g;
      memset(&g, 0, sizeof(g));
      g.A = dy;
      g.lda = s.D;
      g.B = w_o + (int64_t)ch.h0 * d;
      g.ldb = (int64_t)s.Hq * d;
      g.C = staging[sl];
      g.ldc = s.hc * d;
      g.M = (int)s.L;
      g.N = s.hc * d;
      g.K = s.D;
      g.k_per_split = s.D;
      UPIPE_TRY(timed(UPIPE_KERNEL_GEMM, sq, [&]() { return launch_gemm(GEMM_NN, EPI_STORE_BF16, g, sq); }));
      pd.src_do = staging[sl];
      pd.do_ld = s.hc * d;

      // dW_o[:, cols] = dy^T O_c   (reduction over the sequence, split-K)
      const int splits = gemm_reduction_splits(s.L, s.D, s.hc * d);
      GemmArgs w;
      memset(&w, 0, sizeof(w));
      w.A = dy;
      w.lda = s.D;
      w.B = o_chunk;
      w.ldb = o_chunk_ld;
      w.C = dw_acc[sl];
      w.M = s.D;
      w.N = s.hc * d;
      w.K = (int)s.L;
      w.k_per_split = gemm_k_per_split(s.L, splits);
      UPIPE_TRY(timed(UPIPE_KERNEL_GEMM, sq, [&]() { return launch_gemm(GEMM_TN, EPI_ATOMIC_F32, w, sq); }));
      RowSegments ident;
      memset(&ident, 0, sizeof(ident));
      UPIPE_TRY(timed(UPIPE_KERNEL_FINALIZE, sq, [&]() {
        return launch_acc_to_bf16(dw_acc[sl], s.D, s.hc * d, dw_o + (int64_t)ch.h0 * d,
                                  (int64_t)s.Hq * d, ident, sq);
      }));
    } else {
      pd.src_do = dy + (int64_t)ch.h0 * d;
      pd.do_ld = (int64_t)s.Hq * d;
    }
    UPIPE_TRY(timed(UPIPE_KERNEL_PREP_DOUT, sq, [&]() { return launch_prep_dout(pd, sq); }));
    return UPIPE_OK;
  };

  // ---- stage 2 of chunk c on the caller's stream: the attention backward
  // (dK/dV of the chunk's KV groups, dQ of its heads), then dx and dW_qkv
  auto stage_attend = [&](int c, int sl, int kl) -> int {
    const Chunk ch = chunk_info(s, c);
    if (ch.kv_first) {  // the cross-chunk dK/dV accumulators start at this chunk
      UPIPE_TRY(debug_fill(dk_acc, (size_t)s.kc * s.Lp * d * 4, st));
      UPIPE_TRY(debug_fill(dv_acc, (size_t)s.kc * s.Lp * d * 4, st));
    }
    // 3. attention backward: dK/dV of the chunk's KV groups, dQ of its heads
    BwdArgs ba;
    ba.q = q_rm[sl];
    ba.k = k_rm[kl];
    ba.v = v_rm[kl];
    ba.dO = do_rm[sl];
    ba.lse2 = lse2[sl];
    ba.dvec = dvec[sl];
    ba.dk_acc = dk_acc;
    ba.dv_acc = dv_acc;
    ba.kv_first = ch.kv_first ? 1 : 0;
    ba.kv_last = ch.kv_last ? 1 : 0;
    if (s.proj) {   // rows of [dq | dk | dv] for this chunk, in the staging buffer
      ba.dq_out = staging[sl];
      ba.dq_ld = width;
      ba.dk_out = staging[sl] + s.hc * d;
      ba.dv_out = staging[sl] + (s.hc + s.kc) * d;
      ba.out_ld = width;
    } else {        // straight into the caller's dqkv
      ba.dq_out = dx + (int64_t)ch.h0 * d;
      ba.dq_ld = qkv_ld;
      ba.dk_out = dx + (int64_t)(s.Hq + ch.g0) * d;
      ba.dv_out = dx + (int64_t)(s.Hq + s.Hkv + ch.g0) * d;
      ba.out_ld = qkv_ld;
    }
    ba.nh = s.hc;
    ba.nkv = s.kc;
    ba.group = s.G;
    ba.q_head0 = ch.h0;
    ba.kv_head0 = ch.g0;
    ba.L = s.L;
    ba.Lp = s.Lp;
    ba.scale = 1.f / sqrtf((float)d);
    ba.dk_scale = ba.scale / q_prescale(d);
    ba.rope = rope;
    UPIPE_LAUNCH(UPIPE_KERNEL_ATTN_BWD_DKDV, launch_flash_bwd_dkdv(ba, st));
    UPIPE_LAUNCH(UPIPE_KERNEL_ATTN_BWD_DQ, launch_flash_bwd_dq(ba, st));

    // 4. dx (+)= [dq | dk | dv] W_qkv[rows], dW_qkv[rows] = [dq | dk | dv]^T x
    if (s.proj) {
      const int ncols = ch.kv_last ? width : s.hc * d;
      RowSegments seg;
      memset(&seg, 0, sizeof(seg));
      seg.count = ch.kv_last ? 3 : 1;
      seg.end[0] = s.hc * d;
      seg.row0[0] = (int64_t)ch.h0 * d;
      seg.end[1] = (s.hc + s.kc) * d;
      seg.row0[1] = (int64_t)(s.Hq + ch.g0) * d;
      seg.end[2] = width;
      seg.row0[2] = (int64_t)(s.Hq + s.Hkv + ch.g0) * d;

      GemmArgs g;
      memset(&g, 0, sizeof(g));
      g.A = staging[sl];
      g.lda = width;
      g.B = w_qkv;
      g.ldb = s.D;
      g.bseg = seg;
      g.C = dx;
      g.ldc = s.D;
      g.M = (int)s.L;
      g.N = s.D;
      g.K = ncols;
      g.k_per_split = ncols;
      if (c == 0)
        UPIPE_LAUNCH(UPIPE_KERNEL_GEMM, launch_gemm(GEMM_NN, EPI_STORE_BF16, g, st));
      else
        UPIPE_LAUNCH(UPIPE_KERNEL_GEMM_ACCUM, launch_gemm(GEMM_NN, EPI_ACCUM_BF16, g, st));

      const int splits = gemm_reduction_splits(s.L, ncols, s.D);
      GemmArgs w;
      memset(&w, 0, sizeof(w));
      w.A = staging[sl];
      w.lda = width;
      w.B = x;
      w.ldb = s.D;
      w.C = dw_acc[sl];
      w.M = ncols;
      w.N = s.D;
      w.K = (int)s.L;
      w.k_per_split = gemm_k_per_split(s.L, splits);
      UPIPE_LAUNCH(UPIPE_KERNEL_GEMM, launch_gemm(GEMM_TN, EPI_ATOMIC_F32, w, st));
      UPIPE_LAUNCH(UPIPE_KERNEL_FINALIZE, launch_acc_to_bf16(dw_acc[sl], ncols, s.D, dw_qkv, s.D, seg, st));
    }
    return UPIPE_OK;
  };

  if (!pipelined || nchunks == 1) {
    for (int c = 0; c < nchunks; ++c) {
      rc = stage_prepare(c, 0, 0, st);
      if (rc != UPIPE_OK) return rc;
      rc = stage_attend(c, 0, 0);
      if (rc != UPIPE_OK) return rc;
    }
    return UPIPE_OK;
  }

  // ---- two-slot schedule: chunk c+1's preparation (projection, RoPE and
  // layout, dO, dW_o) runs on a second stream into the other slot while
  // chunk c's attention backward and dx/dW_qkv run on the caller's stream.
  // Chunk c uses slot c % 2; a KV group's k/v use the slot after the
  // previous group's.  The preparation of chunk c waits for chunk c - 2's
  // stage 2 (the last reader of every buffer of its slot; a KV slot's last
  // reader is at least as early), stage 2 of chunk c for its preparation.
  // Stage 2 runs in chunk order on one stream, which orders the dK/dV
  // accumulators and the dx accumulate.
  Side* side = nullptr;
  rc = side_stream(&side);
  if (rc != UPIPE_OK) return rc;
  hipStream_t sb = side->stream;
  UPIPE_TRY(hipEventRecord(side->fork, st));   // after the accumulator fills
  UPIPE_TRY(hipStreamWaitEvent(sb, side->fork, 0));
  int kslot_of[2] = {0, 0};                     // KV slot of the chunk in each slot
  int kslot = 1;
  auto prepare = [&](int c) -> int {
    const Chunk ch = chunk_info(s, c);
    const int sl = c & 1;
    if (ch.kv_first) kslot ^= 1;
    kslot_of[sl] = kslot;
    if (c >= 2) UPIPE_TRY(hipStreamWaitEvent(sb, side->done[sl], 0));
    const int r = stage_prepare(c, sl, kslot, sb);
    if (r != UPIPE_OK) return r;
    UPIPE_TRY(hipEventRecord(side->ready[sl], sb));
    return UPIPE_OK;
  };
  rc = prepare(0);
  if (rc != UPIPE_OK) return rc;
  for (int c = 0; c < nchunks; ++c) {
    const int sl = c & 1;
    const int kl = kslot_of[sl];
    if (c + 1 < nchunks) {
      rc = prepare(c + 1);
      if (rc != UPIPE_OK) return rc;
    }
    // the ready event of this slot was recorded for chunk c before chunk
    // c+1's preparation re-recorded the other slot's
    UPIPE_TRY(hipStreamWaitEvent(st, side->ready[sl], 0));
    rc = stage_attend(c, sl, kl);
    if (rc != UPIPE_OK) return rc;
    UPIPE_TRY(hipEventRecord(side->done[sl], st));
  }
  return UPIPE_OK;
}

}  // extern "C"
