/*
 * upipe_attn.h - C ABI of the headwise-chunked causal GQA attention layer
 * (UPipe, "Untied Ulysses") on one MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * One GPU's share of a context-parallel attention layer: full-sequence causal
 * self-attention over this GPU's Hq query heads and Hkv key/value heads,
 * processed one head chunk at a time.  Per chunk of `head_chunk` query heads:
 * the chunk's rows of W_qkv project q (and k, v when a KV group is first
 * touched), RoPE rotates q and k, causal attention runs and the chunk's
 * per-head output (its partial result) is stored in o_saved.  After the last
 * chunk the output projection accumulates every chunk's partial result
 * through its columns of W_o into y (fp32 accumulation, one bf16 rounding).
 * The buffers for q/k/v and all intermediates are carved from one
 * caller-owned workspace that every chunk reuses, so workspace grows with
 * head_chunk, not with Hq.
 *   - method: "Untied Ulysses Pushes Llama-3-8B Training to 5 Million Tokens",
 *     Untied Ulysses section (one group of heads at a time, a partial result
 *     stored per group, buffers reused; tailored to grouped-query attention)
 *     and its chunk-size ablation paragraph (chunk size trades memory for
 *     throughput; pick the chunk that fits the memory budget);
 *   - exact attention: "Untied Ulysses: Memory-Efficient Context Parallelism
 *     via Headwise Chunking", Abstract and Builds-on list (Attention Is All You
 *     Need, RoFormer, FlashAttention).
 * Conventions where the pages are silent: scale 1/sqrt(head_dim); query i sees
 * keys j <= i; q head h uses KV head h / (Hq/Hkv); W_qkv rows are packed
 * [Q heads | K heads | V heads], head_dim rows per head, no bias (nn.Linear
 * [out, in] layout); W_o is [hidden, Hq*head_dim]; RoPE rotates consecutive
 * pairs (2i, 2i+1) by p * theta^(-2i/head_dim) at position p = 0..L-1.
 *
 * Common argument rules (every entry point)
 * -----------------------------------------
 *  - All tensor pointers are DEVICE memory owned by the caller; the library
 *    never allocates or frees device memory and keeps no pointer after return.
 *  - bfloat16 tensors are passed as uint16_t bit patterns, row-major and
 *    contiguous; every pointer must be 16-byte aligned, the workspace
 *    256-byte aligned.
 *  - Batch is 1 and attention is causal.
 *  - hidden == 0 selects q/k/v-given mode: x is packed q|k|v
 *    [L, (Hq+2Hkv)*head_dim] (already projected, not yet rotated), the
 *    weights and y / dw_* must be NULL, dy is dO [L, Hq*head_dim] and dx is
 *    dqkv [L, (Hq+2Hkv)*head_dim].
 *  - Supported: head_dim == 128, hidden a multiple of 128 (or 0),
 *    1 <= L <= 2^24, Hq % Hkv == 0, Hq % head_chunk == 0 and either
 *    head_chunk % G == 0 or G % head_chunk == 0 (G = Hq/Hkv), so that no chunk
 *    holds part of two KV groups' query heads; and no kernel grid reaches
 *    2^32 threads: with L_256 = L rounded up to 256, kc = the KV heads one
 *    chunk touches and w = (head_chunk + 2 kc) * 128,
 *    L_256 * head_chunk < 2^31, L_256 * kc < 2^30,
 *    L_256 * max(hidden, w) < 2^39 and hidden * w < 2^34
 *    (UPIPE_EUNSUPPORTED otherwise; all hold for L <= 2^24 with
 *    head_chunk <= 32 and hidden <= 16384).
 *  - All checks run on the host before the first launch; on any error nothing
 *    is launched and outputs are untouched.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *    null stream) and is asynchronous: the call returns before the GPU is
 *    done.  The library never synchronizes.  Calls that share a workspace
 *    must be ordered on one stream.
 *  - Calls run on the current HIP device.  With pipelining enabled (off by
 *    default, see upipe_pipeline_enable) the forward also uses a second
 *    stream of the library's own, forked from and joined back into `stream`
 *    with events, so work after the call on `stream` sees every result.
 *    Calls on one device must not run concurrently from several host
 *    threads.
 *  - HIP graph capture: with pipelining and profiling off (the defaults)
 *    every entry point enqueues kernel launches on `stream` only (no
 *    allocation, memset, event or synchronization), so a caller may
 *    capture a forward and backward into a graph and replay it; a replay
 *    reads whatever the captured input buffers hold at that time and gives
 *    the eager call's bits.  The pipelined and profiled schedules use the
 *    library's own stream and events and are not meant for capture.
 *  - Outputs are fully overwritten (never accumulated into).
 *
 * Precision
 * ---------
 *  - The projections and the score product Q K^T take bf16 operands with
 *    fp32 accumulation; the rotated q and k are held in bf16 (q multiplied
 *    by log2(e)/sqrt(head_dim) in fp32 first, so that the scores come out
 *    as base-2 exponents; the relative rounding is unchanged).
 *  - The forward's O = P V product takes fp16 operands (P in [0, 256], v
 *    converted from bf16 to fp16) with fp32 accumulation: fp16's 10-bit
 *    mantissa keeps O inside its error budget where bf16's 7 bits do not.
 *    Finite |v| > 65504 therefore saturates to +-65504 in the forward (the
 *    backward uses the bf16 v as given, so its gradients are those of the
 *    unsaturated v): such inputs are outside the supported range.  NaN and
 *    +-Inf in v propagate: a non-finite v_j makes that column of O
 *    non-finite for every query row from j's 64-key tile on (rows of the
 *    tile before j included, since masked keys enter the tile's product
 *    with P = 0).
 */
#ifndef UPIPE_ATTN_H
#define UPIPE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define UPIPE_OK 0
#define UPIPE_EINVAL (-1)       /* bad size, count, or pointer combination        */
#define UPIPE_EUNSUPPORTED (-2) /* head_dim != 128, hidden % 128 != 0, L > 2^24,
                                   or a kernel grid of 2^32 threads or more       */
#define UPIPE_ECHUNK (-3)       /* head_chunk does not divide Hq or straddles a KV group */
#define UPIPE_EWORKSPACE (-4)   /* workspace NULL, misaligned or smaller than required */
#define UPIPE_EHIP (-5)         /* the HIP runtime reported an error at launch    */
#define UPIPE_ESCRATCH (-6)     /* upipe_attn_fwd_static: the shapes need more
                                   workspace than its static scratch holds        */

#define UPIPE_PASS_FWD 0
#define UPIPE_PASS_BWD 1
#define UPIPE_PASS_BWD_RECOMPUTE 2  /* upipe_attn_bwd with o_saved == NULL */
#define UPIPE_PASS_FWD_PIPELINED 3  /* upipe_attn_fwd with pipelining enabled */
#define UPIPE_PASS_BWD_PIPELINED 4  /* upipe_attn_bwd (o_saved given) with pipelining enabled */

/*
 * Workspace size query.  Writes to *bytes the workspace that upipe_attn_fwd
 * (pass = UPIPE_PASS_FWD; UPIPE_PASS_FWD_PIPELINED while pipelining is
 * enabled), upipe_attn_bwd (pass = UPIPE_PASS_BWD; UPIPE_PASS_BWD_PIPELINED
 * while pipelining is enabled) or upipe_attn_bwd in full-recompute mode
 * (pass = UPIPE_PASS_BWD_RECOMPUTE, projection mode only; never pipelined)
 * needs for these shapes.  The size is affine in head_chunk (per-chunk q-side buffers
 * plus the resident KV group): choosing head_chunk is how a caller fits the
 * layer into its memory budget (chunk-size ablation paragraph of the
 * talk write-up).  Returns UPIPE_OK or the error the entry point itself would
 * return for these shapes.  Host only; touches no GPU.
 */
int upipe_attn_workspace_bytes(int64_t seq_len, int32_t hidden, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t head_chunk,
                               int32_t pass, size_t* bytes);

/*
 * Chunk choice for a memory budget: writes to *head_chunk the largest valid
 * head chunk (it divides n_q_heads and keeps KV groups whole) whose
 * workspace for `pass` is at most budget_bytes, and that workspace to
 * *bytes.  Larger chunks run faster and need more memory, so the training
 * run picks the chunk that fits its budget (chunk-size ablation paragraph
 * of "Untied Ulysses Pushes Llama-3-8B Training to 5 Million Tokens").
 * Returns UPIPE_EWORKSPACE when no chunk fits, otherwise as
 * upipe_attn_workspace_bytes.  Host only.
 */
int upipe_attn_choose_chunk(int64_t seq_len, int32_t hidden, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, int32_t pass,
                            size_t budget_bytes, int32_t* head_chunk, size_t* bytes);

/*
 * Forward pass: for each head chunk in turn, project the chunk's q (k and v
 * when the chunk opens a KV group), rotate, run causal attention and store
 * the chunk's per-head output; then y = o_saved W_o^T.  The head-at-a-time
 * schedule with buffers reused by the next group is the one described in
 * the Untied Ulysses section of "Untied Ulysses Pushes Llama-3-8B Training
 * to 5 Million Tokens"; the attention itself is exact causal softmax
 * attention with RoPE ("Untied Ulysses: Memory-Efficient Context
 * Parallelism via Headwise Chunking", Builds-on list).
 *  x        [L, hidden] bf16 (projection mode) or packed q|k|v (hidden == 0)
 *  w_qkv    [(Hq+2Hkv)*head_dim, hidden] bf16, NULL iff hidden == 0
 *  w_o      [hidden, Hq*head_dim] bf16, NULL iff hidden == 0
 *  y        [L, hidden] bf16 out, NULL iff hidden == 0
 *  o_saved  [L, Hq*head_dim] bf16 out: per-head attention output (before W_o);
 *           upipe_attn_bwd reads it back
 *  lse      [Hq, L] fp32 out: natural-log sum of exp of the scaled scores of
 *           each query row; upipe_attn_bwd reads it back
 *  workspace, workspace_bytes: caller-owned scratch of at least the size the
 *           query returns for UPIPE_PASS_FWD (UPIPE_PASS_FWD_PIPELINED while
 *           pipelining is enabled); contents on entry are ignored
 *  stream   hipStream_t or NULL
 */
int upipe_attn_fwd(int64_t seq_len, int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, double rope_theta, int32_t head_chunk,
                   const uint16_t* x, const uint16_t* w_qkv, const uint16_t* w_o,
                   uint16_t* y, uint16_t* o_saved, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same computation, arguments and results as
 * upipe_attn_fwd with the one-stream schedule, but the workspace is a
 * static device array of the library, UPIPE_STATIC_SCRATCH_BYTES (256 MiB)
 * per GPU, held from library load until the process ends (each GPU the
 * library runs on has its own copy; its address is looked up on the first
 * call on that device).  The call allocates nothing: no device memory, no
 * stream or event (pipelining and profiling are not applied to it).
 * Returns UPIPE_ESCRATCH, before any GPU work, when upipe_attn_workspace_bytes
 * for UPIPE_PASS_FWD exceeds the scratch (for example L = 32768, hidden 4096,
 * 32 q / 8 KV heads fits up to head_chunk 8); otherwise as upipe_attn_fwd.
 * Every call on one GPU uses the same scratch and leaves its contents
 * behind: calls on one GPU that may overlap in time (different streams,
 * host threads or processes sharing the library instance) race on it and
 * must be serialized by the caller.  Nothing in the scratch needs to start
 * at any value.
 */
#define UPIPE_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
int upipe_attn_fwd_static(int64_t seq_len, int32_t hidden, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, double rope_theta,
                          int32_t head_chunk, const uint16_t* x, const uint16_t* w_qkv,
                          const uint16_t* w_o, uint16_t* y, uint16_t* o_saved, float* lse,
                          void* stream);

/*
 * Backward pass: the chain rule of the forward, run chunk by chunk in the
 * same head-group order with the same buffer reuse (Untied Ulysses section
 * of "Untied Ulysses Pushes Llama-3-8B Training to 5 Million Tokens");
 * q/k/v are recomputed per chunk from x, so only o_saved and lse are kept
 * from the forward.
 *  x, w_qkv, w_o   as in upipe_attn_fwd
 *  o_saved, lse    the forward's outputs for the same inputs.  In projection
 *           mode o_saved may be NULL ("full recompute"): each chunk's
 *           attention output is then recomputed from the recomputed q/k/v
 *           and the saved lse, in one pass (P = exp(S - lse) needs no
 *           running maximum or row sum; 4*head_dim FLOPs more per causal
 *           pair and q head), into per-chunk workspace, so nothing of size
 *           L*Hq*head_dim has to outlive the forward: activation
 *           checkpointing, one step of the memory progression in "Untied
 *           Ulysses Pushes Llama-3-8B Training to 5 Million Tokens", applied
 *           to this layer's own saved output.  Needs the
 *           UPIPE_PASS_BWD_RECOMPUTE workspace.  The recomputed O differs
 *           from the forward's by rounding (it is normalised by the saved
 *           lse instead of its own row sum), so the gradients match those
 *           of the o_saved call to about 2e-3 relative, not bit for bit.
 *           With o_saved, dx is bitwise reproducible from run to run;
 *           dw_qkv and dw_o are too when the weight-gradient GEMMs split
 *           their reduction over L in at most two parts (short L); with
 *           more parts the parts meet by fp32 atomic adds in an order that
 *           varies from run to run, so a few bf16 values may differ by one
 *           unit in the last place between any two calls.
 *  dy       [L, hidden] bf16 upstream gradient of y, or dO [L, Hq*head_dim]
 *  dx       [L, hidden] bf16 out, or dqkv [L, (Hq+2Hkv)*head_dim] (hidden == 0)
 *  dw_qkv   [(Hq+2Hkv)*head_dim, hidden] bf16 out, NULL iff hidden == 0
 *  dw_o     [hidden, Hq*head_dim] bf16 out, NULL iff hidden == 0
 *  workspace, workspace_bytes: at least the UPIPE_PASS_BWD query size
 *           (UPIPE_PASS_BWD_PIPELINED while pipelining is enabled,
 *           UPIPE_PASS_BWD_RECOMPUTE when o_saved is NULL)
 */
int upipe_attn_bwd(int64_t seq_len, int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, double rope_theta, int32_t head_chunk,
                   const uint16_t* x, const uint16_t* w_qkv, const uint16_t* w_o,
                   const uint16_t* o_saved, const float* lse, const uint16_t* dy,
                   uint16_t* dx, uint16_t* dw_qkv, uint16_t* dw_o,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing for measurement tools (not needed to use the layer).
 * upipe_profile_enable(mask) clears previous records and, until
 * upipe_profile_enable(0), brackets each kernel launch of upipe_attn_fwd /
 * upipe_attn_bwd whose class bit (1 << kind) is set in mask with a pair of
 * HIP events recorded on the caller's stream (UPIPE_PROFILE_ALL: every
 * class).  Each bracket adds two event records to the stream; bracketing
 * every launch of a layer step costs about 1% of its time, one class a
 * fraction of that.  upipe_profile_read(kind, ...) waits for the recorded
 * events and returns the summed GPU milliseconds and the number of launches
 * of one kernel class:
 *   UPIPE_KERNEL_ATTN_FWD      causal attention forward
 *   UPIPE_KERNEL_ATTN_BWD_DKDV causal attention backward, dK and dV
 *   UPIPE_KERNEL_ATTN_BWD_DQ   causal attention backward, dQ
 *   UPIPE_KERNEL_GEMM          projection / gradient GEMMs (except below)
 *   UPIPE_KERNEL_PREP          RoPE / layout pass of q, k, v
 *   UPIPE_KERNEL_FINALIZE      accumulator conversion, fills
 *   UPIPE_KERNEL_GEMM_ACCUM    the dx GEMMs of the second and later chunks,
 *                              whose epilogue accumulates into dx in bf16
 *   UPIPE_KERNEL_PREP_DOUT     dO preparation (D = dO . O, base-2 LSE)
 * State is process-wide and not thread-safe.  Events are host-side HIP
 * objects; no device memory is allocated.  Returns UPIPE_OK, UPIPE_EINVAL
 * (a mask outside 0 .. UPIPE_PROFILE_ALL, a bad kind or NULL output) or
 * UPIPE_EHIP.
 */
#define UPIPE_KERNEL_ATTN_FWD 0
#define UPIPE_KERNEL_ATTN_BWD_DKDV 1
#define UPIPE_KERNEL_ATTN_BWD_DQ 2
#define UPIPE_KERNEL_GEMM 3
#define UPIPE_KERNEL_PREP 4
#define UPIPE_KERNEL_FINALIZE 5
#define UPIPE_KERNEL_GEMM_ACCUM 6
#define UPIPE_KERNEL_PREP_DOUT 7
#define UPIPE_PROFILE_ALL 0xFF
int upipe_profile_enable(int mask);
int upipe_profile_read(int kind, double* total_ms, int64_t* launches);

/*
 * Two-slot pipelining (off by default): the next chunk's preparation runs on
 * a second stream, into a second set of per-chunk workspace buffers, while
 * the current chunk's attention runs on the caller's stream (the overlap of
 * the next group's work with the current group's, "Untied Ulysses Pushes
 * Llama-3-8B Training to 5 Million Tokens", Untied Ulysses section).
 *   forward:  chunk c+1's QKV projection and RoPE/layout pass overlap chunk
 *             c's attention (needs the UPIPE_PASS_FWD_PIPELINED workspace);
 *   backward: chunk c+1's projection recompute, RoPE/layout pass, dO GEMM,
 *             dW_o GEMM and dO preparation overlap chunk c's attention
 *             backward and its dx / dW_qkv GEMMs (UPIPE_PASS_BWD_PIPELINED
 *             workspace; the full-recompute backward, o_saved == NULL, keeps
 *             the one-stream schedule).
 * While enabled, the calls need those workspaces (else UPIPE_EWORKSPACE).
 * The stream (default priority) and five events are created on a device's
 * first pipelined call and kept until the process ends; no device memory is
 * allocated.  Results are identical either way (the same kernels read the
 * same inputs; only buffers and streams differ), except that the weight
 * gradients' split-K fp32 atomics are order-dependent as in any two calls.
 * On one GPU the overlap gains little (the attention kernels keep every CU
 * busy, so the overlapped work mostly takes CUs from them), hence off by
 * default.  Process-wide setting; returns UPIPE_OK.
 */
int upipe_pipeline_enable(int on);

/*
 * Debug mode (off by default), a check for workspace reuse between chunks:
 * before each chunk (and each tile of upipe_mlp_fwd / upipe_mlp_bwd and
 * upipe_loss_fwd / upipe_loss_bwd) the
 * library fills that chunk's workspace buffers with 0xFF bytes (NaN in
 * bf16, fp16 and fp32) by a fill kernel on the stream that then writes
 * them, so a kernel that read a buffer before the chunk wrote it, or read a
 * previous chunk's leftovers, would turn results into NaN.  Buffers that
 * legitimately carry state across chunks (a KV group's k, v and dK/dV
 * accumulators while the group spans chunks, the weight-gradient
 * accumulators) are filled when that state begins.  Results are identical
 * with and without it; it costs extra HBM writes.  Process-wide setting;
 * returns UPIPE_OK.
 */
int upipe_debug_enable(int on);

/*
 * The HIP error behind the calling thread's most recent UPIPE_EHIP (as an
 * int hipError_t value, 0 if none was recorded) and its HIP description
 * (static text, never NULL).  Host-side state only.
 */
int upipe_last_hip_error(void);
const char* upipe_last_hip_error_string(void);

/* Static, human-readable text for a status code.  Never NULL. */
const char* upipe_strerror(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int upipe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_ATTN_H */
