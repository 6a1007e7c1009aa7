/*
 * upipe_mlp.h - C ABI of the sequence-tiled SwiGLU MLP on one MI355X
 * (gfx950), the companion of the attention layer in upipe_attn.h.
 *
 * What the library computes
 * -------------------------
 * The gated MLP of "GLU Variants Improve Transformer" (Builds-on list of
 * "Untied Ulysses: Memory-Efficient Context Parallelism via Headwise
 * Chunking"), with nn.Linear [out, in] weights and no bias:
 *     h = x W_gate^T,  u = x W_up^T,  a = silu(h) * u,  y = a W_down^T,
 * silu(z) = z / (1 + exp(-z)), and its chain-rule backward.  The sequence
 * is processed `tile_rows` rows at a time: the step of the memory
 * progression in "Untied Ulysses Pushes Llama-3-8B Training to 5 Million
 * Tokens" that tiles losses and MLPs along the sequence (Arctic Long
 * Sequence Training), so that no intermediate spans the whole sequence.
 * The intermediates h, u, a (and the backward's da, dh, du) exist for one
 * tile at a time in a caller-owned workspace that every tile reuses; the
 * backward recomputes h and u per tile from x, so nothing of size L x ffn
 * is kept between the passes.  The weight gradients are summed over tiles
 * in fp32 accumulators held in the workspace (their size is that of the
 * weights, independent of L and of the tile).
 *
 * Conventions where the pages are silent: the MLP is the SwiGLU MLP of the
 * Llama models the pages train; gate and up weights are packed into one
 * w_gate_up [2 ffn, hidden], gate rows first; tiles are consecutive rows,
 * the last one ragged.
 *
 * Argument rules
 * --------------
 *  - As in upipe_attn.h: DEVICE pointers owned by the caller, bf16 passed
 *    as uint16_t bits, row-major and contiguous, 16-byte aligned, the
 *    workspace 256-byte aligned; the library never allocates, never
 *    synchronizes and enqueues on `stream` (hipStream_t as void*); all
 *    checks run on the host before the first launch, on any error nothing
 *    is launched; outputs are fully overwritten; status codes are the
 *    UPIPE_* codes of upipe_attn.h.
 *  - Every call enqueues kernel launches on `stream` only, so it may be
 *    captured into a HIP graph and replayed (as in upipe_attn.h).
 *  - Supported: 1 <= L <= 2^24, hidden and ffn multiples of 128 with
 *    hidden * ffn < 2^33, tile_rows >= 1 (a tile larger than L is L).
 *  - Precision: bf16 operands with fp32 accumulation; h, u, a, da, dh, du
 *    are held in bf16 between the GEMMs; the activation runs in fp32.
 *  - y and dx are bitwise reproducible from run to run.  Across tile sizes
 *    they are bit for bit equal whenever the hidden-wide GEMMs split their
 *    reduction the same number of times (not at all once a tile gives them
 *    256 output tiles of 256 x 256; short tiles split into fp32 slices
 *    summed in a fixed order).  The weight gradients accumulate
 *    over tiles in fp32, tile by tile in order; a tile whose weight-
 *    gradient GEMM splits its reduction (short tiles of wide layers) adds
 *    its parts by fp32 atomics, whose order can vary from run to run.
 */
#ifndef UPIPE_MLP_H
#define UPIPE_MLP_H

#include <stddef.h>
#include <stdint.h>

#include "upipe_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Workspace size query for upipe_mlp_fwd (pass = UPIPE_PASS_FWD) or
 * upipe_mlp_bwd (pass = UPIPE_PASS_BWD): one tile's [tile, 2 ffn] and
 * [tile, ffn] bf16 intermediates; for tiles too short to give the hidden-
 * wide GEMMs 256 output tiles of 256 x 256, s fp32 [tile, hidden] slices of
 * their split reduction (s = min(ceil(256 / output tiles), K / 512), K = ffn
 * forward and 2 ffn backward); and, for the backward, the fp32
 * weight-gradient accumulators (4 * 3 * hidden * ffn bytes).  Returns
 * UPIPE_OK or the error the entry point would return for these shapes.
 * Host only.
 */
int upipe_mlp_workspace_bytes(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t tile_rows,
                              int32_t pass, size_t* bytes);

/*
 * Tile choice for a memory budget: writes to *tile_rows the longest tile
 * (a multiple of 256 rows, or the whole sequence) whose workspace for
 * `pass` is at most budget_bytes, and that workspace to *bytes.  Longer
 * tiles run faster.  Returns UPIPE_EWORKSPACE when no tile fits.  Host only.
 */
int upipe_mlp_choose_tile(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t pass,
                          size_t budget_bytes, int32_t* tile_rows, size_t* bytes);

/*
 * Forward: y = (silu(x W_gate^T) * (x W_up^T)) W_down^T, tile by tile.
 *  x          [L, hidden] bf16
 *  w_gate_up  [2 ffn, hidden] bf16: rows 0 .. ffn-1 W_gate, ffn .. 2ffn-1 W_up
 *  w_down     [hidden, ffn] bf16
 *  y          [L, hidden] bf16 out
 *  workspace  at least the UPIPE_PASS_FWD query size; contents ignored
 */
int upipe_mlp_fwd(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t tile_rows,
                  const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                  uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward (chain rule of the forward; h and u are recomputed per tile):
 *  x, w_gate_up, w_down  as in upipe_mlp_fwd
 *  dy          [L, hidden] bf16 upstream gradient of y
 *  dx          [L, hidden] bf16 out
 *  dw_gate_up  [2 ffn, hidden] bf16 out
 *  dw_down     [hidden, ffn] bf16 out
 *  workspace   at least the UPIPE_PASS_BWD query size; contents ignored
 */
int upipe_mlp_bwd(int64_t seq_len, int32_t hidden, int32_t ffn, int32_t tile_rows,
                  const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                  const uint16_t* dy, uint16_t* dx, uint16_t* dw_gate_up, uint16_t* dw_down,
                  void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_MLP_H */
