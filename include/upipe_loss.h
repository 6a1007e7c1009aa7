/*
 * upipe_loss.h - C ABI of the sequence-tiled language-model loss on one
 * MI355X (gfx950), the companion of the attention layer in upipe_attn.h and
 * of the MLP in upipe_mlp.h.
 *
 * What the library computes
 * -------------------------
 * The mean cross-entropy of next-token training: the final hidden states h
 * [L, hidden] are projected onto the vocabulary by the output weight W
 * [vocab, hidden] (nn.Linear [out, in], no bias), logits = h W^T, and
 *     loss = mean over counted rows r of ( log sum_j exp(logits_rj)
 *                                          - logits_r,target(r) ),
 * a row counting unless its target is ignore_index; and the chain-rule
 * backward with upstream gradient dloss:
 *     dlogits_r = (softmax(logits_r) - onehot(target_r)) * dloss / count,
 *     dh = dlogits W,   dW = dlogits^T h.
 * The sequence is processed `tile_rows` rows at a time: the step of the
 * memory progression in "Untied Ulysses Pushes Llama-3-8B Training to 5
 * Million Tokens" that tiles losses and MLPs along the sequence (Arctic Long
 * Sequence Training), so that no buffer of size L x vocab exists.  The
 * logits never reach memory in fp32: in the forward, the GEMM that forms a
 * tile's logits reduces each row over each 256-column tile to its maximum
 * and sum of exponentials in its epilogue, and the forward returns the
 * per-row log-sum-exp; the backward recomputes the tile's logits and its
 * GEMM epilogue writes the bf16 dlogits from them and that log-sum-exp; dW
 * is summed over tiles in an fp32 accumulator held in the workspace (the
 * size of W, independent of L and of the tile).
 *
 * Conventions where the pages are silent: the loss is the mean cross-entropy
 * of the Llama models the pages train; rows whose target is ignore_index
 * (the caller's choice, e.g. -100) are left out of the mean; when every row
 * is ignored the loss is 0 and so are the gradients (a mean over no terms
 * taken as 0); a target outside [0, vocab) that is not ignore_index makes
 * its row's loss, the mean and that row's gradients NaN (and, through the
 * sum, dW); tiles are consecutive rows, the last one ragged.  Inputs are
 * expected finite: a NaN or Inf in h or W gives unspecified (possibly
 * finite) results, since the row maxima are taken without NaN handling.
 *
 * Argument rules
 * --------------
 *  - As in upipe_attn.h: DEVICE pointers owned by the caller, bf16 passed
 *    as uint16_t bits, row-major and contiguous, bf16 arrays 16-byte
 *    aligned, int32/fp32 arrays 4-byte aligned, the workspace 256-byte
 *    aligned; the library never allocates, never synchronizes and enqueues
 *    on `stream` (hipStream_t as void*); all checks run on the host before
 *    the first launch (target values are device data and are not checked
 *    there, see above), on any error nothing is launched; outputs are fully
 *    overwritten; status codes are the UPIPE_* codes of upipe_attn.h.
 *  - Every call enqueues kernel launches on `stream` only, so it may be
 *    captured into a HIP graph and replayed (as in upipe_attn.h).
 *  - Supported: 1 <= L <= 2^24, hidden and vocab multiples of 128 (pad the
 *    vocabulary; padded rows of W take part in the softmax), hidden * vocab
 *    < 2^33, tile_rows >= 1 (a tile larger than L is L).
 *  - Precision: bf16 operands with fp32 accumulation; the logits are fp32
 *    (in registers), the log-sum-exp and the loss are evaluated in fp32
 *    (the mean's sum in fp64); dlogits is rounded to bf16 between the
 *    backward's GEMMs.
 *  - The loss, the log-sum-exp, dh and dW are bitwise reproducible from run
 *    to run (no atomics: the mean is summed by one workgroup in a fixed
 *    order, dW accumulates tile by tile, and short tiles split dh's
 *    vocabulary reduction into fp32 slices summed in a fixed order).
 */
#ifndef UPIPE_LOSS_H
#define UPIPE_LOSS_H

#include <stddef.h>
#include <stdint.h>

#include "upipe_attn.h"

/* pass value of the workspace query and tile choice for upipe_loss_fwd_bwd */
#define UPIPE_PASS_FWD_BWD 5

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Workspace size query for upipe_loss_fwd (pass = UPIPE_PASS_FWD): per row
 * of a tile one fp32 (max, sum) pair per 256-column tile of the vocabulary
 * and the target's logit, and 4 bytes per row of the sequence (the per-row
 * loss); or for upipe_loss_bwd (pass = UPIPE_PASS_BWD): one tile's bf16
 * dlogits [tile, vocab], for tiles too short to give the dh GEMM 256 output
 * tiles of 256 x 256 the fp32 slices of its split reduction (s [tile,
 * hidden], s = min(ceil(256 / output tiles), vocab / 512)), and the fp32 dW
 * accumulator (4 * vocab * hidden bytes); or for upipe_loss_fwd_bwd (pass
 * = UPIPE_PASS_FWD_BWD): the forward's buffers and the backward's (its
 * [tile, vocab] 2-byte tile first holds fp16 logits, then the bf16 dlogits).
 * Returns UPIPE_OK or the error the entry point would return for these
 * shapes.  Host only.
 */
int upipe_loss_workspace_bytes(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                               int32_t pass, size_t* bytes);

/*
 * Tile choice for a memory budget: writes to *tile_rows the longest tile (a
 * multiple of 256 rows, or the whole sequence) whose workspace for `pass`
 * is at most budget_bytes, and that workspace to *bytes.  Longer tiles run
 * faster.  Returns UPIPE_EWORKSPACE when no tile fits.  Host only.
 */
int upipe_loss_choose_tile(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t pass,
                           size_t budget_bytes, int32_t* tile_rows, size_t* bytes);

/*
 * Forward: the mean cross-entropy, tile by tile.
 *  h             [L, hidden] bf16 final hidden states
 *  w             [vocab, hidden] bf16 output weight
 *  targets       [L] int32 target token of each row
 *  ignore_index  rows with this target do not count
 *  loss          one fp32 out: the mean over counted rows
 *  lse           [L] fp32 out: each row's log-sum-exp (natural log), the
 *                backward's input (ignored rows included)
 *  workspace     at least the UPIPE_PASS_FWD query size; contents ignored
 */
int upipe_loss_fwd(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                   const uint16_t* h, const uint16_t* w, const int32_t* targets,
                   int32_t ignore_index, float* loss, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Backward (chain rule of the forward; each tile's logits are recomputed):
 *  h, w, targets, ignore_index  as in upipe_loss_fwd
 *  lse     [L] fp32 from upipe_loss_fwd with the same h, w
 *  dloss   upstream gradient of the loss (host value; 1 for loss.backward())
 *  dh      [L, hidden] bf16 out
 *  dw      [vocab, hidden] bf16 out
 *  workspace  at least the UPIPE_PASS_BWD query size; contents ignored
 */
int upipe_loss_bwd(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                   const uint16_t* h, const uint16_t* w, const int32_t* targets,
                   int32_t ignore_index, const float* lse, float dloss, uint16_t* dh,
                   uint16_t* dw, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward and backward in one pass, for a caller that knows dloss when the
 * forward runs (e.g. 1 for loss.backward(), or a fixed loss scale): the
 * outputs of upipe_loss_fwd and of upipe_loss_bwd with that dloss.  Each
 * tile's logits are formed once instead of twice: the logits GEMM's epilogue
 * also stores them in fp16 (finite values beyond +-65504 saturate), and an
 * in-place pass turns them into the bf16 dlogits, so a quarter of the
 * GEMM work of the separate passes is saved for no extra memory.  The loss
 * and lse equal upipe_loss_fwd's bit for bit; dh and dW differ from
 * upipe_loss_bwd's by the fp16 rounding of the logits (relative 2^-11 *
 * |logit| in each probability, below dlogits' own bf16 rounding for
 * |logit| < 4).
 *  h, w, targets, ignore_index, dloss  as above
 *  loss, lse   out, as upipe_loss_fwd
 *  dh, dw      out, as upipe_loss_bwd
 *  workspace   at least the UPIPE_PASS_FWD_BWD query size; contents ignored
 */
int upipe_loss_fwd_bwd(int64_t seq_len, int32_t hidden, int32_t vocab, int32_t tile_rows,
                       const uint16_t* h, const uint16_t* w, const int32_t* targets,
                       int32_t ignore_index, float dloss, float* loss, float* lse, uint16_t* dh,
                       uint16_t* dw, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UPIPE_LOSS_H */
