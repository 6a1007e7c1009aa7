// Host-side launch interface of the gfx950 kernels (internal to the library;
// the public ABI is include/upipe_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace upipe {

// ------------------------------------------------------------------ GEMM
// C[m][n] = sum_k A(m,k) B(k,n) with bf16 operands and fp32 accumulation.
//   A(m,k) = A[m*lda + k]  (a_kmajor)   or  A[k*lda + m]
//   B(k,n) = Brow(n)[k]    (b_kmajor)   or  Brow(k)[n]
// where Brow(r) = B + map(r)*ldb and map() sends a logical B row (n when
// b_kmajor, k otherwise) through up to three contiguous segments; this is how
// a head chunk picks its rows of W_qkv without a copy.
struct RowSegments {
  int count;           // 0 = identity map
  int end[3];          // exclusive logical end of each segment (ascending)
  int64_t row0[3];     // memory row of the segment's first logical row
};

// A quiet NaN built from its bits behind an empty asm: device code is built
// with -fno-honor-nans, under which a NaN constant is undefined.
__device__ __forceinline__ float quiet_nan() {
  uint32_t b = 0x7fc00000u;
  asm volatile("" : "+v"(b));
  return __builtin_bit_cast(float, b);
}

enum GemmLayout { GEMM_NT = 0, GEMM_NN = 1, GEMM_TN = 2 };
// EPI_STORE_F32 writes each split's fp32 partial tile into its own [M][N]
// slice of C (slice s at C + s*M*N; one split: C itself); EPI_ADD_F32 adds
// the fp32 tile into C with plain stores (TN, one split: each element has
// one writer); EPI_ATOMIC_F32 adds with atomics (any split count).  The
// cross-entropy epilogues (NT, one split) take C = logits of sequence rows
// ce_row0 + m: EPI_CE_STATS stores no logits, only each row's maximum and
// sum of 2^(y - max) (y = logit log2 e) over every 256-column tile, and the
// target's logit; EPI_CE_GRAD stores bf16 (exp(logit - lse) - onehot) *
// scale.
enum GemmEpilogue {
  EPI_STORE_BF16 = 0,
  EPI_ACCUM_BF16 = 1,
  EPI_ATOMIC_F32 = 2,
  EPI_STORE_F32 = 3,
  EPI_ADD_F32 = 4,
  EPI_CE_STATS = 5,
  EPI_CE_GRAD = 6
};

struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  RowSegments bseg;
  void* C;            // bf16 [M][ldc], or an fp32 [M][N] accumulator (split-K atomics)
  int64_t ldc;
  int M, N, K;        // M, N multiples of 8; K a multiple of 64 when an operand is
                      // k-contiguous (NT, NN); any K for TN (the tail is zeroed)
  int k_per_split;    // multiple of 64; ceil(K / k_per_split) splits
  // bf16 store epilogue only: output columns n < rope_cols are rotated (RoPE,
  // position = row m, pair = (n % 128) / 2) in fp32 before the one rounding
  int rope_cols;
  // bf16 store epilogue only: if > 0, output columns n >= f16_from are stored
  // as fp16 (saturated to +-65504) instead of bf16
  int f16_from;
  // bf16 store epilogue only: columns n < hm_end go to the attention
  // kernels' head-major buffers [head][Lp][128] instead of C: n < hm_split
  // to hm_q (head n / 128), the rest to hm_k (head (n - hm_split) / 128);
  // row m at m * 128 of its head, heads hm_stride elements apart; every row
  // m < M is stored there
  uint16_t* hm_q;
  uint16_t* hm_k;
  int hm_split, hm_end;
  int64_t hm_stride;
  // factor applied to the hm_q columns after RoPE, before the rounding
  // (the attention kernels take q pre-multiplied by log2(e) / sqrt(d))
  float hm_q_scale;
  // NT only, if > 0: rows of A that exist (reads of later rows clamp to the
  // last one) and rows of C that are stored; M may then exceed it, for the
  // head-major columns' padding rows
  int rows_valid;
  // cross-entropy epilogues: targets and ignore index of the sequence rows
  // (row m of C is row ce_row0 + m); EPI_CE_STATS writes ce_stats [M][ceil(N
  // / 256)] (max, sum) pairs and ce_tlogit [M] (rows whose target lies in
  // [0, N)); EPI_CE_GRAD reads ce_lse [L] (natural log) and *ce_scale
  const int32_t* ce_targets;
  int ce_ignore;
  int64_t ce_row0;
  float* ce_stats;
  float* ce_tlogit;
  uint16_t* ce_logits16;  // EPI_CE_STATS, optional: [M][N] fp16 logits

  const float* ce_lse;
  const float* ce_scale;
  RopeTable rope;
};

hipError_t launch_gemm(GemmLayout layout, GemmEpilogue epi, const GemmArgs& a, hipStream_t s);

// The HIP error behind the most recent UPIPE_EHIP of the calling thread,
// kept for upipe_last_hip_error (hipSuccess when none)
void note_hip_error(hipError_t e);

// bf16 dst rows = the sum of nslices fp32 [M][N] slices, in slice order
// (the partial results of a GEMM whose splits store into their own slices)
hipError_t launch_sum_slices(const float* slices, int nslices, int M, int N, uint16_t* dst,
                             int64_t ld, hipStream_t s);

// Split count and k extent per split (a multiple of the k step) for a TN
// GEMM reducing over L rows into an M x N fp32 accumulator (host side).
int gemm_reduction_splits(int64_t L, int M, int N);
int gemm_k_per_split(int64_t L, int splits);

// fp32 accumulator [M][N] -> bf16 dst rows dst[map(m)*ld_dst + n]; clears the
// accumulator for the next split-K GEMM.
hipError_t launch_acc_to_bf16(float* acc, int M, int N, uint16_t* dst, int64_t ld_dst,
                              const RowSegments& rows, hipStream_t s);

// ---------------------------------------------------------------- prep
// Copies a chunk's heads into the attention kernels' head-major layout
// [head][Lp][128], padded with zero rows to Lp, rotating q and k heads (RoPE)
// on the way unless the source is already rotated (the projection GEMM
// rotates in its epilogue), and converting v between bf16 and fp16.
struct PrepArgs {
  const uint16_t* src_q;   // head j of each kind starts at src + j*128; rows every src_ld
  const uint16_t* src_k;
  const uint16_t* src_v;
  int64_t src_ld;
  int nq, nkv;
  uint16_t* q_rm;          // [nq][Lp][128]
  uint16_t* k_rm;          // [nkv][Lp][128]
  uint16_t* v_rm;          // [nkv][Lp][128]
  int64_t L, Lp;
  int rotate;              // apply RoPE to q and k heads
  int v_src_f16;           // v source holds fp16 bits (else bf16)
  int v_out_f16;           // write v as fp16 (else bf16)
  int v_tiles;             // write v (fp16) as the forward's transposed
                           // 64-key tiles instead of row-major (see prep.hip)
  int v_only;              // only the v heads (the q and k heads are skipped)
  float q_scale;           // q heads are multiplied by this (after RoPE) before rounding
};
hipError_t launch_prep_qkv(const PrepArgs& a, const RopeTable& t, hipStream_t s);

// dO prep for the backward: head-major dO, D_i = dO_i . O_i and the base-2
// log-sum-exp of each row, all padded to Lp; D and the log-sum-exp are
// stored negated (they start the backward kernels' accumulators).
struct PrepDoutArgs {
  const uint16_t* src_do;  // head j at src_do + j*128, row stride do_ld
  int64_t do_ld;
  const uint16_t* o;       // head j at o + j*128, row stride o_ld
  int64_t o_ld;
  const float* lse;        // head j at lse + j*L
  int nh;
  uint16_t* do_rm;         // [nh][Lp][128]
  float* lse2;             // [nh][Lp] -LSE in base 2, negated
  float* dvec;             // [nh][Lp] -D = -(dO . O), negated
  int64_t L, Lp;
};
hipError_t launch_prep_dout(const PrepDoutArgs& a, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// fills whole 16-byte chunks of [p, p + bytes) with a 32-bit pattern
hipError_t launch_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t s);
// debug mode (upipe_debug_enable): workspace buffers are filled with 0xFF
// bytes (NaN in bf16, fp16 and fp32) before each chunk or tile writes them
extern bool g_debug_fill;

// ---------------------------------------------------------- attention
// q arrives rotated and pre-multiplied by log2(e) / sqrt(d) (by the
// projection GEMM's epilogue or by prep_qkv), so q . k is the score in
// base-2 units and the softmax needs no scaling.
struct FwdArgs {
  const uint16_t* q;    // [nh][Lp][128], rotated, times log2(e)/sqrt(d)
  const uint16_t* k;    // [nkv][Lp][128], rotated
  const uint16_t* v;    // [nkv][Lp/64] transposed fp16 tiles of 128 x 64 (prep.hip)
  int nh;               // query heads in this chunk
  int group;            // G = Hq / Hkv
  int q_head0;          // global index of the chunk's first q head
  int kv_head0;         // global index of kv buffer 0
  int o_head0;          // global q head stored at column 0 of o / row 0 of lse
  uint16_t* o;          // [L][o_ld]; q head h at column (h - o_head0)*128
  int64_t o_ld;
  float* lse;           // [.][L]; q head h at row h - o_head0
  int64_t L, Lp;
  const float* lse_in;  // launch_flash_fwd_lse: [Hq][L] saved LSE (natural log),
                        // q head h at row h; lse is not written then
};
hipError_t launch_flash_fwd(const FwdArgs& a, hipStream_t s);
// O only, from the forward's saved LSE (the backward's full recompute)
hipError_t launch_flash_fwd_lse(const FwdArgs& a, hipStream_t s);

struct BwdArgs {
  const uint16_t* q;     // [nh][Lp][128] rotated, times log2(e)/sqrt(d) (as FwdArgs)
  const uint16_t* k;     // [nkv][Lp][128] rotated
  const uint16_t* v;     // [nkv][Lp][128]
  const uint16_t* dO;    // [nh][Lp][128]
  const float* lse2;     // [nh][Lp] -LSE in base 2 (negated: it starts the S accumulators)
  const float* dvec;     // [nh][Lp] -D (negated: it starts the dP accumulators)
  float* dk_acc;         // [nkv][Lp][128] fp32 cross-chunk accumulators
  float* dv_acc;
  int kv_first, kv_last; // this chunk starts / finishes its KV groups
  uint16_t* dk_out;      // bf16 rows: dk of kv j at dk_out + row*out_ld + j*128 (when kv_last)
  uint16_t* dv_out;
  uint16_t* dq_out;      // bf16 rows: dq of q head j at dq_out + row*dq_ld + j*128
  int64_t out_ld, dq_ld;
  int nh, nkv;
  int group;             // G
  int q_head0, kv_head0; // global indices (q head h uses kv head h / G)
  int64_t L, Lp;
  float dk_scale;        // dK = dk_scale * dS^T q: 1/sqrt(d) over q's factor
  float scale;           // 1/sqrt(d) (dQ = scale * dS K)
  RopeTable rope;
};
// dK, dV of the chunk's KV heads (key-stationary) ...
hipError_t launch_flash_bwd_dkdv(const BwdArgs& a, hipStream_t s);
// ... and dQ of its q heads (query-stationary), written inverse-rotated in bf16
hipError_t launch_flash_bwd_dq(const BwdArgs& a, hipStream_t s);

}  // namespace upipe
