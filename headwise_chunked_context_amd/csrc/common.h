// Shared device helpers for the gfx950 kernels: bf16 packing, MFMA wrappers,
// RoPE angle evaluation.  CDNA4 only (64-lane wavefronts, bf16 MFMA 32x32x16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace upipe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// RoPE: per-pair frequency divided by 2*pi, i.e. revolutions per position,
// theta^(-2i/d) / (2 pi) for i < d/2, evaluated in fp64 on the host.
struct RopeTable {
  double rev_per_pos[kHeadDim / 2];
};

// ---------------------------------------------------------------- MFMA
// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies A row (l % 32) and B column (l % 32), eight k values each
// (slot 8*(l/32) .. +7 of the 16); the result element (row i, col j) sits in
// lane j + 32*((i/4) % 2), register 4*(i/8) + i%4.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies A row
// (l % 16) and B column (l % 16), eight k values each (slot 8*(l/16) .. +7 of
// the 32); the result element (row i, col j) sits in lane j + 16*(i/4),
// register i % 4.  Same FLOPs per cycle as the 32x32x16 shape with half the
// accumulator traffic per FLOP.
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Same shape with fp16 operands (10-bit mantissa); used where bf16's 7 bits
// cost too much accuracy (the probabilities and values of O = P V).
__device__ __forceinline__ f32x16 mfma32_f16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Combine a per-lane value with the one of the lane in the other 32-lane half
// (lane ^ 32).  A single bpermute; the permlane32 swap builtin is not used
// because the optimizer folds its two results into one.
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32); }

// Row of the 32x32 accumulator element held in register r by a lane of half g.
__device__ __forceinline__ int acc_row(int r, int g) { return (r >> 2) * 8 + g * 4 + (r & 3); }

// ---------------------------------------------------------------- LDS tiles
// Row-major tiles of 128 16-bit elements per row (256 B, no padding).  The
// 16-byte chunk c of row r is stored at chunk position c ^ swz(r), where
// swz swaps the two 2-bit halves of r % 16.  With it both access patterns
// the kernels use are free of bank conflicts:
//  * row-per-lane 16-byte reads (lane i of 16 reads row r0+i, one chunk):
//    swz is a bijection on 16 consecutive rows;
//  * transposed 8-byte reads (ds_read_b64_tr_b16, 4 rows x 32 bytes per
//    16-lane group): rows r..r+3 (r % 4 == 0) land in four different
//    64-byte quarters of the bank space.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int tile_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte pieces addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// A-operand of a 32x32x16 MFMA whose m index runs along a row-major tile's
// columns and whose k index runs down its rows (a transposed operand): lane
// l gets column m0 + l % 32 and rows {k0 + 4g + j, k0 + 8 + 4g + j}, j < 4,
// g = l / 32 -- the k order of the 32x32 accumulator layout, so the matching
// B operand can come straight from accumulator registers.
__device__ __forceinline__ u32x4 tile_read_t(const uint16_t* tile, int k0, int m0, int lane) {
  const int s = lane & 15, grp2 = (lane >> 4) & 1, g = lane >> 5;
  const int col = m0 + 16 * grp2 + 4 * (s & 3);
  const int chunk = col >> 3, half = (col & 7);
  const int r0 = k0 + 4 * g + (s >> 2);
  u32x2 lo = lds_read_tr16(tile + tile_off(r0, chunk) + half);
  u32x2 hi = lds_read_tr16(tile + tile_off(r0 + 8, chunk) + half);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Same, k in natural order: lane l gets rows {k0 + 8g + j, k0 + 8g + 4 + j},
// i.e. k0 + 8g .. k0 + 8g + 7, the order of a row-per-lane operand.
__device__ __forceinline__ u32x4 tile_read_t_nat(const uint16_t* tile, int k0, int m0, int lane) {
  const int s = lane & 15, grp2 = (lane >> 4) & 1, g = lane >> 5;
  const int col = m0 + 16 * grp2 + 4 * (s & 3);
  const int chunk = col >> 3, half = (col & 7);
  const int r0 = k0 + 8 * g + (s >> 2);
  u32x2 lo = lds_read_tr16(tile + tile_off(r0, chunk) + half);
  u32x2 hi = lds_read_tr16(tile + tile_off(r0 + 4, chunk) + half);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Row-per-lane operand: row r, eight elements starting at column 8*chunk.
__device__ __forceinline__ u32x4 tile_read_row(const uint16_t* tile, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(tile + tile_off(row, chunk));
}

// Asynchronous global -> LDS copy (global_load_lds_dwordx4 / _dword): each
// lane fetches 16 (or 4) bytes and the wave's data lands in consecutive LDS
// from the address in M0 (lane i at M0 + 16i).  Issued as inline asm, so the
// compiler does not know that a copy into LDS is in flight and does not
// make later LDS reads wait for it: it cannot tell the two buffers of a
// double-buffered loop apart for every read form (transpose reads in
// particular) and would otherwise wait for the copy into the other buffer
// before each of them.  The caller owns completion: lds_dma_wait() and a
// barrier before the destination is read, and no copy into a buffer until
// every wave has passed the barrier that follows its last read.  M0 is
// listed as clobbered; the compiler keeps no value in it across other code
// (it sets M0 right before each of its own uses), which the warning about
// clobbering a reserved register concerns.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_untracked(const void* src, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_dst)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_untracked(const void* src, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(lds_dst)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// 16-byte LDS read at byte address addr + off (off a compile-time constant
// that folds into the instruction's offset field)
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
      (uintptr_t)(addr + off));
}
// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// wait for this wave's outstanding vector-memory operations (vmcnt = 0)
__device__ __forceinline__ void lds_dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// fp16 pack of the forward's value operand: finite values beyond the fp16
// range saturate to +-65504, NaN and +-Inf pass through unchanged.  The
// finiteness test is on the exponent bits, hidden from the optimizer by an
// empty asm: device code is built with -fno-honor-nans, under which the
// compiler turns a visible bit test into a class test that assumes no NaN
// (and a NaN would then be clamped to -65504).
__device__ __forceinline__ float sat_f16_range(float x) {
  uint32_t b = __builtin_bit_cast(uint32_t, x);
  asm volatile("" : "+v"(b));
  const float c = fminf(fmaxf(x, -65504.f), 65504.f);
  return (b & 0x7f800000u) == 0x7f800000u ? x : c;
}
__device__ __forceinline__ uint32_t pack_f16x2_sat(float lo, float hi) {
  lo = sat_f16_range(lo);
  hi = sat_f16_range(hi);
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
}

// ---------------------------------------------------------------- RoPE
// cos/sin of the rotation angle of pair i at position pos.  The angle is
// reduced to [-0.5, 0.5) revolutions in fp64 (positions reach 2^24, where an
// fp32 product would be off by whole radians), then the hardware sin/cos
// (argument in revolutions) evaluate it in fp32.
__device__ __forceinline__ void rope_cos_sin(const RopeTable& t, int64_t pos, int i, float& c,
                                             float& s) {
  double rev = static_cast<double>(pos) * t.rev_per_pos[i];
  rev -= __builtin_rint(rev);
  float r = static_cast<float>(rev);
  c = __builtin_amdgcn_cosf(r);
  s = __builtin_amdgcn_sinf(r);
}

__device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

}  // namespace upipe
