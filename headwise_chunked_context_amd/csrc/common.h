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

// Same shape with fp16 operands (10-bit mantissa); used where bf16's 7 bits
// cost too much accuracy (the probabilities and values of O = P V).
__device__ __forceinline__ f32x16 mfma32_f16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Row of the 32x32 accumulator element held in register r by a lane of half g.
__device__ __forceinline__ int acc_row(int r, int g) { return (r >> 2) * 8 + g * 4 + (r & 3); }

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// fp16 pack; values beyond the fp16 range saturate to +-65504
__device__ __forceinline__ uint32_t pack_f16x2_sat(float lo, float hi) {
  lo = fminf(fmaxf(lo, -65504.f), 65504.f);
  hi = fminf(fmaxf(hi, -65504.f), 65504.f);
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
