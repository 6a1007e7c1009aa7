// Memory-bound passes around the attention kernels (gfx950):
//   prep_qkv    head-major copies of a chunk's q/k/v, RoPE on q and k,
//               zero padding to Lp rows, v converted between bf16 and fp16
//               as the consumer needs; for the forward, v goes out as
//               transposed 64-key tiles (below);
//   prep_dout   the same for dO, plus D_i = dO_i . O_i and LSE in base 2;
//   zero        fill kernel (used instead of hipMemsetAsync).
// Each workgroup owns 64 rows x 128 columns of one head: coalesced 16-byte
// reads and writes along the rows.
#include "kernels.h"

namespace upipe {
namespace {

constexpr int ROWS = 64;

// rotate 8 consecutive elements (4 pairs starting at pair p0) of one row
// and multiply them by mul, in fp32 before the one rounding
__device__ __forceinline__ u32x4 rotate8(u32x4 v, const RopeTable& t, int64_t pos, int p0, float mul) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float c, s;
    rope_cos_sin(t, pos, p0 + j, c, s);
    float e = bf16_lo(v[j]), o = bf16_hi(v[j]);
    out[j] = pack_bf16x2((e * c - o * s) * mul, (e * s + o * c) * mul);
  }
  return out;
}
// multiply 8 bf16 elements by mul
__device__ __forceinline__ u32x4 scale8(u32x4 v, float mul) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = pack_bf16x2(bf16_lo(v[j]) * mul, bf16_hi(v[j]) * mul);
  return out;
}

// The forward's V operand: for every 64 keys one 128 x 64 fp16 tile of V^T
// (row = d, 128 bytes per row), stored exactly as the LDS tile the forward
// kernel reads, so the kernel copies it with contiguous 16-byte loads:
//  * the 16-byte chunk c = 2*st + g of row d holds keys 16st + 4g + {0..3}
//    followed by 16st + 8 + 4g + {0..3}: the key order in which the score
//    accumulator hands P^T to the O^T = V^T P^T MFMA as its B operand;
//  * chunk c of row d sits at position c ^ ((d >> 1) & 7), which makes the
//    kernel's row-per-lane 16-byte reads of 16 consecutive rows hit 16
//    different 16-byte bank groups.
__device__ void write_v_tiles(const PrepArgs& a, const uint16_t* src, uint16_t* dst, int64_t r0,
                              int tid) {
  __shared__ __attribute__((aligned(16))) uint16_t vs[ROWS][136];  // [key][d] fp16 bits
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int c = tid + 256 * it;
    int r = c >> 4, cc = c & 15;
    int64_t row = r0 + r;
    u32x4 v = {0, 0, 0, 0};
    if (row < a.L) {
      v = *reinterpret_cast<const u32x4*>(src + row * a.src_ld + cc * 8);
      if (!a.v_src_f16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack_f16x2_sat(bf16_lo(v[j]), bf16_hi(v[j]));
      }
    }
    *reinterpret_cast<u32x4*>(&vs[r][cc * 8]) = v;
  }
  __syncthreads();
  uint16_t* tile = dst + r0 * 128;  // tile r0 / 64 of the head
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int q = tid + 256 * it;  // 16-byte position in the tile
    int d = q >> 3;
    int c = (q & 7) ^ ((d >> 1) & 7);
    int kb = (c >> 1) * 16 + (c & 1) * 4;
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      w[j] = (uint32_t)vs[kb + 2 * j][d] | ((uint32_t)vs[kb + 2 * j + 1][d] << 16);
      w[2 + j] = (uint32_t)vs[kb + 8 + 2 * j][d] | ((uint32_t)vs[kb + 8 + 2 * j + 1][d] << 16);
    }
    *reinterpret_cast<u32x4*>(tile + q * 8) = w;
  }
}

// one workgroup per 64 rows of one head slot (q heads, then k, then v)
__global__ __launch_bounds__(256) void prep_qkv_kernel(PrepArgs a, RopeTable t) {
  const int slot = blockIdx.y + (a.v_only ? a.nq + a.nkv : 0);
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  const uint16_t* src;
  uint16_t* dst;
  bool rot = a.rotate != 0, is_v = false, is_q = false;
  if (slot < a.nq) {
    is_q = true;
    src = a.src_q + slot * 128;
    dst = a.q_rm + (int64_t)slot * a.Lp * 128;
  } else if (slot < a.nq + a.nkv) {
    const int j = slot - a.nq;
    src = a.src_k + j * 128;
    dst = a.k_rm + (int64_t)j * a.Lp * 128;
  } else {
    const int j = slot - a.nq - a.nkv;
    src = a.src_v + j * 128;
    dst = a.v_rm + (int64_t)j * a.Lp * 128;
    rot = false;
    is_v = true;
  }
  const int tid = threadIdx.x;
  if (is_v && a.v_tiles) {  // uniform: the whole workgroup has one slot
    write_v_tiles(a, src, dst, r0, tid);
    return;
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int c = tid + 256 * it;  // 64 rows x 16 chunks of 8
    int r = c >> 4, cc = c & 15;
    int64_t row = r0 + r;
    u32x4 v = {0, 0, 0, 0};
    if (row < a.L) {
      v = *reinterpret_cast<const u32x4*>(src + row * a.src_ld + cc * 8);
      if (rot)
        v = rotate8(v, t, row, cc * 4, is_q ? a.q_scale : 1.f);
      else if (is_q)
        v = scale8(v, a.q_scale);
      if (is_v && a.v_src_f16 && !a.v_out_f16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(f16_lo(v[j]), f16_hi(v[j]));
      } else if (is_v && !a.v_src_f16 && a.v_out_f16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = pack_f16x2_sat(bf16_lo(v[j]), bf16_hi(v[j]));
      }
    }
    *reinterpret_cast<u32x4*>(dst + row * 128 + cc * 8) = v;
  }
}

__global__ __launch_bounds__(256) void prep_dout_kernel(PrepDoutArgs a) {
  const int h = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * ROWS;
  const uint16_t* src = a.src_do + h * 128;
  const uint16_t* o = a.o + h * 128;
  uint16_t* rm = a.do_rm + (int64_t)h * a.Lp * 128;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    int c = tid + 256 * it;
    int r = c >> 4, cc = c & 15;  // 16 consecutive lanes share one row
    int64_t row = r0 + r;
    u32x4 v = {0, 0, 0, 0};
    float dot = 0.f;
    if (row < a.L) {
      v = *reinterpret_cast<const u32x4*>(src + row * a.do_ld + cc * 8);
      u32x4 ov = *reinterpret_cast<const u32x4*>(o + row * a.o_ld + cc * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dot += bf16_lo(v[j]) * bf16_lo(ov[j]) + bf16_hi(v[j]) * bf16_hi(ov[j]);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    *reinterpret_cast<u32x4*>(rm + row * 128 + cc * 8) = v;
    if (cc == 0) {
      a.dvec[(int64_t)h * a.Lp + row] = -dot;  // stored negated: -D
      a.lse2[(int64_t)h * a.Lp + row] = row < a.L ? -a.lse[(int64_t)h * a.L + row] * kLog2e : 0.f;
    }
  }
}

// fills n16 16-byte chunks with a 32-bit pattern (0: the accumulator
// clears; 0xFFFFFFFF: debug mode's NaN fill)
__global__ __launch_bounds__(256) void zero_kernel(u32x4* p, int64_t n16, uint32_t pattern) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * 256;
  for (; i < n16; i += stride) p[i] = u32x4{pattern, pattern, pattern, pattern};
}

}  // namespace

hipError_t launch_prep_qkv(const PrepArgs& a, const RopeTable& t, hipStream_t s) {
  dim3 grid((unsigned)(a.Lp / ROWS), a.v_only ? a.nkv : a.nq + 2 * a.nkv);
  hipLaunchKernelGGL(prep_qkv_kernel, grid, dim3(256), 0, s, a, t);
  return hipGetLastError();
}

hipError_t launch_prep_dout(const PrepDoutArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.Lp / ROWS), a.nh);
  hipLaunchKernelGGL(prep_dout_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t s) {
  int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<u32x4*>(p), n16, pattern);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) { return launch_fill(p, bytes, 0u, s); }

}  // namespace upipe
