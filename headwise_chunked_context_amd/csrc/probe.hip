// Sustained bf16 MFMA rate probe (include/upipe_probe.h): four independent
// accumulator chains of v_mfma_f32_32x32x16_bf16 per wave over operand
// fragments loaded once, with the shader and constant clocks read around the
// loop.
#include "../../include/upipe_probe.h"
#include "kernels.h"

using namespace upipe;

namespace {

constexpr int64_t kFragments = int64_t(1) << 20;  // 16-byte fragments in 16 MiB
// 64 KB of (unused) LDS per workgroup caps a CU at two workgroups, i.e. two
// waves per SIMD, whatever the register count would allow
constexpr unsigned kLdsBytes = 64 * 1024;

__global__ __launch_bounds__(256) void mfma_probe_kernel(const u32x4* ops, int iters, float* sink,
                                                         uint64_t* clocks) {
  const int tid = threadIdx.x;
  const int64_t gid = (int64_t)blockIdx.x * 256 + tid;
  u32x4 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    a[f] = ops[(gid * 16 + f) & (kFragments - 1)];
    b[f] = ops[(gid * 16 + 8 + f) & (kFragments - 1)];
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32(a[(j + c) & 7], b[(j + 3 * c) & 7], acc[c]);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[gid] = s;
  if ((tid & 63) == 0) {
    const int64_t w = gid >> 6;
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int upipe_probe_mfma(const uint16_t* operands, size_t operand_bytes, int32_t iters,
                                int32_t workgroups, float* sink, uint64_t* clocks, void* stream) {
  if (!operands || !sink || !clocks || iters < 1 || workgroups < 1 || workgroups > (1 << 22))
    return UPIPE_EINVAL;
  if (operand_bytes < (size_t)kFragments * 16 || (reinterpret_cast<uintptr_t>(operands) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3) != 0 || (reinterpret_cast<uintptr_t>(clocks) & 7) != 0)
    return UPIPE_EINVAL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)workgroups), dim3(256), kLdsBytes, st,
                     reinterpret_cast<const u32x4*>(operands), iters, sink, clocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return UPIPE_EHIP;
  }
  return UPIPE_OK;
}
