// Dense matrix-core throughput probe (measurement aid; see fa355_probe.h).
#include "fa355_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters,
                                                         uint64_t* clocks,
                                                         float* sink) {
  const int lane = threadIdx.x & 63;
  const bool first = blockIdx.x == 0 && threadIdx.x < 64;
  uint64_t t0 = 0, r0 = 0;
  if (first) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  if (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(1e-3f * (float)((lane + e) & 7));
      b[e] = (__bf16)(1e-3f * (float)((lane * 3 + e) & 7));
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  } else {
    // E4M3 codes of small values (0x08..0x0f: subnormal-free normals near
    // 2^-6), varied per lane.
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x20202020 + ((lane + e) & 7);
      b[e] = 0x20202020 + ((lane * 3 + e) & 7);
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, b, acc[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
  if (first) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      clocks[0] = t0;
      clocks[1] = t1;
      clocks[2] = r0;
      clocks[3] = r1;
    }
  }
}

}  // namespace

extern "C" int fa355_mfma_probe(int kind, int iters, int blocks,
                                uint64_t* clocks, float* sink, void* stream) {
  if ((kind != 0 && kind != 1) || iters < 1 || blocks < 1 || !clocks || !sink)
    return 1;
  (void)hipGetLastError();
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0,
                       (hipStream_t)stream, iters, clocks, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0,
                       (hipStream_t)stream, iters, clocks, sink);
  return (int)hipGetLastError();
}
