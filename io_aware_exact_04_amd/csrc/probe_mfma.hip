// Dense matrix-core throughput probe (measurement aid; see fa355_probe.h).
#include "fa355_probe.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kCoexecModes = 23;
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

// ---------------------------------------------------------------- co-issue
//
// One workgroup of eight waves per CU (waves w and w + 4 share a SIMD); each
// wave runs one of the roles below for `iters` iterations and reports its
// shader-clock and 100 MHz reference-clock spans.
enum Role { kIdle, kMfma, kFma, kExp, kLds, kLdsTr, kMfmaExp, kMfmaFma,
            kMfmaBurstFma, kMix2, kMix4, kMix6, kMix8, kMix5e1 };

// Roles of waves 0-3 and 4-7 in each mode.
__constant__ int kModeRoles[kCoexecModes][2] = {
    {kMfma, kMfma}, {kMfma, kIdle},  {kMfma, kFma},    {kMfma, kExp},
    {kIdle, kFma},  {kIdle, kExp},   {kFma, kFma},     {kLds, kLds},
    {kLdsTr, kLdsTr}, {kMfmaExp, kIdle}, {kMfmaFma, kIdle}, {kMfma, kLds},
    {kMfma, kLdsTr}, {kExp, kExp},   {kLds, kIdle},
    {kMfmaFma, kMfmaFma}, {kMfmaExp, kMfmaExp}, {kMfmaBurstFma, kMfmaBurstFma},
    {kMix2, kMix2}, {kMix4, kMix4}, {kMix6, kMix6}, {kMix8, kMix8},
    {kMix5e1, kMix5e1}};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short lds_bf16x4 __attribute__((ext_vector_type(4)));

template <int ROLE>
__device__ __attribute__((noinline)) float coexec_work(int iters, int lane,
                                                       const char* lds) {
  float s = 0.f;
  if constexpr (ROLE == kMfma || ROLE == kMfmaExp || ROLE == kMfmaFma ||
                ROLE == kMfmaBurstFma) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(1e-3f * (float)((lane + e) & 7));
      b[e] = (__bf16)(1e-3f * (float)((lane * 3 + e) & 7));
    }
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 1e-3f * (float)(lane + j);
    for (int i = 0; i < iters; ++i) {
      if constexpr (ROLE == kMfmaBurstFma) {
        // The 8 MFMAs back to back, then the 128 FMAs.
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int u = 0; u < 16; ++u)
            asm volatile("v_fma_f32 %0, %0, %1, %1"
                         : "+v"(x[u]) : "v"(x[(u + 1) & 15]));
        __builtin_amdgcn_sched_barrier(0);
        continue;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
        if constexpr (ROLE == kMfmaExp) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            asm volatile("v_exp_f32 %0, %0" : "+v"(x[(4 * j + u) & 15]));
        } else if constexpr (ROLE == kMfmaFma) {
#pragma unroll
          for (int u = 0; u < 16; ++u)
            asm volatile("v_fma_f32 %0, %0, %1, %1"
                         : "+v"(x[u]) : "v"(x[(u + 1) & 15]));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc[j][r];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
  } else if constexpr (ROLE == kFma || ROLE == kExp) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = 1e-3f * (float)(lane + j);
    for (int i = 0; i < iters; ++i) {
      if constexpr (ROLE == kFma) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int u = 0; u < 16; ++u)
            asm volatile("v_fma_f32 %0, %0, %1, %1"
                         : "+v"(x[u]) : "v"(x[(u + 1) & 15]));
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u) asm volatile("v_exp_f32 %0, %0" : "+v"(x[u]));
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
  } else if constexpr (ROLE == kLds || ROLE == kLdsTr) {
    // Eight reads per iteration, each wave-wide: 1 KiB (16 bytes per lane)
    // or 512 bytes (ds_read_b64_tr_b16); addresses stay inside the 64 KiB
    // array.
    i32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = i32x4{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = (lane * 16 + ((i * 8 + j) & 63) * 1024) & 0xFFF0;
        if constexpr (ROLE == kLds) {
          v[j] ^= *(const i32x4*)(lds + off);
        } else {
          const lds_bf16x4 r = __builtin_bit_cast(
              lds_bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                              (__attribute__((address_space(3))) bf16x4*)(
                                  (__attribute__((address_space(3))) char*)(lds + off))));
          v[j].x ^= (int)r.x;
          v[j].y ^= (int)r.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s += (float)(v[j].x ^ v[j].y ^ v[j].z ^ v[j].w);
  }
  return s;
}

// The 8 MFMA chains with NF independent FMAs and NE exponentials issued
// after every MFMA: the instruction mix of a wave that interleaves its
// matrix and vector work (the attention kernels issue about 5-6 vector
// instructions and one exponential per MFMA).
template <int NF, int NE>
__device__ __attribute__((noinline)) float coexec_mix(int iters, int lane) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((lane + e) & 7));
    b[e] = (__bf16)(1e-3f * (float)((lane * 3 + e) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 1e-3f * (float)(lane + j);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < NF; ++u)
        asm volatile("v_fma_f32 %0, %0, %1, %1"
                     : "+v"(x[(NF * j + u) & 15])
                     : "v"(x[(NF * j + u + 1) & 15]));
#pragma unroll
      for (int u = 0; u < NE; ++u)
        asm volatile("v_exp_f32 %0, %0" : "+v"(x[(NE * j + u + 8) & 15]));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  return s;
}

__global__ __launch_bounds__(512, 1) void coexec_probe_kernel(int mode, int iters,
                                                              uint64_t* cycles,
                                                              float* sink) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int i = threadIdx.x; i < 65536 / 4; i += 512)
    ((float*)lds)[i] = (float)(i & 7);
  __syncthreads();
  const int role = kModeRoles[mode][wave < 4 ? 0 : 1];
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  switch (role) {
    case kMfma: s = coexec_work<kMfma>(iters, lane, lds); break;
    case kFma: s = coexec_work<kFma>(iters, lane, lds); break;
    case kExp: s = coexec_work<kExp>(iters, lane, lds); break;
    case kLds: s = coexec_work<kLds>(iters, lane, lds); break;
    case kLdsTr: s = coexec_work<kLdsTr>(iters, lane, lds); break;
    case kMfmaExp: s = coexec_work<kMfmaExp>(iters, lane, lds); break;
    case kMfmaFma: s = coexec_work<kMfmaFma>(iters, lane, lds); break;
    case kMfmaBurstFma: s = coexec_work<kMfmaBurstFma>(iters, lane, lds); break;
    case kMix2: s = coexec_mix<2, 0>(iters, lane); break;
    case kMix4: s = coexec_mix<4, 0>(iters, lane); break;
    case kMix6: s = coexec_mix<6, 0>(iters, lane); break;
    case kMix8: s = coexec_mix<8, 0>(iters, lane); break;
    case kMix5e1: s = coexec_mix<5, 1>(iters, lane); break;
    default: break;
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 512 + threadIdx.x] = s;
  if (lane == 0) {
    cycles[blockIdx.x * 16 + wave] = t1 - t0;
    cycles[blockIdx.x * 16 + 8 + wave] = r1 - r0;
  }
}


// Atomic-accumulation probe: workgroup (head, 128-key block) walks the
// 64-row query tiles its keys see (all of them, or those from the block's
// first key on under a causal mask) and adds a 64 x d fp32 tile into
// dq[head] with global fp32 atomic adds -- the HBM traffic of a dQ formed
// inside the key-outer backward kernel, one partial tile per key block and
// query tile.  Workgroups run in the head-grouped order of that kernel.
__global__ __launch_bounds__(512) void atomic_probe_kernel(int BH, int N,
                                                           int d, int causal,
                                                           float* dq) {
  const int nkb = (N + 127) / 128;
  const int bid = (int)blockIdx.x;
  int head, kb;
  if ((BH & 7) == 0) {
    const int x = bid & 7, sq = bid >> 3;
    const int hl = sq / nkb;
    head = hl * 8 + x;
    kb = sq - hl * nkb;
  } else {
    kb = bid / BH;
    head = bid - kb * BH;
  }
  float* base = dq + (int64_t)head * N * d;
  for (int i0 = causal ? kb * 128 : 0; i0 < N; i0 += 64) {
    float* t = base + (int64_t)i0 * d;
    const int lim = min(64, N - i0) * d;
    for (int e = (int)threadIdx.x; e < lim; e += 512)
      atomicAdd(t + e, 0.0009765625f);
  }
}

}  // namespace

extern "C" int fa355_coexec_probe(int mode, int iters, int blocks,
                                  uint64_t* cycles, float* sink, void* stream) {
  if (mode < 0 || mode >= kCoexecModes || iters < 1 || blocks < 1 || !cycles ||
      !sink)
    return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(coexec_probe_kernel, dim3(blocks), dim3(512), 0,
                     (hipStream_t)stream, mode, iters, cycles, sink);
  return (int)hipGetLastError();
}

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

extern "C" int fa355_atomic_probe(int BH, int N, int d, int causal, float* dq,
                                  void* stream) {
  if (BH < 1 || N < 1 || (d != 64 && d != 128) || !dq) return 1;
  (void)hipGetLastError();
  const int blocks = BH * ((N + 127) / 128);
  hipLaunchKernelGGL(atomic_probe_kernel, dim3(blocks), dim3(512), 0,
                     (hipStream_t)stream, BH, N, d, causal ? 1 : 0, dq);
  return (int)hipGetLastError();
}
