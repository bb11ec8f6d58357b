// Internal declarations shared by the fa355 HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// log2(e) and ln(2) in float.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Geometry of one attention problem, shared by every kernel.
struct Geom {
  int B, H, N;
  int64_t sb, sh, sn;   // element strides of [B,H,N,d] tensors
  const uint8_t* mask;  // device block mask or nullptr
  int mask_block;       // rows/cols per mask block
  int nmb;              // mask blocks per mask row
  float scale;          // softmax scale applied to Q K^T
  float scale_log2;     // scale * log2(e)
};

struct FwdArgs {
  Geom g;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
};

struct BwdArgs {
  Geom g;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // workspace: D [B,H,N]
  float* dq_acc;  // workspace: fp32 dQ accumulator [B,H,N,d] (bf16 path)
};

// Host-side launchers, one per kernel family.  Each returns hipSuccess or
// the launch error; none synchronises.
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal,
                          hipStream_t s);
hipError_t launch_bwd_pre(const BwdArgs& a, int d, bool bf16, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int d, bool causal,
                                hipStream_t s);
hipError_t launch_bwd_dq_convert(const BwdArgs& a, int d, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int d, bool causal,
                          hipStream_t s);

// ------------------------------------------------------------ device helpers

// Exchange a value with the lane 32 away (lanes l and l^32) and combine.
__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Whether the block mask keeps the tile (query row qrow, key column kcol).
__device__ __forceinline__ bool mask_keeps(const Geom& g, int qrow, int kcol) {
  return g.mask[(qrow / g.mask_block) * g.nmb + (kcol / g.mask_block)] != 0;
}

// 64-bit element offset of head (b, h).
__device__ __forceinline__ int64_t head_offset(const Geom& g, int b, int h) {
  return (int64_t)b * g.sb + (int64_t)h * g.sh;
}

}  // namespace fa

namespace fa {

// Workgroup barrier that waits for this wave's LDS operations and for all
// but its last VMCNT vector-memory operations.  Vector-memory operations of a
// wave complete in issue order on this architecture, so the loads issued
// before the last VMCNT operations (for example LDS-bound loads issued before
// a batch of atomics) are complete when the barrier is passed, while the
// younger operations may stay in flight.  The "memory" clobber keeps the
// compiler from moving memory accesses across it.
template <int VMCNT>
__device__ __forceinline__ void barrier_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VMCNT)
               : "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace fa
