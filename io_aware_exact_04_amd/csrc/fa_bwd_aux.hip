// Memory-bound pre-pass of the fp32 backward pass (the bf16 dQ kernel forms
// the same row terms itself): the softmax gradient's row term
// D = rowsum(dO * O) ("FlashAttention: making attention IO-aware", "The
// backward pass: recompute, don't store": it comes from vectors the forward
// already produced, so no N x N matrix is needed), one fp32 value per query
// row, and next to it the row's logsumexp in base-2 units, L * log2(e) (+inf
// for a row with no key, so that exp2(S * scale * log2(e) - it) = 0), which
// the key-outer kernel streams into LDS with the query tiles.  Every byte of O and dO is read once with 16-byte coalesced accesses;
// one row of d elements is handled by d/8 neighbouring lanes.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void unpack8(const uint4& w, float (&x)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    x[2 * p] = __uint_as_float(u[p] << 16);
    x[2 * p + 1] = __uint_as_float(u[p] & 0xffff0000u);
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;             // lanes per row
  constexpr int RPB = kThreads / TPR;    // rows per block
  const Geom& g = a.g;
  const int64_t rows = (int64_t)g.B * g.H * g.N;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (r < rows) {
    const int head = (int)(r / g.N);
    const int q = (int)(r - (int64_t)head * g.N);
    const int b = head / g.H, h = head - b * g.H;
    const int64_t off = head_offset(g, b, h) + (int64_t)q * g.sn + 8 * part;
    float o[8], d[8];
    if (BF16) {
      unpack8(*(const uint4*)((const __bf16*)a.o + off), o);
      unpack8(*(const uint4*)((const __bf16*)a.dout + off), d);
    } else {
      const float4* po = (const float4*)((const float*)a.o + off);
      const float4* pd = (const float4*)((const float*)a.dout + off);
      const float4 o0 = po[0], o1 = po[1], d0 = pd[0], d1 = pd[1];
      o[0] = o0.x; o[1] = o0.y; o[2] = o0.z; o[3] = o0.w;
      o[4] = o1.x; o[5] = o1.y; o[6] = o1.z; o[7] = o1.w;
      d[0] = d0.x; d[1] = d0.y; d[2] = d0.z; d[3] = d0.w;
      d[4] = d1.x; d[5] = d1.y; d[6] = d1.z; d[7] = d1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(o[e], d[e], acc);
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (r < rows && part == 0) {
    a.delta[r] = acc;
    const float L = a.lse[r];
    a.lse2[r] = L == -INFINITY ? INFINITY : L * kLog2e;
  }
}

}  // namespace

hipError_t launch_bwd_pre(const BwdArgs& a, int d, bool bf16, hipStream_t s) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.N;
  const int rpb = kThreads / (d / 8);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (d == 64) {
    if (bf16)
      hipLaunchKernelGGL((bwd_pre_kernel<64, true>), grid, dim3(kThreads), 0,
                         s, a);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<64, false>), grid, dim3(kThreads), 0,
                         s, a);
  } else {
    if (bf16)
      hipLaunchKernelGGL((bwd_pre_kernel<128, true>), grid, dim3(kThreads), 0,
                         s, a);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<128, false>), grid, dim3(kThreads),
                         0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fa
