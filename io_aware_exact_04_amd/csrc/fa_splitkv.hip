// Merge step of the split-KV forward ("FlashAttention: making attention
// IO-aware", "In practice": Flash-Decoding splits the keys across
// workgroups and combines the partial results with the logsumexp rescaling
// of the online softmax).  Split s of a query row produced its own
// normalised output O_s and logsumexp L_s over its keys; over all keys
//     L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s.
// Evaluated with the largest L_s subtracted; splits with no keys for the row
// (L_s = -inf) weigh zero, and a row with no keys at all gets O = 0 and
// L = -inf.  Memory-bound: every partial is read once, 16 bytes per lane,
// d/8 neighbouring lanes per row.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void splitkv_merge_kernel(FwdArgs a) {
  constexpr int TPR = D / 8;            // lanes per row
  constexpr int RPB = kThreads / TPR;   // rows per block
  const Geom& g = a.g;
  const int64_t rows = (int64_t)g.B * g.H * g.N;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (r >= rows) return;
  const int head = (int)(r / g.N);
  const int q = (int)(r - (int64_t)head * g.N);
  const int b = head / g.H, h = head - b * g.H;

  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.part_l[s * rows + r]);
  float sum = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      const float w = expf(a.part_l[s * rows + r] - mx);
      sum += w;
      const float4* po =
          (const float4*)(a.part_o + (s * rows + r) * D + 8 * part);
      const float4 x0 = po[0], x1 = po[1];
      o[0] = fmaf(w, x0.x, o[0]);
      o[1] = fmaf(w, x0.y, o[1]);
      o[2] = fmaf(w, x0.z, o[2]);
      o[3] = fmaf(w, x0.w, o[3]);
      o[4] = fmaf(w, x1.x, o[4]);
      o[5] = fmaf(w, x1.y, o[5]);
      o[6] = fmaf(w, x1.z, o[6]);
      o[7] = fmaf(w, x1.w, o[7]);
    }
  }
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  bf16x8 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (__bf16)(o[e] * inv);
  *(bf16x8*)((__bf16*)a.o + head_offset(g, b, h) + (int64_t)q * g.sn +
             8 * part) = y;
  if (part == 0) a.lse[r] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

}  // namespace

hipError_t launch_splitkv_merge(const FwdArgs& a, int d, hipStream_t s) {
  const int64_t rows = (int64_t)a.g.B * a.g.H * a.g.N;
  const int rpb = kThreads / (d / 8);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (d == 64)
    hipLaunchKernelGGL((splitkv_merge_kernel<64>), grid, dim3(kThreads), 0, s,
                       a);
  else
    hipLaunchKernelGGL((splitkv_merge_kernel<128>), grid, dim3(kThreads), 0, s,
                       a);
  return hipGetLastError();
}

}  // namespace fa
