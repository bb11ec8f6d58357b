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

// Split-KV decode, one query row per (b, h): the per-split pass of the
// split-KV forward when there is a single query, which reads each key and
// value once and does 4 d flops per key -- HBM-bound, so it runs on the
// vector ALUs in fp32 instead of the 128-row matrix-core forward (which
// would spend a whole 128-row block of MFMA work on one row).  A workgroup
// of 4 waves takes split `split` of head (b, h); a lane group of 16 lanes
// takes one key row (d/16 dims per lane) and wave w the key batches
// w, w + 4, ... of 64 keys (key base + 4u + group, u < 16, so that one load
// instruction reads four whole rows), all loads of a batch issued before the
// first is used.  Each of the 16 (wave, group) streams keeps its own online
// softmax state (running maximum m in base-2 units, sum l and unnormalised
// output) over its keys; at the end they are combined with the logsumexp
// rescaling ("FlashAttention: making attention IO-aware", "Online softmax")
// into the split's normalised output and logsumexp, the same partials the
// merge kernel above reads.
constexpr int kDecThreads = 256;
constexpr int kDecU = 16;  // keys per lane group and batch

// Sum over the 16 lanes of a DPP row, the same bits in every lane: each
// step adds a value and its partner's, and both partners add the same two
// numbers (xor 1, xor 2, then the mirrors within 8 and 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF,
                                         false);
  return v + __int_as_float(o);
}
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x = dpp_add<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x = dpp_add<0x141>(x);  // row_half_mirror
  x = dpp_add<0x140>(x);  // row_mirror
  return x;
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(FwdArgs a) {
  constexpr int DPL = D / 16;  // dims per lane
  typedef int ivec __attribute__((ext_vector_type(DPL / 2)));
  const Geom& g = a.g;
  const int BH = g.B * g.H;
  const int split = (int)blockIdx.x / BH;
  const int head = (int)blockIdx.x - split * BH;
  const int b = head / g.H, h = head - b * g.H;
  const int lane = (int)threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int grp = lane >> 4, part = lane & 15;
  const int kbeg = split * a.split_len;
  const int kend = min(g.Nk, kbeg + a.split_len);
  const float c = g.scale_log2;

  // The query's dims DPL * part .. +DPL-1, times scale * log2(e).
  float qv[DPL];
  {
    const ivec w = *(const ivec*)((const __bf16*)a.q + head_offset(g, b, h) +
                                  DPL * part);
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i) {
      qv[2 * i] = __uint_as_float((uint32_t)w[i] << 16) * c;
      qv[2 * i + 1] = __uint_as_float((uint32_t)w[i] & 0xffff0000u) * c;
    }
  }
  const int64_t kvoff = (int64_t)b * g.ksb + (int64_t)h * g.ksh;
  const uint32_t kv_bytes = (uint32_t)(((int64_t)(g.Nk - 1) * g.ksn + D) * 2);
  const __amdgpu_buffer_rsrc_t kr =
      make_rsrc((const __bf16*)a.k + kvoff, kv_bytes);
  const __amdgpu_buffer_rsrc_t vr =
      make_rsrc((const __bf16*)a.v + kvoff, kv_bytes);

  float m = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  constexpr int KB = 4 * kDecU;  // keys per wave batch
  for (int base = kbeg + wave * KB; base < kend; base += 4 * KB) {
    ivec kx[kDecU], vx[kDecU];
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const int key = base + 4 * u + grp;
      const int off = (key * (int)g.ksn + DPL * part) * 2;
      if constexpr (DPL == 8) {
        kx[u] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
        vx[u] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
      } else {
        kx[u] = __builtin_amdgcn_raw_buffer_load_b64(kr, off, 0, 0);
        vx[u] = __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0);
      }
    }
    float sc[kDecU];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      float d0 = 0.f;
#pragma unroll
      for (int i = 0; i < DPL / 2; ++i) {
        d0 = fmaf(qv[2 * i], __uint_as_float((uint32_t)kx[u][i] << 16), d0);
        d0 = fmaf(qv[2 * i + 1],
                  __uint_as_float((uint32_t)kx[u][i] & 0xffff0000u), d0);
      }
      const float sv = row16_sum(d0);
      sc[u] = base + 4 * u + grp < kend ? sv : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    const float m_new = fmaxf(m, mx);
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - mu);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const float p = fast_exp2(sc[u] - mu);
      l += p;
#pragma unroll
      for (int i = 0; i < DPL / 2; ++i) {
        acc[2 * i] =
            fmaf(p, __uint_as_float((uint32_t)vx[u][i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(
            p, __uint_as_float((uint32_t)vx[u][i] & 0xffff0000u), acc[2 * i + 1]);
      }
    }
    m = m_new;
  }

  // Combine the 16 (wave, group) states: M = max m, weights 2^(m - M).
  __shared__ float sm[16], sl[16], sacc[16][D];
  const int st = wave * 4 + grp;
  if (part == 0) {
    sm[st] = m;
    sl[st] = l;
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) sacc[st][DPL * part + i] = acc[i];
  __syncthreads();
  const int t = (int)threadIdx.x;
  if (t < D) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, sm[i]);
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float wgt = fast_exp2(sm[i] - M);
        L = fmaf(sl[i], wgt, L);
        o = fmaf(sacc[i][t], wgt, o);
      }
    }
    const int64_t rows = BH;  // one query row per head
    a.part_o[((int64_t)split * rows + head) * D + t] = L > 0.f ? o / L : 0.f;
    if (t == 0)
      a.part_l[(int64_t)split * rows + head] =
          L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode_split_bf16(const FwdArgs& a, int d, hipStream_t s) {
  const dim3 grid((unsigned)(a.g.B * a.g.H * a.splits));
  if (d == 64)
    hipLaunchKernelGGL((decode_split_kernel<64>), grid, dim3(kDecThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<128>), grid, dim3(kDecThreads), 0,
                       s, a);
  return hipGetLastError();
}

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
