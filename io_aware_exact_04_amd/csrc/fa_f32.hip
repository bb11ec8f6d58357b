// fp32 storage path: the same tiled algorithm computed entirely in fp32 on
// the vector ALUs (no bf16 anywhere, so the fp32 workload keeps fp32
// accuracy end to end).
//
// Forward ("FlashAttention: making attention IO-aware": "Tiling: never
// materialise S", "Online softmax"; the merge of partial results by their
// logsumexp is the one "In practice" describes for Flash-Decoding): a
// workgroup owns 64 query rows, one per lane, and its four waves split the
// key tiles among themselves (wave w takes tiles w, w + 4, ...).  Each wave
// keeps, per row, a reference maximum in base-2 units that moves only when a
// tile's maximum exceeds it by more than 8, the sum of exp2(s - reference)
// and the unnormalised output over its own keys.  The four partial states are
// then rescaled to their common maximum and summed through LDS.
//
// Backward ("The backward pass: recompute, don't store"): P = exp(S - L) is
// recomputed; D = rowsum(dO * O) comes from the pre-pass.  A key-outer kernel
// (one key row per lane, query tiles streamed through LDS) accumulates dK and
// dV; a query-outer kernel (one query row per lane, key tiles streamed)
// accumulates dQ in registers and writes it once.  In both, four waves split
// the streamed tiles and add their partial sums at the end.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kRows = 64;  // rows per workgroup (one per lane)

template <int D>
__device__ __forceinline__ void stage_rows(float* dst, int dst_stride,
                                           const float* src, int r0, int nrows,
                                           int N, int sn, int tid) {
  // nrows x D floats, 64 threads, 16-byte chunks.
  constexpr int CPR = D / 4;
  for (int c = tid; c < nrows * CPR; c += kRows) {
    const int row = c / CPR, col = (c % CPR) * 4;
    const int gr = r0 + row;
    const float4 x = gr < N ? *(const float4*)(src + gr * sn + col)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    float* p = dst + row * dst_stride + col;
    p[0] = x.x; p[1] = x.y; p[2] = x.z; p[3] = x.w;
  }
}

constexpr int kFwdWaves = 4;         // waves splitting the keys of 64 rows
constexpr int kFwdTile = 16;         // keys per wave and tile
constexpr float kMoveRef = 8.0f;     // log2 units

template <int D>
struct F32FwdLds {
  // Key and value tiles of each wave; after the key loop the same bytes
  // hold the four waves' partial outputs, half a row at a time.
  static constexpr int TILES = kFwdWaves * 2 * kFwdTile * D;
  static constexpr int MERGE = kFwdWaves * (D / 2) * kRows;
  static constexpr int FLOATS = TILES > MERGE ? TILES : MERGE;
};

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kRows * kFwdWaves, 1) void fwd_f32_kernel(
    FwdArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[F32FwdLds<D>::FLOATS];
  __shared__ float m_part[kFwdWaves][kRows];
  __shared__ float l_part[kFwdWaves][kRows];
  const Geom& g = a.g;
  const int N = g.N, sn = (int)g.sn;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int BH = g.B * g.H;
  const int nqb = (N + kRows - 1) / kRows;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int qb = CAUSAL ? nqb - 1 - rank : rank;
  const int b = head / g.H, h = head - b * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const float* kh = (const float*)a.k + hoff;
  const float* vh = (const float*)a.v + hoff;
  const int i0 = qb * kRows;
  const int row = i0 + lane;
  const float c2 = g.scale_log2;

  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = row < N ? ((const float*)a.q)[hoff + (int64_t)row * sn + e] : 0.f;
    acc[e] = 0.f;
  }
  float ref = -INFINITY, sum = 0.f;
  // Keys this row may see: all, or those up to the row itself.
  const int row_end = row >= N ? 0 : (CAUSAL ? row + 1 : N);
  const int block_end = CAUSAL ? min(N, i0 + kRows) : N;
  float* Ks = lds + wave * 2 * kFwdTile * D;
  float* Vs = Ks + kFwdTile * D;
  // Every wave runs the same number of rounds (the workgroup barrier of
  // the merge needs all of them); a wave whose tile is past the end idles.
  const int rounds = (block_end + kFwdWaves * kFwdTile - 1) /
                     (kFwdWaves * kFwdTile);
  for (int t = 0; t < rounds; ++t) {
    const int j0 = (t * kFwdWaves + wave) * kFwdTile;
    if (j0 >= block_end || (MASK && !mask_keeps(g, i0, j0))) continue;
    // The wave's own tile: staged and read by this wave only, so the
    // hardware's in-order LDS queue of the wave orders the accesses; the
    // wave barriers keep the compiler from moving them.
    __builtin_amdgcn_wave_barrier();
    stage_rows<D>(Ks, D, kh, j0, kFwdTile, N, sn, lane);
    stage_rows<D>(Vs, D, vh, j0, kFwdTile, N, sn, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Scores in base-2 units; keys past this row's limit do not exist.
    const int valid = min(max(row_end - j0, 0), kFwdTile);
    float s[kFwdTile];
    float top = -INFINITY;
#pragma unroll
    for (int c = 0; c < kFwdTile; ++c) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(q[e], Ks[c * D + e], dot);
      s[c] = c < valid ? dot * c2 : -INFINITY;
      top = fmaxf(top, s[c]);
    }
    if (top > ref + kMoveRef) {
      // Move the reference up to this tile's maximum (the first time from
      // -inf: nothing accumulated yet, factor 0).
      const float f = ref == -INFINITY ? 0.f : exp2f(ref - top);
      sum *= f;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] *= f;
      ref = top;
    }
    if (ref == -INFINITY) continue;   // no key of this row seen yet
#pragma unroll
    for (int c = 0; c < kFwdTile; ++c) {
      const float p = exp2f(s[c] - ref);   // 0 for keys that do not exist
      sum += p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(p, Vs[c * D + e], acc[e]);
    }
  }

  // Merge the four partial states of each row: rescale to the common
  // maximum, add the sums and the outputs.
  m_part[wave][lane] = ref;
  __syncthreads();
  float top = -INFINITY;
#pragma unroll
  for (int w = 0; w < kFwdWaves; ++w) top = fmaxf(top, m_part[w][lane]);
  const float f = ref == -INFINITY ? 0.f : exp2f(ref - top);
  l_part[wave][lane] = sum * f;
  __syncthreads();
  float total = 0.f;
#pragma unroll
  for (int w = 0; w < kFwdWaves; ++w) total += l_part[w][lane];
  const float inv = total > 0.f ? 1.0f / total : 0.f;
  float* oh = (float*)a.o + hoff;
  constexpr int HALF = D / 2, PER_WAVE = HALF / kFwdWaves;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // Partial outputs of this half row, [wave][dim][row].
#pragma unroll
    for (int e = 0; e < HALF; ++e)
      lds[(wave * HALF + e) * kRows + lane] = acc[half * HALF + e] * f;
    __syncthreads();
    // Wave w finishes dims [w PER_WAVE, (w + 1) PER_WAVE) of the half for
    // all 64 rows (row = lane).
    if (row < N) {
#pragma unroll
      for (int e = 0; e < PER_WAVE; ++e) {
        const int dim = wave * PER_WAVE + e;
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < kFwdWaves; ++w) x += lds[(w * HALF + dim) * kRows + lane];
        oh[(int64_t)row * sn + half * HALF + dim] = x * inv;
      }
    }
    __syncthreads();
  }
  if (wave == 0 && row < N)
    a.lse[(int64_t)head * N + row] =
        total > 0.f ? (top + log2f(total)) * kLn2 : -INFINITY;
}

// Backward, fp32.  A workgroup owns 64 rows (keys for dK and dV, queries
// for dQ), one per lane of each of its four waves; the waves split the
// streamed tiles of the other side (wave w takes tiles w, w + 4, ...), each
// staging its own 16-row tile in LDS, and at the end the four waves' partial
// sums are added through LDS, each wave finishing a quarter of the columns.
constexpr int kBwdWaves = 4;
constexpr int kBwdTile = 16;

// nrows x D floats into LDS rows of stride dst_stride, by NT threads.
template <int D, int NT>
__device__ __forceinline__ void stage_rows_by(float* dst, int dst_stride,
                                              const float* src, int r0,
                                              int nrows, int N, int sn,
                                              int tid) {
  constexpr int CPR = D / 4;
  for (int c = tid; c < nrows * CPR; c += NT) {
    const int row = c / CPR, col = (c % CPR) * 4;
    const int gr = r0 + row;
    const float4 x = gr < N ? *(const float4*)(src + (int64_t)gr * sn + col)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    float* p = dst + row * dst_stride + col;
    p[0] = x.x; p[1] = x.y; p[2] = x.z; p[3] = x.w;
  }
}

template <int D>
struct F32BwdLds {
  static constexpr int OWN = D + 1;                           // padded rows
  static constexpr int ROWS = 2 * kRows * OWN;                // two own arrays
  static constexpr int TILES = kBwdWaves * 2 * kBwdTile * D;  // per-wave pairs
  static constexpr int MERGE = kBwdWaves * (D / 2) * kRows;   // half the columns
  static constexpr int SCRATCH = TILES > MERGE ? TILES : MERGE;
};

// Adds the four waves' partial rows x[D] (row = lane) and writes
// out[row * sn + col] = factor * sum, through `buf` (F32BwdLds::SCRATCH
// floats).  Every thread of the workgroup must call it.
template <int D>
__device__ __forceinline__ void merge_rows(float (&x)[D], float* buf,
                                           float* out, int64_t row_off,
                                           bool valid, float factor,
                                           int wave, int lane) {
  constexpr int HALF = D / 2, PER_WAVE = HALF / kBwdWaves;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < HALF; ++e)
      buf[(wave * HALF + e) * kRows + lane] = x[half * HALF + e];
    __syncthreads();
    if (valid) {
#pragma unroll
      for (int e = 0; e < PER_WAVE; ++e) {
        const int col = wave * PER_WAVE + e;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < kBwdWaves; ++w) y += buf[(w * HALF + col) * kRows + lane];
        out[row_off + half * HALF + col] = y * factor;
      }
    }
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kRows * kBwdWaves, 1) void bwd_dkdv_f32_kernel(
    BwdArgs a) {
  using L = F32BwdLds<D>;
  constexpr int OWN = L::OWN;
  __shared__ __attribute__((aligned(16))) float own[L::ROWS];
  __shared__ __attribute__((aligned(16))) float scratch_tiles[L::SCRATCH];
  __shared__ float ld[kBwdWaves][2][kBwdTile];
  const Geom& g = a.g;
  const int N = g.N, sn = (int)g.sn;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = g.B * g.H;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int b = head / g.H, h = head - b * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const float* qh = (const float*)a.q + hoff;
  const float* doh = (const float*)a.dout + hoff;
  const float* lse_h = a.lse + (int64_t)head * N;
  const float* del_h = a.delta + (int64_t)head * N;
  const int j0 = rank * kRows;
  const int myk = j0 + lane;

  float* Kown = own;
  float* Vown = own + kRows * OWN;
  stage_rows_by<D, kRows * kBwdWaves>(Kown, OWN, (const float*)a.k + hoff, j0,
                                      kRows, N, sn, tid);
  stage_rows_by<D, kRows * kBwdWaves>(Vown, OWN, (const float*)a.v + hoff, j0,
                                      kRows, N, sn, tid);
  __syncthreads();
  float dk[D], dv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const float* kr = Kown + lane * OWN;
  const float* vr = Vown + lane * OWN;
  float* Qs = scratch_tiles + wave * 2 * kBwdTile * D;
  float* dOs = Qs + kBwdTile * D;
  // Query tiles that can see this block's keys: from the block's first key
  // (causal) or 0, to the end.
  const int i_first = CAUSAL ? j0 : 0;
  const int ntiles = N > i_first ? (N - i_first + kBwdTile - 1) / kBwdTile : 0;
  for (int t = wave; t < ntiles; t += kBwdWaves) {
    const int i0 = i_first + t * kBwdTile;
    if (MASK && !mask_keeps(g, i0, j0)) continue;
    // This wave's own tile: the wave barriers keep the compiler from moving
    // the staging across the reads (the wave's LDS accesses are in order).
    __builtin_amdgcn_wave_barrier();
    stage_rows_by<D, kRows>(Qs, D, qh, i0, kBwdTile, N, sn, lane);
    stage_rows_by<D, kRows>(dOs, D, doh, i0, kBwdTile, N, sn, lane);
    if (lane < kBwdTile) {
      const int r = i0 + lane;
      ld[wave][0][lane] = r < N ? lse_h[r] : -INFINITY;
      ld[wave][1][lane] = r < N ? del_h[r] : 0.f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (myk >= N) continue;
    for (int qi = 0; qi < kBwdTile; ++qi) {
      const int qrow = i0 + qi;
      const float Lq = ld[wave][0][qi];
      if (qrow >= N || Lq == -INFINITY || (CAUSAL && myk > qrow)) continue;
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        sc = fmaf(Qs[qi * D + e], kr[e], sc);
        dp = fmaf(dOs[qi * D + e], vr[e], dp);
      }
      const float p = expf(sc * g.scale - Lq);
      const float ds = p * (dp - ld[wave][1][qi]);
#pragma unroll
      for (int e = 0; e < D; ++e) {
        dv[e] = fmaf(p, dOs[qi * D + e], dv[e]);
        dk[e] = fmaf(ds, Qs[qi * D + e], dk[e]);
      }
    }
  }
  // The four waves' partial dK, dV of each key row, summed.
  const bool valid = myk < N;
  const int64_t row_off = (int64_t)myk * sn;
  merge_rows<D>(dk, scratch_tiles, (float*)a.dk + hoff, row_off, valid,
                g.scale, wave, lane);
  merge_rows<D>(dv, scratch_tiles, (float*)a.dv + hoff, row_off, valid, 1.0f,
                wave, lane);
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kRows * kBwdWaves, 1) void bwd_dq_f32_kernel(
    BwdArgs a) {
  using L = F32BwdLds<D>;
  constexpr int OWN = L::OWN;
  __shared__ __attribute__((aligned(16))) float own[L::ROWS];
  __shared__ __attribute__((aligned(16))) float scratch_tiles[L::SCRATCH];
  const Geom& g = a.g;
  const int N = g.N, sn = (int)g.sn;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = g.B * g.H;
  const int nqb = (N + kRows - 1) / kRows;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int qb = CAUSAL ? nqb - 1 - rank : rank;
  const int b = head / g.H, h = head - b * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const float* kh = (const float*)a.k + hoff;
  const float* vh = (const float*)a.v + hoff;
  const int i0 = qb * kRows;
  const int myq = i0 + lane;

  float* Qown = own;
  float* dOown = own + kRows * OWN;
  stage_rows_by<D, kRows * kBwdWaves>(Qown, OWN, (const float*)a.q + hoff, i0,
                                      kRows, N, sn, tid);
  stage_rows_by<D, kRows * kBwdWaves>(dOown, OWN, (const float*)a.dout + hoff,
                                      i0, kRows, N, sn, tid);
  __syncthreads();
  const float Lq = myq < N ? a.lse[(int64_t)head * N + myq] : -INFINITY;
  const float Dq = myq < N ? a.delta[(int64_t)head * N + myq] : 0.f;
  float dq[D];
#pragma unroll
  for (int e = 0; e < D; ++e) dq[e] = 0.f;
  const float* qr = Qown + lane * OWN;
  const float* dor = dOown + lane * OWN;
  float* Ks = scratch_tiles + wave * 2 * kBwdTile * D;
  float* Vs = Ks + kBwdTile * D;
  const int jend = CAUSAL ? min(N, i0 + kRows) : N;
  const int ntiles = (jend + kBwdTile - 1) / kBwdTile;
  for (int t = wave; t < ntiles; t += kBwdWaves) {
    const int j0 = t * kBwdTile;
    if (MASK && !mask_keeps(g, i0, j0)) continue;
    __builtin_amdgcn_wave_barrier();
    stage_rows_by<D, kRows>(Ks, D, kh, j0, kBwdTile, N, sn, lane);
    stage_rows_by<D, kRows>(Vs, D, vh, j0, kBwdTile, N, sn, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (myq >= N || Lq == -INFINITY) continue;
    for (int cI = 0; cI < kBwdTile; ++cI) {
      const int key = j0 + cI;
      if (key >= N || (CAUSAL && key > myq)) continue;
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        sc = fmaf(qr[e], Ks[cI * D + e], sc);
        dp = fmaf(dor[e], Vs[cI * D + e], dp);
      }
      const float p = expf(sc * g.scale - Lq);
      const float ds = p * (dp - Dq);
#pragma unroll
      for (int e = 0; e < D; ++e) dq[e] = fmaf(ds, Ks[cI * D + e], dq[e]);
    }
  }
  merge_rows<D>(dq, scratch_tiles, (float*)a.dq + hoff, (int64_t)myq * sn,
                myq < N, g.scale, wave, lane);
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.g.N + kRows - 1) / kRows;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, MASK>),
                     dim3((unsigned)(a.g.B * a.g.H * nqb)),
                     dim3(kRows * kFwdWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool MASK, bool DQ>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  const int nb = (a.g.N + kRows - 1) / kRows;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nb));
  const dim3 block(kRows * kBwdWaves);
  if (DQ)
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL, MASK>), grid, block, 0, s,
                       a);
  else
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL, MASK>), grid, block, 0,
                       s, a);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_d(const FwdArgs& a, bool causal, hipStream_t s) {
  const bool mask = a.g.mask != nullptr;
  if (causal)
    return mask ? launch_fwd<D, true, true>(a, s)
                : launch_fwd<D, true, false>(a, s);
  return mask ? launch_fwd<D, false, true>(a, s)
              : launch_fwd<D, false, false>(a, s);
}

template <int D, bool DQ>
hipError_t bwd_d(const BwdArgs& a, bool causal, hipStream_t s) {
  const bool mask = a.g.mask != nullptr;
  if (causal)
    return mask ? launch_bwd<D, true, true, DQ>(a, s)
                : launch_bwd<D, true, false, DQ>(a, s);
  return mask ? launch_bwd<D, false, true, DQ>(a, s)
              : launch_bwd<D, false, false, DQ>(a, s);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal,
                          hipStream_t s) {
  return d == 64 ? fwd_d<64>(a, causal, s) : fwd_d<128>(a, causal, s);
}

hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, bool causal,
                               hipStream_t s) {
  return d == 64 ? bwd_d<64, false>(a, causal, s)
                 : bwd_d<128, false>(a, causal, s);
}

hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, bool causal,
                             hipStream_t s) {
  return d == 64 ? bwd_d<64, true>(a, causal, s)
                 : bwd_d<128, true>(a, causal, s);
}

}  // namespace fa
