// Backward pass of exact attention, bf16 storage, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware", "The backward pass:
// recompute, don't store"): the forward kept only O and the row logsumexp L.
// Every probability tile is rebuilt from Q and K as P = exp(S - L), already
// normalised, and the softmax gradient's row term is the closed form
// D = rowsum(dO * O), computed beforehand by the pre-pass kernel.  Per tile:
//     dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P * (dP - D_i),
//     dK_j += scale dS^T Q_i,  dQ_i += scale dS K_j.
// No N x N matrix reaches memory.
//
// gfx950 mapping (key-block outer):
//   * workgroup = 4 waves x 32 keys = 128 keys; grid = B*H*ceil(N/128), the
//     causally heaviest key blocks (those seen by the most queries) first,
//     heads the fastest index;
//   * each wave keeps its K_j and V_j rows in registers as MFMA B operands and
//     accumulates its own dK_j, dV_j rows (no cross-wave reduction);
//   * query tiles of 64 rows are staged through LDS twice: row-major (A
//     operand of S = Q K^T and dP = dO V^T) and transposed (B operand of
//     dK and dV, read in the key-slot order of the accumulator layout);
//   * S and dP come out with one key per lane, so P and dS feed the dV and
//     dK contractions straight from registers;
//   * dS goes through LDS once so the four waves can form dQ_i = dS K_j over
//     all 128 keys of the block (K_j^T is staged in LDS once per
//     workgroup); the result is added with fp32 atomics into the dQ
//     accumulator in the workspace, later converted to bf16.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBk = 128;  // keys per workgroup
constexpr int kBq = 64;   // queries per tile

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;
  static constexpr int QPAD = D + 8;     // Qs / dOs row stride
  static constexpr int TPAD = kBq + 4;   // Qt / dOt row stride
  static constexpr int SPAD = kBk + 8;   // dSs row stride
  static constexpr int KTPAD = kBk + 8;  // Kt row stride
  static constexpr int Q_ELEMS = kBq * QPAD;
  static constexpr int T_ELEMS = D * TPAD;
  static constexpr int S_ELEMS = kBq * SPAD;
  static constexpr int KT_ELEMS = D * KTPAD;
  static constexpr int TB = (kBq / 4) * CPR;       // 4x8 blocks per tensor
  static constexpr int NIT = (2 * TB) / kThreads;  // blocks per thread
  static constexpr int KT_NIT = ((kBk / 4) * CPR) / kThreads;
  static constexpr int DQB = DB / 2;               // dQ blocks per wave
};

__device__ __forceinline__ uint32_t comp(const uint4& x, int p) {
  return p == 0 ? x.x : p == 1 ? x.y : p == 2 ? x.z : x.w;
}

// Write a 4-row x 8-column register block both row-major (if rm != nullptr)
// and transposed.
__device__ __forceinline__ void store_block(__bf16* rm, int rm_stride,
                                            __bf16* tr, int tr_stride,
                                            const uint4 (&w)[4], int rg,
                                            int cc) {
  if (rm != nullptr) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *(uint4*)(rm + (4 * rg + u) * rm_stride + 8 * cc) = w[u];
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w0 = comp(w[0], p), w1 = comp(w[1], p);
    const uint32_t w2 = comp(w[2], p), w3 = comp(w[3], p);
    uint2 lo, hi;
    lo.x = (w0 & 0xffffu) | (w1 << 16);
    lo.y = (w2 & 0xffffu) | (w3 << 16);
    hi.x = (w0 >> 16) | (w1 & 0xffff0000u);
    hi.y = (w2 >> 16) | (w3 & 0xffff0000u);
    *(uint2*)(tr + (8 * cc + 2 * p) * tr_stride + 4 * rg) = lo;
    *(uint2*)(tr + (8 * cc + 2 * p + 1) * tr_stride + 4 * rg) = hi;
  }
}

template <int D>
struct QStage {
  uint4 w[BwdCfg<D>::NIT][4];
  float ld;  // L*log2(e) (threads 0..63) or D (threads 64..127)
};

template <int D>
__device__ __forceinline__ void load_q(QStage<D>& st, const __bf16* qh,
                                       const __bf16* doh, const float* lse_h,
                                       const float* del_h, int i0, int N,
                                       int sn, int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int it = 0; it < C::NIT; ++it) {
    const int id = it * kThreads + tid;
    const int tensor = id / C::TB, blk = id % C::TB;
    const int rg = blk / C::CPR, cc = blk % C::CPR;
    const __bf16* src = tensor == 0 ? qh : doh;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = i0 + 4 * rg + u;
      st.w[it][u] = row < N ? *(const uint4*)(src + row * sn + 8 * cc)
                            : make_uint4(0, 0, 0, 0);
    }
  }
  if (tid < kBq) {
    const int row = i0 + tid;
    float L = row < N ? lse_h[row] : -INFINITY;
    // An empty row (L = -inf) or a padding row must give P = 0:
    // exp2(s*c - (+inf)) = 0.
    st.ld = L == -INFINITY ? INFINITY : L * kLog2e;
  } else if (tid < 2 * kBq) {
    const int row = i0 + tid - kBq;
    st.ld = row < N ? del_h[row] : 0.f;
  }
}

template <int D>
__device__ __forceinline__ void store_q(const QStage<D>& st, __bf16* Qs,
                                        __bf16* Qt, __bf16* dOs, __bf16* dOt,
                                        float* Ls, float* Ds, int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int it = 0; it < C::NIT; ++it) {
    const int id = it * kThreads + tid;
    const int tensor = id / C::TB, blk = id % C::TB;
    const int rg = blk / C::CPR, cc = blk % C::CPR;
    if (tensor == 0)
      store_block(Qs, C::QPAD, Qt, C::TPAD, st.w[it], rg, cc);
    else
      store_block(dOs, C::QPAD, dOt, C::TPAD, st.w[it], rg, cc);
  }
  if (tid < kBq)
    Ls[tid] = st.ld;
  else if (tid < 2 * kBq)
    Ds[tid - kBq] = st.ld;
}

__device__ __forceinline__ bf16x8 cvt8(const f32x16& x, int off) {
  f32x4 a = {x[off + 0], x[off + 1], x[off + 2], x[off + 3]};
  f32x4 b = {x[off + 4], x[off + 5], x[off + 6], x[off + 7]};
  bf16x4 ya = __builtin_convertvector(a, bf16x4);
  bf16x4 yb = __builtin_convertvector(b, bf16x4);
  return bf16x8{ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]};
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_bf16_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Qs[C::Q_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 dOs[C::Q_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Qt[C::T_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 dOt[C::T_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 dSs[C::S_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 Kt[C::KT_ELEMS];
  __shared__ __attribute__((aligned(16))) float Ls[kBq];
  __shared__ __attribute__((aligned(16))) float Ds[kBq];

  const Geom& g = a.g;
  const int N = g.N;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  const int BH = g.B * g.H;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int b = head / g.H, h = head - (head / g.H) * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const __bf16* qh = (const __bf16*)a.q + hoff;
  const __bf16* kh = (const __bf16*)a.k + hoff;
  const __bf16* vh = (const __bf16*)a.v + hoff;
  const __bf16* doh = (const __bf16*)a.dout + hoff;
  const float* lse_h = a.lse + (int64_t)head * N;
  const float* del_h = a.delta + (int64_t)head * N;
  float* dqa_h = a.dq_acc + (int64_t)head * N * D;

  const int j0 = rank * kBk;       // first key of the workgroup
  const int kw0 = j0 + 32 * wave;  // first key of this wave
  const int myk = kw0 + l32;
  const float c = g.scale_log2;

  // K_j^T into LDS for the dQ contraction.
#pragma unroll
  for (int it = 0; it < C::KT_NIT; ++it) {
    const int blk = it * kThreads + tid;
    const int rg = blk / C::CPR, cc = blk % C::CPR;
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = j0 + 4 * rg + u;
      w[u] = row < N ? *(const uint4*)(kh + row * sn + 8 * cc)
                     : make_uint4(0, 0, 0, 0);
    }
    store_block(nullptr, 0, Kt, C::KTPAD, w, rg, cc);
  }
  // This wave's key and value rows as B operands (lane: key myk, 8 dims).
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (myk < N) {
      kf[ks] = *(const bf16x8*)(kh + myk * sn + 16 * ks + 8 * hh);
      vf[ks] = *(const bf16x8*)(vh + myk * sn + 16 * ks + 8 * hh);
    } else {
      kf[ks] = bf16x8{};
      vf[ks] = bf16x8{};
    }
  }

  f32x16 dK[C::DB], dV[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dK[db] = f32x16{};
    dV[db] = f32x16{};
  }

  const int nq = N;
  const int mcol = MASK ? j0 / g.mask_block : 0;
  auto kept = [&](int i) {
    return !MASK || g.mask[(i / g.mask_block) * g.nmb + mcol] != 0;
  };
  int i = CAUSAL ? j0 : 0;  // j0 is a multiple of kBq
  while (i < nq && !kept(i)) i += kBq;

  QStage<D> st;
  if (i < nq) load_q<D>(st, qh, doh, lse_h, del_h, i, N, sn, tid);

  while (i < nq) {
    store_q<D>(st, Qs, Qt, dOs, dOt, Ls, Ds, tid);
    __syncthreads();
    int in = i + kBq;
    while (in < nq && !kept(in)) in += kBq;
    if (in < nq) load_q<D>(st, qh, doh, lse_h, del_h, in, N, sn, tid);

    const bool active = kw0 < N && (!CAUSAL || i + kBq - 1 >= kw0);
    if (active) {
      f32x16 S[2], dP[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        S[qb] = f32x16{};
        dP[qb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const int off = (32 * qb + l32) * C::QPAD + 16 * ks + 8 * hh;
          const bf16x8 qa = *(const bf16x8*)(Qs + off);
          const bf16x8 da = *(const bf16x8*)(dOs + off);
          S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], S[qb],
                                                          0, 0, 0);
          dP[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ks], dP[qb],
                                                           0, 0, 0);
        }
      }
      // Lane holds key myk and queries i + 32qb + 8(r/4) + 4hh + r%4.
      const bool need_mask = (CAUSAL && i < kw0 + 31) || (kw0 + 31 >= N);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int qo = 32 * qb + 8 * grp + 4 * hh;
          const f32x4 lv = *(const f32x4*)(Ls + qo);
          const f32x4 dv = *(const f32x4*)(Ds + qo);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * grp + e;
            float p = fast_exp2(fmaf(S[qb][r], c, -lv[e]));
            if (need_mask) {
              const int qrow = i + qo + e;
              const bool ok = myk < N && (!CAUSAL || myk <= qrow);
              if (!ok) p = 0.f;
            }
            S[qb][r] = p;
            dP[qb][r] = p * (dP[qb][r] - dv[e]);
          }
        }
      // dV += P^T dO, dK += dS^T Q (scale applied at the end).
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int qb = kk >> 1, off = 8 * (kk & 1);
        const bf16x8 pa = cvt8(S[qb], off);
        const bf16x8 sa = cvt8(dP[qb], off);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int toff = (32 * db + l32) * C::TPAD + 16 * kk + 4 * hh;
          const bf16x4 d0 = *(const bf16x4*)(dOt + toff);
          const bf16x4 d1 = *(const bf16x4*)(dOt + toff + 8);
          const bf16x4 q0 = *(const bf16x4*)(Qt + toff);
          const bf16x4 q1 = *(const bf16x4*)(Qt + toff + 8);
          const bf16x8 dob = {d0[0], d0[1], d0[2], d0[3],
                              d1[0], d1[1], d1[2], d1[3]};
          const bf16x8 qtb = {q0[0], q0[1], q0[2], q0[3],
                              q1[0], q1[1], q1[2], q1[3]};
          dV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, dob, dV[db],
                                                           0, 0, 0);
          dK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, qtb, dK[db],
                                                           0, 0, 0);
        }
        // dS (bf16) into LDS, [query][key].
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int q = 32 * qb + 16 * (kk & 1) + 8 * (e >> 2) + 4 * hh +
                        (e & 3);
          dSs[q * C::SPAD + 32 * wave + l32] = sa[e];
        }
      }
    } else {
      // This wave's keys are all masked for the tile: its dS columns are 0.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          dSs[q * C::SPAD + 32 * wave + l32] = (__bf16)0.f;
        }
    }
    __syncthreads();

    // dQ_i += scale * dS K_j over the workgroup's 128 keys.
    {
      const int qb = wave >> 1;
#pragma unroll
      for (int t = 0; t < C::DQB; ++t) {
        const int db = (wave & 1) * C::DQB + t;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int gk = 0; gk < kBk / 16; ++gk) {
          const bf16x8 sa = *(const bf16x8*)(dSs + (32 * qb + l32) * C::SPAD +
                                              16 * gk + 8 * hh);
          const bf16x8 kb = *(const bf16x8*)(Kt + (32 * db + l32) * C::KTPAD +
                                              16 * gk + 8 * hh);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, kb, acc, 0, 0, 0);
        }
        // Lane holds dim 32db + l32, queries 32qb + 8(r/4) + 4hh + r%4.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = i + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (qrow < N)
            unsafeAtomicAdd(dqa_h + (int64_t)qrow * D + 32 * db + l32,
                            acc[r] * g.scale);
        }
      }
    }
    i = in;
  }

  // dK, dV rows of this wave: lane holds dim 32db + l32, keys
  // kw0 + 8(r/4) + 4hh + r%4.
  __bf16* dkh = (__bf16*)a.dk + hoff;
  __bf16* dvh = (__bf16*)a.dv + hoff;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key < N) {
        dkh[key * sn + 32 * db + l32] = (__bf16)(dK[db][r] * g.scale);
        dvh[key * sn + 32 * db + l32] = (__bf16)dV[db][r];
      }
    }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const int nkb = (a.g.N + kBk - 1) / kBk;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nkb));
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, MASK>), grid,
                     dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, bool causal, hipStream_t s) {
  const bool mask = a.g.mask != nullptr;
  if (causal)
    return mask ? launch<D, true, true>(a, s) : launch<D, true, false>(a, s);
  return mask ? launch<D, false, true>(a, s) : launch<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int d, bool causal,
                                hipStream_t s) {
  if (d == 64) return launch_d<64>(a, causal, s);
  return launch_d<128>(a, causal, s);
}

}  // namespace fa
