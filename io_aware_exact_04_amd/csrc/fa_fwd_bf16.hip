// Forward pass of exact attention, bf16 storage, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware": "Tiling: never
// materialise S", "Online softmax", "FlashAttention-2: better parallelism"):
// a workgroup owns one block of query rows and streams key/value tiles past
// it.  Each score tile lives only in MFMA accumulators; it is folded into a
// running row maximum m, a running sum l and an unnormalised output acc, with
// everything accumulated so far rescaled by exp(m_old - m_new).  After the
// last tile O = acc / l and L = m + ln l are written; nothing of size N x N
// reaches memory.  Tiles entirely above the causal diagonal, or removed by
// the block mask, are skipped without being loaded.
//
// gfx950 mapping:
//   * workgroup = 4 waves x 32 query rows = 128 rows; grid = B*H*ceil(N/128),
//     heaviest causal blocks dispatched first, heads the fastest index so
//     that (with B*H a multiple of 8) every query block of a head lands on
//     the same XCD and shares its L2;
//   * each wave owns its 32 rows outright (the per-row statistics never
//     leave the wave);
//   * S^T = K_j Q_i^T on v_mfma_f32_32x32x16_bf16: the wave's Q fragments
//     stay in registers, K_j is read from LDS.  In the accumulator layout a
//     lane holds one query and 16 of the tile's 32 keys, so the row max and
//     row sum are in-lane reductions plus one exchange with the lane 32
//     away (v_permlane32_swap);
//   * O^T += V_j^T P^T on the same MFMA: the exponentiated score registers
//     are the B operand directly (the key order inside a 16-key step is the
//     accumulator's, and V^T is read from LDS in that same order);
//   * K_j is staged row-major and V_j transposed into LDS, double-buffered;
//     the next tile's global loads are in flight while the current tile is
//     computed;
//   * exponentials are exp2 with scale*log2(e) folded into one FMA; L is
//     exported in natural log.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBr = 128;

template <int D>
struct FwdCfg {
  static constexpr int BC = 8192 / D;   // keys per tile (64 or 128)
  static constexpr int NKB = BC / 32;   // 32-key blocks per tile
  static constexpr int NKK = BC / 16;   // 16-key MFMA steps of P V
  static constexpr int KS = D / 16;     // 16-wide steps of Q K^T
  static constexpr int DB = D / 32;     // 32-dim blocks of O
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int KPAD = D + 8;    // K tile row stride (elements)
  static constexpr int VPAD = BC + 4;   // V^T tile row stride (elements)
  static constexpr int K_ELEMS = BC * KPAD;
  static constexpr int V_ELEMS = D * VPAD;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
};

struct Stage {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ uint32_t comp(const uint4& x, int p) {
  return p == 0 ? x.x : p == 1 ? x.y : p == 2 ? x.z : x.w;
}

// Global -> registers for key/value tile starting at key j0.
template <int D>
__device__ __forceinline__ void load_kv(Stage& st, const __bf16* kh,
                                        const __bf16* vh, int j0, int N,
                                        int sn, int tid) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = u * kThreads + tid;
    const int row = c / C::CPR, col = (c % C::CPR) * 8;
    const int key = j0 + row;
    st.k[u] = key < N ? *(const uint4*)(kh + key * sn + col)
                      : make_uint4(0, 0, 0, 0);
  }
  const int rg = tid / C::CPR, cc = tid % C::CPR;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int key = j0 + 4 * rg + u;
    st.v[u] = key < N ? *(const uint4*)(vh + key * sn + cc * 8)
                      : make_uint4(0, 0, 0, 0);
  }
}

// Registers -> LDS: K row-major [BC][KPAD], V transposed [D][VPAD].
template <int D>
__device__ __forceinline__ void store_kv(__bf16* buf, const Stage& st,
                                         int tid) {
  using C = FwdCfg<D>;
  __bf16* Ks = buf;
  __bf16* Vt = buf + C::K_ELEMS;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = u * kThreads + tid;
    const int row = c / C::CPR, col = (c % C::CPR) * 8;
    *(uint4*)(Ks + row * C::KPAD + col) = st.k[u];
  }
  const int rg = tid / C::CPR, cc = tid % C::CPR;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t w0 = comp(st.v[0], p), w1 = comp(st.v[1], p);
    const uint32_t w2 = comp(st.v[2], p), w3 = comp(st.v[3], p);
    uint2 lo, hi;
    lo.x = (w0 & 0xffffu) | (w1 << 16);
    lo.y = (w2 & 0xffffu) | (w3 << 16);
    hi.x = (w0 >> 16) | (w1 & 0xffff0000u);
    hi.y = (w2 >> 16) | (w3 & 0xffff0000u);
    *(uint2*)(Vt + (8 * cc + 2 * p) * C::VPAD + 4 * rg) = lo;
    *(uint2*)(Vt + (8 * cc + 2 * p + 1) * C::VPAD + 4 * rg) = hi;
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::BUF_ELEMS];

  const Geom& g = a.g;
  const int N = g.N;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  const int BH = g.B * g.H;
  const int nqb = (N + kBr - 1) / kBr;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int qb = CAUSAL ? (nqb - 1 - rank) : rank;
  const int b = head / g.H, h = head - (head / g.H) * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const __bf16* qh = (const __bf16*)a.q + hoff;
  const __bf16* kh = (const __bf16*)a.k + hoff;
  const __bf16* vh = (const __bf16*)a.v + hoff;
  __bf16* oh = (__bf16*)a.o + hoff;

  const int i0 = qb * kBr;
  const int q0w = i0 + 32 * wave;
  const int myq = q0w + l32;
  const float c = g.scale_log2;

  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (myq < N)
      qf[ks] = *(const bf16x8*)(qh + myq * sn + 16 * ks + 8 * hh);
    else
      qf[ks] = bf16x8{};
  }

  const int jend = CAUSAL ? min(N, i0 + kBr) : N;
  const uint8_t* mrow =
      MASK ? g.mask + (i0 / g.mask_block) * g.nmb : nullptr;
  auto kept = [&](int j) {
    return !MASK || mrow[j / g.mask_block] != 0;
  };
  int j = 0;
  while (j < jend && !kept(j)) j += BC;

  float m_run = -INFINITY;
  float l_part = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  Stage st;
  int buf = 0;
  if (j < jend) {
    load_kv<D>(st, kh, vh, j, N, sn, tid);
    store_kv<D>(smem, st, tid);
  }
  __syncthreads();

  while (j < jend) {
    int jn = j + BC;
    while (jn < jend && !kept(jn)) jn += BC;
    if (jn < jend) load_kv<D>(st, kh, vh, jn, N, sn, tid);

    const __bf16* Ks = smem + buf * C::BUF_ELEMS;
    const __bf16* Vt = Ks + C::K_ELEMS;
    const bool active = q0w < N && (!CAUSAL || j <= q0w + 31);
    if (active) {
      // S^T tile: lane holds query myq, keys j + 32kb + 8(r/4) + 4hh + r%4.
      f32x16 s[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(Ks + (32 * kb + l32) * C::KPAD +
                                              16 * ks + 8 * hh);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb],
                                                          0, 0, 0);
        }
      }
      const bool need_mask = (CAUSAL && j + BC - 1 > q0w) || (j + BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= myq);
            if (!ok) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = swap_halves_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], c, -m_use));
          s[kb][r] = p;
          rs += p;
        }
      l_part = l_part * alpha + rs;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
      m_run = m_new;

      bf16x8 pb[C::NKK];
#pragma unroll
      for (int kk = 0; kk < C::NKK; ++kk) {
        const int kb = kk >> 1, off = 8 * (kk & 1);
        f32x4 x0 = {s[kb][off + 0], s[kb][off + 1], s[kb][off + 2],
                    s[kb][off + 3]};
        f32x4 x1 = {s[kb][off + 4], s[kb][off + 5], s[kb][off + 6],
                    s[kb][off + 7]};
        bf16x4 y0 = __builtin_convertvector(x0, bf16x4);
        bf16x4 y1 = __builtin_convertvector(x1, bf16x4);
        pb[kk] = bf16x8{y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk) {
          const __bf16* vp = Vt + (32 * db + l32) * C::VPAD + 16 * kk + 4 * hh;
          const bf16x4 lo = *(const bf16x4*)vp;
          const bf16x4 hi = *(const bf16x4*)(vp + 8);
          const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3],
                             hi[0], hi[1], hi[2], hi[3]};
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kk], acc[db],
                                                            0, 0, 0);
        }
      }
    }
    if (jn < jend) store_kv<D>(smem + (buf ^ 1) * C::BUF_ELEMS, st, tid);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  const float l = swap_halves_sum(l_part);
  if (myq < N) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        f32x4 x = {acc[db][4 * grp + 0] * inv, acc[db][4 * grp + 1] * inv,
                   acc[db][4 * grp + 2] * inv, acc[db][4 * grp + 3] * inv};
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        *(bf16x4*)(oh + myq * sn + 32 * db + 8 * grp + 4 * hh) = y;
      }
    if (hh == 0)
      a.lse[(int64_t)head * N + myq] =
          l > 0.f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.g.N + kBr - 1) / kBr;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nqb));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, MASK>), grid, dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, bool causal, hipStream_t s) {
  const bool mask = a.g.mask != nullptr;
  if (causal)
    return mask ? launch<D, true, true>(a, s) : launch<D, true, false>(a, s);
  return mask ? launch<D, false, true>(a, s) : launch<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal,
                           hipStream_t s) {
  if (d == 64) return launch_d<64>(a, causal, s);
  return launch_d<128>(a, causal, s);
}

}  // namespace fa
