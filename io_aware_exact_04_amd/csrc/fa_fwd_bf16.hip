// Forward pass of exact attention, bf16 storage, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware": "Tiling: never
// materialise S", "Online softmax", "FlashAttention-2: better parallelism"):
// a workgroup owns one block of query rows and streams key/value tiles past
// it.  Each score tile lives only in MFMA accumulators; it is folded into a
// running row maximum, a running sum l and an unnormalised output acc.  After
// the last tile O = acc / l and L = m + ln l are written; nothing of size
// N x N reaches memory.  Tiles entirely above the causal diagonal, or removed
// by the block mask, are skipped without being loaded.
//
// gfx950 mapping:
//   * workgroup = 4 waves x 64 query rows = 256 rows; grid = B*H*ceil(N/256),
//     heaviest causal blocks dispatched first, heads the fastest index so
//     that (with B*H a multiple of 8) every query block of a head lands on
//     the same XCD and shares its L2;
//   * each wave owns its 64 rows outright as two 32-row halves; every K or V
//     fragment read from LDS feeds one MFMA per half, which halves the LDS
//     bytes per MFMA (LDS bandwidth, not the matrix cores, is the scarce
//     resource at one fragment per MFMA);
//   * S^T = K_j Q_i^T on v_mfma_f32_32x32x16_bf16 with the wave's Q
//     fragments in registers and K_j read row-major from LDS.  A lane of the
//     accumulator holds one query and 16 of every 32 keys, so the row max and
//     row sum are in-lane reductions plus one v_permlane32_swap;
//   * O^T += V_j^T P^T on the same MFMA: the exponentiated accumulator
//     registers are the B operand as they are (the key order inside each
//     16-key step is the accumulator's); the V^T operand is read from the
//     row-major V tile with ds_read_b64_tr_b16, which hands each lane four
//     consecutive keys of one column;
//   * K and V tiles go from HBM straight into LDS (buffer_load ... lds, no
//     registers on the way; rows past N arrive as zeros through the buffer
//     range check), double-buffered: the next tile's loads are in flight
//     while the current one is computed.  Tiles are row-major with the
//     16-byte units of each row XOR-swizzled so that both the 16-byte K
//     reads and the transposed V reads are free of bank conflicts on the
//     64-bank LDS;
//   * exponentials are exp2 with scale*log2(e) folded into one FMA;
//   * the output is rescaled lazily: the reference maximum of a row only
//     moves (and acc, l are multiplied by exp2(m_old - m_new)) when the tile
//     maximum exceeds it by more than 8 (a factor 256), and only if some row
//     of the wave needs it.  The result is the same exact softmax -- every
//     term of acc and l carries the same factor exp2(-m_ref) -- with P kept
//     below 256.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 64;
constexpr int kBr = 4 * kRowsPerWave;
constexpr float kLazyThreshold = 8.0f;  // log2 units

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct FwdCfg {
  static constexpr int BC = 8192 / D;   // keys per tile (64 or 128)
  static constexpr int NKB = BC / 32;   // 32-key blocks per tile
  static constexpr int NKK = BC / 16;   // 16-key MFMA steps of P V
  static constexpr int KS = D / 16;     // 16-wide steps of Q K^T
  static constexpr int DB = D / 32;     // 32-dim blocks of O
  static constexpr int TILE = BC * D;   // elements per K or V tile
};

// S^T for the 32-key sub-tile kb of the staged K tile, both 32-row halves:
// one K fragment (16-byte LDS read) feeds two MFMAs.
template <int D>
__device__ __forceinline__ void compute_s(f32x16 (&s)[2], const char* Ks,
                                          const int (&koff)[FwdCfg<D>::KS],
                                          const bf16x8 (&qf)[2][FwdCfg<D>::KS],
                                          int kb) {
  using C = FwdCfg<D>;
  bf16x8 kf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    kf[ks] = *(const bf16x8*)(Ks + koff[ks] + 32 * kb * 2 * D);
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[0][ks], s[0], 0,
                                                   0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[1][ks], s[1], 0,
                                                   0, 0);
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  // Two K and two V tiles, each its own LDS object: while one pair is read,
  // the next tile streams into the other, and the compiler can tell the two
  // apart (no wait for the in-flight loads before reading the current tile).
  __shared__ __attribute__((aligned(16))) __bf16 K0[C::TILE];
  __shared__ __attribute__((aligned(16))) __bf16 V0[C::TILE];
  __shared__ __attribute__((aligned(16))) __bf16 K1[C::TILE];
  __shared__ __attribute__((aligned(16))) __bf16 V1[C::TILE];

  const Geom& g = a.g;
  const int N = g.N;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: keep it in a scalar register
  // so that per-wave branches stay scalar.
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int BH = g.B * g.H;
  const int nqb = (N + kBr - 1) / kBr;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int qb = CAUSAL ? (nqb - 1 - rank) : rank;
  const int b = head / g.H, h = head - b * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const uint32_t head_bytes = (uint32_t)(((int64_t)(N - 1) * sn + D) * 2);
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const __bf16*)a.q + hoff,
                                              head_bytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + hoff,
                                              head_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + hoff,
                                              head_bytes);
  const __amdgpu_buffer_rsrc_t orr = make_rsrc((__bf16*)a.o + hoff,
                                               head_bytes);
  const __amdgpu_buffer_rsrc_t lr =
      make_rsrc(a.lse + (int64_t)head * N, (uint32_t)N * 4u);

  const int i0 = qb * kBr;
  const int q0w = i0 + kRowsPerWave * wave;
  const float c = g.scale_log2;

  // Q fragments (B operand of S^T): lane holds query q0w + 32qa + l32 and
  // dims 16ks + 8hh .. +7.
  bf16x8 qf[2][C::KS];
#pragma unroll
  for (int qa = 0; qa < 2; ++qa)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int off = ((q0w + 32 * qa + l32) * sn + 16 * ks + 8 * hh) * 2;
      const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
      qf[qa][ks] = __builtin_bit_cast(bf16x8, x);
    }

  // Mask rows of this workgroup (a 256-row block spans at most two) and of
  // this wave (64 rows never straddle a mask row).
  const int mb = g.mask_block;
  const uint8_t* mrow0 = MASK ? g.mask + (i0 / mb) * g.nmb : nullptr;
  const int r1 = MASK ? min(N - 1, i0 + kBr - 1) / mb : 0;
  const uint8_t* mrow1 = MASK ? g.mask + r1 * g.nmb : nullptr;
  const uint8_t* mroww =
      MASK ? g.mask + (min(q0w, N - 1) / mb) * g.nmb : nullptr;
  auto wg_keeps = [&](int j) {
    return !MASK || mrow0[j / mb] != 0 || mrow1[j / mb] != 0;
  };

  const int jend = CAUSAL ? min(N, i0 + kBr) : N;
  int j = 0;
  while (j < jend && !wg_keeps(j)) j += BC;

  float m_ref[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};
  f32x16 acc[2][C::DB];
#pragma unroll
  for (int qa = 0; qa < 2; ++qa)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) acc[qa][db] = f32x16{};

  // Per-lane LDS byte offsets.  K (16-byte reads): lane reads row
  // 32kb + l32, unit 2ks + hh.  V (transposed reads): lane group of 16 reads
  // rows 16kk + 4hh + gi/4 (+8), columns 32db + 16(gg&1) + 4(gi&3).
  const int gi = lane & 15, gg = lane >> 4;
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    koff[ks] = l32 * 2 * D + 16 * ((2 * ks + hh) ^ swz<D>(l32));
  const int vrow = 4 * hh + (gi >> 2);
  // (Rows r and r + 8 are swizzled differently: one offset for each.)
  int voff[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int r = vrow + 8 * sec;
      voff[db][sec] = r * 2 * D +
                     16 * ((4 * db + 2 * (gg & 1) + ((gi & 3) >> 1)) ^ swz<D>(r)) +
                     8 * (gi & 1);
    }

  auto next_tile = [&](int jj) {
    jj += BC;
    while (jj < jend && !wg_keeps(jj)) jj += BC;
    return jj;
  };
  // One tile: compute on (Kc, Vc) while the tile after it streams into
  // (Kn, Vn).  Instantiated twice with the buffers swapped.
  auto step = [&](const __bf16* Kc, const __bf16* Vc, __bf16* Kn, __bf16* Vn) {
    const int jn = next_tile(j);
    if (jn < jend) {
      load_rows_lds<BC, D>((char*)Kn, kr, jn, sn, wave, lane);
      load_rows_lds<BC, D>((char*)Vn, vr, jn, sn, wave, lane);
    }
    const char* Ks = (const char*)Kc;
    const char* Vs = (const char*)Vc;
      const bool active = q0w < N && (!CAUSAL || j <= q0w + kRowsPerWave - 1) &&
                          (!MASK || mroww[j / mb] != 0);
      if (active) {
        // The tile is folded in 32-key sub-tiles.  S^T of sub-tile kb+1 is
        // issued before the softmax of sub-tile kb so that the matrix cores
        // stay busy while the vector ALUs work.
        // (At d = 128 the registers of a second S^T tile do not fit beside
        // the Q fragments, so there the sub-tiles run one after the other.)
        constexpr bool kPipeline = D <= 64;
        f32x16 s_next[2];
        if (kPipeline) compute_s<D>(s_next, Ks, koff, qf, 0);
  #pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const int jk = j + 32 * kb;
          // Sub-tiles entirely above the diagonal contribute nothing.
          const bool skip = CAUSAL && jk > q0w + kRowsPerWave - 1;
          f32x16 s[2];
          if (kPipeline) {
            s[0] = s_next[0];
            s[1] = s_next[1];
            if (kb + 1 < C::NKB) compute_s<D>(s_next, Ks, koff, qf, kb + 1);
          } else if (!skip) {
            compute_s<D>(s, Ks, koff, qf, kb);
          }
          if (skip) continue;
          // Lane holds query q0w + 32qa + l32 and keys jk + 8(r/4) + 4hh + r%4.
          if ((CAUSAL && jk + 31 > q0w) || jk + 32 > N) {
            // (An opaque statement keeps this rare path a real branch instead
            // of being if-converted into selects on every sub-tile.)
            asm volatile("");
  #pragma unroll
            for (int qa = 0; qa < 2; ++qa) {
              const int q = q0w + 32 * qa + l32;
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = jk + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool ok = key < N && (!CAUSAL || key <= q);
                if (!ok) s[qa][r] = -INFINITY;
              }
            }
          }
          // Online softmax with a lazily moved reference maximum.
          float m_new[2];
          bool need = false;
  #pragma unroll
          for (int qa = 0; qa < 2; ++qa) {
            float t = -INFINITY;
  #pragma unroll
            for (int r = 0; r < 16; ++r) t = fmaxf(t, s[qa][r]);
            const float mx = swap_halves_max(t) * c;
            m_new[qa] = mx > m_ref[qa] + kLazyThreshold ? mx : m_ref[qa];
            need |= m_new[qa] != m_ref[qa];
          }
          if (__builtin_amdgcn_ballot_w64(need) != 0) {
            asm volatile("");
  #pragma unroll
            for (int qa = 0; qa < 2; ++qa) {
              const float alpha = m_new[qa] == m_ref[qa]
                                      ? 1.0f
                                      : fast_exp2(m_ref[qa] - m_new[qa]);
              l_part[qa] *= alpha;
  #pragma unroll
              for (int db = 0; db < C::DB; ++db) acc[qa][db] *= alpha;
              m_ref[qa] = m_new[qa];
            }
          }
          bf16x8 pb[2][2];
  #pragma unroll
          for (int qa = 0; qa < 2; ++qa) {
            const float m_use = m_ref[qa] == -INFINITY ? 0.f : m_ref[qa];
            float rs = 0.f;
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pr = fast_exp2(fmaf(s[qa][r], c, -m_use));
              s[qa][r] = pr;
              rs += pr;
            }
            l_part[qa] += rs;
  #pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int off = 8 * half;
              const f32x4 x0 = {s[qa][off + 0], s[qa][off + 1], s[qa][off + 2],
                                s[qa][off + 3]};
              const f32x4 x1 = {s[qa][off + 4], s[qa][off + 5], s[qa][off + 6],
                                s[qa][off + 7]};
              const bf16x4 y0 = __builtin_convertvector(x0, bf16x4);
              const bf16x4 y1 = __builtin_convertvector(x1, bf16x4);
              pb[qa][half] = bf16x8{y0[0], y0[1], y0[2], y0[3],
                                    y1[0], y1[1], y1[2], y1[3]};
            }
          }
          // O^T += V^T P^T: one V fragment feeds both 32-row halves.
  #pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int kk = 2 * kb + half;
  #pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              const bf16x4 lo = tr_read(Vs + voff[db][0] + 16 * kk * 2 * D);
              const bf16x4 hi = tr_read(Vs + voff[db][1] + 16 * kk * 2 * D);
              const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3],
                                 hi[0], hi[1], hi[2], hi[3]};
              acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  vf, pb[0][half], acc[0][db], 0, 0, 0);
              acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  vf, pb[1][half], acc[1][db], 0, 0, 0);
            }
          }
        }
      }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    j = jn;
  };

  if (j < jend) {
    load_rows_lds<BC, D>((char*)K0, kr, j, sn, wave, lane);
    load_rows_lds<BC, D>((char*)V0, vr, j, sn, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  while (j < jend) {
    step(K0, V0, K1, V1);
    if (j >= jend) break;
    step(K1, V1, K0, V0);
  }

  // ---- epilogue: O = acc / l (rows past N are dropped by the range check).
#pragma unroll
  for (int qa = 0; qa < 2; ++qa) {
    const float l = swap_halves_sum(l_part[qa]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int q = q0w + 32 * qa + l32;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const f32x4 x = {acc[qa][db][4 * grp + 0] * inv,
                         acc[qa][db][4 * grp + 1] * inv,
                         acc[qa][db][4 * grp + 2] * inv,
                         acc[qa][db][4 * grp + 3] * inv};
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        const int off = (q * sn + 32 * db + 8 * grp + 4 * hh) * 2;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, y),
                                              orr, off, 0, 0);
      }
    if (hh == 0) {
      const float L = l > 0.f ? (m_ref[qa] + log2f(l)) * kLn2 : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(L), lr, q * 4, 0, 0);
    }
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
