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
//   * workgroup = 4 waves x 32 query rows = 128 rows; 64-key tiles; at
//     most 256 VGPRs per wave and 64 KiB of LDS at d = 128 (168 VGPRs and
//     32 KiB at d = 64), so that two (three) workgroups share a CU and every
//     SIMD runs two (three) waves: while one wave is in the softmax (vector
//     ALU, exponentials) another keeps the matrix core busy.  The
//     workgroups synchronise independently, so their phases drift apart by
//     themselves;
//   * grid = B*H*ceil(N/128).  Causal: heaviest blocks dispatched first,
//     heads the fastest index, so that (with B*H a multiple of 8) every query
//     block of a head lands on the same XCD and shares its L2.  Otherwise
//     (all blocks cost the same) each XCD runs the query blocks of one head
//     after another, so that the blocks sharing K and V also run together;
//   * S^T = K_j Q_i^T on v_mfma_f32_32x32x16_bf16 with the wave's Q
//     fragments in registers and K_j read row-major from LDS.  A lane of the
//     accumulator holds one query and 16 of every 32 keys, so the row max and
//     row sum are in-lane reductions plus one v_permlane32_swap;
//   * O^T += V_j^T P^T on the same MFMA: the exponentiated accumulator
//     registers are the B operand as they are (the key order inside each
//     16-key step is the accumulator's); the V^T operand is read from the
//     row-major V tile with ds_read_b64_tr_b16, which hands each lane four
//     consecutive keys of one column;
//   * the scores of the next 32-key sub-tile are issued to the matrix core
//     before the softmax of the current one, so that within a wave too the
//     MFMAs overlap the vector work;
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;
constexpr float kLazyThreshold = 8.0f;  // log2 units

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct FwdCfg {
  static constexpr int BC = 64;         // keys per tile
  static constexpr int NKB = BC / 32;   // 32-key sub-tiles per tile
  static constexpr int KS = D / 16;     // 16-wide steps of Q K^T
  static constexpr int DB = D / 32;     // 32-dim blocks of O
  static constexpr int TILE = BC * D * 2;  // bytes per K or V tile
};

// S^T for the 32-key sub-tile kb of the staged K tile.
template <int D>
__device__ __forceinline__ f32x16 compute_s(const char* Ks,
                                            const int (&koff)[FwdCfg<D>::KS],
                                            const bf16x8 (&qf)[FwdCfg<D>::KS],
                                            int kb) {
  using C = FwdCfg<D>;
  bf16x8 kf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    kf[ks] = *(const bf16x8*)(Ks + koff[ks] + 32 * kb * 2 * D);
  f32x16 s = {};
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
  return s;
}

template <int D, bool CAUSAL, bool MASK, bool SPLIT, bool PACKED, bool DROP>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void fwd_bf16_kernel(
    FwdArgs a) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  // Two (K, V) tile pairs: while one is read the next streams into the other.
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];

  const Geom& g = a.g;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: keep it in a scalar register
  // so that per-wave branches stay scalar.
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int BH = g.B * g.H;
  const int nqb = (g.N + kBr - 1) / kBr;
  // Split-KV: the split index is outermost.
  const int split = SPLIT ? (int)blockIdx.x / (BH * nqb) : 0;
  const int bid = (int)blockIdx.x - split * BH * nqb;
  // Causal: heaviest blocks first, heads fastest.  Otherwise the blocks of
  // a head run together on one XCD and share its K and V in that XCD's L2
  // (block-masked: in the head's heaviest-first order, below).
  int rank, head;
  if (!CAUSAL && !SPLIT && !PACKED) {
    map_block(bid, BH, nqb, head, rank);
  } else {
    rank = bid / BH;
    head = bid - rank * BH;
  }
  // (Block-masked: a head's query blocks heaviest first.)
  const int qb = CAUSAL ? (nqb - 1 - rank)
                 : MASK && !SPLIT && !PACKED
                     ? heavy_first<kWaves>(g.mask, g.nmb, g.mask_block / kBr,
                                           nqb, snake4(rank, nqb), false,
                                           (int*)smem)
                     : rank;
  const int b = head / g.H, h = head - b * g.H;
  const HeadView hv = head_view<PACKED>(g, b, h);
  const int N = hv.N;  // rows of this head (of this sequence when packed)
  // (Blocks past a short packed sequence have nothing to do.)
  if (PACKED && qb * kBr >= N) return;
  const int64_t hoff = hv.off;
  const uint32_t head_bytes = (uint32_t)(((int64_t)(N - 1) * sn + D) * 2);
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const __bf16*)a.q + hoff,
                                              head_bytes);
  // Keys and values: Nk rows with their own strides (the query geometry
  // except in a split-KV call); query q keeps keys <= q + off when causal.
  constexpr bool packed = PACKED;
  const int Nk = packed ? N : g.Nk;
  const int off = CAUSAL ? g.causal_off : 0;
  const int snk = packed ? sn : (int)g.ksn;
  const int64_t hoff_kv =
      packed ? hoff : (int64_t)b * g.ksb + (int64_t)h * g.ksh;
  const uint32_t kv_bytes = (uint32_t)(((int64_t)(Nk - 1) * snk + D) * 2);
  const __bf16* kbase = (const __bf16*)a.k + hoff_kv;
  const __bf16* vbase = (const __bf16*)a.v + hoff_kv;
  // This workgroup's keys: all (or the first kv_lens[b] with key padding),
  // or split `split` of them.
  const int klim = g.kv_lens ? min(max(g.kv_lens[b], 0), Nk) : Nk;
  const int kbeg = SPLIT ? split * a.split_len : 0;
  const int kend = SPLIT ? min(klim, kbeg + a.split_len) : klim;
  const __amdgpu_buffer_rsrc_t orr = make_rsrc((__bf16*)a.o + hoff,
                                               head_bytes);
  const __amdgpu_buffer_rsrc_t lr =
      make_rsrc(a.lse + hv.lrow, (uint32_t)N * 4u);

  const int i0 = qb * kBr;
  const int q0w = i0 + kRowsPerWave * wave;
  const float c = g.scale_log2;

  // Q fragments (B operand of S^T): lane holds query q0w + l32 and dims
  // 16ks + 8hh .. +7.
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int off = ((q0w + l32) * sn + 16 * ks + 8 * hh) * 2;
    const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  // The block-mask row of this workgroup (128 rows never straddle one);
  // a tile of 64 keys never straddles a mask block either.
  const int mb = g.mask_block;
  MaskScan scan(MASK ? g.mask + (i0 / mb) * g.nmb : nullptr, 1,
                MASK ? g.nmb : 0);
  const int jend = CAUSAL ? min(kend, i0 + kBr + off) : kend;
  // The first kept tile at or after key jj (jend or beyond if none).
  auto kept_from = [&](int jj) {
    return MASK && jj < jend ? scan.first_kept(jj, mb) : jj;
  };
  int j = kept_from(kbeg);

  float m_ref = -INFINITY;
  float l_part = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

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

  auto next_tile = [&](int jj) { return kept_from(jj + BC); };
  // LDS: K tiles in slots 0, 1, V tiles in slots 2, 3.
  const uint32_t smem_lds = lds_addr(smem);
  // (K and V tiles share the row geometry, so one set of lane offsets.)
  const TileDma<BC, D, kWaves> tdma(snk, wave, lane);
  auto fetch_k = [&](int jj, int slot) {
    tdma.load(smem_lds + slot * C::TILE, kbase, kv_bytes, jj, snk, wave);
  };
  auto fetch_v = [&](int jj, int slot) {
    tdma.load(smem_lds + (2 + slot) * C::TILE, vbase, kv_bytes, jj, snk, wave);
  };
  // Whether this wave has unmasked keys in the tile at key jj.
  auto active = [&](int jj) {
    return q0w < N && (!CAUSAL || jj <= q0w + kRowsPerWave - 1 + off);
  };

  // Software pipeline over the kept tiles t = 0, 1, ...: while the softmax
  // of tile t runs on the vector ALUs, the matrix core forms the scores of
  // tile t+1, then P_t V_t.  K is therefore staged one tile ahead of V: in
  // step t the waves read K(t+1) and V(t) while K(t+2) and V(t+1) stream in.
  f32x16 S[C::NKB];
  int jc = j;
  int jn = jc < jend ? next_tile(jc) : jend;
  if (jc < jend) {
    fetch_k(jc, 0);
    fetch_v(jc, 0);
  }
  if (jn < jend) fetch_k(jn, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (jc < jend && active(jc)) {
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) S[kb] = compute_s<D>(smem, koff, qf, kb);
  }
  // Every wave has read K(0) before K(2) overwrites it.
  barrier_lds();
  // One step of the pipeline: softmax and P V of tile jc (its scores in Sc)
  // while the next tile's scores are formed into Sx.  Instantiated twice per
  // loop iteration with the two score arrays swapped, so that no registers
  // are copied between steps.
  int slot = 0;
  auto step = [&](f32x16 (&Sc)[C::NKB], f32x16 (&Sx)[C::NKB]) {
    const int jnn = jn < jend ? next_tile(jn) : jend;
    if (jnn < jend) fetch_k(jnn, slot);
    if (jn < jend) fetch_v(jn, slot ^ 1);
    if (active(jc)) {
      const char* Kn = smem + (slot ^ 1) * C::TILE;
      const char* Vs = smem + (2 + slot) * C::TILE;
      // Lane holds query q0w + l32 and keys jc + 32kb + 8(r/4) + 4hh + r%4.
      if ((CAUSAL && jc + BC - 1 > q0w + off) || jc + BC > kend) {
        // (An opaque statement keeps this rare path a real branch instead of
        // being if-converted into selects on every tile.)
        asm volatile("");
        const int q = q0w + l32;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = jc + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < kend && (!CAUSAL || key <= q + off);
            if (!ok) Sc[kb][r] = -INFINITY;
          }
      }
      // Online softmax over the whole tile, with a lazily moved reference
      // maximum.
      float t = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          t = fmaxf(fmaxf(t, Sc[kb][r]), Sc[kb][r + 1]);
      const float mx = swap_halves_max(t) * c;
      const float m_new = mx > m_ref + kLazyThreshold ? mx : m_ref;
      if (__builtin_amdgcn_ballot_w64(m_new != m_ref) != 0) {
        asm volatile("");
        const float alpha = m_new == m_ref ? 1.0f : fast_exp2(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
        m_ref = m_new;
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      // Scores of the next tile (harmless if there is none: the slot then
      // holds stale keys and the result is dropped) interleaved with the
      // exponentials of this one.
      bf16x8 pb[C::NKB][2];
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        Sx[kb] = compute_s<D>(Kn, koff, qf, kb);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          Sc[kb][r] = fast_exp2(fmaf(Sc[kb][r], c, -m_use));
          Sc[kb][r + 1] = fast_exp2(fmaf(Sc[kb][r + 1], c, -m_use));
          rs0 += Sc[kb][r];
          rs1 += Sc[kb][r + 1];
        }
        if (DROP) {
          // Dropout after the row sum: l normalises the undropped P.
          uint32_t y[4];
          drop_bytes_qrow(g, b, h, q0w + 4 * (l32 >> 2), jc + 32 * kb + 4 * hh,
                          lane & 3, y);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
              if (!drop_keeps(y[i], cc, g.p8)) Sc[kb][4 * i + cc] = 0.f;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int off = 8 * half;
          const f32x4 x0 = {Sc[kb][off + 0], Sc[kb][off + 1], Sc[kb][off + 2],
                            Sc[kb][off + 3]};
          const f32x4 x1 = {Sc[kb][off + 4], Sc[kb][off + 5], Sc[kb][off + 6],
                            Sc[kb][off + 7]};
          pb[kb][half] = cat(__builtin_convertvector(x0, bf16x4),
                             __builtin_convertvector(x1, bf16x4));
        }
      }
      l_part += rs0 + rs1;
      // O^T += V^T P^T.
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kk = 2 * kb + half;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const bf16x8 vf = cat(tr_read(Vs + voff[db][0] + 16 * kk * 2 * D),
                                  tr_read(Vs + voff[db][1] + 16 * kk * 2 * D));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kb][half],
                                                              acc[db], 0, 0, 0);
          }
        }
    }
    // Every wave is done with K(t+1) and V(t); K(t+2) and V(t+1) have landed.
    barrier_vmcnt<0>();
    jc = jn;
    jn = jnn;
    slot ^= 1;
  };
  f32x16 S2[C::NKB];
  while (jc < jend) {
    step(S, S2);
    if (jc >= jend) break;
    step(S2, S);
  }

  // ---- epilogue: O = acc / l (rows past N are dropped by the range check).
  const float l = swap_halves_sum(l_part);
  const float inv = l > 0.f ? (DROP ? g.drop_scale : 1.0f) / l : 0.f;
  const int q = q0w + l32;
  if (SPLIT) {
    // This split's normalised partial output and logsumexp, fp32.
    const int64_t slab = (int64_t)split * BH + head;
    const __amdgpu_buffer_rsrc_t por =
        make_rsrc(a.part_o + slab * N * D, (uint32_t)N * D * 4u);
    const __amdgpu_buffer_rsrc_t plr =
        make_rsrc(a.part_l + slab * N, (uint32_t)N * 4u);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const f32x4 x = {acc[db][4 * grp + 0] * inv, acc[db][4 * grp + 1] * inv,
                         acc[db][4 * grp + 2] * inv,
                         acc[db][4 * grp + 3] * inv};
        const int po = (q * D + 32 * db + 8 * grp + 4 * hh) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x),
                                               por, po, 0, 0);
      }
    if (hh == 0) {
      const float L = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(L), plr, q * 4, 0,
                                            0);
    }
    return;
  }
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 x = {acc[db][4 * grp + 0] * inv, acc[db][4 * grp + 1] * inv,
                       acc[db][4 * grp + 2] * inv, acc[db][4 * grp + 3] * inv};
      const bf16x4 y = __builtin_convertvector(x, bf16x4);
      const int off = (q * sn + 32 * db + 8 * grp + 4 * hh) * 2;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, y), orr,
                                            off, 0, 0);
    }
  if (hh == 0) {
    const float L = l > 0.f ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(L), lr, q * 4, 0, 0);
  }
}

template <int D, bool CAUSAL, bool MASK, bool SPLIT = false,
          bool PACKED = false, bool DROP = false>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int nqb = (a.g.N + kBr - 1) / kBr;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nqb * (SPLIT ? a.splits : 1)));
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, MASK, SPLIT, PACKED, DROP>), grid,
                     dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, bool causal, hipStream_t s) {
  if (a.g.cu != nullptr)
    return causal ? launch<D, true, false, false, true>(a, s)
                  : launch<D, false, false, false, true>(a, s);
  if (a.g.p8 > 0)  // dropout: no block mask, not packed
    return causal ? launch<D, true, false, false, false, true>(a, s)
                  : launch<D, false, false, false, false, true>(a, s);
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

hipError_t launch_fwd_splitkv_bf16(const FwdArgs& a, int d, bool causal,
                                   hipStream_t s) {
  if (d == 64)
    return causal ? launch<64, true, false, true>(a, s)
                  : launch<64, false, false, true>(a, s);
  return causal ? launch<128, true, false, true>(a, s)
                : launch<128, false, false, true>(a, s);
}

}  // namespace fa
