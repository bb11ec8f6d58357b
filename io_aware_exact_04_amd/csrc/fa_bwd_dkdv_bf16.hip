// Backward pass of exact attention, dK and dV, bf16 storage, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware", "The backward pass:
// recompute, don't store"): the forward kept only O and the row logsumexp L.
// Every probability tile is rebuilt from Q and K as P = exp(S - L), already
// normalised, and the softmax gradient's row term is the closed form
// D = rowsum(dO * O), formed beforehand by the dQ kernel.  Per tile:
//     dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P * (dP - D_i),
//     dK_j += scale dS^T Q_i.
// No N x N matrix reaches memory.  dQ_i = scale dS K_j is formed by the
// query-outer kernel, so that every gradient row is written exactly once
// and no atomics are needed.
//
// gfx950 mapping (key-block outer, two specialised waves per key slice):
//   * workgroup = 128 keys in four 32-key slices, eight waves.  For each
//     slice a "P wave" keeps K in registers and owns dV: it forms
//     S = Q K^T, P = exp(S - L) and dV += P^T dO; its partner "dS wave" keeps
//     V in registers and owns dK: it forms dP = dO V^T, takes P from its
//     partner through LDS, and forms dS = P (dP - D) and dK += dS^T Q.  Each
//     wave then holds one key-side operand and one accumulator, which fits
//     two waves per SIMD (the pair shares a SIMD), so one wave's vector work
//     overlaps the other's MFMAs;
//   * the dS waves run one query tile behind the P waves: in step t the P
//     waves work on tile t while the dS waves finish tile t-1 with the P
//     written in step t-1, so one workgroup barrier per tile orders both the
//     P hand-over and the tile buffers;
//   * query tiles of 64 rows, 32 at d = 64 (Q, dO, and L * log2(e) and D of
//     those rows, written by the dQ kernel) go from HBM straight into LDS
//     (buffer_load ... lds, so no register waits on them), triple-buffered:
//     tile t+1
//     streams in while tiles t and t-1 are read.  Rows past N arrive as
//     zeros.  Tiles are row-major with the 16-byte units of each row
//     XOR-swizzled so that neither read below meets a bank conflict: 16-byte
//     reads give the A operand of S = Q K^T and dP = dO V^T, and
//     ds_read_b64_tr_b16 (four consecutive rows of one column per lane) the
//     B operand of dV += P^T dO and dK += dS^T Q -- no transposed copies;
//   * S and dP come out with one key per lane and the same layout, so P and
//     dS feed the dV and dK contractions straight from registers and the P
//     hand-over is lane to lane (bf16, as the MFMA operand);
//   * grid = B*H*ceil(N/128) in map_block's order: with B*H a multiple of
//     8, each XCD takes whole heads one after another, all key blocks of a
//     head in a row (so a head's Q and dO are read from HBM once into that
//     XCD's L2); otherwise block ranks are outermost.  Rank 0 is the key
//     block seen by the most queries under a causal mask, so the heaviest
//     blocks start first (with a block mask and no causal mask, a head's
//     key blocks are taken in order of kept mask blocks, heaviest first);
//     causal masking is applied only on tiles that cross the diagonal.
#include "fa_internal.h"

#include <math.h>

#include <type_traits>

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlices = 4;              // 32-key slices per workgroup
constexpr int kBk = 32 * kSlices;       // keys per workgroup
constexpr int kSets = 3;                // query-tile buffers
constexpr int kPSlot = 64 * 32;         // bytes of one half's P hand-over

template <int D>
struct BwdCfg {
  // Queries per tile: 64 at d = 128; 32 at d = 64, where the smaller tiles
  // bring the LDS to 42 KiB so that two workgroups share a CU.
  static constexpr int BQ = D == 64 ? 32 : 64;
  static constexpr int NH = BQ / 32;              // 32-query halves per tile
  static constexpr int WPC = D == 64 ? 2 : 1;     // workgroups per CU
  // Waves that stream a tile pair (a whole number of 16-byte units each).
  static constexpr int DMA_WAVES = BQ * (D / 8) / 64 >= kWaves ? kWaves
                                                              : BQ * (D / 8) / 64;
  static constexpr int KS = D / 16;               // 16-wide steps over d
  static constexpr int DB = D / 32;               // 32-column blocks over d
  static constexpr int QT = BQ * D * 2;           // bytes of a Q or dO tile
  static constexpr int SET = 2 * QT + 2 * BQ * 4;  // Q, dO, L, D
  // P hand-over: three slots (one per buffer set) x four slices x the
  // 32-query halves of a tile.
  static constexpr int PBASE = kSets * SET;
  static constexpr int LDS = PBASE + kSets * kSlices * NH * kPSlot;
};

__device__ __forceinline__ bf16x8 cvt8(const f32x16& x, int off) {
  const f32x4 a = {x[off + 0], x[off + 1], x[off + 2], x[off + 3]};
  const f32x4 b = {x[off + 4], x[off + 5], x[off + 6], x[off + 7]};
  return cat(__builtin_convertvector(a, bf16x4),
             __builtin_convertvector(b, bf16x4));
}

// An LDS access is a per-lane register plus an immediate offset, which has
// 16 bits.  Regions that start at or above 64 KiB are addressed from copies
// of the per-lane offsets raised by 64 KiB (kept opaque, so that the compiler
// does not fold the 64 KiB back into a vector add at every access).
constexpr int kLdsHi = 65536;
template <bool HI, typename T>
__device__ __forceinline__ const T& lanes(const T& lo, const T& hi) {
  if constexpr (HI) return hi;
  else return lo;
}

// A += X Y^T over d for one 32-query half: X rows (Q or dO) are 16-byte
// A-operand reads from the LDS tile, Y (K or V rows of this slice) the
// B operand in registers.
template <int D>
__device__ __forceinline__ f32x16 contract_d(const char* Xs, int qh,
                                             const int (&aoff)[D / 16],
                                             const bf16x8 (&yf)[D / 16],
                                             f32x16 acc = f32x16{}) {
  constexpr int KS = D / 16;
  constexpr int BATCH = KS / 2;
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += BATCH) {
    bf16x8 xa[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      xa[u] = *(const bf16x8*)(Xs + aoff[k0 + u] + 32 * qh * 2 * D);
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[u], yf[k0 + u], acc, 0,
                                                    0, 0);
  }
  return acc;
}

// G += W^T X over one half's 32 queries: W^T (P^T or dS^T) comes from the
// registers w, X (dO or Q) through transposed reads of the LDS tile.
template <int D>
__device__ __forceinline__ void accumulate_t(f32x16 (&G)[D / 32],
                                             const bf16x8 (&w)[2],
                                             const char* Xs, int qh,
                                             const int (&toff)[D / 32][2]) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8 xb[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int o = 16 * (2 * qh + half) * 2 * D;
      xb[db] = cat(tr_read(Xs + toff[db][0] + o), tr_read(Xs + toff[db][1] + o));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
      G[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[half], xb[db], G[db],
                                                      0, 0, 0);
  }
}

template <int D, bool CAUSAL, bool MASK, bool PACKED, bool DROP>
__global__ __launch_bounds__(kThreads, BwdCfg<D>::WPC) void bwd_dkdv_bf16_kernel(
    BwdArgs a) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const Geom& g = a.g;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  // Wave index, role and slice are uniform across the wave: keep them in
  // scalar registers so that per-wave branches stay scalar.
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < kSlices;        // P/dV wave, else dS/dK wave
  const int slice = pwave ? wave : wave - kSlices;
  const int l32 = lane & 31, hh = lane >> 5;
  const int gi = lane & 15, gg = lane >> 4;

  const int BH = g.B * g.H;
  int head, rank;
  const int nkb = (g.N + kBk - 1) / kBk;
  map_block(blockIdx.x, BH, nkb, head, rank);
  // (Causal: rank 0 is the heaviest; block-masked: a head's key blocks
  // heaviest first.  Both dealt evenly over the shader engines.)
  if (CAUSAL && !PACKED) rank = snake4(rank, nkb);
  if (MASK && !CAUSAL && !PACKED)
    rank = heavy_first<kWaves>(g.mask, g.nmb, g.mask_block / kBk, nkb,
                               snake4(rank, nkb), true, (int*)smem);
  const int b = head / g.H, h = head - b * g.H;
  const HeadView hv = head_view<PACKED>(g, b, h);
  const int N = hv.N;  // rows of this head (of this sequence when packed)
  // (Blocks past a short packed sequence have nothing to do.)
  if (PACKED && rank * kBk >= N) return;
  // Keys: all, or the first kv_lens[b] with key padding (the others get
  // zero gradients).
  const int kend = g.kv_lens ? min(max(g.kv_lens[b], 0), N) : N;
  const int64_t hoff = hv.off;
  const uint32_t head_bytes = (uint32_t)(((int64_t)(N - 1) * sn + D) * 2);
  const __bf16* qbase = (const __bf16*)a.q + hoff;
  const __bf16* dobase = (const __bf16*)a.dout + hoff;
  // L * log2(e) and D of the head's rows (from the dQ kernel, which runs
  // first).
  const float* lse2_h = a.lse2 + hv.lrow;
  const float* del_h = a.delta + hv.lrow;

  const int j0 = rank * kBk;         // first key of the workgroup
  const int kw0 = j0 + 32 * slice;   // first key of this wave's slice
  const int myk = kw0 + l32;
  const float c = g.scale_log2;

  // The block-mask column of this workgroup (128 keys never straddle one);
  // a query tile never straddles a mask block either.
  MaskScan scan(MASK ? g.mask + j0 / g.mask_block : nullptr, g.nmb,
                MASK ? g.nmb : 0);
  // The first kept query tile at or after row ii (N or beyond if none).
  auto kept_from = [&](int ii) {
    return MASK && ii < N ? scan.first_kept(ii, g.mask_block) : ii;
  };
  auto next_tile = [&](int ii) { return kept_from(ii + C::BQ); };
  const uint32_t smem_lds = lds_addr(smem);
  // Stream the tile at query row ii into buffer `set`, all by DMA: Q and dO
  // (the DMA waves split the 16-byte units), and L * log2(e) and D of its
  // rows (the last wave).  Rows past N arrive as zeros; their Q and dO rows
  // are zero too, so they add nothing to dK and dV whatever P they get.
  // (Q and dO tiles share the row geometry, so one set of lane offsets.)
  const TileDma<C::BQ, D, C::DMA_WAVES> tdma(
      sn, wave < C::DMA_WAVES ? wave : 0, lane);
  auto fetch = [&](int ii, int set) {
    const uint32_t base = smem_lds + set * C::SET;
    if (wave < C::DMA_WAVES) {
      tdma.load(base, qbase, head_bytes, ii, sn, wave);
      tdma.load(base + C::QT, dobase, head_bytes, ii, sn, wave);
    }
    if (wave == kWaves - 1 && lane < C::BQ) {
      const uint32_t left = (uint32_t)(N - ii) * 4u;
      dma_b32(__builtin_amdgcn_readfirstlane(base + 2 * C::QT),
              rsrc_words(lse2_h + ii, left), 4 * lane);
      dma_b32(__builtin_amdgcn_readfirstlane(base + 2 * C::QT + 4 * C::BQ),
              rsrc_words(del_h + ii, left), 4 * lane);
    }
  };
  // Whether the 32-query half at q0 of a tile sees any key of the slice
  // (only tiles that cross the diagonal or the last key can miss).
  auto half_active = [&](bool diag, int q0) {
    return !diag || (kw0 < kend && (!CAUSAL || q0 + 31 >= kw0));
  };
  auto is_diag = [&](int i) {
    int d = __builtin_amdgcn_readfirstlane(
        (CAUSAL && i < j0 + kBk - 1) || j0 + kBk > kend);
    // (Opaque, so that the loop is not unswitched into copies.)
    asm volatile("" : "+s"(d));
    return d != 0;
  };

  int i_first = CAUSAL ? j0 : 0;  // j0 is a multiple of the tile height
  if (j0 >= kend) i_first = N;     // all keys padding: dK = dV = 0
  i_first = kept_from(i_first);
  if (i_first < N) fetch(i_first, 0);

  // The slice's K rows (P wave) or V rows (dS wave) as B operands (lane:
  // key myk, dims 16ks + 8hh .. +7); rows past N read as zero.  Loaded
  // after the first tile's loads are issued, so that the two latencies
  // overlap (using these registers makes the wave wait for them); the
  // per-lane LDS offsets below are formed while both are in flight.
  bf16x8 yf[C::KS];
  {
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(
        (const __bf16*)(pwave ? a.k : a.v) + hoff, head_bytes);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int off = (myk * sn + 16 * ks + 8 * hh) * 2;
      yf[ks] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(yr, off, 0, 0));
    }
    // (dS waves without dropout hold -V, so that the dP contraction started
    // from D yields D - dP.)
    if (!pwave && !DROP) {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        i32x4_t w = __builtin_bit_cast(i32x4_t, yf[ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] ^= (int)0x80008000u;
        yf[ks] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }
  // Per-lane LDS byte offsets.
  //  * 16-byte A-operand reads of Q / dO: row 32qh + l32, unit 2ks + hh;
  //  * transposed B-operand reads of Q / dO: rows 16kk + 4hh + gi/4 (+8),
  //    columns 32db + 16(gg&1) + 4(gi&3).
  int aoff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    aoff[ks] = l32 * 2 * D + 16 * ((2 * ks + hh) ^ swz<D>(l32));
  const int trow = 4 * hh + (gi >> 2);
  // (Rows r and r + 8 are swizzled differently: one offset for each.)
  int toff[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int r = trow + 8 * sec;
      toff[db][sec] = r * 2 * D +
                     16 * ((4 * db + 2 * (gg & 1) + ((gi & 3) >> 1)) ^ swz<D>(r)) +
                     8 * (gi & 1);
    }

  // Lane offset of the row terms (f32x4 reads: queries 8grp + 4hh ..).
  const int loff = 16 * hh;
  // The same offsets raised by 64 KiB, for regions above it (d = 128).
  int aoff_hi[C::KS], toff_hi[C::DB][2], loff_hi = 0;
  if constexpr (C::LDS > kLdsHi) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      aoff_hi[ks] = aoff[ks] + kLdsHi;
      asm volatile("" : "+v"(aoff_hi[ks]));
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        toff_hi[db][sec] = toff[db][sec] + kLdsHi;
        asm volatile("" : "+v"(toff_hi[db][sec]));
      }
    loff_hi = loff + kLdsHi;
    asm volatile("" : "+v"(loff_hi));
  }

  // dV (P wave) or dK / scale (dS wave) of the slice: lane holds dim
  // 32db + l32 and keys kw0 + 8(r/4) + 4hh + r%4.
  f32x16 G[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) G[db] = f32x16{};

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Both roles step through the same tile sequence with one barrier per
  // step; each role has its own loop so that its accumulator stays in place.
  // Step t: the P waves work on tile t (buffer set t % 3, P slot t % 3), the
  // dS waves on tile t-1 (set and P slot (t + 2) % 3), and tile t+1 streams
  // into set (t + 1) % 3.  The loops are unrolled three times so that set
  // and slot are constants and every LDS address an immediate offset from a
  // per-lane register.
  int i_cur = i_first, i_prev = N;
  auto running = [&]() { return i_cur < N || i_prev < N; };
  auto begin_step = [&](int set_next) {
    const int i_next = i_cur < N ? next_tile(i_cur) : N;
    if (i_next < N) fetch(i_next, set_next);
    return i_next;
  };
  auto end_step = [&](int i_next) {
    // Every wave is done with the tiles and P it read, the P written this
    // step is visible, and the next tile has landed.
    barrier_vmcnt<0>();
    i_prev = i_cur;
    i_cur = i_next;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  if (pwave) {
    auto step = [&](auto kc) {
      constexpr int K = decltype(kc)::value;
      const int i_next = begin_step((K + 1) % kSets);
      if (i_cur < N) {
          // P = exp(S - L) and dV += P^T dO for tile i_cur; P goes to the
          // partner through LDS.
          const int i = i_cur;
          // Q, dO and L of set K, each addressed from the low or the raised
          // lane offsets (region bases are compile-time constants).
          constexpr int QB = K * C::SET, OB = QB + C::QT, LB = QB + 2 * C::QT;
          constexpr bool QH = QB >= kLdsHi, OH = OB >= kLdsHi, LH = LB >= kLdsHi;
          const char* Qs = smem + (QH ? QB - kLdsHi : QB);
          const char* dOs = smem + (OH ? OB - kLdsHi : OB);
          const char* Ls = smem + (LH ? LB - kLdsHi : LB) + (LH ? loff_hi : loff);
          const auto& qa = lanes<QH>(aoff, aoff_hi);
          const auto& ot = lanes<OH>(toff, toff_hi);
          const bool diag = is_diag(i);
          char* Pw =
              smem + C::PBASE + ((K * kSlices + slice) * C::NH) * kPSlot;
#pragma unroll
          for (int qh = 0; qh < C::NH; ++qh) {
            const int q0 = i + 32 * qh;
            if (!half_active(diag, q0)) continue;
            f32x16 S = contract_d<D>(Qs, qh, qa, yf);
            // Lane: key myk, queries q0 + 8grp + 4hh + e.
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
              const f32x4 lv = *(const f32x4*)(Ls + 4 * (32 * qh + 8 * grp));
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * grp + e;
                S[r] = fast_exp2(fmaf(S[r], c, -lv[e]));
              }
            }
            if (diag) {
              asm volatile("");
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int qrow = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool ok = myk < kend && (!CAUSAL || myk <= qrow);
                if (!ok) S[r] = 0.f;
              }
            }
            if (DROP) {
              // dV takes the dropped P; the partner gets P with the sign bit
              // set where dropped (P >= 0, so the sign carries the decision).
              uint32_t y[4];
              drop_bytes_kcol(g, b, h, kw0 + 4 * (l32 >> 2), q0 + 4 * hh,
                              lane & 3, y);
              f32x16 Pd;
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int r = 4 * i + e;
                  const bool keep = drop_keeps(y[i], e, g.p8);
                  Pd[r] = keep ? S[r] : 0.f;
                  S[r] = keep ? S[r] : -S[r];
                }
              const bf16x8 pt[2] = {cvt8(S, 0), cvt8(S, 8)};
              *(bf16x8*)(Pw + qh * kPSlot + 16 * lane) = pt[0];
              *(bf16x8*)(Pw + qh * kPSlot + 1024 + 16 * lane) = pt[1];
              const bf16x8 pd[2] = {cvt8(Pd, 0), cvt8(Pd, 8)};
              accumulate_t<D>(G, pd, dOs, qh, ot);
            } else {
              const bf16x8 pa[2] = {cvt8(S, 0), cvt8(S, 8)};
              *(bf16x8*)(Pw + qh * kPSlot + 16 * lane) = pa[0];
              *(bf16x8*)(Pw + qh * kPSlot + 1024 + 16 * lane) = pa[1];
              accumulate_t<D>(G, pa, dOs, qh, ot);
            }
          }
      }
      end_step(i_next);
    };
    while (running()) {
      step(I0{});
      if (!running()) break;
      step(I1{});
      if (!running()) break;
      step(I2{});
    }
  } else {
    auto step = [&](auto kc) {
      constexpr int KP = (decltype(kc)::value + kSets - 1) % kSets;
      const int i_next = begin_step((decltype(kc)::value + 1) % kSets);
      if (i_prev < N) {
          // dP = dO V^T, dS = P (dP - D) and dK += dS^T Q for tile i_prev,
          // with the P its partner wrote in the previous step.
          const int i = i_prev;
          constexpr int QB = KP * C::SET, OB = QB + C::QT,
                        DB_ = QB + 2 * C::QT + 4 * C::BQ;
          constexpr bool QH = QB >= kLdsHi, OH = OB >= kLdsHi, DH = DB_ >= kLdsHi;
          const char* Qs = smem + (QH ? QB - kLdsHi : QB);
          const char* dOs = smem + (OH ? OB - kLdsHi : OB);
          const char* Dl = smem + (DH ? DB_ - kLdsHi : DB_) + (DH ? loff_hi : loff);
          const auto& qt = lanes<QH>(toff, toff_hi);
          const auto& oa = lanes<OH>(aoff, aoff_hi);
          const bool diag = is_diag(i);
          const char* Pr =
              smem + C::PBASE + ((KP * kSlices + slice) * C::NH) * kPSlot;
#pragma unroll
          for (int qh = 0; qh < C::NH; ++qh) {
            const int q0 = i + 32 * qh;
            if (!half_active(diag, q0)) continue;
            f32x16 dinit;
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
              const f32x4 dv = *(const f32x4*)(Dl + 4 * (32 * qh + 8 * grp));
#pragma unroll
              for (int e = 0; e < 4; ++e) dinit[4 * grp + e] = dv[e];
            }
            // Without dropout: D - dP (V negated, D as the start value);
            // with dropout: dP.
            f32x16 dP = DROP ? contract_d<D>(dOs, qh, oa, yf)
                             : contract_d<D>(dOs, qh, oa, yf, dinit);
            const bf16x8 pa[2] = {
                *(const bf16x8*)(Pr + qh * kPSlot + 16 * lane),
                *(const bf16x8*)(Pr + qh * kPSlot + 1024 + 16 * lane)};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = (float)pa[r >> 3][r & 7];
              if (DROP) {
                // dP reaching P is (dO V^T) Z s; a set sign bit = dropped.
                const float dz = signbit(p) ? 0.f : dP[r] * g.drop_scale;
                dP[r] = fabsf(p) * (dz - dinit[r]);
              } else {
                dP[r] = -p * dP[r];
              }
            }
            const bf16x8 sa[2] = {cvt8(dP, 0), cvt8(dP, 8)};
            accumulate_t<D>(G, sa, Qs, qh, qt);
          }
      }
      end_step(i_next);
    };
    while (running()) {
      step(I0{});
      if (!running()) break;
      step(I1{});
      if (!running()) break;
      step(I2{});
    }
  }

  // dV (P waves) or dK = scale * G (dS waves) leave through LDS, so that
  // each lane stores 16 bytes (8 dims of one key) instead of one value per
  // 2-byte store: the wave writes its 32 keys x D tile transposed (row =
  // dim, 4 keys per 8-byte write; lane holds dim 32db + l32, keys
  // 8(r/4) + 4hh + r%4) into a region of its own, and transposed reads give
  // lane j of a 16-lane group dims R .. R+3 of key C + j.  Keys past N fall
  // outside the range.
  const float gs = pwave ? (DROP ? g.drop_scale : 1.0f) : g.scale;
  constexpr int RS = 32 * 2 + 8;  // bytes per dim row (padded)
  static_assert(kWaves * D * RS <= C::LDS, "epilogue tiles exceed the LDS");
  __syncthreads();                // every wave is done with tiles and P
  char* T = smem + wave * (D * RS);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = {G[db][4 * q + 0] * gs, G[db][4 * q + 1] * gs,
                       G[db][4 * q + 2] * gs, G[db][4 * q + 3] * gs};
      *(bf16x4*)(T + (32 * db + l32) * RS + (8 * q + 4 * hh) * 2) =
          __builtin_convertvector(x, bf16x4);
    }
  // Store n: group gg takes keys 16(gg&1) + gi and dims 8o .. 8o+7,
  // o = 2n + gg/2.
  const __amdgpu_buffer_rsrc_t gr =
      make_rsrc((__bf16*)(pwave ? a.dv : a.dk) + hoff, head_bytes);
  const int key = 16 * (gg & 1) + gi;
  const int rd = T - smem + (gi >> 2) * RS + (16 * (gg & 1) + 4 * (gi & 3)) * 2;
#pragma unroll
  for (int n = 0; n < D / 16; ++n) {
    const int o = 2 * n + (gg >> 1);
    const bf16x8 y = cat(tr_read(smem + rd + 8 * o * RS),
                         tr_read(smem + rd + (8 * o + 4) * RS));
    const int off = ((kw0 + key) * sn + 8 * o) * 2;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, y), gr,
                                           off, 0, 0);
  }
}

template <int D, bool CAUSAL, bool MASK, bool PACKED = false,
          bool DROP = false>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const int nkb = (a.g.N + kBk - 1) / kBk;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nkb));
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, MASK, PACKED, DROP>),
                     grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, bool causal, hipStream_t s) {
  if (a.g.p8 > 0)  // dropout: no block mask, not packed
    return causal ? launch<D, true, false, false, true>(a, s)
                  : launch<D, false, false, false, true>(a, s);
  if (a.g.cu != nullptr)
    return causal ? launch<D, true, false, true>(a, s)
                  : launch<D, false, false, true>(a, s);
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
