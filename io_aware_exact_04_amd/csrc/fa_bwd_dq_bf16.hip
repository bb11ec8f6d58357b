// Backward pass of exact attention, dQ, bf16 storage, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware", "The backward pass:
// recompute, don't store"): dQ_i = scale * sum_j dS_ij K_j with the
// probability tile rebuilt as P = exp(S - L) from Q and K, dP = dO V^T and
// dS = P * (dP - D), D = rowsum(dO * O).  This kernel is query-outer: a
// workgroup owns a block of query rows, streams the key and value tiles
// past it and keeps dQ in registers, so every dQ row is written once by one
// workgroup -- no atomics and no fp32 accumulator in memory.  It runs first
// in the backward pass and also forms each of its rows' D and L * log2(e)
// (it holds the row's dO already; O is one more 16-byte load per lane and
// step over d) into the workspace for the key-outer kernel, which produces
// dK and dV; the price of the split is that S and dP are formed twice.
//
// gfx950 mapping (the forward kernel's, with dP and dS in place of the
// online softmax):
//   * workgroup = 4 waves x 32 query rows = 128 rows, 64-key tiles, at most
//     256 VGPRs per wave and 64 KiB of LDS (168 and 32 KiB at d = 64), so
//     that two (three at d = 64) workgroups share a CU and the waves on each
//     SIMD overlap one's vector work with another's MFMAs; grid = B*H*ceil(N/128), heaviest causal blocks first, heads the
//     fastest index (without causal mask: the blocks of a head one after
//     another on one XCD);
//   * the wave's Q and dO rows stay in registers as MFMA B operands;
//     S^T = K_j Q_i^T and dP^T = V_j dO_i^T on v_mfma_f32_32x32x16_bf16 with
//     K_j and V_j read row-major from LDS;
//   * a lane of the accumulators holds one query, so L_i and D_i are
//     per-lane scalars;
//   * dQ^T += K_j^T dS^T: the dS accumulator registers, rounded to bf16, are
//     the B operand as they are (the key order inside each 16-key step is
//     the accumulator's) and K_j^T is read from the same row-major K tile
//     with ds_read_b64_tr_b16;
//   * K and V tiles go HBM -> LDS with buffer_load ... lds, double-buffered,
//     16-byte units XOR-swizzled against LDS bank conflicts; rows past N
//     arrive as zeros and their scores are masked.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct DqCfg {
  static constexpr int BC = 64;         // keys per tile
  static constexpr int NKB = BC / 32;   // 32-key blocks per tile
  static constexpr int KS = D / 16;     // 16-wide steps over d
  static constexpr int DB = D / 32;     // 32-dim blocks of dQ
  static constexpr int TILE = BC * D * 2;  // bytes per K or V tile
};

__device__ __forceinline__ bf16x8 cvt8(const f32x16& x, int off) {
  const f32x4 a = {x[off + 0], x[off + 1], x[off + 2], x[off + 3]};
  const f32x4 b = {x[off + 4], x[off + 5], x[off + 6], x[off + 7]};
  return cat(__builtin_convertvector(a, bf16x4),
             __builtin_convertvector(b, bf16x4));
}

template <int D, bool CAUSAL, bool MASK, bool PACKED, bool DROP>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void bwd_dq_bf16_kernel(
    BwdArgs a) {
  using C = DqCfg<D>;
  constexpr int BC = C::BC;
  // Two (K, V) tile pairs: while one is read the next streams into the other.
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];

  const Geom& g = a.g;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int gi = lane & 15, gg = lane >> 4;

  const int BH = g.B * g.H;
  const int nqb = (g.N + kBr - 1) / kBr;
  // Causal: heaviest blocks first, heads fastest.  Otherwise the blocks of
  // a head run together on one XCD and share its K and V in that L2.
  int rank, head;
  if (!CAUSAL && !PACKED) {
    map_block((int)blockIdx.x, BH, nqb, head, rank);
  } else {
    rank = (int)blockIdx.x / BH;
    head = (int)blockIdx.x - rank * BH;
  }
  // (Block-masked: a head's query blocks heaviest first.)
  const int qb = CAUSAL ? (nqb - 1 - rank)
                 : MASK && !PACKED
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
  const __bf16* kbase = (const __bf16*)a.k + hoff;
  const __bf16* vbase = (const __bf16*)a.v + hoff;
  const __amdgpu_buffer_rsrc_t dor = make_rsrc((const __bf16*)a.dout + hoff,
                                               head_bytes);
  const __amdgpu_buffer_rsrc_t dqr = make_rsrc((__bf16*)a.dq + hoff,
                                               head_bytes);
  const __amdgpu_buffer_rsrc_t orr = make_rsrc((const __bf16*)a.o + hoff,
                                               head_bytes);
  const float* lse_h = a.lse + hv.lrow;

  const int i0 = qb * kBr;
  const int q0w = i0 + kRowsPerWave * wave;
  const float c = g.scale_log2;

  // Q and dO fragments (B operands of S^T and dP^T), and O: lane holds
  // query q0w + l32 and dims 16ks + 8hh .. +7; rows past N read as zero.
  bf16x8 qf[C::KS], df[C::KS], of[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int off = ((q0w + l32) * sn + 16 * ks + 8 * hh) * 2;
    qf[ks] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
    df[ks] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(dor, off, 0, 0));
    of[ks] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(orr, off, 0, 0));
  }
  const int myq = q0w + l32;
  const float Lq = myq < N ? lse_h[myq] : -INFINITY;

  // The block-mask row of this workgroup (128 rows never straddle one);
  // a tile of 64 keys never straddles a mask block either.
  const int mb = g.mask_block;
  MaskScan scan(MASK ? g.mask + (i0 / mb) * g.nmb : nullptr, 1,
                MASK ? g.nmb : 0);

  // Keys: all, or the first kv_lens[b] with key padding.
  const int kend = g.kv_lens ? min(max(g.kv_lens[b], 0), N) : N;
  const int jend = CAUSAL ? min(kend, i0 + kBr) : kend;
  // The first kept tile at or after key jj (jend or beyond if none).
  auto kept_from = [&](int jj) {
    return MASK && jj < jend ? scan.first_kept(jj, mb) : jj;
  };
  int j = kept_from(0);

  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  // Per-lane LDS byte offsets.  K and V rows (16-byte reads): lane reads row
  // 32kb + l32, unit 2ks + hh.  K^T (transposed reads): lane group of 16
  // reads rows 16kk + 4hh + gi/4 (+8), columns 32db + 16(gg&1) + 4(gi&3).
  // They include the current buffer set's offset (2 TILE bytes per set,
  // above every in-tile offset, so one XOR flips the set) and are flipped
  // once per tile; every read is then a register plus an immediate.
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    koff[ks] = l32 * 2 * D + 16 * ((2 * ks + hh) ^ swz<D>(l32));
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

  auto next_tile = [&](int jj) { return kept_from(jj + BC); };
  const uint32_t smem_lds = lds_addr(smem);
  // (K and V tiles share the row geometry, so one set of lane offsets.)
  const TileDma<BC, D, kWaves> tdma(sn, wave, lane);
  auto fetch = [&](int jj, int set) {
    const uint32_t base = smem_lds + set * 2 * C::TILE;
    tdma.load(base, kbase, head_bytes, jj, sn, wave);
    tdma.load(base + C::TILE, vbase, head_bytes, jj, sn, wave);
  };

  int set = 0;
  if (j < jend) fetch(j, 0);
  // (The lane offsets address rows below 32 of a 64-row tile, so they stay
  // below TILE; with TILE a power of two, XOR by 2 TILE adds or removes
  // exactly one set.)
  static_assert((C::TILE & (C::TILE - 1)) == 0, "TILE must be a power of two");
  // The row terms of the lane's query, from vectors the forward already
  // produced ("FlashAttention: making attention IO-aware", "The backward
  // pass: recompute, don't store"): D = rowsum(dO * O) -- this lane holds
  // half of the row's dims, lane l ^ 32 the other half -- and L * log2(e)
  // (+inf for an empty or padding row, so that P = 0).  Both go to the
  // workspace for the key-outer kernel, which runs after this one.  (Formed
  // after the first tiles' loads are issued, so that the wait for O and dO
  // overlaps theirs.)
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dpart = fmaf((float)of[ks][e], (float)df[ks][e], dpart);
  const float dsum = swap_halves_sum(dpart);
  const float lc = Lq == -INFINITY ? INFINITY : Lq * kLog2e;
  const float dl = myq < N ? dsum : 0.f;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (hh == 0 && myq < N) {
    a.delta[hv.lrow + myq] = dl;
    a.lse2[hv.lrow + myq] = lc;
  }
  // Without dropout the dP^T contraction starts from -D (every accumulator
  // slot of a lane belongs to its one query), so it yields dP - D and dS is
  // one multiply per element.
  f32x16 neg_d;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_d[r] = -dl;
  while (j < jend) {
    const int jn = next_tile(j);
    if (jn < jend) fetch(jn, set ^ 1);
    const char* Ks = smem;  // (the set is in koff and toff)
    const char* Vs = smem + C::TILE;
    // Sub-tiles at or past this key start above the wave's causal diagonal
    // or past the last key.
    const int kstop =
        min(CAUSAL ? min(j + BC, q0w + kRowsPerWave) : j + BC, kend);
    if (q0w < N) {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        const int jk = j + 32 * kb;
        if (jk >= kstop) break;
        // S^T and dP^T for the 32 keys jk..
        f32x16 s = {}, dp = DROP ? f32x16{} : neg_d;
        {
          constexpr int BATCH = C::KS / 2;
#pragma unroll
          for (int k0 = 0; k0 < C::KS; k0 += BATCH) {
            bf16x8 kf[BATCH], vf[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
              kf[u] = *(const bf16x8*)(Ks + koff[k0 + u] + 32 * kb * 2 * D);
              vf[u] = *(const bf16x8*)(Vs + koff[k0 + u] + 32 * kb * 2 * D);
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[u], qf[k0 + u], s,
                                                          0, 0, 0);
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u], df[k0 + u],
                                                           dp, 0, 0, 0);
            }
          }
        }
        // dS = P (dP - D), P = exp2(S c - L log2 e) (without dropout dp
        // already holds dP - D).  Lane holds query
        // q0w + l32 and keys jk + 8(r/4) + 4hh + r%4.
        if (DROP) {
          // dP reaching P is (dO V^T) Z s: zero where dropped.
          uint32_t y[4];
          drop_bytes_qrow(g, b, h, q0w + 4 * (l32 >> 2), jk + 4 * hh, lane & 3,
                          y);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
              const int r = 4 * i + cc;
              dp[r] = drop_keeps(y[i], cc, g.p8) ? dp[r] * g.drop_scale : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[r], c, -lc));
          s[r] = DROP ? p * (dp[r] - dl) : p * dp[r];
        }
        if ((CAUSAL && jk + 31 > q0w) || jk + 32 > kend) {
          // (An opaque statement keeps this rare path a real branch instead
          // of being if-converted into selects on every sub-tile.)
          asm volatile("");
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = jk + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < kend && (!CAUSAL || key <= myq);
            if (!ok) s[r] = 0.f;
          }
        }
        const bf16x8 sb[2] = {cvt8(s, 0), cvt8(s, 8)};
        // dQ^T += K^T dS^T.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kk = 2 * kb + half;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const bf16x8 kt = cat(tr_read(Ks + toff[db][0] + 16 * kk * 2 * D),
                                  tr_read(Ks + toff[db][1] + 16 * kk * 2 * D));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt, sb[half],
                                                              acc[db], 0, 0, 0);
          }
        }
      }
    }
    // Every wave is done with the current pair, and the next one has landed.
    barrier_vmcnt<0>();
    j = jn;
    set ^= 1;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) koff[ks] ^= 2 * C::TILE;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      toff[db][0] ^= 2 * C::TILE;
      toff[db][1] ^= 2 * C::TILE;
    }
  }

  // dQ = scale * acc: lane holds query q0w + l32 and dims
  // 32db + 8grp + 4hh .. +3; rows past N fall outside the range.
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const f32x4 x = {acc[db][4 * grp + 0] * g.scale,
                       acc[db][4 * grp + 1] * g.scale,
                       acc[db][4 * grp + 2] * g.scale,
                       acc[db][4 * grp + 3] * g.scale};
      const bf16x4 y = __builtin_convertvector(x, bf16x4);
      const int off = (myq * sn + 32 * db + 8 * grp + 4 * hh) * 2;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, y), dqr,
                                            off, 0, 0);
    }
}

template <int D, bool CAUSAL, bool MASK, bool PACKED = false,
          bool DROP = false>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const int nqb = (a.g.N + kBr - 1) / kBr;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nqb));
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, MASK, PACKED, DROP>),
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

hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int d, bool causal,
                              hipStream_t s) {
  if (d == 64) return launch_d<64>(a, causal, s);
  return launch_d<128>(a, causal, s);
}

}  // namespace fa
