// Backward pass of exact attention, dK and dV, bf16 storage, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware", "The backward pass:
// recompute, don't store"): the forward kept only O and the row logsumexp L.
// Every probability tile is rebuilt from Q and K as P = exp(S - L), already
// normalised, and the softmax gradient's row term is the closed form
// D = rowsum(dO * O), computed beforehand by the pre-pass kernel.  Per tile:
//     dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P * (dP - D_i),
//     dK_j += scale dS^T Q_i.
// No N x N matrix reaches memory.  dQ_i = scale dS K_j is formed by the
// query-outer kernel, so that every gradient row is written exactly once
// and no atomics are needed.
//
// gfx950 mapping (key-block outer):
//   * workgroup = 4 waves x 32 keys = 128 keys; grid = B*H*ceil(N/128), the
//     causally heaviest key blocks (those seen by the most queries) first,
//     heads the fastest index;
//   * each wave keeps its K_j and V_j rows in registers as MFMA B operands and
//     accumulates its own dK_j, dV_j rows (no cross-wave reduction);
//   * query tiles of 64 rows (Q, dO) go from HBM straight into LDS
//     (buffer_load ... lds, double-buffered, rows past N arrive as zeros),
//     row-major with the 16-byte units of each row XOR-swizzled so that
//     neither read below meets a bank conflict.  They are read twice: with 16-byte reads as the A
//     operand of S = Q K^T and dP = dO V^T, and with ds_read_b64_tr_b16 (four
//     consecutive rows of one column per lane) as the B operand of
//     dK += dS^T Q and dV += P^T dO -- no transposed copies;
//   * S and dP come out with one key per lane, so P and dS feed the dV and
//     dK contractions straight from registers; the tile is processed in two
//     32-query halves to keep them few;
//   * causal masking is applied only on tiles that cross the diagonal.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBk = 128;  // keys per workgroup
constexpr int kBq = 64;   // queries per tile

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 16;     // 16-wide steps over d
  static constexpr int DB = D / 32;     // 32-column blocks over d
  static constexpr int QT = kBq * D;    // elements of one Q or dO tile
};

__device__ __forceinline__ bf16x8 cvt8(const f32x16& x, int off) {
  const f32x4 a = {x[off + 0], x[off + 1], x[off + 2], x[off + 3]};
  const f32x4 b = {x[off + 4], x[off + 5], x[off + 6], x[off + 7]};
  return cat(__builtin_convertvector(a, bf16x4),
             __builtin_convertvector(b, bf16x4));
}

// S = Q K^T and dP = dO V^T for one 32-query half: the 16-byte A-operand
// fragments are all requested first, then the MFMAs run.
template <int D>
__device__ __forceinline__ void sdp_half(f32x16& S, f32x16& dP,
                                         const char* Qs, const char* dOs,
                                         int qb, const int (&aoff)[D / 16],
                                         const bf16x8 (&kf)[D / 16],
                                         const bf16x8 (&vf)[D / 16]) {
  constexpr int KS = D / 16;
  constexpr int BATCH = 4;  // fragments requested ahead of their MFMAs
  S = f32x16{};
  dP = f32x16{};
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += BATCH) {
    bf16x8 qa[BATCH], da[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      qa[u] = *(const bf16x8*)(Qs + aoff[k0 + u] + 32 * qb * 2 * D);
      da[u] = *(const bf16x8*)(dOs + aoff[k0 + u] + 32 * qb * 2 * D);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[u], kf[k0 + u], S, 0, 0,
                                                  0);
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[u], vf[k0 + u], dP, 0, 0,
                                                   0);
    }
  }
}

// P = exp(S - L) and dS = P (dP - D) for one half (lane: key myk, queries
// q0 + 8(r/4) + 4hh + r%4), masked on diagonal tiles; returns them as bf16
// MFMA operands.
template <bool MASKED, bool CAUSAL>
__device__ __forceinline__ void softmax_grad_half(
    f32x16& S, f32x16& dP, bf16x8 (&pa)[2], bf16x8 (&sa)[2], const float* Ls,
    const float* Dl, int qb, int q0, int myk, int N, float c, int hh) {
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int qo = 32 * qb + 8 * grp + 4 * hh;
    const f32x4 lv = *(const f32x4*)(Ls + qo);
    const f32x4 dv = *(const f32x4*)(Dl + qo);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * grp + e;
      float p = fast_exp2(fmaf(S[r], c, -lv[e]));
      if (MASKED) {
        const int qrow = q0 + 8 * grp + 4 * hh + e;
        const bool ok = myk < N && (!CAUSAL || myk <= qrow);
        p = ok ? p : 0.f;
      }
      S[r] = p;
      dP[r] = p * (dP[r] - dv[e]);
    }
  }
  pa[0] = cvt8(S, 0);
  pa[1] = cvt8(S, 8);
  sa[0] = cvt8(dP, 0);
  sa[1] = cvt8(dP, 8);
}

// dV += P^T dO and dK += dS^T Q over one half's 32 queries: the transposed
// B-operand fragments are all requested first, then the MFMAs run.
template <int D>
__device__ __forceinline__ void dkdv_half(f32x16 (&dK)[D / 32],
                                          f32x16 (&dV)[D / 32],
                                          const bf16x8 (&pa)[2],
                                          const bf16x8 (&sa)[2],
                                          const char* Qs, const char* dOs,
                                          int qb, const int (&toff)[D / 32][2]) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8 dob[DB], qtb[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int o0 = toff[db][0] + 16 * (2 * qb + half) * 2 * D;
      const int o1 = toff[db][1] + 16 * (2 * qb + half) * 2 * D;
      dob[db] = cat(tr_read(dOs + o0), tr_read(dOs + o1));
      qtb[db] = cat(tr_read(Qs + o0), tr_read(Qs + o1));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dV[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[half], dob[db],
                                                       dV[db], 0, 0, 0);
      dK[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[half], qtb[db],
                                                       dK[db], 0, 0, 0);
    }
  }
}

// One 64-query tile for this wave.  Straight-line on tiles below the
// diagonal; MASKED adds per-element masks and skips halves that see none of
// this wave's keys.
template <int D, bool CAUSAL, bool MASKED>
__device__ __forceinline__ void tile_body(
    const char* Qs, const char* dOs, const float* Ls, const float* Dl, int i,
    int kw0, int myk, int N, float c, const int (&aoff)[D / 16],
    const int (&toff)[D / 32][2], const bf16x8 (&kf)[D / 16],
    const bf16x8 (&vf)[D / 16], f32x16 (&dK)[D / 32], f32x16 (&dV)[D / 32]) {
  const int hh = (threadIdx.x & 63) >> 5;
  // (At d = 128 the registers of a second S/dP pair do not fit beside the
  // dK/dV accumulators, so there the halves run one after the other.)
  if (!MASKED && D <= 64) {
    // Two halves, software-pipelined: the second half's S/dP MFMAs are
    // issued before the first half's exponentials, and the first half's
    // dV/dK MFMAs before the second half's exponentials.
    f32x16 S0, dP0, S1, dP1;
    bf16x8 pa0[2], sa0[2], pa1[2], sa1[2];
    sdp_half<D>(S0, dP0, Qs, dOs, 0, aoff, kf, vf);
    sdp_half<D>(S1, dP1, Qs, dOs, 1, aoff, kf, vf);
    softmax_grad_half<false, CAUSAL>(S0, dP0, pa0, sa0, Ls, Dl, 0, i, myk, N,
                                     c, hh);
    dkdv_half<D>(dK, dV, pa0, sa0, Qs, dOs, 0, toff);
    softmax_grad_half<false, CAUSAL>(S1, dP1, pa1, sa1, Ls, Dl, 1, i + 32,
                                     myk, N, c, hh);
    dkdv_half<D>(dK, dV, pa1, sa1, Qs, dOs, 1, toff);
    return;
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q0 = i + 32 * qb;
    const bool active =
        !MASKED || (kw0 < N && (!CAUSAL || q0 + 31 >= kw0));
    if (active) {
      f32x16 S, dP;
      bf16x8 pa[2], sa[2];
      sdp_half<D>(S, dP, Qs, dOs, qb, aoff, kf, vf);
      softmax_grad_half<MASKED, CAUSAL>(S, dP, pa, sa, Ls, Dl, qb, q0, myk, N,
                                        c, hh);
      dkdv_half<D>(dK, dV, pa, sa, Qs, dOs, qb, toff);
    }
  }
}

template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_bf16_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  // LDS: two sets of (Q tile, dO tile, L and D of the tile's rows).  While
  // one set is read the next tile streams into the other.
  constexpr int SET = 2 * C::QT * 2 + 2 * kBq * 4;  // bytes per set
  __shared__ __attribute__((aligned(1024))) char smem[2 * SET];

  const Geom& g = a.g;
  const int N = g.N;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: keep it in a scalar register
  // so that per-wave branches stay scalar.
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int gi = lane & 15, gg = lane >> 4;

  const int BH = g.B * g.H;
  const int rank = blockIdx.x / BH;
  const int head = blockIdx.x - rank * BH;
  const int b = head / g.H, h = head - b * g.H;
  const int64_t hoff = head_offset(g, b, h);
  const uint32_t head_bytes = (uint32_t)(((int64_t)(N - 1) * sn + D) * 2);
  const i32x4_t qr = rsrc_words((const __bf16*)a.q + hoff, head_bytes);
  const i32x4_t dor = rsrc_words((const __bf16*)a.dout + hoff, head_bytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const __bf16*)a.k + hoff,
                                              head_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const __bf16*)a.v + hoff,
                                              head_bytes);
  const float* lse_h = a.lse + (int64_t)head * N;
  const float* del_h = a.delta + (int64_t)head * N;

  const int j0 = rank * kBk;       // first key of the workgroup
  const int kw0 = j0 + 32 * wave;  // first key of this wave
  const int myk = kw0 + l32;
  const float c = g.scale_log2;

  // This wave's key and value rows as B operands of S and dP (lane: key
  // myk, dims 16ks + 8hh .. +7); rows past N read as zero.
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int off = (myk * sn + 16 * ks + 8 * hh) * 2;
    kf[ks] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
    vf[ks] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
  }

  // Per-lane LDS byte offsets.
  //  * 16-byte A-operand reads of Q / dO: row 32qb + l32, unit 2ks + hh;
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

  f32x16 dK[C::DB], dV[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dK[db] = f32x16{};
    dV[db] = f32x16{};
  }

  const int mcol = MASK ? j0 / g.mask_block : 0;
  auto kept = [&](int i) {
    return !MASK || g.mask[(i / g.mask_block) * g.nmb + mcol] != 0;
  };
  int i = CAUSAL ? j0 : 0;  // j0 is a multiple of kBq
  while (i < N && !kept(i)) i += kBq;

  // L (as L*log2(e), +inf for empty or padding rows so that P = 0) and D of
  // the tile starting at query row i0, one value per thread 0..127.
  auto load_ld = [&](int i0) -> float {
    if (tid < kBq) {
      const int row = i0 + tid;
      const float L = row < N ? lse_h[row] : -INFINITY;
      return L == -INFINITY ? INFINITY : L * kLog2e;
    }
    if (tid < 2 * kBq) {
      const int row = i0 + tid - kBq;
      return row < N ? del_h[row] : 0.f;
    }
    return 0.f;
  };
  auto store_ld = [&](float* ld, float v) {
    if (tid < 2 * kBq) ld[tid] = v;
  };

  auto next_tile = [&](int ii) {
    ii += kBq;
    while (ii < N && !kept(ii)) ii += kBq;
    return ii;
  };
  const uint32_t smem_lds = lds_addr(smem);
  // Stream the tile at query row ii into set `set`: Q and dO by DMA, and
  // this thread's L/D value, returned for store_ld after the compute.
  auto fetch = [&](int ii, int set) -> float {
    const uint32_t base = smem_lds + set * SET;
    dma_rows<kBq, D>(base, qr, ii, sn, wave, lane);
    dma_rows<kBq, D>(base + C::QT * 2, dor, ii, sn, wave, lane);
    return load_ld(ii);
  };

  int set = 0;
  if (i < N) store_ld((float*)(smem + 2 * C::QT * 2), fetch(i, 0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  while (i < N) {
    // Fresh (opaque) copies of the lane offsets each tile, so that the LDS
    // addresses are formed inside the loop rather than hoisted as one
    // register per (set, offset) pair.
#pragma unroll
    for (int k = 0; k < C::KS; ++k) asm volatile("" : "+v"(aoff[k]));
#pragma unroll
    for (int k = 0; k < C::DB; ++k) {
      asm volatile("" : "+v"(toff[k][0]));
      asm volatile("" : "+v"(toff[k][1]));
    }
    const int in = next_tile(i);
    float ld_next = 0.f;
    if (in < N) ld_next = fetch(in, set ^ 1);
    const char* Qs = smem + set * SET;
    const char* dOs = Qs + C::QT * 2;
    const float* Ls = (const float*)(Qs + 2 * C::QT * 2);
    const float* Dl = Ls + kBq;
    // Tiles that cross the causal diagonal or the end of the keys take the
    // masked path; all others run the straight-line path.
    int diag = __builtin_amdgcn_readfirstlane(
        (CAUSAL && i < j0 + kBk - 1) || j0 + kBk > N);
    // (Opaque, so that the loop is not unswitched into two copies.)
    asm volatile("" : "+s"(diag));
    if (diag)
      tile_body<D, CAUSAL, true>(Qs, dOs, Ls, Dl, i, kw0, myk, N, c, aoff,
                                 toff, kf, vf, dK, dV);
    else
      tile_body<D, CAUSAL, false>(Qs, dOs, Ls, Dl, i, kw0, myk, N, c, aoff,
                                  toff, kf, vf, dK, dV);
    if (in < N) store_ld((float*)(smem + (set ^ 1) * SET + 2 * C::QT * 2),
                         ld_next);
    // Every wave is done with the current set, and the next one has landed.
    barrier_vmcnt<0>();
    i = in;
    set ^= 1;
  }

  // dK, dV rows of this wave: lane holds dim 32db + l32, keys
  // kw0 + 8(r/4) + 4hh + r%4; keys past N fall outside the range.
  const __amdgpu_buffer_rsrc_t dkr = make_rsrc((__bf16*)a.dk + hoff,
                                               head_bytes);
  const __amdgpu_buffer_rsrc_t dvr = make_rsrc((__bf16*)a.dv + hoff,
                                               head_bytes);
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const int off = (key * sn + 32 * db + l32) * 2;
      const __bf16 kv = (__bf16)(dK[db][r] * g.scale);
      const __bf16 vv = (__bf16)dV[db][r];
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, kv), dkr,
                                            off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, vv), dvr,
                                            off, 0, 0);
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
