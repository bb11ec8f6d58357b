// FP8 forward of exact attention with incoherent processing, for gfx950.
//
// Method ("FlashAttention: making attention IO-aware", section
// "FlashAttention-3: Hopper asynchrony and FP8"): both products of the
// forward run in FP8; to keep outliers from ruining the 3-bit mantissas, Q
// and K are first multiplied by a random orthogonal matrix built from a
// Hadamard matrix, and every operand is quantised per block.  Concretely:
//   * rotation: x -> (x o signs) H_d with H_d the Sylvester Hadamard matrix
//     (entries +-1).  Since H H^T = d I, (Q M)(K M)^T = d Q K^T and the
//     softmax scale carries a factor 1/d (a power of two);
//   * blocks of 64 rows of one head share a power-of-two scale 2^e, e the
//     smallest integer with max|x| <= 448 * 2^e; the codes are OCP E4M3
//     (largest finite value 448), rounded to nearest even;
//   * P = 2^4 exp2(s - m_ref) is rounded to E4M3 for the second product
//     (m_ref is the lazily moved row reference, at most 4 below the running
//     maximum, so P <= 2^8 < 448); the row sum l uses the unrounded P.
//
// Two kernels:
//   fp8_quantize_kernel -- one workgroup per (tensor, head, 64-row block):
//     loads the bf16 rows, applies the fast Walsh-Hadamard transform to Q
//     and K rows (butterflies in registers and across the 4 lanes of a row
//     with DPP), reduces the block maximum, writes E4M3 codes and the E8M0
//     scale code.  V is written transposed, [d][keys], with the keys of each
//     64-key group in the order in which the P operand of the FP8 MFMA holds
//     them, so that the forward reads V^T fragments with plain 16-byte LDS
//     reads;
//   fwd_fp8_kernel -- the bf16 forward's structure (4 waves x 32 rows per
//     workgroup, two workgroups per CU, K/V tiles DMA'd to LDS, software
//     pipelined S, ping-pong score registers, lazy rescale) on
//     v_mfma_scale_f32_32x32x64_f8f6f4: the per-block scales of Q, K and V
//     enter the MFMA as E8M0 operand scales, so dequantisation costs nothing.
#include "fa_internal.h"

#include <math.h>

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockRows = 64;     // rows per quantisation block
constexpr int kE8M0Bias = 127;
constexpr int kPShift = 4;         // P is formed times 2^4
constexpr float kLazyFp8 = 4.0f;   // reference moves when exceeded by 2^4

// Transposed V: key r of a 64-key group is stored at position
//   32 ((r >> 2) & 1) + 16 (r >> 5) + 4 ((r >> 3) & 3) + (r & 3)
// of the group.  The P operand of the FP8 MFMA (B, 32 x 64) gives lane half
// hh the bytes 32 hh .. 32 hh + 31 of the contraction; byte i of half hh is
// element i % 16 of the score accumulator of keys 32 (i / 16) .. +31, and
// accumulator element j of a lane in half hh holds key 8 (j / 4) + 4 hh +
// j % 4: in this order a V^T fragment is 32 consecutive bytes.

__device__ __forceinline__ i32x8 cat8(i32x4 lo, i32x4 hi) {
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Two floats -> two E4M3 bytes (round to nearest even) in byte lanes
// 2 HI, 2 HI + 1 of `old`.
template <bool HI>
__device__ __forceinline__ int pack_fp8(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Lane exchange inside groups of four lanes (DPP quad permutations).
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// Smallest e with amax <= 448 * 2^e (amax = f 2^x, f in [0.5, 1): e = x - 9
// when f <= 0.875, else x - 8), at least -127; amax == 0 gives -127.
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.f)) return -kE8M0Bias;
  int x;
  const float f = frexpf(amax, &x);
  return max(f <= 0.875f ? x - 9 : x - 8, -kE8M0Bias);
}

// ------------------------------------------------------------ quantisation
//
// One workgroup of LPR * 64 threads (LPR = d / 32) per (tensor, head, 64-row
// block); every thread holds 32 values.
//
// Lane l of a row holds the 32 columns 8 l + 8 LPR p + e (p = 0..3,
// e = 0..7), so the column index bits are e (bits 0-2, in registers), l (1
// or 2 bits, across lanes) and p (2 bits, in registers): the butterflies of
// the bits in registers are adds and subtracts, those across lanes a DPP
// exchange and one FMA with the lane's sign.
//
// V (not rotated) is loaded the same way and transposed through LDS.
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void fp8_quantize_kernel(
    Fp8Args a) {
  constexpr int LPR = D / 32;
  constexpr int NT = 64 * LPR;
  constexpr int NW = NT / 64;
  __shared__ float wave_max[NW];
  __shared__ __attribute__((aligned(16))) uint8_t vtile[D * kBlockRows];

  const Geom& g = a.g;
  const int BH = g.B * g.H;
  const int nblk = a.Np / kBlockRows;
  const int t = (int)blockIdx.x / (BH * nblk);  // 0: Q, 1: K, 2: V
  const int rem = (int)blockIdx.x - t * BH * nblk;
  const int bh = rem / nblk, blk = rem - bh * nblk;
  const int b = bh / g.H, h = bh - b * g.H;
  const int tid = threadIdx.x;
  const int sn = (int)g.sn;

  const void* src = t == 0 ? a.q : (t == 1 ? a.k : a.v);
  const int64_t hoff = (int64_t)b * g.sb + (int64_t)h * g.sh;
  const uint32_t head_bytes = (uint32_t)(((int64_t)(g.N - 1) * sn + D) * 2);
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc((const __bf16*)src + hoff, head_bytes);
  const int row0 = blk * kBlockRows;

  // Rows past N read as zeros (the buffer range ends with row N - 1).
  float x[32];
  const int r = tid / LPR, l = tid % LPR;
  {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int col0 = 8 * l + 8 * LPR * p;
      const i32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
          sr, ((row0 + r) * sn + col0) * 2, 0, 0);
      const bf16x8 v = __builtin_bit_cast(bf16x8, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * p + e] = (float)v[e];
    }
    if (t < 2 && a.rotate) {
      // x o signs, then the butterflies of H_d, one per column bit (in
      // exact arithmetic their order does not matter).
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        // Columns 8 l + 8 LPR p + 0..7 lie in one 64-bit sign word.
        const int col0 = 8 * l + 8 * LPR * p;
        const uint64_t word = col0 < 64 ? a.sign_lo : a.sign_hi;
        const uint32_t bits = (uint32_t)(word >> (col0 & 63)) & 0xffu;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[8 * p + e] = __uint_as_float(__float_as_uint(x[8 * p + e]) ^
                                         (((bits >> e) & 1u) << 31));
      }
#pragma unroll
      for (int bit = 1; bit < 32; bit <<= 1)     // e and p bits
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (!(i & bit)) {
            const float u = x[i], w = x[i | bit];
            x[i] = u + w;
            x[i | bit] = u - w;
          }
      // l bits: the partner lane holds the same (p, e) of the other column;
      // the lower lane forms x + y, the upper y - x, both as fma(+-1, x, y).
#pragma unroll
      for (int lb = 0; lb < (LPR == 4 ? 2 : 1); ++lb) {
        const float sgn = ((l >> lb) & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float y = lb == 0 ? quad_xor1(x[i]) : quad_xor2(x[i]);
          x[i] = fmaf(sgn, x[i], y);
        }
      }
    }
  }

  // Block maximum of |x|.
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  float amax = wave_max[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) amax = fmaxf(amax, wave_max[w]);
  const int e8 = block_exponent(amax);
  const float inv = ldexpf(1.0f, -e8);

  int32_t* exps = t == 0 ? a.qe : (t == 1 ? a.ke : a.ve);
  if (tid == 0) exps[(int64_t)bh * nblk + blk] = e8 + kE8M0Bias;

  if (t < 2) {
    uint8_t* dst = (t == 0 ? a.qc : a.kc) + ((int64_t)bh * a.Np + row0 + r) * D;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      i32x2 c;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const float* y = x + 8 * p + 4 * w;
        const int lo = pack_fp8<false>(y[0] * inv, y[1] * inv, 0);
        c[w] = pack_fp8<true>(y[2] * inv, y[3] * inv, lo);
      }
      *(i32x2*)(dst + 8 * l + 8 * LPR * p) = c;
    }
    return;
  }
  // V: transpose through LDS into [d][64 positions] (the key order above),
  // then 16-byte rows out.
  const int pos = 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) +
                  (r & 3);
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int word = pack_fp8<false>(x[8 * p + e] * inv, x[8 * p + e + 1] * inv, 0);
      const int col = 8 * l + 8 * LPR * p + e;
      vtile[col * kBlockRows + pos] = (uint8_t)(word & 0xff);
      vtile[(col + 1) * kBlockRows + pos] = (uint8_t)((word >> 8) & 0xff);
    }
  __syncthreads();
  uint8_t* vdst = a.vt + (int64_t)bh * D * a.Np + row0;
  constexpr int UNITS = D * kBlockRows / 16;
#pragma unroll
  for (int u = tid; u < UNITS; u += NT) {
    const int d = u >> 2, part = u & 3;
    *(i32x4*)(vdst + (int64_t)d * a.Np + 16 * part) =
        *(const i32x4*)(vtile + d * kBlockRows + 16 * part);
  }
}

// ----------------------------------------------------------------- forward

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBr = kWaves * kRowsPerWave;

template <int D>
struct F8Cfg {
  static constexpr int BC = 64;          // keys per tile (= one scale block)
  static constexpr int NKB = BC / 32;    // 32-key sub-tiles
  static constexpr int KC = D / 64;      // 64-deep chunks of Q K^T
  static constexpr int DB = D / 32;      // 32-row blocks of O^T
  static constexpr int TILE = BC * D;    // bytes of a K tile (= a V tile)
  static constexpr int KUPR = D / 16;    // 16-byte units per K row
};

// XOR swizzle of the 16-byte units of LDS rows, so that 16 lanes reading
// one logical unit of 16 consecutive rows hit 16 distinct 16-byte bank
// groups of the 64-bank LDS.  K rows are d bytes (2 or 4 rows per 256
// bytes), V^T rows 64 bytes.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
__device__ __forceinline__ int swz_v(int r) { return (r >> 2) & 3; }

// HBM -> LDS of ROWS rows of UPR 16-byte units (row r at byte
// r * stride + col0 of the buffer), swizzled with SWZ, by the 4 waves.
template <int ROWS, int UPR, typename Swz>
__device__ __forceinline__ void dma_tile(uint32_t dst, i32x4_t src, int stride,
                                         int col0, int wave, int lane, Swz swz) {
  constexpr int PER_WAVE = ROWS * UPR / (kWaves * 64);
  static_assert(PER_WAVE * kWaves * 64 == ROWS * UPR, "whole loads");
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int base = (wave * PER_WAVE + u) * 64;
    const int p = base + lane;
    const int r = p / UPR;
    const int unit = (p % UPR) ^ swz(r);
    dma_b128(__builtin_amdgcn_readfirstlane(dst + 16 * base), src,
             r * stride + col0 + 16 * unit);
  }
}

// S^T of the 32-key sub-tile kb of the staged K tile (K block scale code
// ke, Q block scale code qe).
template <int D>
__device__ __forceinline__ f32x16 compute_s8(const char* Ks,
                                             const int (&koff)[F8Cfg<D>::KC][2],
                                             const i32x8 (&qf)[F8Cfg<D>::KC],
                                             int kb, int ke, int qe) {
  using C = F8Cfg<D>;
  f32x16 s = {};
#pragma unroll
  for (int c = 0; c < C::KC; ++c) {
    const i32x8 kf = cat8(*(const i32x4*)(Ks + koff[c][0] + 32 * kb * D),
                          *(const i32x4*)(Ks + koff[c][1] + 32 * kb * D));
    s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[c], s, 0, 0, 0,
                                                        ke, 0, qe);
  }
  return s;
}

// Per-64-row block values of one head (the E8M0 block scale codes), held 64
// at a time in one register (lane l: block w0 + l) and picked out with
// readlane: a tile's scale costs no memory access inside the loop, so no
// wait on it can also catch the tile loads in flight.  Every lane of the
// wave calls get() together, with the same block.
struct BlockCodes {
  const int32_t* p;
  int n;   // blocks of the head
  int w0;  // first block held
  int v;   // this lane's block w0 + lane
  __device__ __forceinline__ BlockCodes(const int32_t* ptr, int count)
      : p(ptr), n(count), w0(-64), v(0) {}
  __device__ __forceinline__ int get(int blk) {
    if (blk < w0 || blk >= w0 + 64) {
      w0 = blk;
      const int i = blk + (int)(threadIdx.x & 63);
      v = i < n ? p[i] : 0;
      // (Used here, so that the wait for this load stays on this rare
      // path instead of the join that every step passes.)
      asm volatile("" : "+v"(v));
    }
    return __builtin_amdgcn_readlane(v, blk - w0);
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_kernel(Fp8Args a) {
  using C = F8Cfg<D>;
  constexpr int BC = C::BC;
  // Two (K, V^T) tile pairs: K in slots 0, 1 and V^T in slots 2, 3.
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];

  const Geom& g = a.g;
  const int sn = (int)g.sn;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int BH = g.B * g.H;
  const int N = g.N;
  const int Np = a.Np;
  const int nblk = Np / kBlockRows;
  const int nqb = (N + kBr - 1) / kBr;
  const int rank = (int)blockIdx.x / BH;
  const int head = (int)blockIdx.x - rank * BH;
  const int qb = CAUSAL ? (nqb - 1 - rank) : rank;
  const int b = head / g.H, h = head - b * g.H;

  const uint32_t op_bytes = (uint32_t)Np * D;
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(a.qc + (int64_t)head * op_bytes, op_bytes);
  const i32x4_t kr = rsrc_words(a.kc + (int64_t)head * op_bytes, op_bytes);
  const i32x4_t vr = rsrc_words(a.vt + (int64_t)head * op_bytes, op_bytes);
  const int32_t* qe_h = a.qe + (int64_t)head * nblk;
  BlockCodes ke_h(a.ke + (int64_t)head * nblk, nblk);
  BlockCodes ve_h(a.ve + (int64_t)head * nblk, nblk);
  const int64_t hoff = (int64_t)b * g.sb + (int64_t)h * g.sh;
  const uint32_t head_bytes = (uint32_t)(((int64_t)(N - 1) * sn + D) * 2);
  const __amdgpu_buffer_rsrc_t orr = make_rsrc((__bf16*)a.o + hoff, head_bytes);
  const __amdgpu_buffer_rsrc_t lr =
      make_rsrc(a.lse + (int64_t)head * N, (uint32_t)N * 4u);

  const int i0 = qb * kBr;
  const int q0w = i0 + kRowsPerWave * wave;
  const float c = g.scale_log2;
  // The wave's 32 rows lie in one 64-row block of Q.
  const int qe = q0w < Np ? qe_h[q0w / kBlockRows] : kE8M0Bias;

  // Q fragments (B operand of S^T): lane holds query q0w + l32, bytes
  // 64 c + 32 hh .. +31 of its row.
  i32x8 qf[C::KC];
#pragma unroll
  for (int cc = 0; cc < C::KC; ++cc) {
    const int off = (q0w + l32) * D + 64 * cc + 32 * hh;
    qf[cc] = cat8(__builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0),
                  __builtin_amdgcn_raw_buffer_load_b128(qr, off + 16, 0, 0));
  }

  const int jend = CAUSAL ? min(N, i0 + kBr) : N;

  float m_ref = -INFINITY;
  float l_part = 0.f;
  f32x16 acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) acc[db] = f32x16{};

  // Per-lane LDS byte offsets.  K: row 32 kb + l32, units 4 c + 2 hh (+1).
  // V^T: row 32 db + l32, units 2 hh (+1).
  int koff[C::KC][2];
#pragma unroll
  for (int cc = 0; cc < C::KC; ++cc)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      koff[cc][j] = l32 * D + 16 * ((4 * cc + 2 * hh + j) ^ swz_k<D>(l32));
  int voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    voff[j] = l32 * BC + 16 * ((2 * hh + j) ^ swz_v(l32));

  const uint32_t smem_lds = lds_addr(smem);
  auto fetch_k = [&](int jj, int slot) {
    dma_tile<BC, C::KUPR>(smem_lds + slot * C::TILE, kr, D, jj * D, wave,
                          lane, [](int r) { return swz_k<D>(r); });
  };
  auto fetch_v = [&](int jj, int slot) {
    dma_tile<D, BC / 16>(smem_lds + (2 + slot) * C::TILE, vr, Np, jj, wave,
                         lane, [](int r) { return swz_v(r); });
  };
  auto active = [&](int jj) {
    return q0w < N && (!CAUSAL || jj <= q0w + kRowsPerWave - 1);
  };

  // The same software pipeline as the bf16 forward: K is staged one tile
  // ahead of V, and the scores of tile t+1 are formed while the softmax of
  // tile t runs.
  f32x16 S[C::NKB];
  int jc = 0;
  int jn = jc + BC < jend ? jc + BC : jend;
  if (jc < jend) {
    fetch_k(jc, 0);
    fetch_v(jc, 0);
  }
  if (jn < jend) fetch_k(jn, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (jc < jend && active(jc)) {
    const int ke = ke_h.get(jc / kBlockRows);
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb)
      S[kb] = compute_s8<D>(smem, koff, qf, kb, ke, qe);
  }
  barrier_lds();
  int slot = 0;
  auto step = [&](f32x16 (&Sc)[C::NKB], f32x16 (&Sx)[C::NKB]) {
    const int jnn = jn + BC < jend ? jn + BC : jend;
    if (jnn < jend) fetch_k(jnn, slot);
    if (jn < jend) fetch_v(jn, slot ^ 1);
    if (active(jc)) {
      const char* Kn = smem + (slot ^ 1) * C::TILE;
      const char* Vs = smem + (2 + slot) * C::TILE;
      // Lane holds query q0w + l32 and keys jc + 32 kb + 8 (r/4) + 4 hh + r%4.
      if ((CAUSAL && jc + BC - 1 > q0w) || jc + BC > N) {
        asm volatile("");
        const int q = q0w + l32;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = jc + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= q);
            if (!ok) Sc[kb][r] = -INFINITY;
          }
      }
      float t = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          t = fmaxf(fmaxf(t, Sc[kb][r]), Sc[kb][r + 1]);
      const float mx = swap_halves_max(t) * c;
      const float m_new = mx > m_ref + kLazyFp8 ? mx : m_ref;
      if (__builtin_amdgcn_ballot_w64(m_new != m_ref) != 0) {
        asm volatile("");
        const float alpha = m_new == m_ref ? 1.0f : fast_exp2(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) acc[db] *= alpha;
        m_ref = m_new;
      }
      // P = 2^4 exp2(s c - m_ref) <= 2^8.
      const float m_use = (m_ref == -INFINITY ? 0.f : m_ref) - (float)kPShift;
      const int ken = jn < jend ? ke_h.get(jn / kBlockRows) : kE8M0Bias;
      const int vec = ve_h.get(jc / kBlockRows);
      int pw[8];
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        Sx[kb] = compute_s8<D>(Kn, koff, qf, kb, ken, qe);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          Sc[kb][r] = fast_exp2(fmaf(Sc[kb][r], c, -m_use));
          Sc[kb][r + 1] = fast_exp2(fmaf(Sc[kb][r + 1], c, -m_use));
          rs0 += Sc[kb][r];
          rs1 += Sc[kb][r + 1];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int lo = pack_fp8<false>(Sc[kb][4 * w], Sc[kb][4 * w + 1], 0);
          pw[4 * kb + w] =
              pack_fp8<true>(Sc[kb][4 * w + 2], Sc[kb][4 * w + 3], lo);
        }
      }
      l_part += rs0 + rs1;
      const i32x8 pf = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
      // O^T += V^T P^T (V block scale on the A operand, P unscaled).
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const i32x8 vf =
            cat8(*(const i32x4*)(Vs + voff[0] + 32 * db * BC),
                 *(const i32x4*)(Vs + voff[1] + 32 * db * BC));
        acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            vf, pf, acc[db], 0, 0, 0, vec, 0, kE8M0Bias);
      }
    }
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

  // ---- epilogue: O = acc / l, L = (m_use + log2 l) ln 2.
  const float l = swap_halves_sum(l_part);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const int q = q0w + l32;
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
    const float m_use = m_ref - (float)kPShift;
    const float L = l > 0.f ? (m_use + log2f(l)) * kLn2 : -INFINITY;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(L), lr, q * 4, 0, 0);
  }
}

template <int D>
hipError_t quantize_d(const Fp8Args& a, hipStream_t s) {
  const int nblk = a.Np / kBlockRows;
  const dim3 grid((unsigned)(3 * a.g.B * a.g.H * nblk));
  hipLaunchKernelGGL((fp8_quantize_kernel<D>), grid, dim3(64 * (D / 32)), 0, s,
                     a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t fwd_d(const Fp8Args& a, hipStream_t s) {
  const int nqb = (a.g.N + kBr - 1) / kBr;
  const dim3 grid((unsigned)(a.g.B * a.g.H * nqb));
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8Args& a, int d, hipStream_t s) {
  return d == 64 ? quantize_d<64>(a, s) : quantize_d<128>(a, s);
}

hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? fwd_d<64, true>(a, s) : fwd_d<64, false>(a, s);
  return causal ? fwd_d<128, true>(a, s) : fwd_d<128, false>(a, s);
}

}  // namespace fa
