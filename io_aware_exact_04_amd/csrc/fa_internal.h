// Internal declarations shared by the fa355 HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// log2(e) and ln(2) in float.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Geometry of one attention problem, shared by every kernel.
struct Geom {
  int B, H, N;
  int64_t sb, sh, sn;   // element strides of [B,H,N,d] tensors
  const uint8_t* mask;  // device block mask or nullptr
  int mask_block;       // rows/cols per mask block
  int nmb;              // mask blocks per mask row
  float scale;          // softmax scale applied to Q K^T
  float scale_log2;     // scale * log2(e)
  // Keys and values (split-KV forward only; otherwise Nk = N and the K/V
  // strides are the Q strides): length, strides, and the causal offset
  // (query q keeps keys <= q + causal_off).
  int Nk;
  int causal_off;
  int64_t ksb, ksh, ksn;
  // Packed variable-length batch (nullptr otherwise): sequence b is rows
  // cu[b] .. cu[b+1]-1 of [total, H, d] tensors (element strides sh, sn),
  // with L and D stored [H, total]; B counts the sequences and N is the
  // longest sequence (the grid is sized by it).
  const int* cu;
  int total;
  // Key padding (nullptr otherwise): batch b keeps keys < kv_lens[b]
  // (clamped into [0, Nk]).
  const int* kv_lens;
  // Dropout (p8 > 0): an element is dropped when its generator byte is
  // < p8; kept probabilities are scaled by drop_scale = 256 / (256 - p8).
  // The generator is Philox4x32-10 keyed by the seed (drop_bytes_*).
  int p8;
  uint32_t seed_lo, seed_hi;
  float drop_scale;
};

// Rows of one (sequence b, head h): its length, the element offset of its
// row 0 in the [.., d] tensors and the index of its row 0 in L and D.
struct HeadView {
  int N;
  int64_t off;
  int64_t lrow;
};

template <bool PACKED>
__device__ __forceinline__ HeadView head_view(const Geom& g, int b, int h) {
  HeadView v;
  if (!PACKED) {
    v.N = g.N;
    v.off = (int64_t)b * g.sb + (int64_t)h * g.sh;
    v.lrow = ((int64_t)b * g.H + h) * g.N;
  } else {
    // Offsets are clamped into [0, total] and lengths to the longest
    // sequence, so that malformed offsets cannot address outside the
    // tensors (such sequences come out empty or cut short).
    const int s = min(max(g.cu[b], 0), g.total);
    const int e = min(min(max(g.cu[b + 1], s), g.total), s + g.N);
    v.N = e - s;
    v.off = (int64_t)s * g.sn + (int64_t)h * g.sh;
    v.lrow = (int64_t)h * g.total + s;
  }
  return v;
}

struct FwdArgs {
  Geom g;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  // Split-KV forward: keys [s * split_len, (s + 1) * split_len) form split
  // s; its normalised partial output and logsumexp go to part_o
  // [splits][B*H][N][d] and part_l [splits][B*H][N] (fp32).
  int splits;
  int split_len;
  float* part_o;
  float* part_l;
};

struct BwdArgs {
  Geom g;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // workspace: D [B,H,N]
  float* lse2;    // workspace: L * log2(e), +inf where L = -inf, [B,H,N]
};

// FP8 forward with incoherent processing.  The quantised operands live in a
// caller workspace, per head h (of B*H) and with Np = N rounded up to 64:
//   qc, kc: [B*H][Np][d] E4M3 codes (row-major, rows past N are zero);
//   vt:     [B*H][d][Np] E4M3 codes of V transposed, the 64 keys of each
//           64-key group stored in the order the P operand of the FP8 MFMA
//           holds them (fa_fp8.hip, key_position);
//   qe, ke, ve: [B*H][Np/64] E8M0 block scale codes (scale = 2^(code-127)).
struct Fp8Args {
  Geom g;        // bf16 Q, K, V, O geometry; scale_log2 includes the rotation's 1/d
  int Np;
  uint8_t* qc;
  uint8_t* kc;
  uint8_t* vt;
  int32_t* qe;
  int32_t* ke;
  int32_t* ve;
  const void* q;
  const void* k;
  const void* v;
  uint64_t sign_lo, sign_hi;  // bit i: negate dimension i before the transform
  int rotate;                 // Q and K go through diag(signs) H_d
  void* o;
  float* lse;
};

// Host-side launchers, one per kernel family.  Each returns hipSuccess or
// the launch error; none synchronises.
hipError_t launch_fwd_bf16(const FwdArgs& a, int d, bool causal,
                           hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int d, bool causal,
                          hipStream_t s);
hipError_t launch_fwd_splitkv_bf16(const FwdArgs& a, int d, bool causal,
                                   hipStream_t s);
hipError_t launch_splitkv_merge(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_decode_split_bf16(const FwdArgs& a, int d, hipStream_t s);
hipError_t launch_fp8_quantize(const Fp8Args& a, int d, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_pre(const BwdArgs& a, int d, bool bf16, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int d, bool causal,
                                hipStream_t s);
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, int d, bool causal,
                              hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, int d, bool causal,
                               hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdArgs& a, int d, bool causal,
                             hipStream_t s);

// ------------------------------------------------------------ device helpers

// Exchange a value with the lane 32 away (lanes l and l^32) and combine.
__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Whether the block mask keeps the tile (query row qrow, key column kcol).
__device__ __forceinline__ bool mask_keeps(const Geom& g, int qrow, int kcol) {
  return g.mask[(qrow / g.mask_block) * g.nmb + (kcol / g.mask_block)] != 0;
}

// Kept blocks along one line of the block mask -- a row (stride 1) or a
// column (stride nmb) -- for stepping from one kept tile to the next.  The
// mask bytes are read 64 at a time, one per lane, and held as a 64-bit
// window of kept bits in scalar registers (a ballot), so finding the next
// kept block is a bit scan instead of one dependent byte load per skipped
// tile.  Every lane of the wave calls it together.
struct MaskScan {
  const uint8_t* line;
  int stride, n;  // n blocks along the line
  int w0;         // first block of the window
  uint64_t bits;  // bit k set: block w0 + k is kept
  __device__ __forceinline__ MaskScan(const uint8_t* p, int s, int count)
      : line(p), stride(s), n(count), w0(-64), bits(0) {}
  __device__ __forceinline__ void fill(int w) {
    const int blk = w + (int)(threadIdx.x & 63);
    const bool keep = blk < n && line[(int64_t)blk * stride] != 0;
    bits = __builtin_amdgcn_ballot_w64(keep);
    w0 = w;
  }
  // The first kept block at or after block b, or n if there is none.
  __device__ __forceinline__ int next(int b) {
    while (b < n) {
      if (b < w0 || b >= w0 + 64) fill(b);
      const uint64_t m = bits >> (b - w0);
      if (m != 0) return b + __builtin_ctzll(m);
      b = w0 + 64;
    }
    return n;
  }
  // The first position at or after pos (a tile start, never straddling a
  // block of mb) inside a kept block; past the line's end if none.
  __device__ __forceinline__ int first_kept(int pos, int mb) {
    const int b = pos / mb;
    const int k = next(b);
    return k == b ? pos : k * mb;
  }
};

// Within an XCD, workgroups go to its four shader engines in turn (the
// engine follows the position in the XCD's sequence, mod 4), and dispatch
// is in order: an engine with no free CU holds up the rest.  Where a head's
// blocks run heaviest first (causal dK/dV, block-masked launches), position
// p takes block rank snake4(p): groups of four ranks alternately forwards
// and backwards, so that with costs falling linearly in the rank every
// engine gets the same work from each pair of groups (the last, incomplete
// group keeps its order).
__device__ __forceinline__ int snake4(int p, int n) {
  const int m = p >> 2;
  if (4 * m + 4 > n || (m & 1) == 0) return p;
  return 8 * m + 3 - p;
}

// Workgroup id -> (head, block rank).  Workgroup ids are dealt round-robin
// over the 8 XCDs (id % 8), each with its own L2.  When the head count is a
// multiple of 8, XCD x takes heads x, x + 8, ... one after the other, all
// block ranks of a head in a row, so that the workgroups running together
// on an XCD share one or two heads' K and V (or Q and dO) in its L2.
// Otherwise ranks are outermost.  Rank 0 comes first in both orders.
__device__ __forceinline__ void map_block(int bid, int BH, int nblk,
                                          int& head, int& rank) {
  if ((BH & 7) == 0) {
    const int x = bid & 7, sq = bid >> 3;
    const int hl = sq / nblk;
    head = hl * 8 + x;
    rank = sq - hl * nblk;
  } else {
    rank = bid / BH;
    head = bid - rank * BH;
  }
}

// ------------------------------------------------------------- dropout
//
// Philox4x32-10 ("Parallel random numbers: as easy as 1, 2, 3", Salmon et
// al., SC 2011): per round (hi0, lo0) = 0xD2511F53 c0 and (hi1, lo1) =
// 0xCD9E8D57 c2 as 64-bit products; the state becomes (hi1 ^ c1 ^ k0, lo1,
// hi0 ^ c3 ^ k1, lo0); the key is bumped by (0x9E3779B9, 0xBB67AE85)
// between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1,
                                              uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1,
                                              uint32_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// x from the lane with index lane ^ B inside each group of four lanes
// (DPP quad permutation).
template <int B>
__device__ __forceinline__ uint32_t quad_swap(uint32_t x) {
  static_assert(B == 1 || B == 2, "quad lane bit");
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, B == 1 ? 0xB1 : 0x4E, 0xF,
                                            0xF, false);
}

// 4 x 4 transpose across a quad: with m = lane & 3, word r of lane m
// becomes word m of lane r (each lane bit is exchanged with the word bit).
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int m) {
#pragma unroll
  for (int r = 0; r < 4; r += 2) {         // lane bit 0 <-> word bit 0
    const bool up = m & 1;
    const uint32_t got = quad_swap<1>(up ? x[r] : x[r + 1]);
    if (up) x[r] = got; else x[r + 1] = got;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {            // lane bit 1 <-> word bit 1
    const bool up = m & 2;
    const uint32_t got = quad_swap<2>(up ? x[r] : x[r + 2]);
    if (up) x[r] = got; else x[r + 2] = got;
  }
}

// 4 x 4 byte transpose inside a lane: byte c of word r becomes byte r of
// word c.
__device__ __forceinline__ void byte_transpose(uint32_t (&x)[4]) {
  // v_perm_b32 (a, b, sel): result byte i = byte sel_i of {b (0-3), a (4-7)}.
  const uint32_t t0 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  x[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  x[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  x[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// The generator covers 4 x 4 blocks of (query, key) of one (b, h): counter
// (key / 4, query / 4, h, b), key = the seed, and byte 4 r + c of its output
// (words in order, bytes little-endian) belongs to (query 4 qq + r, key
// 4 kq + c).  Both helpers are called by the four lanes of a quad together.
//
// Query-per-lane layout (forward, dQ): the quad holds queries qbase ..
// qbase + 3 (lane m: qbase + m) and, in each of four 4-key groups i, the
// keys key0 + 8 i .. + 3.  Returns y with byte c of y[i] = the byte of
// (qbase + m, key0 + 8 i + c).
__device__ __forceinline__ void drop_bytes_qrow(const Geom& g, int b, int h,
                                                int qbase, int key0, int m,
                                                uint32_t (&y)[4]) {
  philox4x32_10((uint32_t)(key0 + 8 * m) >> 2, (uint32_t)qbase >> 2,
                (uint32_t)h, (uint32_t)b, g.seed_lo, g.seed_hi, y);
  quad_transpose(y, m);
}

// Key-per-lane layout (dK/dV): the quad holds keys kbase .. kbase + 3 (lane
// m: kbase + m) and four 4-query groups i, queries q0 + 8 i .. + 3.
// Returns y with byte e of y[i] = the byte of (q0 + 8 i + e, kbase + m).
__device__ __forceinline__ void drop_bytes_kcol(const Geom& g, int b, int h,
                                                int kbase, int q0, int m,
                                                uint32_t (&y)[4]) {
  philox4x32_10((uint32_t)kbase >> 2, (uint32_t)(q0 + 8 * m) >> 2,
                (uint32_t)h, (uint32_t)b, g.seed_lo, g.seed_hi, y);
  byte_transpose(y);
  quad_transpose(y, m);
}

// Whether byte c of w keeps its element.
__device__ __forceinline__ bool drop_keeps(uint32_t w, int c, int p8) {
  return ((w >> (8 * c)) & 0xffu) >= (uint32_t)p8;
}

// 64-bit element offset of head (b, h).
__device__ __forceinline__ int64_t head_offset(const Geom& g, int b, int h) {
  return (int64_t)b * g.sb + (int64_t)h * g.sh;
}

}  // namespace fa

namespace fa {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Buffer resource over [p, p + bytes): loads past the end return zero,
// stores and atomics past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)bytes, 0x00020000);
}

// ds_read_b64_tr_b16: if lane i of a 16-lane group addresses row R + i/4,
// columns C + 4(i%4) .. +3 of a row-major bf16 tile, lane j of the group
// receives rows R .. R+3 of column C + j.
__device__ __forceinline__ bf16x4 tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)p));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// XOR swizzle of the 16-byte units of row r of a d-wide bf16 tile in LDS.
// gfx950 LDS has 64 banks of 4 bytes; a 16-byte read is served 16 lanes per
// cycle and an 8-byte (transposed) read 32 lanes per cycle.  Reads of one
// logical unit by 16 consecutive rows (MFMA A/B fragments) and transposed
// reads of 4 consecutive rows x 4 units then hit distinct banks:
//   d = 128 (256-byte rows): unit ^ ((r%4) << 2 | (r/4)%4);
//   d = 64  (128-byte rows, two rows per bank sweep):
//            unit ^ (((r/2)%2) << 2 | (r/4)%4).
// The pattern repeats every 16 rows; rows r and r + 8 differ by XOR 2.
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dimension");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Buffer resource words for inline assembly (the same descriptor as
// make_rsrc: base, stride 0, num_records = bytes), forced into SGPRs.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  i32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Byte address of an LDS object, as a 32-bit LDS offset.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16-byte HBM -> LDS DMA: lane l loads the 16 bytes at byte offset voff of
// the buffer (zeros past its range) and writes them to LDS at
// lds_base + 16 l.  Issued as inline assembly, so the compiler does not
// count these loads as possible writers of every LDS object (it would
// otherwise wait for all of them before each LDS read).  The caller orders
// them: s_waitcnt vmcnt(0) and a barrier before the data is read, and a
// barrier after the last read of the destination before the next DMA to it.
__device__ __forceinline__ void dma_b128(uint32_t lds_base, i32x4_t rsrc,
                                         int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// 4-byte HBM -> LDS DMA: lane l loads the dword at byte offset voff of the
// buffer (zero past its range) and writes it to LDS at lds_base + 4 l;
// ordered by the caller like dma_b128.
__device__ __forceinline__ void dma_b32(uint32_t lds_base, i32x4_t rsrc,
                                        int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// HBM -> LDS of ROWS rows of a d-wide bf16 tensor into the swizzled
// row-major tile at an LDS address, by NW waves: the waves split the 16-byte
// units; lane l of a load writes the unit at LDS position base + l, fetching
// the global unit the swizzle places there.  The per-lane part of the
// addressing is computed once (lane_off[u]: byte offset of this lane's unit
// within a tile of row stride sn elements) and the tile's first row goes
// into the buffer descriptor (base + r0 * sn * 2, range shortened to match),
// so a load needs no vector arithmetic; the descriptor's range check still
// zero-fills rows past the end of the tensor.
template <int ROWS, int D, int NW = 4>
struct TileDma {
  static constexpr int UPR = D / 8;
  static constexpr int PER_WAVE = ROWS * UPR / (NW * 64);
  static_assert(PER_WAVE * NW * 64 == ROWS * UPR, "tile not a whole number of loads");
  int lane_off[PER_WAVE];
  __device__ __forceinline__ TileDma(int sn, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      const int p = (wave * PER_WAVE + u) * 64 + lane;
      const int row = p / UPR;
      const int unit = (p % UPR) ^ swz<D>(row);
      lane_off[u] = (row * sn + 8 * unit) * 2;
    }
  }
  // Rows r0 .. r0 + ROWS - 1 of the tensor at `base` (total_bytes long)
  // into the swizzled tile at LDS address dst.
  __device__ __forceinline__ void load(uint32_t dst, const void* base,
                                       uint32_t total_bytes, int r0, int sn,
                                       int wave) const {
    const uint32_t skip = (uint32_t)r0 * (uint32_t)sn * 2u;
    const uint32_t left = total_bytes - min(skip, total_bytes);
    const i32x4_t rsrc = rsrc_words((const char*)base + skip, left);
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u)
      dma_b128(__builtin_amdgcn_readfirstlane(dst + 16 * (wave * PER_WAVE + u) * 64),
               rsrc, lane_off[u]);
  }
};

// Heaviest-first order of the row (or column) blocks of a block-masked,
// non-causal launch.  The blocks of one head run in rank order; if that
// order followed the mask's row order, the launch would end on whatever
// heavy blocks happen to come last, with most CUs idle.  Ranking the lines
// of the mask by their kept blocks, heaviest first (longest processing time
// first), makes the blocks that start last the short ones.
//
// Lines are mask rows (cols = false) or mask columns (cols = true), nmb of
// them; each covers rpb blocks of the launch (the last line possibly fewer:
// nblk in all).  Returns the block that the workgroup of the given rank
// takes: the lines in order of kept-block count (descending, then line
// index ascending), each line's blocks in ascending order.  The NW waves of
// the workgroup read the mask one row per load (lane j: column j), wave w
// rows w, w + NW, ...; their per-line counts meet in `part` (NW x 64 ints of
// LDS, free again on return: a workgroup barrier follows the last read).
// Masks wider than 64 blocks keep the natural order.  Every thread of the
// workgroup calls it together with the same arguments.
template <int NW>
__device__ __forceinline__ int heavy_first(const uint8_t* mask, int nmb,
                                           int rpb, int nblk, int rank,
                                           bool cols, int* part) {
  if (nmb > 64) return rank;
  constexpr int RPW = 64 / NW;  // rows per wave
  const int lane = (int)(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(mask, (uint32_t)(nmb * nmb));
  // All loads first (one memory latency); out-of-range ones read zero.
  int byte[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int r = wave + NW * k;
    const int off = r < nmb && lane < nmb ? r * nmb + lane : nmb * nmb;
    byte[k] = __builtin_amdgcn_raw_buffer_load_b8(mr, off, 0, 0);
  }
  // v: this wave's share of the count of line `lane`.
  int v = 0;
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    if (cols) {
      v += byte[k] != 0 ? 1 : 0;
    } else {
      const int c = __builtin_popcountll(__builtin_amdgcn_ballot_w64(byte[k] != 0));
      v = lane == wave + NW * k ? c : v;
    }
  }
  part[wave * 64 + lane] = v;
  __syncthreads();
  int w = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) w += part[i * 64 + lane];
  __syncthreads();
  // Order: larger key first; keys differ (the low bits hold 63 - line).
  const bool valid = lane < nmb;
  const int key = (w << 6) | (63 - lane);
  // Only the last line can hold fewer than rpb blocks: nl of them, at
  // position pl (the number of larger keys).  Ranks before it map rpb to a
  // line, then nl, then rpb.
  const int nl = nblk - (nmb - 1) * rpb;
  const int klast = __builtin_amdgcn_readlane(key, nmb - 1);
  const int pl = __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid && key > klast));
  int p, o;
  if (rank < pl * rpb) {
    p = rank / rpb;
    o = rank - p * rpb;
  } else if (rank < pl * rpb + nl) {
    p = pl;
    o = rank - pl * rpb;
  } else {
    const int s = rank - pl * rpb - nl;
    p = pl + 1 + s / rpb;
    o = s - (p - pl - 1) * rpb;
  }
  // The line at position p holds the (p+1)-th largest key: the largest t
  // with more than p keys >= t, found bit by bit from the top (keys are
  // below 2^13).
  int t = 0;
#pragma unroll
  for (int bit = 12; bit >= 0; --bit) {
    const int cand = t | (1 << bit);
    const int n = __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid && key >= cand));
    t = n > p ? cand : t;
  }
  return (63 - (t & 63)) * rpb + o;
}

// Workgroup barrier that waits for this wave's LDS operations and for all
// but its last VMCNT vector-memory operations.  Vector-memory operations of a
// wave complete in issue order on this architecture, so the loads issued
// before the last VMCNT operations (for example LDS-bound loads issued before
// a batch of atomics) are complete when the barrier is passed, while the
// younger operations may stay in flight.  The "memory" clobber keeps the
// compiler from moving memory accesses across it.
template <int VMCNT>
__device__ __forceinline__ void barrier_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VMCNT)
               : "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace fa
