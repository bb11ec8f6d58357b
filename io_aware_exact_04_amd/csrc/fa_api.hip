// C ABI of fa355: argument validation, workspace layout and dispatch.
// Validation touches only host memory and happens before any HIP call, so
// an invalid call launches nothing and writes nothing.
#include "fa355.h"
#include "fa_internal.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <utility>

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const char* what) {
  g_last_error = what;
  return s;
}

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// True if no two rows of a strided layout share an element.  A row is
// `row` contiguous elements; dims are (size, stride) pairs.  Taken in order
// of stride, each dimension of size > 1 must step past everything inside it
// (the rows of a broadcast dimension, stride 0, all coincide).  Outputs take
// the strides of the inputs, so overlapping rows would be written by several
// workgroups at once.
bool rows_disjoint(int64_t row, std::initializer_list<std::pair<int64_t, int64_t>> dims) {
  std::pair<int64_t, int64_t> v[3];
  int n = 0;
  for (const auto& e : dims)
    if (e.first > 1 && n < 3) v[n++] = {e.second, e.first};
  std::sort(v, v + n);
  int64_t span = row;
  for (int i = 0; i < n; ++i) {
    if (v[i].first < span) return false;
    const int64_t step = v[i].second - 1;
    span = v[i].first > (INT64_MAX - span) / step ? INT64_MAX
                                                  : span + step * v[i].first;
  }
  return true;
}

// Descriptor checks shared by both directions.  Sets *empty for B*H*N == 0.
fa_status check_desc(const fa_desc* d, bool* empty) {
  if (d == nullptr) return fail(FA_ERR_NULL, "desc is NULL");
  if (d->B < 0 || d->H < 0 || d->N < 0)
    return fail(FA_ERR_SHAPE, "B, H and N must be >= 0");
  if (d->reserved != 0) return fail(FA_ERR_SHAPE, "desc.reserved must be 0");
  if (d->d != 64 && d->d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  if (d->dtype != FA_F32 && d->dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype must be FA_F32 or FA_BF16");
  *empty = (int64_t)d->B * d->H * d->N == 0;
  if (*empty) return FA_OK;
  if (d->sn < d->d || d->sh < 0 || d->sb < 0)
    return fail(FA_ERR_SHAPE, "strides must satisfy sn >= d, sh >= 0, sb >= 0");
  if (!rows_disjoint(d->d, {{d->N, d->sn}, {d->H, d->sh}, {d->B, d->sb}}))
    return fail(FA_ERR_SHAPE, "strides make rows of different (b, h, n) overlap");
  const int64_t elt = d->dtype == FA_BF16 ? 2 : 4;
  const int64_t q16 = 16 / elt;  // elements per 16 bytes
  if (d->sn % q16 || d->sh % q16 || d->sb % q16)
    return fail(FA_ERR_ALIGN, "strides must be multiples of 16 bytes");
  if ((__int128)(d->N - 1) * d->sn + d->d >= ((int64_t)1 << 31))
    return fail(FA_ERR_ALIGN, "one head spans more than 2^31 elements");
  // bf16 kernels address one head with 32-bit byte offsets that may run up
  // to 256 rows past its end (range-checked loads of a ragged last tile).
  if (d->dtype == FA_BF16 &&
      ((__int128)d->N + 256) * d->sn * 2 >= ((int64_t)1 << 31))
    return fail(FA_ERR_ALIGN, "one head spans more than 2^31 bytes");
  // Largest grid: B*H*ceil(N/64) workgroups.
  if ((int64_t)d->B * d->H * ((d->N + 63) / 64) >= ((int64_t)1 << 31))
    return fail(FA_ERR_SHAPE, "problem too large for one launch");
  return FA_OK;
}

fa_status check_common(const fa_desc* d, float scale,
                       const uint8_t* block_mask, int32_t mask_block) {
  if (!(isfinite(scale) && scale > 0.f))
    return fail(FA_ERR_UNSUPPORTED, "scale must be finite and > 0");
  if (block_mask != nullptr && (mask_block <= 0 || mask_block % 128 != 0))
    return fail(FA_ERR_MASK, "mask_block must be a positive multiple of 128");
  (void)d;
  return FA_OK;
}

fa::Geom make_geom(const fa_desc* d, float scale, const uint8_t* block_mask,
                   int32_t mask_block) {
  fa::Geom g;
  g.B = d->B;
  g.H = d->H;
  g.N = d->N;
  g.sb = d->sb;
  g.sh = d->sh;
  g.sn = d->sn;
  g.mask = block_mask;
  g.mask_block = block_mask ? mask_block : 128;
  g.nmb = block_mask ? (d->N + mask_block - 1) / mask_block : 0;
  g.scale = scale;
  g.scale_log2 = scale * fa::kLog2e;
  g.Nk = d->N;
  g.causal_off = 0;
  g.ksb = d->sb;
  g.ksh = d->sh;
  g.ksn = d->sn;
  g.cu = nullptr;
  g.total = 0;
  g.kv_lens = nullptr;
  g.p8 = 0;
  g.seed_lo = g.seed_hi = 0;
  g.drop_scale = 1.0f;
  return g;
}

fa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  return fail(FA_ERR_HIP, hipGetErrorString(e));
}

}  // namespace

// Options of fa_fwd_ex / fa_bwd_ex: validation and application to a Geom.
namespace {

fa_status check_opts(const fa_desc* d, const fa_opts* o) {
  if (o == nullptr) return FA_OK;
  if (o->reserved != 0) return fail(FA_ERR_SHAPE, "opts.reserved must be 0");
  if (!(o->dropout_p >= 0.f && o->dropout_p < 1.f))
    return fail(FA_ERR_UNSUPPORTED, "dropout_p must be in [0, 1)");
  if ((int)floorf(256.f * o->dropout_p + 0.5f) > 255)
    return fail(FA_ERR_UNSUPPORTED, "dropout_p rounds to 1 (p8 > 255)");
  if ((o->dropout_p > 0.f || o->kv_lens != nullptr) && d->dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED,
                "dropout and key padding need FA_BF16 tensors");
  if (((uintptr_t)o->kv_lens & 3u) != 0)
    return fail(FA_ERR_ALIGN, "kv_lens must be 4-byte aligned");
  return FA_OK;
}

void apply_opts(fa::Geom& g, const fa_opts* o) {
  if (o == nullptr) return;
  g.kv_lens = o->kv_lens;
  g.p8 = (int)floorf(256.f * o->dropout_p + 0.5f);
  g.seed_lo = (uint32_t)o->seed;
  g.seed_hi = (uint32_t)(o->seed >> 32);
  g.drop_scale = g.p8 > 0 ? 256.0f / (float)(256 - g.p8) : 1.0f;
}

}  // namespace

// FP8 forward helpers.
namespace {

// Workspace sections of the FP8 forward, each 256-byte aligned.
fa_fp8_layout fp8_layout(const fa_desc* d) {
  fa_fp8_layout L;
  const size_t bh = (size_t)d->B * d->H;
  const size_t np = ((size_t)d->N + 63) / 64 * 64;
  const size_t codes = round_up(bh * np * d->d);
  const size_t scales = round_up(bh * (np / 64) * sizeof(int32_t));
  L.q_codes = 0;
  L.k_codes = codes;
  L.v_codes = 2 * codes;
  L.q_scales = 3 * codes;
  L.k_scales = 3 * codes + scales;
  L.v_scales = 3 * codes + 2 * scales;
  L.bytes = 3 * codes + 3 * scales;
  L.rows = (int32_t)np;
  L.reserved = 0;
  return L;
}

fa_status check_fp8_desc(const fa_desc* d, bool* empty) {
  fa_status st = check_desc(d, empty);
  if (st != FA_OK || *empty) return st;
  if (d->dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "the FP8 forward takes FA_BF16 tensors");
  if ((int64_t)3 * d->B * d->H * ((d->N + 63) / 64) >= ((int64_t)1 << 31))
    return fail(FA_ERR_SHAPE, "problem too large for one launch");
  return FA_OK;
}

fa::Fp8Args fp8_args(const fa_desc* d, void* ws, float scale, int rotate) {
  const fa_fp8_layout L = fp8_layout(d);
  char* w = (char*)ws;
  fa::Fp8Args a;
  memset(&a, 0, sizeof(a));
  // The rotation multiplies Q K^T by d: the score scale takes 1/d.
  a.g = make_geom(d, rotate ? scale / (float)d->d : scale, nullptr, 128);
  a.Np = L.rows;
  a.qc = (uint8_t*)(w + L.q_codes);
  a.kc = (uint8_t*)(w + L.k_codes);
  a.vt = (uint8_t*)(w + L.v_codes);
  a.qe = (int32_t*)(w + L.q_scales);
  a.ke = (int32_t*)(w + L.k_scales);
  a.ve = (int32_t*)(w + L.v_scales);
  a.rotate = rotate != 0;
  return a;
}

}  // namespace

namespace {

constexpr int kMaxSplits = 1024;
constexpr int kKeyTile = 64;  // split lengths are whole key tiles

fa_status check_kv(const fa_desc* d, const fa_kv_desc* kv, int causal,
                   int32_t num_splits) {
  if (kv == nullptr) return fail(FA_ERR_NULL, "kv descriptor is NULL");
  if (kv->reserved != 0) return fail(FA_ERR_SHAPE, "kv.reserved must be 0");
  if (kv->N < 1) return fail(FA_ERR_SHAPE, "kv.N must be >= 1");
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(FA_ERR_SHAPE, "num_splits must be in [1, 1024]");
  if (causal && kv->N < d->N)
    return fail(FA_ERR_SHAPE,
                "causal split-KV needs at least as many keys as queries");
  if (kv->sn < d->d || kv->sh < 0 || kv->sb < 0)
    return fail(FA_ERR_SHAPE,
                "kv strides must satisfy sn >= d, sh >= 0, sb >= 0");
  if (kv->sn % 8 || kv->sh % 8 || kv->sb % 8)  // 16 bytes of bf16
    return fail(FA_ERR_ALIGN, "kv strides must be multiples of 16 bytes");
  if ((__int128)(kv->N - 1) * kv->sn + d->d >= ((int64_t)1 << 31) ||
      ((__int128)kv->N + 256) * kv->sn * 2 >= ((int64_t)1 << 31))
    return fail(FA_ERR_ALIGN, "one key head spans more than 2^31 bytes");
  return FA_OK;
}

// Keys per split (whole key tiles) and the number of non-empty splits.
void split_geometry(int nk, int num_splits, int* len, int* splits) {
  int l = (nk + num_splits - 1) / num_splits;
  l = (l + kKeyTile - 1) / kKeyTile * kKeyTile;
  *len = l;
  *splits = (nk + l - 1) / l;
}

}  // namespace

namespace {

fa_status check_varlen(const fa_varlen_desc* d, bool* empty) {
  if (d == nullptr) return fail(FA_ERR_NULL, "desc is NULL");
  if (d->num_seqs < 0 || d->H < 0 || d->total < 0 || d->max_seqlen < 0)
    return fail(FA_ERR_SHAPE,
                "num_seqs, H, total and max_seqlen must be >= 0");
  if (d->reserved != 0) return fail(FA_ERR_SHAPE, "desc.reserved must be 0");
  if (d->d != 64 && d->d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
  if (d->dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "packed batches support FA_BF16 only");
  *empty = (int64_t)d->num_seqs * d->H == 0 || d->total == 0 ||
           d->max_seqlen == 0;
  if (*empty) return FA_OK;
  if (d->cu_seqlens == nullptr)
    return fail(FA_ERR_NULL, "cu_seqlens must be non-NULL");
  if ((uintptr_t)d->cu_seqlens & 3u)
    return fail(FA_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  if (d->sn < d->d || d->sh < 0)
    return fail(FA_ERR_SHAPE, "strides must satisfy sn >= d, sh >= 0");
  if (!rows_disjoint(d->d, {{d->total, d->sn}, {d->H, d->sh}}))
    return fail(FA_ERR_SHAPE, "strides make rows of different (row, h) overlap");
  if (d->sn % 8 || d->sh % 8)  // 16 bytes of bf16
    return fail(FA_ERR_ALIGN, "strides must be multiples of 16 bytes");
  if ((__int128)(d->total - 1) * d->sn + (__int128)(d->H - 1) * d->sh +
              d->d >= ((int64_t)1 << 31) ||
      ((__int128)d->total + 256) * d->sn * 2 >= ((int64_t)1 << 31))
    return fail(FA_ERR_ALIGN, "the packed tensors span more than 2^31 bytes");
  if ((int64_t)d->num_seqs * d->H * ((d->max_seqlen + 63) / 64) >=
      ((int64_t)1 << 31))
    return fail(FA_ERR_SHAPE, "problem too large for one launch");
  return FA_OK;
}

fa::Geom make_varlen_geom(const fa_varlen_desc* d, float scale) {
  fa::Geom g;
  g.B = d->num_seqs;
  g.H = d->H;
  g.N = d->max_seqlen;
  g.sb = 0;
  g.sh = d->sh;
  g.sn = d->sn;
  g.mask = nullptr;
  g.mask_block = 128;
  g.nmb = 0;
  g.scale = scale;
  g.scale_log2 = scale * fa::kLog2e;
  g.Nk = d->max_seqlen;
  g.causal_off = 0;
  g.ksb = 0;
  g.ksh = d->sh;
  g.ksn = d->sn;
  g.cu = d->cu_seqlens;
  g.total = d->total;
  g.kv_lens = nullptr;
  g.p8 = 0;
  g.seed_lo = g.seed_hi = 0;
  g.drop_scale = 1.0f;
  return g;
}

}  // namespace

// ------------------------------------------------- allocation-free backward
//
// fa_bwd_noalloc keeps the backward's row terms (D, then L * log2(e), one
// region of kScratchRows values each) in this file-scope device array
// instead of a caller workspace.  Every GPU the library runs on holds
// its own copy (allocated when the code object is loaded there) until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: the device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
namespace {

constexpr size_t kScratchRows = (size_t)1 << 22;  // B*H*N limit
static __device__ __align__(256) float scratch[2 * kScratchRows];  // 32 MiB

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the calling thread's current device.
fa_status scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr)
      return fail(FA_ERR_HIP, "no device address for the scratch array");
    g_scratch_dev[dev] = (float*)p;
  }
  *out = g_scratch_dev[dev];
  return FA_OK;
}

}  // namespace

extern "C" {


static fa_status fwd_impl(const fa_desc* desc, const void* q, const void* k,
                          const void* v, float scale, int causal,
                          const uint8_t* block_mask, int32_t mask_block,
                          const fa_opts* opts, void* o, float* lse,
                          void* stream) {
  bool empty = false;
  fa_status st = check_desc(desc, &empty);
  if (st != FA_OK) return st;
  st = check_opts(desc, opts);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  st = check_common(desc, scale, block_mask, mask_block);
  if (st != FA_OK) return st;

  fa::FwdArgs a;
  a.g = make_geom(desc, scale, block_mask, mask_block);
  apply_opts(a.g, opts);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.splits = 1;
  a.split_len = desc->N;
  a.part_o = nullptr;
  a.part_l = nullptr;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // clear an unrelated sticky launch error
  if (desc->dtype == FA_BF16)
    return hip_status(fa::launch_fwd_bf16(a, desc->d, causal != 0, s));
  return hip_status(fa::launch_fwd_f32(a, desc->d, causal != 0, s));
}

fa_status fa_fwd(const fa_desc* desc, const void* q, const void* k,
                 const void* v, float scale, int causal,
                 const uint8_t* block_mask, int32_t mask_block, void* o,
                 float* lse, void* stream) {
  return fwd_impl(desc, q, k, v, scale, causal, block_mask, mask_block,
                  nullptr, o, lse, stream);
}

fa_status fa_fwd_ex(const fa_desc* desc, const void* q, const void* k,
                    const void* v, float scale, int causal,
                    const fa_opts* opts, void* o, float* lse, void* stream) {
  return fwd_impl(desc, q, k, v, scale, causal, nullptr, 128, opts, o, lse,
                  stream);
}

size_t fa_bwd_workspace_bytes(const fa_desc* desc) {
  bool empty = false;
  if (check_desc(desc, &empty) != FA_OK || empty) return 0;
  const size_t rows = (size_t)desc->B * desc->H * desc->N;
  return round_up(2 * rows * sizeof(float));  // D, then L * log2(e)
}

// Checks of a backward call's arguments other than the workspace; sets
// *empty for an empty problem (then nothing else is looked at).
static fa_status check_bwd(const fa_desc* desc, int first, int last,
                           const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           float scale, const uint8_t* block_mask,
                           int32_t mask_block, const fa_opts* opts, void* dq,
                           void* dk, void* dv, bool* empty) {
  fa_status st = check_desc(desc, empty);
  if (st != FA_OK) return st;
  st = check_opts(desc, opts);
  if (st != FA_OK) return st;
  if (first < 0 || last > 1 || first > last)
    return fail(FA_ERR_UNSUPPORTED, "stage must be 0 or 1");
  if (*empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(FA_ERR_NULL, "q, k, v, o, lse, dout, dq, dk, dv must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  return check_common(desc, scale, block_mask, mask_block);
}

// Enqueue backward stages first..last with the row term D at `delta` and
// L * log2(e) at `lse2` (B*H*N values each).
static fa_status launch_bwd(const fa_desc* desc, int first, int last,
                            const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dout,
                            float scale, int causal, const uint8_t* block_mask,
                            int32_t mask_block, const fa_opts* opts, void* dq,
                            void* dk, void* dv, float* delta, float* lse2,
                            void* stream) {
  fa::BwdArgs a;
  a.g = make_geom(desc, scale, block_mask, mask_block);
  apply_opts(a.g, opts);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.lse2 = lse2;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = desc->dtype == FA_BF16;
  (void)hipGetLastError();
  for (int stage = first; stage <= last; ++stage) {
    hipError_t e = hipSuccess;
    if (stage == 0) {
      // dQ, and the row terms into the workspace: the bf16 dQ kernel forms
      // them itself; in fp32 the memory-bound pre-pass runs first.
      if (bf16) {
        e = fa::launch_bwd_dq_bf16(a, desc->d, causal != 0, s);
      } else {
        e = fa::launch_bwd_pre(a, desc->d, false, s);
        if (e == hipSuccess)
          e = fa::launch_bwd_dq_f32(a, desc->d, causal != 0, s);
      }
    } else {
      e = bf16 ? fa::launch_bwd_dkdv_bf16(a, desc->d, causal != 0, s)
               : fa::launch_bwd_dkdv_f32(a, desc->d, causal != 0, s);
    }
    if (e != hipSuccess) return hip_status(e);
  }
  return FA_OK;
}

static fa_status bwd_impl(const fa_desc* desc, int first, int last,
                          const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout,
                          float scale, int causal, const uint8_t* block_mask,
                          int32_t mask_block, const fa_opts* opts, void* dq,
                          void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  bool empty = false;
  fa_status st = check_bwd(desc, first, last, q, k, v, o, lse, dout, scale,
                           block_mask, mask_block, opts, dq, dk, dv, &empty);
  if (st != FA_OK || empty) return st;
  const size_t need = fa_bwd_workspace_bytes(desc);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace))
    return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
  const size_t rows = (size_t)desc->B * desc->H * desc->N;
  return launch_bwd(desc, first, last, q, k, v, o, lse, dout, scale, causal,
                    block_mask, mask_block, opts, dq, dk, dv,
                    (float*)workspace, (float*)workspace + rows, stream);
}

fa_status fa_bwd(const fa_desc* desc, const void* q, const void* k,
                 const void* v, const void* o, const float* lse,
                 const void* dout, float scale, int causal,
                 const uint8_t* block_mask, int32_t mask_block, void* dq,
                 void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return bwd_impl(desc, 0, 1, q, k, v, o, lse, dout, scale, causal,
                  block_mask, mask_block, nullptr, dq, dk, dv, workspace,
                  workspace_bytes, stream);
}

fa_status fa_bwd_ex(const fa_desc* desc, const void* q, const void* k,
                    const void* v, const void* o, const float* lse,
                    const void* dout, float scale, int causal,
                    const fa_opts* opts, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(desc, 0, 1, q, k, v, o, lse, dout, scale, causal, nullptr,
                  128, opts, dq, dk, dv, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_stage(const fa_desc* desc, int stage, const void* q,
                       const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, float scale,
                       int causal, const uint8_t* block_mask,
                       int32_t mask_block, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       void* stream) {
  return bwd_impl(desc, stage, stage, q, k, v, o, lse, dout, scale, causal,
                  block_mask, mask_block, nullptr, dq, dk, dv, workspace,
                  workspace_bytes, stream);
}

size_t fa_bwd_noalloc_max_rows(void) { return kScratchRows; }

fa_status fa_bwd_noalloc(const fa_desc* desc, const void* q, const void* k,
                         const void* v, const void* o, const float* lse,
                         const void* dout, float scale, int causal,
                         const uint8_t* block_mask, int32_t mask_block,
                         void* dq, void* dk, void* dv, void* stream) {
  bool empty = false;
  fa_status st = check_bwd(desc, 0, 1, q, k, v, o, lse, dout, scale,
                           block_mask, mask_block, nullptr, dq, dk, dv,
                           &empty);
  if (st != FA_OK || empty) return st;
  if ((size_t)desc->B * desc->H * desc->N > kScratchRows)
    return fail(FA_ERR_WORKSPACE,
                "B*H*N exceeds the allocation-free backward's scratch "
                "(4194304 rows); use fa_bwd with a workspace");
  float* delta = nullptr;
  st = scratch_on_current_device(&delta);
  if (st != FA_OK) return st;
  return launch_bwd(desc, 0, 1, q, k, v, o, lse, dout, scale, causal,
                    block_mask, mask_block, nullptr, dq, dk, dv, delta,
                    delta + kScratchRows, stream);
}

// ---------------------------------------------------------------- split-KV


size_t fa_fwd_splitkv_workspace_bytes(const fa_desc* desc,
                                      const fa_kv_desc* kv,
                                      int32_t num_splits) {
  bool empty = false;
  if (check_desc(desc, &empty) != FA_OK || empty) return 0;
  if (desc->dtype != FA_BF16 || check_kv(desc, kv, 0, num_splits) != FA_OK)
    return 0;
  int len = 0, splits = 0;
  split_geometry(kv->N, num_splits, &len, &splits);
  const size_t rows = (size_t)desc->B * desc->H * desc->N;
  return round_up(rows * splits * desc->d * sizeof(float)) +
         round_up(rows * splits * sizeof(float));
}

fa_status fa_fwd_splitkv(const fa_desc* desc, const fa_kv_desc* kv,
                         const void* q, const void* k, const void* v,
                         float scale, int causal, int32_t num_splits, void* o,
                         float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  bool empty = false;
  fa_status st = check_desc(desc, &empty);
  if (st != FA_OK || empty) return st;
  if (desc->dtype != FA_BF16)
    return fail(FA_ERR_UNSUPPORTED, "split-KV forward supports FA_BF16 only");
  st = check_kv(desc, kv, causal, num_splits);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  st = check_common(desc, scale, nullptr, 0);
  if (st != FA_OK) return st;
  int len = 0, splits = 0;
  split_geometry(kv->N, num_splits, &len, &splits);
  if ((int64_t)desc->B * desc->H * ((desc->N + 127) / 128) * splits >=
      ((int64_t)1 << 31))
    return fail(FA_ERR_SHAPE, "problem too large for one launch");
  const size_t need = fa_fwd_splitkv_workspace_bytes(desc, kv, num_splits);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace))
    return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");

  fa::FwdArgs a;
  a.g = make_geom(desc, scale, nullptr, 0);
  a.g.Nk = kv->N;
  a.g.causal_off = causal ? kv->N - desc->N : 0;
  a.g.ksb = kv->sb;
  a.g.ksh = kv->sh;
  a.g.ksn = kv->sn;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.splits = splits;
  a.split_len = len;
  const size_t rows = (size_t)desc->B * desc->H * desc->N;
  a.part_o = (float*)workspace;
  a.part_l = (float*)((char*)workspace +
                      round_up(rows * splits * desc->d * sizeof(float)));
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  // One query row (decoding): the streaming vector-ALU pass; otherwise the
  // matrix-core forward over each split.
  hipError_t e = desc->N == 1
                     ? fa::launch_decode_split_bf16(a, desc->d, s)
                     : fa::launch_fwd_splitkv_bf16(a, desc->d, causal != 0, s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(fa::launch_splitkv_merge(a, desc->d, s));
}

// ------------------------------------------------------ packed (varlen) batches


fa_status fa_fwd_varlen(const fa_varlen_desc* desc, const void* q,
                        const void* k, const void* v, float scale, int causal,
                        void* o, float* lse, void* stream) {
  bool empty = false;
  fa_status st = check_varlen(desc, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !lse)
    return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!(isfinite(scale) && scale > 0.f))
    return fail(FA_ERR_UNSUPPORTED, "scale must be finite and > 0");
  fa::FwdArgs a;
  a.g = make_varlen_geom(desc, scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.splits = 1;
  a.split_len = desc->max_seqlen;
  a.part_o = nullptr;
  a.part_l = nullptr;
  (void)hipGetLastError();
  return hip_status(
      fa::launch_fwd_bf16(a, desc->d, causal != 0, (hipStream_t)stream));
}

size_t fa_bwd_varlen_workspace_bytes(const fa_varlen_desc* desc) {
  bool empty = false;
  if (check_varlen(desc, &empty) != FA_OK || empty) return 0;
  // D, then L * log2(e), [H, total] each.
  return round_up(2 * (size_t)desc->H * desc->total * sizeof(float));
}

fa_status fa_bwd_varlen(const fa_varlen_desc* desc, const void* q,
                        const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, float scale,
                        int causal, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        void* stream) {
  bool empty = false;
  fa_status st = check_varlen(desc, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(FA_ERR_NULL,
                "q, k, v, o, lse, dout, dq, dk, dv must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!(isfinite(scale) && scale > 0.f))
    return fail(FA_ERR_UNSUPPORTED, "scale must be finite and > 0");
  if (workspace == nullptr ||
      workspace_bytes < fa_bwd_varlen_workspace_bytes(desc))
    return fail(FA_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace))
    return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
  fa::BwdArgs a;
  a.g = make_varlen_geom(desc, scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float*)workspace;
  a.lse2 = a.delta + (size_t)desc->H * desc->total;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  // dQ first: it writes every packed row's D and L * log2(e), laid out
  // [H, total] like L, for the key-outer kernel.
  hipError_t e = fa::launch_bwd_dq_bf16(a, desc->d, causal != 0, s);
  if (e == hipSuccess)
    e = fa::launch_bwd_dkdv_bf16(a, desc->d, causal != 0, s);
  return hip_status(e);
}


fa_status fa_fp8_workspace_layout(const fa_desc* desc, fa_fp8_layout* out) {
  if (out == nullptr) return fail(FA_ERR_NULL, "out is NULL");
  memset(out, 0, sizeof(*out));
  bool empty = false;
  fa_status st = check_fp8_desc(desc, &empty);
  if (st != FA_OK || empty) return st;
  *out = fp8_layout(desc);
  return FA_OK;
}

fa_status fa_fp8_quantize(const fa_desc* desc, const void* q, const void* k,
                          const void* v, const int8_t* signs, int rotate,
                          void* workspace, size_t workspace_bytes,
                          void* stream) {
  bool empty = false;
  fa_status st = check_fp8_desc(desc, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v) return fail(FA_ERR_NULL, "q, k and v must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const fa_fp8_layout L = fp8_layout(desc);
  if (workspace == nullptr || workspace_bytes < L.bytes)
    return fail(FA_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace))
    return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
  uint64_t lo = 0, hi = 0;
  if (rotate && signs != nullptr) {
    for (int i = 0; i < desc->d; ++i) {
      if (signs[i] != 1 && signs[i] != -1)
        return fail(FA_ERR_UNSUPPORTED, "signs must be +1 or -1");
      if (signs[i] < 0) (i < 64 ? lo : hi) |= (uint64_t)1 << (i & 63);
    }
  }
  fa::Fp8Args a = fp8_args(desc, workspace, 1.0f, rotate);
  a.q = q;
  a.k = k;
  a.v = v;
  a.sign_lo = lo;
  a.sign_hi = hi;
  (void)hipGetLastError();
  return hip_status(
      fa::launch_fp8_quantize(a, desc->d, (hipStream_t)stream));
}

fa_status fa_fwd_fp8_quantized(const fa_desc* desc, const void* workspace,
                               size_t workspace_bytes, float scale, int causal,
                               int rotate, void* o, float* lse, void* stream) {
  bool empty = false;
  fa_status st = check_fp8_desc(desc, &empty);
  if (st != FA_OK || empty) return st;
  if (!o || !lse) return fail(FA_ERR_NULL, "o and lse must be non-NULL");
  if (!aligned16(o) || ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!(isfinite(scale) && scale > 0.f))
    return fail(FA_ERR_UNSUPPORTED, "scale must be finite and > 0");
  const fa_fp8_layout L = fp8_layout(desc);
  if (workspace == nullptr || workspace_bytes < L.bytes)
    return fail(FA_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(workspace))
    return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
  fa::Fp8Args a = fp8_args(desc, const_cast<void*>(workspace), scale, rotate);
  a.o = o;
  a.lse = lse;
  (void)hipGetLastError();
  return hip_status(
      fa::launch_fwd_fp8(a, desc->d, causal != 0, (hipStream_t)stream));
}

fa_status fa_fwd_fp8(const fa_desc* desc, const void* q, const void* k,
                     const void* v, float scale, int causal,
                     const int8_t* signs, int rotate, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  fa_status st = check_fp8_desc(desc, &empty);
  if (st != FA_OK || empty) return st;
  // Validate the forward's own arguments before the quantisation is queued,
  // so that an error launches nothing.
  if (!o || !lse) return fail(FA_ERR_NULL, "o and lse must be non-NULL");
  if (!aligned16(o) || ((uintptr_t)lse & 3u))
    return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (!(isfinite(scale) && scale > 0.f))
    return fail(FA_ERR_UNSUPPORTED, "scale must be finite and > 0");
  st = fa_fp8_quantize(desc, q, k, v, signs, rotate, workspace,
                       workspace_bytes, stream);
  if (st != FA_OK) return st;
  return fa_fwd_fp8_quantized(desc, workspace, workspace_bytes, scale, causal,
                              rotate, o, lse, stream);
}

const char* fa_status_str(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer";
    case FA_ERR_SHAPE: return "invalid shape or strides";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or scale";
    case FA_ERR_MASK: return "invalid block mask";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_ALIGN: return "misaligned pointer or stride";
  }
  return "unknown status";
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

const char* fa_last_hip_error(void) { return g_last_error.c_str(); }

int32_t fa_version(void) { return 100; }

}  // extern "C"
