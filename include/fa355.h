/*
 * fa355 -- exact tiled softmax attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor pointer is a DEVICE pointer owned by the caller; the
 * library never allocates device memory, keeps no pointer after a call
 * returns, and holds no mutable global state (calls are thread-safe).  Work
 * is enqueued asynchronously on the caller's HIP stream; no call
 * synchronises the host.  No exception crosses this boundary.
 *
 * Every argument is validated on the host BEFORE any HIP call: on an error
 * status nothing has been launched and no output has been written.  Launch
 * failures are reported as FA_ERR_HIP, with the runtime's text available
 * from fa_last_error() (alias fa_last_hip_error()) on the calling thread.
 *
 * Operation ("FlashAttention: making attention IO-aware", sections "Tiling:
 * never materialise S", "Online softmax", "The backward pass: recompute,
 * don't store"; "Why is FlashAttention faster?", "Why is FlashAttention
 * faster on long sequences?"): for every batch b and head h,
 *     S = scale * Q K^T,   masked entries -inf,
 *     P = row softmax(S),  O = P V,  L = row logsumexp(S) (natural log),
 * computed tile by tile so that no N x N matrix is ever written to memory.
 * A query row whose keys are all masked gets O = 0 and L = -inf, and
 * contributes no gradient.
 *
 * Tensor layout: Q, K, V, O, dO, dQ, dK, dV are [B, H, N, d] with element
 * strides (sb, sh, sn, 1), all eight sharing the strides of the descriptor.
 * L is a dense fp32 [B, H, N] array.  Tensors must not overlap one another,
 * and no two rows (b, h, n) of one tensor may share an element: taken in
 * order of stride, each of sn, sh, sb whose dimension has more than one
 * entry must be at least the span of the dimensions inside it, so a
 * broadcast (stride 0) dimension of size > 1 is refused (FA_ERR_SHAPE).
 *
 * Supported: d in {64, 128}; dtype FA_F32 or FA_BF16 (all eight tensors in
 * that one dtype; L and the workspace are fp32); any N >= 1 (a ragged last
 * tile is masked); scale finite and > 0; base pointers 16-byte aligned and
 * sb, sh, sn multiples of 16 bytes; the offset of the last element of one
 * head, (N-1)*sn + d, below 2^31 elements, and for FA_BF16 (N+256)*sn*2
 * below 2^31 bytes (FA_ERR_ALIGN otherwise).  B*H*N == 0 is an empty
 * problem: FA_OK, nothing is launched, the pointers are not inspected.
 *
 * Masks: causal keeps key <= query (sequences of equal length).  A block
 * mask is a DEVICE array uint8 [nb][nb], nb = ceil(N / mask_block), row =
 * query block, column = key block, non-zero = keep; one mask is shared by
 * every (b, h).  mask_block must be a positive multiple of 128.  Tiles that
 * the mask (or causality) removes entirely are skipped, never computed
 * ("FlashAttention: making attention IO-aware", "Counting the IO" and
 * "FlashAttention-2: better parallelism").  causal together with a block
 * mask keeps their intersection.
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  FA_ERR_SHAPE = 2,       /* B, H, N negative; strides too small or rows
                             overlapping                                    */
  FA_ERR_UNSUPPORTED = 3, /* d or dtype not supported; scale not finite > 0 */
  FA_ERR_MASK = 4,        /* mask_block not a positive multiple of 128      */
  FA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required        */
  FA_ERR_HIP = 6,         /* the HIP runtime reported an error              */
  FA_ERR_ALIGN = 7        /* pointer or stride not 16-byte aligned; offsets
                             of one head do not fit 31 bits                 */
} fa_status;

typedef enum fa_dtype { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

typedef struct fa_desc {
  int32_t B, H, N, d;   /* batch, heads, sequence length, head dimension   */
  int32_t dtype;        /* fa_dtype                                         */
  int32_t reserved;     /* must be 0                                        */
  int64_t sb, sh, sn;   /* element strides of b, h, n; the d stride is 1    */
} fa_desc;

/*
 * Forward.  Reads q, k, v; writes o ([B,H,N,d], dtype of desc) and lse
 * ([B,H,N] fp32, natural-log row logsumexp L of the scaled, masked scores).
 * block_mask may be NULL (no block mask; mask_block is then ignored).
 * stream is a hipStream_t (NULL = the null stream).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_MASK,
 * FA_ERR_ALIGN (nothing launched); FA_ERR_HIP (launch failed).
 */
fa_status fa_fwd(const fa_desc* desc, const void* q, const void* k,
                 const void* v, float scale, int causal,
                 const uint8_t* block_mask, int32_t mask_block, void* o,
                 float* lse, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this descriptor: two fp32 row
 * arrays [B,H,N], the softmax row term D and the logsumexp in base-2 units
 * L * log2(e) (rounded up to 256 bytes).  Returns 0 for an invalid
 * descriptor or an empty problem.
 */
size_t fa_bwd_workspace_bytes(const fa_desc* desc);

/*
 * Backward ("FlashAttention: making attention IO-aware", "The backward
 * pass: recompute, don't store").  Reads q, k, v, o and lse exactly as
 * produced by fa_fwd with the same scale, causal flag and block mask, and
 * the output gradient dout; writes dq, dk, dv ([B,H,N,d], dtype of desc)
 * for the loss sum(O * dO).  Probabilities are recomputed tile by tile as
 * P = exp(S - L); the softmax row term is D = rowsum(dO * O).
 * workspace: device memory of at least fa_bwd_workspace_bytes(desc) bytes,
 * 16-byte aligned, owned by the caller, overwritten by the call and free to
 * reuse once the stream has passed this call.
 * Errors: as fa_fwd, plus FA_ERR_WORKSPACE.
 */
fa_status fa_bwd(const fa_desc* desc, const void* q, const void* k,
                 const void* v, const void* o, const float* lse,
                 const void* dout, float scale, int causal,
                 const uint8_t* block_mask, int32_t mask_block, void* dq,
                 void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * One stage of fa_bwd, for callers that schedule or time the stages
 * separately.  Arguments are those of fa_bwd; stage selects
 *   0: the query-outer pass: dQ, each row written once (no atomics, so the
 *      result does not depend on scheduling), and every row's
 *      D = rowsum(dO * O) and L * log2(e) into the workspace;
 *   1: the key-outer kernel: dK and dV, each row written once, from the
 *      row terms that stage 0 left in the workspace.
 * Running stages 0 and 1 in order on one stream with one workspace is
 * exactly fa_bwd.  Errors: as fa_bwd; FA_ERR_UNSUPPORTED for another stage.
 */
fa_status fa_bwd_stage(const fa_desc* desc, int stage, const void* q,
                       const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, float scale,
                       int causal, const uint8_t* block_mask,
                       int32_t mask_block, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The same computation as fa_bwd (the same kernels, so
 * bitwise the same dq, dk, dv) without a workspace argument: the row terms
 * (D and L * log2(e), fa_bwd_noalloc_max_rows() fp32 values each, 32 MiB)
 * live in a static device array inside the library, one copy per GPU, held
 * until the process ends.  The call allocates nothing; its first call on a device looks up
 * that device's copy (hipGetSymbolAddress), so the calling thread's current
 * device must be the one the stream and the tensors belong to.
 * Requires B*H*N <= fa_bwd_noalloc_max_rows() (FA_ERR_WORKSPACE otherwise,
 * nothing launched); no dropout or key-padding options (use fa_bwd_ex).
 * Every call on one GPU shares that array: calls that overlap on one GPU
 * (on different streams, or from different threads without ordering)
 * race and give wrong results.  Calls ordered on one stream are safe: each
 * call rewrites every row term it reads.  Other arguments and errors as
 * fa_bwd.
 */
fa_status fa_bwd_noalloc(const fa_desc* desc, const void* q, const void* k,
                         const void* v, const void* o, const float* lse,
                         const void* dout, float scale, int causal,
                         const uint8_t* block_mask, int32_t mask_block,
                         void* dq, void* dk, void* dv, void* stream);

/* Largest B*H*N fa_bwd_noalloc accepts (4194304). */
size_t fa_bwd_noalloc_max_rows(void);

/*
 * Split-KV forward ("FlashAttention: making attention IO-aware", "In
 * practice": for decoding -- few query rows against a long key/value cache
 * -- the query blocks give too little parallelism, so Flash-Decoding splits
 * the keys across workgroups and merges the partial results with the
 * logsumexp rescaling of the online softmax).
 *
 * Queries and outputs follow desc (Q, O [B, H, N, d] with desc's strides;
 * L [B, H, N] fp32); keys and values have their own length and strides
 * (K, V [B, H, kv->N, d]).  The kv->N keys are cut into num_splits runs of
 * equal length (rounded up to whole 64-key tiles, so fewer runs may be
 * used); each run is processed independently, and its normalised partial
 * output O_s and logsumexp L_s (fp32, in the workspace) are merged as
 *     L = ln sum_s exp(L_s),   O = sum_s exp(L_s - L) O_s.
 * The result equals fa_fwd's up to rounding.  causal keeps key
 * <= query + (kv->N - N): the queries are the last N positions of the key
 * sequence (requires kv->N >= N).  No block mask.  bf16 only.
 *
 * Supported and validated as fa_fwd, plus: dtype FA_BF16 (else
 * FA_ERR_UNSUPPORTED); kv->N >= 1, kv->reserved == 0, 1 <= num_splits <=
 * 1024, kv->N >= N when causal (else FA_ERR_SHAPE); kv strides as desc's
 * (FA_ERR_SHAPE / FA_ERR_ALIGN).  workspace: at least
 * fa_fwd_splitkv_workspace_bytes(desc, kv, num_splits) bytes of device
 * memory, 16-byte aligned, owned by the caller, overwritten by the call.
 * Errors: as fa_fwd, plus FA_ERR_WORKSPACE.
 */
typedef struct fa_kv_desc {
  int32_t N;            /* number of keys (and values), >= 1               */
  int32_t reserved;     /* must be 0                                       */
  int64_t sb, sh, sn;   /* element strides of K and V; the d stride is 1  */
} fa_kv_desc;

/* Bytes of workspace fa_fwd_splitkv needs (0 for an invalid or empty call). */
size_t fa_fwd_splitkv_workspace_bytes(const fa_desc* desc,
                                      const fa_kv_desc* kv,
                                      int32_t num_splits);

fa_status fa_fwd_splitkv(const fa_desc* desc, const fa_kv_desc* kv,
                         const void* q, const void* k, const void* v,
                         float scale, int causal, int32_t num_splits,
                         void* o, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Packed variable-length batches ("FlashAttention: making attention
 * IO-aware", "In practice": varlen kernels take a flat batch of
 * concatenated sequences plus their offsets, so padding costs nothing).
 *
 * Q, K, V, O, dO, dQ, dK, dV are packed [total, H, d] tensors (element
 * strides sn per row, sh per head, 1 within a row; sn = H*d, sh = d when
 * dense; no two (row, head) pairs may share an element, FA_ERR_SHAPE
 * otherwise); sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1, with
 * queries and keys of equal length; attention never crosses sequences.
 * L (and the backward workspace's D and L * log2(e)) are fp32 [H, total].  causal keeps key
 * <= query within each sequence.  No block mask.  bf16 only.
 *
 * cu_seqlens is a DEVICE int32 array [num_seqs + 1], non-decreasing, with
 * cu_seqlens[0] = 0 and cu_seqlens[num_seqs] = total; max_seqlen must be at
 * least the longest sequence (it sizes the grid).  The library cannot read
 * device memory before launching: offsets outside [0, total] are clamped and
 * rows past max_seqlen of a sequence are not computed, so malformed offsets
 * give wrong (never out-of-bounds) results.
 */
typedef struct fa_varlen_desc {
  int32_t num_seqs;     /* sequences in the batch                          */
  int32_t H, d;         /* heads, head dimension (64 or 128)               */
  int32_t dtype;        /* FA_BF16                                         */
  int32_t total;        /* packed rows, cu_seqlens[num_seqs]               */
  int32_t max_seqlen;   /* >= every sequence length                        */
  int32_t reserved;     /* must be 0                                       */
  int32_t pad;          /* ignored                                         */
  const int32_t* cu_seqlens;  /* DEVICE [num_seqs + 1]                    */
  int64_t sh, sn;       /* element strides of head and row; d stride 1    */
} fa_varlen_desc;

/*
 * Forward of a packed batch: writes o (packed like q) and lse ([H, total]).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN
 * (nothing launched); FA_ERR_HIP.  num_seqs * H, total or max_seqlen equal
 * to 0 is an empty problem (FA_OK, nothing launched).
 */
fa_status fa_fwd_varlen(const fa_varlen_desc* desc, const void* q,
                        const void* k, const void* v, float scale,
                        int causal, void* o, float* lse, void* stream);

/* Bytes of workspace fa_bwd_varlen needs: D and L * log2(e), fp32
 * [H, total] each. */
size_t fa_bwd_varlen_workspace_bytes(const fa_varlen_desc* desc);

/*
 * Backward of a packed batch (as fa_bwd, per sequence): reads q, k, v, o,
 * lse from fa_fwd_varlen with the same arguments and dout; writes dq, dk,
 * dv (packed like q).  Errors: as fa_fwd_varlen, plus FA_ERR_WORKSPACE.
 */
fa_status fa_bwd_varlen(const fa_varlen_desc* desc, const void* q,
                        const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, float scale,
                        int causal, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Dropout and key padding (named on the pages among the element-wise steps
 * attention fuses: "FlashAttention: making attention IO-aware", "Attention
 * is memory-bound"; "Why is FlashAttention faster?", "Extra computation can
 * still finish sooner").  fa_fwd_ex / fa_bwd_ex are fa_fwd / fa_bwd without
 * a block mask and with these options (opts == NULL: none):
 *
 *   kv_lens: DEVICE int32 [B] or NULL.  Batch b keeps keys < kv_lens[b]
 *     (values are clamped into [0, N]; the library cannot read them before
 *     launching); combined with causal by intersection.  Rows left without
 *     keys get O = 0 and L = -inf; padded keys get dK = dV = 0.
 *   dropout_p, seed: after the softmax, each probability P[b,h,q,k] is
 *     dropped with probability p8 / 256, p8 = floor(256 dropout_p + 1/2)
 *     (0 <= dropout_p, p8 <= 255; FA_ERR_UNSUPPORTED otherwise), and kept
 *     ones are scaled by 256 / (256 - p8): O = (P o Z) V * 256/(256 - p8).
 *     L stays the logsumexp of S.  The decision for (b, h, q, k) is the
 *     byte 4 (q % 4) + (k % 4) of Philox4x32-10 ("Parallel random numbers:
 *     as easy as 1, 2, 3", Salmon et al., SC 2011) with counter
 *     (k / 4, q / 4, h, b) and key (seed low word, seed high word), the
 *     output words' bytes taken little-endian in order; dropped when that
 *     byte < p8.  The backward regenerates the same decisions: call fa_bwd_ex
 *     with the options (and scale, causal) of the forward.
 *
 * Both options need desc->dtype == FA_BF16 (FA_ERR_UNSUPPORTED otherwise);
 * opts->reserved must be 0 (FA_ERR_SHAPE); kv_lens 4-byte aligned
 * (FA_ERR_ALIGN).  Other errors as fa_fwd / fa_bwd.
 */
typedef struct fa_opts {
  float dropout_p;          /* drop probability, quantised to 1/256        */
  int32_t reserved;         /* must be 0                                   */
  uint64_t seed;            /* generator key                               */
  const int32_t* kv_lens;   /* DEVICE int32 [B] key lengths, or NULL       */
} fa_opts;

fa_status fa_fwd_ex(const fa_desc* desc, const void* q, const void* k,
                    const void* v, float scale, int causal,
                    const fa_opts* opts, void* o, float* lse, void* stream);

fa_status fa_bwd_ex(const fa_desc* desc, const void* q, const void* k,
                    const void* v, const void* o, const float* lse,
                    const void* dout, float scale, int causal,
                    const fa_opts* opts, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward with incoherent processing ("FlashAttention: making attention
 * IO-aware", section "FlashAttention-3: Hopper asynchrony and FP8": FP8
 * products, per-block quantisation, and Q, K multiplied by a random
 * orthogonal Hadamard-based matrix first to spread outliers).
 *
 * Operation, per (b, h), on bf16 Q, K, V [B, H, N, d] (desc->dtype must be
 * FA_BF16; d in {64, 128}; strides as for fa_fwd):
 *   1. rotation (rotate != 0): Q' = Q M, K' = K M with M = diag(signs) H_d,
 *      H_d the Sylvester Hadamard matrix (entries +-1); V is not rotated.
 *      Q' K'^T = d Q K^T, so the score scale becomes scale / d;
 *   2. quantisation: every 64 rows of one head of Q', K', V share a scale
 *      2^e, e the smallest integer with max|x| <= 448 * 2^e (e >= -127);
 *      codes = OCP E4M3 (largest value 448) of x / 2^e, round to nearest
 *      even;
 *   3. S = scale' Qd Kd^T (Qd = codes * 2^e, ...), masked as for fa_fwd
 *      (causal or none; no block mask); P = exp(S - m) with a row
 *      reference m, rounded to E4M3 after multiplication by a power of two;
 *      O = (rounded P) Vd / sum(unrounded P); L = row logsumexp of S
 *      (natural log).  O is written as bf16 with desc's strides, L as fp32
 *      [B, H, N].
 * The products run on the FP8 matrix cores; O differs from exact attention
 * by the rounding of Q', K', V and P to 3-bit mantissas (a few percent
 * relative on unit-variance inputs).
 *
 * signs: HOST array of d int8 values, each +1 or -1 (FA_ERR_UNSUPPORTED
 * otherwise); NULL means all +1; ignored when rotate == 0.  rotate == 0
 * gives plain per-block FP8 attention.
 *
 * Workspace: a DEVICE buffer of at least fa_fp8_layout.bytes (16-byte
 * aligned) that holds the quantised operands between the two steps:
 *   q_codes, k_codes: uint8 [B*H][rows][d] (rows = N rounded up to 64; rows
 *                     past N are zero);
 *   v_codes:          uint8 [B*H][d][rows], V transposed, the keys of each
 *                     64-key group g stored at position
 *                     32 ((r>>2)&1) + 16 (r>>5) + 4 ((r>>3)&3) + (r&3)
 *                     for key 64 g + r (the key order the FP8 matrix core
 *                     consumes);
 *   q_scales, k_scales, v_scales: int32 [B*H][rows/64] E8M0 codes, scale =
 *                     2^(code - 127).
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN,
 * FA_ERR_WORKSPACE (nothing launched); FA_ERR_HIP.  B*H*N == 0 is empty.
 */
typedef struct fa_fp8_layout {
  size_t q_codes, k_codes, v_codes;     /* byte offsets in the workspace  */
  size_t q_scales, k_scales, v_scales;  /* byte offsets in the workspace  */
  size_t bytes;                         /* workspace size required        */
  int32_t rows;                         /* rows per head: N rounded to 64 */
  int32_t reserved;
} fa_fp8_layout;

/* Workspace layout for desc (all zero for an empty problem). */
fa_status fa_fp8_workspace_layout(const fa_desc* desc, fa_fp8_layout* out);

/* Steps 1-2: rotate and quantise q, k, v into the workspace. */
fa_status fa_fp8_quantize(const fa_desc* desc, const void* q, const void* k,
                          const void* v, const int8_t* signs, int rotate,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* Step 3 on a workspace filled by fa_fp8_quantize with the same desc;
 * `rotate` must be the value given to it (it selects the 1/d). */
fa_status fa_fwd_fp8_quantized(const fa_desc* desc, const void* workspace,
                               size_t workspace_bytes, float scale,
                               int causal, int rotate, void* o, float* lse,
                               void* stream);

/* Steps 1-3 in one call (two launches on the stream). */
fa_status fa_fwd_fp8(const fa_desc* desc, const void* q, const void* k,
                     const void* v, float scale, int causal,
                     const int8_t* signs, int rotate, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* fa_status_str(fa_status status);

/* Text of the last FA_ERR_HIP (or validation) failure on this thread
 * (never NULL; empty before the first failure).  The pointer stays valid
 * until the next call that fails on the same thread. */
const char* fa_last_error(void);

/* The same text under the name the backward boundary was specified with:
 * fa_last_hip_error() returns exactly what fa_last_error() returns. */
const char* fa_last_hip_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
