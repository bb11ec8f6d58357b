"""Python binding of fa355, exact tiled softmax attention for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfa355.so`` behind its C ABI (``include/fa355.h``).  PyTorch is
used for device memory and the current stream; there is no fallback path --
if the library is missing or a call fails, an exception is raised.

    o, lse = fa_fwd(q, k, v, causal=True)
    dq, dk, dv = fa_bwd(q, k, v, o, lse, do, causal=True)
    out = attention(q, k, v, causal=True)        # autograd-aware
    o, lse = fa_fwd_splitkv(q, k_cache, v_cache, num_splits=16)  # decoding
    o, lse = fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen)  # packed batch
    o, lse = fa_fwd_fp8(q, k, v, causal=True, signs=signs)  # FP8 products
    o, lse = fa_fwd_ex(q, k, v, causal=True, dropout_p=0.1, seed=7,
                       kv_lens=lens)                # dropout, key padding

Tensors are [B, H, N, d] (d in {64, 128}), bfloat16 or float32, on one GPU.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch

__all__ = ["fa_fwd", "fa_bwd", "fa_fwd_splitkv", "fa_fwd_varlen",
           "fa_bwd_varlen", "attention", "FaError",
           "library_path", "load_library", "workspace_bytes",
           "splitkv_workspace_bytes", "fa_fwd_fp8", "fa_fp8_quantize",
           "fa_fwd_fp8_quantized", "fp8_layout", "fp8_sections",
           "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_noalloc", "noalloc_max_rows"]

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                         "libfa355.so")
_lib = None
_lock = threading.Lock()

FA_F32, FA_BF16 = 0, 1
_STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE",
           3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_MASK", 5: "FA_ERR_WORKSPACE",
           6: "FA_ERR_HIP", 7: "FA_ERR_ALIGN"}


class FaDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


class FaKvDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


class FaVarlenDesc(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("total", ctypes.c_int32), ("max_seqlen", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


class FaFp8Layout(ctypes.Structure):
    _fields_ = [("q_codes", ctypes.c_size_t), ("k_codes", ctypes.c_size_t),
                ("v_codes", ctypes.c_size_t), ("q_scales", ctypes.c_size_t),
                ("k_scales", ctypes.c_size_t), ("v_scales", ctypes.c_size_t),
                ("bytes", ctypes.c_size_t), ("rows", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class FaOpts(ctypes.Structure):
    _fields_ = [("dropout_p", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("kv_lens", ctypes.c_void_p)]


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = _STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfa355.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing; build it with "
                "`python -m io_aware_exact_04_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, f32, i32 = ctypes.c_void_p, ctypes.c_float, ctypes.c_int32
        desc_p = ctypes.POINTER(FaDesc)
        lib.fa_fwd.argtypes = [desc_p, vp, vp, vp, f32, ctypes.c_int, vp, i32,
                               vp, vp, vp]
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_bwd_workspace_bytes.argtypes = [desc_p]
        lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_bwd.argtypes = [desc_p, vp, vp, vp, vp, vp, vp, f32,
                               ctypes.c_int, vp, i32, vp, vp, vp, vp,
                               ctypes.c_size_t, vp]
        lib.fa_bwd.restype = ctypes.c_int
        lib.fa_bwd_stage.argtypes = [desc_p, ctypes.c_int, vp, vp, vp, vp, vp,
                                     vp, f32, ctypes.c_int, vp, i32, vp, vp,
                                     vp, vp, ctypes.c_size_t, vp]
        lib.fa_bwd_stage.restype = ctypes.c_int
        lib.fa_bwd_noalloc.argtypes = [desc_p, vp, vp, vp, vp, vp, vp, f32,
                                       ctypes.c_int, vp, i32, vp, vp, vp, vp]
        lib.fa_bwd_noalloc.restype = ctypes.c_int
        lib.fa_bwd_noalloc_max_rows.argtypes = []
        lib.fa_bwd_noalloc_max_rows.restype = ctypes.c_size_t
        kv_p = ctypes.POINTER(FaKvDesc)
        lib.fa_fwd_splitkv_workspace_bytes.argtypes = [desc_p, kv_p, i32]
        lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_fwd_splitkv.argtypes = [desc_p, kv_p, vp, vp, vp, f32,
                                       ctypes.c_int, i32, vp, vp, vp,
                                       ctypes.c_size_t, vp]
        lib.fa_fwd_splitkv.restype = ctypes.c_int
        vl_p = ctypes.POINTER(FaVarlenDesc)
        lib.fa_fwd_varlen.argtypes = [vl_p, vp, vp, vp, f32, ctypes.c_int, vp,
                                      vp, vp]
        lib.fa_fwd_varlen.restype = ctypes.c_int
        lib.fa_bwd_varlen_workspace_bytes.argtypes = [vl_p]
        lib.fa_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
        lib.fa_bwd_varlen.argtypes = [vl_p, vp, vp, vp, vp, vp, vp, f32,
                                      ctypes.c_int, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
        lib.fa_bwd_varlen.restype = ctypes.c_int
        op_p = ctypes.POINTER(FaOpts)
        lib.fa_fwd_ex.argtypes = [desc_p, vp, vp, vp, f32, ctypes.c_int, op_p,
                                  vp, vp, vp]
        lib.fa_fwd_ex.restype = ctypes.c_int
        lib.fa_bwd_ex.argtypes = [desc_p, vp, vp, vp, vp, vp, vp, f32,
                                  ctypes.c_int, op_p, vp, vp, vp, vp,
                                  ctypes.c_size_t, vp]
        lib.fa_bwd_ex.restype = ctypes.c_int
        lay_p = ctypes.POINTER(FaFp8Layout)
        i8p = ctypes.POINTER(ctypes.c_int8)
        lib.fa_fp8_workspace_layout.argtypes = [desc_p, lay_p]
        lib.fa_fp8_workspace_layout.restype = ctypes.c_int
        lib.fa_fp8_quantize.argtypes = [desc_p, vp, vp, vp, i8p, ctypes.c_int,
                                        vp, ctypes.c_size_t, vp]
        lib.fa_fp8_quantize.restype = ctypes.c_int
        lib.fa_fwd_fp8_quantized.argtypes = [desc_p, vp, ctypes.c_size_t, f32,
                                             ctypes.c_int, ctypes.c_int, vp,
                                             vp, vp]
        lib.fa_fwd_fp8_quantized.restype = ctypes.c_int
        lib.fa_fwd_fp8.argtypes = [desc_p, vp, vp, vp, f32, ctypes.c_int, i8p,
                                   ctypes.c_int, vp, vp, vp, ctypes.c_size_t,
                                   vp]
        lib.fa_fwd_fp8.restype = ctypes.c_int
        lib.fa_status_str.argtypes = [ctypes.c_int]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_last_error.argtypes = []
        lib.fa_last_error.restype = ctypes.c_char_p
        lib.fa_last_hip_error.argtypes = []
        lib.fa_last_hip_error.restype = ctypes.c_char_p
        lib.fa_version.argtypes = []
        lib.fa_version.restype = ctypes.c_int32
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise FaError(status, lib.fa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _desc_for(tensors) -> FaDesc:
    ref = tensors[0]
    code = _dtype_code(ref)
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    for t in tensors:
        if t.shape != ref.shape:
            raise ValueError(f"shape mismatch {tuple(t.shape)} vs "
                             f"{tuple(ref.shape)}")
        if t.dtype != ref.dtype:
            raise TypeError("all tensors must share one dtype")
        if t.device != ref.device or t.device.type != "cuda":
            raise ValueError("all tensors must be on the same GPU")
        if t.stride() != ref.stride() and t.numel() > 1:
            raise ValueError("all tensors must share one stride layout")
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    B, H, N, d = ref.shape
    sb, sh, sn, _ = ref.stride()
    return FaDesc(B, H, N, d, code, 0, sb, sh, sn)


def _empty_as(ref: torch.Tensor) -> torch.Tensor:
    """An uninitialised output with ref's shape AND strides: the kernels
    write every output with the descriptor's strides (those of q), so an
    output allocated with other strides (torch.empty_like gives a non-dense
    q dense strides) would be written past its end."""
    return torch.empty_strided(ref.shape, ref.stride(), dtype=ref.dtype,
                               device=ref.device)


def _check_lse(lse: torch.Tensor, shape, device):
    if (lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape)
            or not lse.is_contiguous() or lse.device != device):
        dims = ", ".join(str(x) for x in shape)
        raise ValueError(f"lse must be a contiguous float32 [{dims}] tensor "
                         "on q's device")


def _same_layout(x: torch.Tensor, ref: torch.Tensor) -> torch.Tensor:
    """x with ref's strides (copied only if they differ)."""
    if x.stride() == ref.stride():
        return x
    y = torch.empty_strided(ref.shape, ref.stride(), dtype=x.dtype,
                            device=x.device)
    y.copy_(x)
    return y


def _mask_args(block_mask, mask_block, N, device):
    if block_mask is None:
        return None, 0, None
    if not isinstance(block_mask, torch.Tensor):
        raise TypeError("block_mask must be a torch.uint8 tensor")
    nb = -(-N // mask_block) if mask_block > 0 else -1
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be uint8 [{nb}, {nb}] for N={N}, "
                         f"mask_block={mask_block}")
    m = block_mask.to(device).contiguous()
    return ctypes.c_void_p(m.data_ptr()), mask_block, m


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fa_fwd(q, k, v, scale=None, causal=False, block_mask=None,
           mask_block=128, out=None, lse=None):
    """Forward: returns (O [B,H,N,d] like q, L [B,H,N] float32)."""
    k = _same_layout(k, q)
    v = _same_layout(v, q)
    desc = _desc_for([q, k, v])
    B, H, N, d = q.shape
    if out is None:
        out = _empty_as(q)
    else:
        _desc_for([q, out])
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_lse(lse, (B, H, N), q.device)
    mptr, mb, _keep = _mask_args(block_mask, mask_block, N, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        st = lib.fa_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                        _scale(scale, d), 1 if causal else 0, mptr, mb,
                        _ptr(out), _ptr(lse), _stream(q.device))
    _check(st)
    return out, lse


def workspace_bytes(q: torch.Tensor) -> int:
    desc = _desc_for([q])
    return int(load_library().fa_bwd_workspace_bytes(ctypes.byref(desc)))


def fa_bwd(q, k, v, o, lse, do, scale=None, causal=False, block_mask=None,
           mask_block=128, workspace=None, stages=None, between=None,
           out=None):
    """Backward: returns (dQ, dK, dV), each like q.

    By default one fa_bwd call.  With ``stages`` (a sequence of stage
    indices, normally ``(0, 1)``: dQ with the row terms, then dK and dV)
    the stages run one by one through
    fa_bwd_stage, and ``between(i)`` (if given) is called after stage i has
    been enqueued -- used to place timing events between the kernels.
    ``out`` may give preallocated (dQ, dK, dV) tensors laid out like q.
    """
    k, v, o, do = (_same_layout(x, q) for x in (k, v, o, do))
    desc = _desc_for([q, k, v, o, do])
    B, H, N, d = q.shape
    _check_lse(lse, (B, H, N), q.device)
    if out is None:
        dq, dk, dv = (_empty_as(q) for _ in range(3))
    else:
        dq, dk, dv = out
        _desc_for([q, dq, dk, dv])
    lib = load_library()
    need = int(lib.fa_bwd_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8,
                                device=q.device)
    mptr, mb, _keep = _mask_args(block_mask, mask_block, N, q.device)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
              _scale(scale, d), 1 if causal else 0, mptr, mb, _ptr(dq),
              _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel())
    with torch.cuda.device(q.device):
        if stages is None:
            _check(lib.fa_bwd(ctypes.byref(desc), *common,
                              _stream(q.device)))
        else:
            for i in stages:
                _check(lib.fa_bwd_stage(ctypes.byref(desc), int(i), *common,
                                        _stream(q.device)))
                if between is not None:
                    between(i)
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, lse, do, scale=None, causal=False,
                   block_mask=None, mask_block=128, out=None):
    """Backward through the allocation-free entry point (the row term lives
    in the library's static device scratch, not in a workspace): returns
    (dQ, dK, dV) like fa_bwd.  Pass ``out`` (preallocated dQ, dK, dV laid
    out like q) where nothing may be allocated.  Calls that overlap on one
    GPU race on that scratch."""
    k, v, o, do = (_same_layout(x, q) for x in (k, v, o, do))
    desc = _desc_for([q, k, v, o, do])
    B, H, N, d = q.shape
    _check_lse(lse, (B, H, N), q.device)
    if out is None:
        dq, dk, dv = (_empty_as(q) for _ in range(3))
    else:
        dq, dk, dv = out
        _desc_for([q, dq, dk, dv])
    mptr, mb, _keep = _mask_args(block_mask, mask_block, N, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_noalloc(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
            _ptr(lse), _ptr(do), _scale(scale, d), 1 if causal else 0, mptr,
            mb, _ptr(dq), _ptr(dk), _ptr(dv), _stream(q.device)))
    return dq, dk, dv


def noalloc_max_rows() -> int:
    """Largest B*H*N the allocation-free backward accepts."""
    return int(load_library().fa_bwd_noalloc_max_rows())


def _kv_desc_for(k: torch.Tensor, v: torch.Tensor, q: torch.Tensor):
    if k.dim() != 4 or k.shape != v.shape:
        raise ValueError("k and v must be [B, H, Nk, d] of one shape")
    B, H, Nk, d = k.shape
    if (B, H, d) != (q.shape[0], q.shape[1], q.shape[3]):
        raise ValueError("k, v must share B, H and d with q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same GPU")
    if d > 1 and (k.stride(-1) != 1 or v.stride(-1) != 1):
        raise ValueError("the head dimension must be contiguous")
    sb, sh, sn, _ = k.stride()
    return FaKvDesc(Nk, 0, sb, sh, sn)


def splitkv_workspace_bytes(q, k, num_splits) -> int:
    desc = _desc_for([q])
    kv = _kv_desc_for(k, k, q)
    return int(load_library().fa_fwd_splitkv_workspace_bytes(
        ctypes.byref(desc), ctypes.byref(kv), int(num_splits)))


def fa_fwd_splitkv(q, k, v, scale=None, causal=False, num_splits=1,
                   out=None, lse=None, workspace=None):
    """Split-KV forward: q [B,H,N,d] against k, v [B,H,Nk,d] (bf16).

    Returns (O like q, L [B,H,N] float32).  causal keeps key <= query +
    (Nk - N).  The keys are split into ``num_splits`` runs whose partial
    results are merged by their logsumexp.
    """
    v = _same_layout(v, k)
    desc = _desc_for([q])
    kv = _kv_desc_for(k, v, q)
    B, H, N, d = q.shape
    if out is None:
        out = _empty_as(q)
    else:
        _desc_for([q, out])
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_lse(lse, (B, H, N), q.device)
    lib = load_library()
    need = int(lib.fa_fwd_splitkv_workspace_bytes(
        ctypes.byref(desc), ctypes.byref(kv), int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8,
                                device=q.device)
    with torch.cuda.device(q.device):
        st = lib.fa_fwd_splitkv(ctypes.byref(desc), ctypes.byref(kv), _ptr(q),
                                _ptr(k), _ptr(v), _scale(scale, d),
                                1 if causal else 0, int(num_splits), _ptr(out),
                                _ptr(lse), _ptr(workspace), workspace.numel(),
                                _stream(q.device))
    _check(st)
    return out, lse


def _varlen_desc(q, cu_seqlens, max_seqlen, tensors):
    if q.dim() != 3:
        raise ValueError("packed tensors must be [total, H, d]")
    if q.dtype != torch.bfloat16:
        raise TypeError("packed batches support bfloat16 only")
    for t in tensors:
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("packed tensors must share shape, dtype, device")
        if t.stride() != q.stride():
            raise ValueError("packed tensors must share one stride layout")
    if q.device.type != "cuda" or q.stride(-1) != 1:
        raise ValueError("packed tensors must be on a GPU, d contiguous")
    if (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or cu_seqlens.device != q.device
            or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 GPU vector")
    total, H, d = q.shape
    return FaVarlenDesc(cu_seqlens.numel() - 1, H, d, FA_BF16, total,
                        int(max_seqlen), 0, 0, cu_seqlens.data_ptr(),
                        q.stride(1), q.stride(0))


def fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale=None, causal=False,
                  out=None, lse=None):
    """Forward of a packed batch: q, k, v [total, H, d] bf16, sequence b is
    rows cu_seqlens[b]:cu_seqlens[b+1].  Returns (O like q, L [H, total]);
    ``out`` / ``lse`` may be given (laid out like q / contiguous fp32)."""
    desc = _varlen_desc(q, cu_seqlens, max_seqlen, [k, v] +
                        ([out] if out is not None else []))
    if out is None:
        out = _empty_as(q)
    if lse is None:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32,
                          device=q.device)
    else:
        _check_lse(lse, (q.shape[1], q.shape[0]), q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_varlen(ctypes.byref(desc), _ptr(q), _ptr(k),
                                 _ptr(v), _scale(scale, q.shape[2]),
                                 1 if causal else 0, _ptr(out), _ptr(lse),
                                 _stream(q.device)))
    return out, lse


def fa_bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, scale=None,
                  causal=False, out=None, workspace=None):
    """Backward of a packed batch: returns (dQ, dK, dV) like q; ``out`` may
    give them (laid out like q), ``workspace`` a uint8 device buffer."""
    desc = _varlen_desc(q, cu_seqlens, max_seqlen, [k, v, o, do] +
                        (list(out) if out is not None else []))
    _check_lse(lse, (q.shape[1], q.shape[0]), q.device)
    if out is None:
        dq, dk, dv = (_empty_as(q) for _ in range(3))
    else:
        dq, dk, dv = out
    lib = load_library()
    need = int(lib.fa_bwd_varlen_workspace_bytes(ctypes.byref(desc)))
    ws = workspace
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_varlen(ctypes.byref(desc), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                 _scale(scale, q.shape[2]),
                                 1 if causal else 0, _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(ws), ws.numel(),
                                 _stream(q.device)))
    return dq, dk, dv


def _opts(q, dropout_p, seed, kv_lens):
    if kv_lens is not None:
        if (kv_lens.dtype != torch.int32 or kv_lens.device != q.device
                or tuple(kv_lens.shape) != (q.shape[0],)
                or not kv_lens.is_contiguous()):
            raise ValueError("kv_lens must be a contiguous int32 [B] tensor "
                             "on q's device")
    return FaOpts(float(dropout_p), 0, int(seed) & (2 ** 64 - 1),
                  None if kv_lens is None else kv_lens.data_ptr())


def fa_fwd_ex(q, k, v, scale=None, causal=False, dropout_p=0.0, seed=0,
              kv_lens=None, out=None, lse=None):
    """Forward with dropout and/or key padding (bf16): returns (O, L)."""
    k = _same_layout(k, q)
    v = _same_layout(v, q)
    desc = _desc_for([q, k, v])
    B, H, N, d = q.shape
    if out is None:
        out = _empty_as(q)
    else:
        _desc_for([q, out])
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_lse(lse, (B, H, N), q.device)
    opts = _opts(q, dropout_p, seed, kv_lens)
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd_ex(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _scale(scale, d),
            1 if causal else 0, ctypes.byref(opts), _ptr(out), _ptr(lse),
            _stream(q.device)))
    return out, lse


def fa_bwd_ex(q, k, v, o, lse, do, scale=None, causal=False, dropout_p=0.0,
              seed=0, kv_lens=None, workspace=None, out=None):
    """Backward of fa_fwd_ex with the same options: returns (dQ, dK, dV)."""
    k, v, o, do = (_same_layout(x, q) for x in (k, v, o, do))
    desc = _desc_for([q, k, v, o, do])
    _check_lse(lse, q.shape[:3], q.device)
    if out is None:
        dq, dk, dv = (_empty_as(q) for _ in range(3))
    else:
        dq, dk, dv = out
        _desc_for([q, dq, dk, dv])
    lib = load_library()
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(q), 16),
                                dtype=torch.uint8, device=q.device)
    opts = _opts(q, dropout_p, seed, kv_lens)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_ex(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
            _ptr(lse), _ptr(do), _scale(scale, q.shape[3]),
            1 if causal else 0, ctypes.byref(opts), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def fp8_layout(q) -> FaFp8Layout:
    """Workspace layout of the FP8 forward for bf16 tensors of q's shape
    (a tensor or a (B, H, N, d) tuple; the layout ignores strides)."""
    B, H, N, d = (int(x) for x in (q.shape if hasattr(q, "shape") else q))
    desc = FaDesc(B, H, N, d, FA_BF16, 0, H * N * d, N * d, d)
    lay = FaFp8Layout()
    _check(load_library().fa_fp8_workspace_layout(ctypes.byref(desc),
                                                  ctypes.byref(lay)))
    return lay


def _signs_arg(signs, d):
    if signs is None:
        return None
    vals = [int(x) for x in (signs.tolist() if hasattr(signs, "tolist")
                             else signs)]
    if len(vals) != d:
        raise ValueError("signs must hold d values")
    return (ctypes.c_int8 * d)(*vals)


def _fp8_workspace(q, workspace):
    need = fp8_layout(q).bytes
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    return workspace


def fa_fp8_quantize(q, k, v, signs=None, rotate=True, workspace=None):
    """Rotation and per-block E4M3 quantisation of bf16 q, k, v into a
    workspace (uint8 tensor), returned."""
    k = _same_layout(k, q)
    v = _same_layout(v, q)
    desc = _desc_for([q, k, v])
    ws = _fp8_workspace(q, workspace)
    sg = _signs_arg(signs, q.shape[3])
    with torch.cuda.device(q.device):
        _check(load_library().fa_fp8_quantize(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), sg,
            1 if rotate else 0, _ptr(ws), ws.numel(), _stream(q.device)))
    return ws


def fa_fwd_fp8_quantized(workspace, out, lse, scale=None, causal=False,
                         rotate=True):
    """The FP8 products on a filled workspace; writes out (bf16
    [B,H,N,d]) and lse (float32 [B,H,N]) and returns them."""
    desc = _desc_for([out])
    B, H, N, d = out.shape
    _check_lse(lse, (B, H, N), out.device)
    with torch.cuda.device(out.device):
        _check(load_library().fa_fwd_fp8_quantized(
            ctypes.byref(desc), _ptr(workspace), workspace.numel(),
            _scale(scale, d), 1 if causal else 0, 1 if rotate else 0,
            _ptr(out), _ptr(lse), _stream(out.device)))
    return out, lse


def fa_fwd_fp8(q, k, v, scale=None, causal=False, signs=None, rotate=True,
               workspace=None, out=None, lse=None):
    """FP8 forward with incoherent processing: returns (O bf16 like q,
    L [B,H,N] float32)."""
    k = _same_layout(k, q)
    v = _same_layout(v, q)
    desc = _desc_for([q, k, v])
    B, H, N, d = q.shape
    if out is None:
        out = _empty_as(q)
    else:
        _desc_for([q, out])
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_lse(lse, (B, H, N), q.device)
    ws = _fp8_workspace(q, workspace)
    sg = _signs_arg(signs, d)
    with torch.cuda.device(q.device):
        _check(load_library().fa_fwd_fp8(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _scale(scale, d),
            1 if causal else 0, sg, 1 if rotate else 0, _ptr(out), _ptr(lse),
            _ptr(ws), ws.numel(), _stream(q.device)))
    return out, lse


def fp8_sections(workspace: torch.Tensor, q: torch.Tensor) -> dict:
    """Views of a filled FP8 workspace (layout in include/fa355.h):
    q_codes, k_codes uint8 [B*H, rows, d]; v_codes uint8 [B*H, d, rows]
    (keys permuted within 64-key groups); *_scales int32 [B*H, rows/64]."""
    lay = fp8_layout(q)
    B, H, N, d = (int(x) for x in (q.shape if hasattr(q, "shape") else q))
    bh, rows = B * H, lay.rows

    def view(off, count, shape, dtype):
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return workspace[off:off + nbytes].view(dtype).view(shape)

    return {
        "q_codes": view(lay.q_codes, bh * rows * d, (bh, rows, d), torch.uint8),
        "k_codes": view(lay.k_codes, bh * rows * d, (bh, rows, d), torch.uint8),
        "v_codes": view(lay.v_codes, bh * rows * d, (bh, d, rows), torch.uint8),
        "q_scales": view(lay.q_scales, bh * rows // 64, (bh, rows // 64),
                         torch.int32),
        "k_scales": view(lay.k_scales, bh * rows // 64, (bh, rows // 64),
                         torch.int32),
        "v_scales": view(lay.v_scales, bh * rows // 64, (bh, rows // 64),
                         torch.int32),
        "rows": rows,
    }


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale, causal, block_mask, mask_block):
        o, lse = fa_fwd(q, k, v, scale, causal, block_mask, mask_block)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (scale, causal, block_mask, mask_block)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        scale, causal, block_mask, mask_block = ctx.args
        dq, dk, dv = fa_bwd(q, k, v, o, lse, do.contiguous(), scale, causal,
                            block_mask, mask_block)
        return dq, dk, dv, None, None, None, None


def attention(q, k, v, scale=None, causal=False, block_mask=None,
              mask_block=128):
    """Exact softmax attention; differentiable (saves only O and L)."""
    return _Attention.apply(q, k, v, scale, causal, block_mask, mask_block)
