"""C-ABI library checks that need no GPU: it loads, exports every declared
symbol, and rejects invalid arguments with the documented status BEFORE any
HIP call.

Every call below that passes stand-in pointer values is constructed so that
validation fails (or the problem is empty); such calls never reach a launch.
"""
import ctypes
import os
import re

import pytest

import io_aware_exact_04_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa355.h")

needs_lib = pytest.mark.skipif(not os.path.exists(fa.library_path()),
                               reason="libfa355.so not built")

OK, NULL, SHAPE, UNSUP, MASK, WS, HIP, ALIGN = range(8)
FAKE = 0x7F0000000000  # 16-byte aligned stand-in, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def desc(B=1, H=2, N=256, d=64, dtype=1, sb=None, sh=None, sn=None,
         reserved=0):
    sn = d if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = H * sh if sb is None else sb
    return fa.FaDesc(B, H, N, d, dtype, reserved, sb, sh, sn)


def p(x=FAKE):
    return ctypes.c_void_p(x)


def fwd(dsc, q=FAKE, k=FAKE, v=FAKE, scale=0.125, causal=0, mask=None,
        mask_block=128, o=FAKE, lse=FAKE):
    lib = fa.load_library()
    return lib.fa_fwd(ctypes.byref(dsc) if dsc is not None else None,
                      p(q), p(k), p(v), scale, causal,
                      None if mask is None else p(mask), mask_block, p(o),
                      p(lse), None)


def bwd(dsc, ws=FAKE, ws_bytes=1 << 40, scale=0.125, mask=None,
        mask_block=128, q=FAKE, dq=FAKE):
    lib = fa.load_library()
    return lib.fa_bwd(ctypes.byref(dsc), p(q), p(), p(), p(), p(), p(),
                      scale, 0, None if mask is None else p(mask), mask_block,
                      p(dq), p(), p(), None if ws is None else p(ws), ws_bytes,
                      None)


@needs_lib
def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_str",
            "fa_last_error", "fa_last_hip_error", "fa_version"} <= set(names)
    lib = ctypes.CDLL(fa.library_path())
    for n in names:
        assert hasattr(lib, n), n


@needs_lib
def test_status_strings_and_version():
    lib = fa.load_library()
    for code in range(8):
        assert lib.fa_status_str(code)
    assert lib.fa_status_str(99) == b"unknown status"
    assert lib.fa_version() == 100


@needs_lib
def test_descriptor_validation():
    lib = fa.load_library()
    assert lib.fa_fwd(None, p(), p(), p(), 0.1, 0, None, 0, p(), p(),
                      None) == NULL
    assert fwd(desc(d=96)) == UNSUP
    assert fwd(desc(d=32)) == UNSUP
    assert fwd(desc(dtype=2)) == UNSUP
    assert fwd(desc(N=-1)) == SHAPE
    assert fwd(desc(B=-3)) == SHAPE
    assert fwd(desc(reserved=1)) == SHAPE
    assert fwd(desc(sn=32)) == SHAPE            # sn < d
    assert fwd(desc(sn=68)) == ALIGN            # 136 bytes, not 16-aligned
    assert fwd(desc(dtype=0, sn=66)) == ALIGN   # fp32: 264 bytes
    assert fwd(desc(sh=1000 * 64 + 4)) == ALIGN
    assert b"16 bytes" in lib.fa_last_error()
    assert fwd(desc(N=1 << 22, sn=1024)) == ALIGN  # head spans > 2^31
    assert b"2^31" in lib.fa_last_error()
    assert lib.fa_last_hip_error() == lib.fa_last_error()


@needs_lib
def test_overlapping_rows_are_refused():
    """Outputs are written with the inputs' strides, so no two rows
    (b, h, n) may share an element; layouts that pass reach the pointer
    checks (q = NULL here), which come after the descriptor's."""
    lib = fa.load_library()
    assert fwd(desc(H=2, sh=0)) == SHAPE                 # heads broadcast
    assert b"overlap" in lib.fa_last_error()
    assert fwd(desc(B=2, sb=0)) == SHAPE                 # batch broadcast
    assert fwd(desc(H=2, N=256, sh=64)) == SHAPE         # sh == sn: rows alias
    assert fwd(desc(B=2, H=2, N=8, sh=1024, sb=256)) == SHAPE  # b cuts rows
    # legal: [B, N, H, d] storage (heads innermost), sizes of 1 broadcast,
    # batch innermost of all
    assert fwd(desc(B=2, H=4, N=8, sn=4 * 64, sh=64, sb=8 * 4 * 64),
               q=0) == NULL
    assert fwd(desc(B=1, H=1, sb=0, sh=0), q=0) == NULL
    assert fwd(desc(B=3, H=2, N=8, sb=64, sh=3 * 64, sn=6 * 64), q=0) == NULL
    assert fwd(desc(B=2, sb=(1 << 62)), q=0) == NULL     # huge: no overflow
    assert fwd(desc(N=1, sn=1 << 62, sh=64, sb=128)) == ALIGN  # bf16 span
    # the workspace query treats an invalid descriptor as no problem at all
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(desc(H=2, sh=0))) == 0


@needs_lib
def test_overlap_check_against_brute_force():
    """The descriptor check against an explicit comparison of every row's
    element range, on random small layouts (strides that are zero, equal,
    interleaved or permuted included): it never accepts a layout whose rows
    overlap.  (It may refuse a disjoint but interleaved one: the header's
    rule asks each stride to cover the dimensions inside it.)  Every dense
    layout, in any order of the three dimensions, is accepted."""
    import itertools
    import random
    rng = random.Random(7)
    d = 64
    accepted = overlapping = 0
    for _ in range(400):
        B, H, N = (rng.randint(1, 4) for _ in range(3))
        pick = lambda: rng.choice([0, 8, 16, 32, 64, 72, 128, 256, 512,  # noqa: E731
                                   1024, 64 * N, 64 * N * H, 72 * N])
        sn = rng.choice([64, 72, 128, 256, 64 * H, 64 * B * H])
        sh, sb = pick(), pick()
        rows = [b_ * sb + h_ * sh + n_ * sn for b_, h_, n_ in
                itertools.product(range(B), range(H), range(N))]
        rows.sort()
        disjoint = all(y - x >= d for x, y in zip(rows, rows[1:]))
        got = fwd(desc(B=B, H=H, N=N, d=d, sn=sn, sh=sh, sb=sb), q=0)
        assert got in (NULL, SHAPE), got
        assert disjoint or got == SHAPE, (B, H, N, sb, sh, sn)
        accepted += got == NULL
        overlapping += not disjoint
    assert accepted > 50 and overlapping > 50   # both kinds were drawn
    for B, H, N in itertools.product((1, 2, 3), repeat=3):
        for order in itertools.permutations("bhn"):
            stride, inner = {}, d
            for dim in order:                    # innermost first
                stride[dim] = inner
                inner *= {"b": B, "h": H, "n": N}[dim]
            got = fwd(desc(B=B, H=H, N=N, d=d, sn=stride["n"],
                           sh=stride["h"], sb=stride["b"]), q=0)
            assert got == NULL, (B, H, N, order)


@needs_lib
def test_empty_problem_is_a_no_op():
    # Nothing is launched and no pointer is looked at.
    lib = fa.load_library()
    d0 = desc(B=0)
    assert lib.fa_fwd(ctypes.byref(d0), None, None, None, 0.1, 0, None, 0,
                      None, None, None) == OK
    assert lib.fa_fwd(ctypes.byref(desc(N=0)), None, None, None, 0.1, 0,
                      None, 0, None, None, None) == OK
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(desc(H=0))) == 0


@needs_lib
def test_pointer_and_argument_validation():
    assert fwd(desc(), q=0) == NULL
    assert fwd(desc(), lse=0) == NULL
    assert fwd(desc(), q=FAKE + 8) == ALIGN
    assert fwd(desc(), o=FAKE + 2) == ALIGN
    assert fwd(desc(), lse=FAKE + 2) == ALIGN
    assert fwd(desc(), scale=0.0) == UNSUP
    assert fwd(desc(), scale=-0.5) == UNSUP
    assert fwd(desc(), scale=float("nan")) == UNSUP
    assert fwd(desc(), scale=float("inf")) == UNSUP
    assert fwd(desc(), mask=FAKE, mask_block=64) == MASK
    assert fwd(desc(), mask=FAKE, mask_block=0) == MASK
    assert fwd(desc(), mask=FAKE, mask_block=200) == MASK


@needs_lib
def test_backward_validation_and_workspace_size():
    lib = fa.load_library()
    d = desc(B=2, H=3, N=100, d=128, dtype=1)
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(d))
    rows = 2 * 3 * 100
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need == r256(2 * rows * 4)   # D and L * log2(e)
    d32 = desc(B=2, H=3, N=100, d=128, dtype=0)
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(d32)) == r256(2 * rows * 4)
    assert lib.fa_bwd_workspace_bytes(None) == 0
    assert bwd(d, q=0) == NULL
    assert bwd(d, dq=0, ws=None) == NULL  # tensor pointers are checked first
    assert bwd(d, q=FAKE + 8) == ALIGN
    # all tensor pointers valid from here on: one other argument is wrong
    lib2 = fa.load_library()

    def full(ws, ws_bytes, scale=0.125, mask=None, mb=128):
        return lib2.fa_bwd(ctypes.byref(d), *[p()] * 6, scale, 0,
                           None if mask is None else p(mask), mb, p(), p(),
                           p(), None if ws is None else p(ws), ws_bytes, None)
    assert full(None, need) == WS
    assert full(FAKE, need - 1) == WS
    assert full(FAKE + 4, need) == ALIGN
    assert full(FAKE, need, scale=0.0) == UNSUP
    assert full(FAKE, need, mask=FAKE, mb=100) == MASK
    # Two stages (0: dQ and the row terms, 1: dK and dV); any other index is
    # rejected before anything is enqueued.
    for stage in (-1, 2, 3):
        assert lib2.fa_bwd_stage(ctypes.byref(d), stage, *[p()] * 6, 0.125,
                                 0, None, 128, p(), p(), p(), p(), need,
                                 None) == UNSUP


def test_binding_rejects_host_tensors_before_calling():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.fa_fwd(q.half(), q.half(), q.half())


def test_product_package_does_not_use_the_oracle():
    pkg = os.path.dirname(fa.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", src, re.M), f
                assert "import workloads" not in src, f


def kvdesc(N=1000, d=64, sn=None, sh=None, sb=None, reserved=0):
    sn = d if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = 2 * sh if sb is None else sb
    return fa.FaKvDesc(N, reserved, sb, sh, sn)


@needs_lib
def test_splitkv_validation_and_workspace_size():
    lib = fa.load_library()
    q = desc(B=1, H=2, N=3, d=64, dtype=1)
    kv = kvdesc(N=1000, d=64)
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731

    def need(kvd, splits, qd=q):
        return lib.fa_fwd_splitkv_workspace_bytes(
            ctypes.byref(qd), None if kvd is None else ctypes.byref(kvd),
            splits)
    # 1000 keys in 4 runs of ceil(250/64)*64 = 256 keys: 4 runs used.
    rows = 1 * 2 * 3
    assert need(kv, 4) == r256(rows * 4 * 64 * 4) + r256(rows * 4 * 4)
    # 16 requested runs of 64 keys: 16 used; 1000 requested: 16 used.
    assert need(kv, 16) == r256(rows * 16 * 64 * 4) + r256(rows * 16 * 4)
    assert need(kv, 1000) == need(kv, 16)
    assert need(kv, 0) == 0 and need(kv, 1025) == 0 and need(None, 4) == 0
    assert need(kv, 4, desc(B=1, H=2, N=3, d=64, dtype=0)) == 0  # fp32

    def call(qd=q, kvd=kv, splits=4, causal=0, ws=FAKE, ws_bytes=1 << 40,
             qp=FAKE):
        return lib.fa_fwd_splitkv(
            ctypes.byref(qd), None if kvd is None else ctypes.byref(kvd),
            p(qp), p(), p(), 0.125, causal, splits, p(), p(),
            None if ws is None else p(ws), ws_bytes, None)
    assert call(kvd=None) == NULL
    assert call(qp=0) == NULL
    assert call(qd=desc(B=1, H=2, N=3, d=64, dtype=0)) == UNSUP
    assert call(kvd=kvdesc(N=0)) == SHAPE
    assert call(kvd=kvdesc(reserved=1)) == SHAPE
    assert call(splits=0) == SHAPE
    assert call(splits=1025) == SHAPE
    assert call(kvd=kvdesc(N=2), causal=1) == SHAPE   # fewer keys than queries
    assert call(kvd=kvdesc(sn=60)) == SHAPE            # sn < d
    assert call(kvd=kvdesc(sn=68)) == ALIGN            # 136-byte rows
    assert call(ws=None) == WS
    assert call(ws_bytes=need(kv, 4) - 1) == WS
    assert call(ws=FAKE + 4, ws_bytes=need(kv, 4)) == ALIGN
    # an empty query batch is a no-op whatever the rest says
    assert call(qd=desc(B=0, H=2, N=3, d=64), kvd=None) == OK


def vdesc(num_seqs=3, H=2, d=64, dtype=1, total=100, max_seqlen=60,
          cu=FAKE, sh=None, sn=None, reserved=0):
    sh = d if sh is None else sh
    sn = H * d if sn is None else sn
    return fa.FaVarlenDesc(num_seqs, H, d, dtype, total, max_seqlen, reserved,
                           0, cu, sh, sn)


@needs_lib
def test_varlen_validation_and_workspace_size():
    lib = fa.load_library()
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    d = vdesc()
    assert (lib.fa_bwd_varlen_workspace_bytes(ctypes.byref(d))
            == r256(2 * 2 * 100 * 4))            # D, L * log2(e): [H, total]
    assert lib.fa_bwd_varlen_workspace_bytes(None) == 0

    def fwdv(dd, q=FAKE, scale=0.125):
        return lib.fa_fwd_varlen(None if dd is None else ctypes.byref(dd),
                                 p(q), p(), p(), scale, 0, p(), p(), None)
    assert fwdv(None) == NULL
    assert fwdv(vdesc(cu=0)) == NULL
    assert fwdv(vdesc(cu=FAKE + 2)) == ALIGN
    assert fwdv(vdesc(dtype=0)) == UNSUP
    assert fwdv(vdesc(d=96)) == UNSUP
    assert fwdv(vdesc(num_seqs=-1)) == SHAPE
    assert fwdv(vdesc(reserved=5)) == SHAPE
    assert fwdv(vdesc(sn=32)) == SHAPE                  # sn < d
    assert fwdv(vdesc(sh=68, sn=256)) == ALIGN          # 136-byte head stride
    assert fwdv(vdesc(sh=0)) == SHAPE                   # heads broadcast
    assert fwdv(vdesc(sh=64, sn=64)) == SHAPE           # rows alias heads
    assert fwdv(vdesc(H=1, sh=0), q=0) == NULL          # one head: fine
    assert fwdv(d, q=0) == NULL
    assert fwdv(d, q=FAKE + 8) == ALIGN
    assert fwdv(d, scale=0.0) == UNSUP
    for empty in (vdesc(num_seqs=0), vdesc(total=0), vdesc(max_seqlen=0),
                  vdesc(H=0)):
        assert fwdv(empty, q=0) == OK                   # nothing inspected
    need = lib.fa_bwd_varlen_workspace_bytes(ctypes.byref(d))

    def bwdv(ws, ws_bytes):
        return lib.fa_bwd_varlen(ctypes.byref(d), *[p()] * 6, 0.125, 0, p(),
                                 p(), p(), None if ws is None else p(ws),
                                 ws_bytes, None)
    assert bwdv(None, need) == WS
    assert bwdv(FAKE, need - 1) == WS
    assert bwdv(FAKE + 4, need) == ALIGN


@needs_lib
def test_varlen_overlap_check_against_brute_force():
    """Packed [total, H, d] layouts: the check never accepts one whose
    (row, head) ranges overlap, and accepts both dense orders."""
    import random
    lib = fa.load_library()
    rng = random.Random(11)
    d = 64

    def call(total, H, sh, sn):
        dd = vdesc(num_seqs=1, H=H, d=d, total=total, max_seqlen=total,
                   sh=sh, sn=sn)
        return lib.fa_fwd_varlen(ctypes.byref(dd), p(0), p(), p(), 0.125, 0,
                                 p(), p(), None)
    accepted = overlapping = 0
    for _ in range(300):
        total, H = rng.randint(1, 6), rng.randint(1, 5)
        sh = rng.choice([0, 8, 64, 72, 128, 64 * total, 72 * total])
        sn = rng.choice([64, 72, 128, 64 * H, 72 * H, 256])
        starts = sorted(r * sn + h * sh for r in range(total) for h in range(H))
        disjoint = all(y - x >= d for x, y in zip(starts, starts[1:]))
        got = call(total, H, sh, sn)
        assert got in (NULL, SHAPE), got
        assert disjoint or got == SHAPE, (total, H, sh, sn)
        accepted += got == NULL
        overlapping += not disjoint
    assert accepted > 30 and overlapping > 30
    for total in (1, 3, 5):
        for H in (1, 2, 4):
            assert call(total, H, d, H * d) == NULL       # heads inside rows
            assert call(total, H, total * d, d) == NULL   # rows inside heads


@needs_lib
def test_dropout_and_padding_options_validation():
    """fa_fwd_ex / fa_bwd_ex refuse bad options before any HIP call; valid
    options reach the pointer checks (q = NULL here)."""
    lib = fa.load_library()

    def opts(p_=0.1, reserved=0, kv=None):
        return fa.FaOpts(p_, reserved, 1, kv)

    def fwd_ex(o, dsc=None, q=0):
        dsc = desc() if dsc is None else dsc
        return lib.fa_fwd_ex(ctypes.byref(dsc), p(q), p(), p(), 0.125, 0,
                             ctypes.byref(o), p(), p(), None)

    def bwd_ex(o, q=0):
        dsc = desc()
        return lib.fa_bwd_ex(ctypes.byref(dsc), p(q), p(), p(), p(), p(),
                             p(), 0.125, 0, ctypes.byref(o), p(), p(), p(),
                             p(), 1 << 40, None)
    for f in (fwd_ex, bwd_ex):
        assert f(opts(-0.1)) == UNSUP
        assert f(opts(1.0)) == UNSUP
        assert f(opts(float("nan"))) == UNSUP
        assert f(opts(0.999)) == UNSUP        # rounds to 256/256: nothing kept
        assert f(opts(reserved=3)) == SHAPE
        assert f(opts(kv=FAKE + 2)) == ALIGN  # kv_lens not 4-byte aligned
        assert f(opts(0.0)) == NULL           # valid: reaches the pointers
        assert f(opts(0.99)) == NULL          # 253/256 dropped, still valid
        assert f(opts(0.5, kv=FAKE)) == NULL
    # dropout and key padding run on bf16 tensors only
    assert fwd_ex(opts(0.1), dsc=desc(dtype=0)) == UNSUP
    assert fwd_ex(opts(0.0, kv=FAKE), dsc=desc(dtype=0)) == UNSUP
    assert fwd_ex(opts(0.0), dsc=desc(dtype=0)) == NULL  # no option in use


@needs_lib
def test_fp8_layout_and_validation():
    lib = fa.load_library()
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    dd = desc(B=2, H=3, N=100, d=128, dtype=1)
    lay = fa.FaFp8Layout()
    assert lib.fa_fp8_workspace_layout(ctypes.byref(dd), ctypes.byref(lay)) == OK
    codes, scales = r256(6 * 128 * 128), r256(6 * 2 * 4)   # rows = 128
    assert lay.rows == 128
    assert (lay.q_codes, lay.k_codes, lay.v_codes) == (0, codes, 2 * codes)
    assert (lay.q_scales, lay.k_scales, lay.v_scales) == (
        3 * codes, 3 * codes + scales, 3 * codes + 2 * scales)
    assert lay.bytes == 3 * codes + 3 * scales
    assert lib.fa_fp8_workspace_layout(ctypes.byref(dd), None) == NULL
    fp32 = desc(B=2, H=3, N=100, d=128, dtype=0)
    assert lib.fa_fp8_workspace_layout(ctypes.byref(fp32),
                                       ctypes.byref(lay)) == UNSUP
    assert lay.bytes == 0
    empty = desc(B=0, H=3, N=100, d=128)
    assert lib.fa_fp8_workspace_layout(ctypes.byref(empty),
                                       ctypes.byref(lay)) == OK
    assert lay.bytes == 0
    need = 3 * codes + 3 * scales

    good = (ctypes.c_int8 * 128)(*([1, -1] * 64))
    bad = (ctypes.c_int8 * 128)(*([1, -1] * 63 + [1, 0]))

    def quant(dsc=dd, q=FAKE, signs=None, rotate=1, ws=FAKE, ws_bytes=need):
        return lib.fa_fp8_quantize(ctypes.byref(dsc), p(q), p(), p(), signs,
                                   rotate, None if ws is None else p(ws),
                                   ws_bytes, None)
    assert quant(q=0) == NULL
    assert quant(dsc=fp32) == UNSUP
    assert quant(dsc=desc(B=2, H=3, N=100, d=96)) == UNSUP
    assert quant(q=FAKE + 8) == ALIGN
    assert quant(ws=None) == WS
    assert quant(ws_bytes=need - 1) == WS
    assert quant(ws=FAKE + 4) == ALIGN
    assert quant(signs=bad) == UNSUP          # a sign that is not +-1
    assert quant(dsc=empty, q=0) == OK        # empty: nothing inspected

    def fwd8(dsc=dd, o=FAKE, lse=FAKE, scale=0.125, ws=FAKE, ws_bytes=need):
        return lib.fa_fwd_fp8_quantized(ctypes.byref(dsc),
                                        None if ws is None else p(ws),
                                        ws_bytes, scale, 1, 1, p(o), p(lse),
                                        None)
    assert fwd8(o=0) == NULL
    assert fwd8(scale=0.0) == UNSUP
    assert fwd8(scale=float("nan")) == UNSUP
    assert fwd8(lse=FAKE + 2) == ALIGN
    assert fwd8(ws_bytes=need - 1) == WS
    assert fwd8(dsc=fp32) == UNSUP

    def fused(signs=good, scale=0.125, o=FAKE, ws_bytes=need):
        return lib.fa_fwd_fp8(ctypes.byref(dd), p(), p(), p(), scale, 1,
                              signs, 1, p(o), p(), p(), ws_bytes, None)
    # Validation of both steps precedes the first launch.
    assert fused(signs=bad) == UNSUP
    assert fused(scale=-1.0) == UNSUP
    assert fused(o=0) == NULL
    assert fused(ws_bytes=need - 1) == WS


PROBE_HEADER = os.path.join(ROOT, "include", "fa355_probe.h")


def test_probe_library_exports_its_header():
    from io_aware_exact_04_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        pytest.skip("libfa355_probe.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fa355_[a-z_0-9]+)\s*\(", text)))
    assert names == ["fa355_atomic_probe", "fa355_coexec_probe",
                     "fa355_mfma_probe"]
    lib = ctypes.CDLL(B.PROBE_LIB)
    for n in names:
        assert hasattr(lib, n)
    for n, modes in (("fa355_mfma_probe", 2), ("fa355_coexec_probe", 23)):
        f = getattr(lib, n)
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        # Argument errors return 1 before any launch.
        assert f(modes, 10, 10, FAKE, FAKE, None) == 1
        assert f(-1, 10, 10, FAKE, FAKE, None) == 1
        assert f(0, 0, 10, FAKE, FAKE, None) == 1
        assert f(0, 10, 0, FAKE, FAKE, None) == 1
        assert f(0, 10, 10, None, FAKE, None) == 1
        assert f(0, 10, 10, FAKE, None, None) == 1
    f = lib.fa355_atomic_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert f(0, 256, 64, 1, FAKE, None) == 1
    assert f(1, 0, 64, 1, FAKE, None) == 1
    assert f(1, 256, 96, 1, FAKE, None) == 1
    assert f(1, 256, 64, 1, None, None) == 1


@pytest.mark.parametrize("header", ["fa355.h", "fa355_probe.h"])
@pytest.mark.parametrize("lang", [("gcc", "c", "-std=c99"),
                                  ("g++", "c++", "-std=c++11")])
def test_header_compiles_standalone(tmp_path, header, lang):
    """The public headers are plain C (usable from C and C++ callers)."""
    import shutil
    import subprocess
    cc, xlang, std = lang
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} not available")
    src = tmp_path / "use.c"
    src.write_text(f'#include "{header}"\nint main(void) {{ return 0; }}\n')
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-fsyntax-only", "-x", xlang,
                        f"-I{os.path.join(ROOT, 'include')}", str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_outputs_keep_the_strides_of_q():
    # The kernels write every output with the descriptor's strides, which
    # are q's: an output allocated for a packed-QKV slice (a non-dense q)
    # must have q's strides and a storage that spans them.
    import torch
    qkv = torch.zeros(10, 3, 4, 64, dtype=torch.bfloat16)
    q = qkv[:, 1]
    assert not q.is_contiguous()
    o = fa._empty_as(q)
    assert o.shape == q.shape and o.stride() == q.stride()
    span = 1 + sum((n - 1) * s for n, s in zip(q.shape, q.stride()))
    assert o.untyped_storage().nbytes() >= span * q.element_size()
    q4 = torch.zeros(2, 5, 3, 128, dtype=torch.float32).permute(0, 2, 1, 3)
    o4 = fa._empty_as(q4)
    assert o4.stride() == q4.stride()


@needs_lib
def test_noalloc_backward_validation():
    # Every case fails validation before any HIP call.
    lib = fa.load_library()
    assert lib.fa_bwd_noalloc_max_rows() == 1 << 22

    def call(dsc, q=FAKE, dq=FAKE, scale=0.125):
        return lib.fa_bwd_noalloc(ctypes.byref(dsc), p(q), p(), p(), p(),
                                  p(), p(), scale, 0, None, 128, p(dq), p(),
                                  p(), None)
    assert call(desc(d=96)) == UNSUP
    assert call(desc(), q=0) == NULL
    assert call(desc(), dq=FAKE + 8) == ALIGN
    assert call(desc(), scale=-1.0) == UNSUP
    # One row beyond the scratch: rejected with a clear message.
    big = desc(B=1, H=1, N=(1 << 22) + 1, d=64)
    assert call(big) == WS
    assert b"scratch" in lib.fa_last_error()
    assert lib.fa_bwd_noalloc(ctypes.byref(desc(B=0)), None, None, None, None,
                              None, None, 0.1, 0, None, 0, None, None, None,
                              None) == OK
