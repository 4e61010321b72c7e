"""The C ABI on the CPU: the library loads, exports every function that
include/attn53.h declares, and rejects invalid arguments before launching anything.

No call here reaches a kernel launch: every argument set is invalid, and validation
returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

import exact_attention_53_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn53.h")

OK, NULL, SHAPE, HEADDIM, STRIDE, ALIGN, WORKSPACE, HIP, ARG, ALIAS = range(10)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.lib_path):
        pytest.fail("libattn53.so is not built: run __graft_entry__.build()")
    return attn.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_bwd_staged", "attn_bwd_workspace_bytes",
            "attn_status_string", "attn_version"} <= set(names)
    raw = ctypes.CDLL(attn.lib_path)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in attn53.h but not exported"


def test_status_strings(lib):
    for s in range(10):
        txt = lib.attn_status_string(s).decode()
        assert txt and txt != "unknown attn_status"
    assert lib.attn_status_string(99).decode() == "unknown attn_status"
    assert lib.attn_version() >= 100


S = attn.Strides
GOOD = 0x10000  # a 16-byte aligned fake device address, never dereferenced


def strides(T=64, NH=2, d=64):
    return S(T * NH * d, d, NH * d)


def fwd(lib, q=GOOD, k=GOOD + 0x100000, v=GOOD + 0x200000, o=GOOD + 0x300000, lse=None,
        B=1, NH=2, T=64, dqk=64, dv=64, scale=0.125, causal=1, sq=None, so=None):
    st = sq or strides(T, NH, dqk)
    return lib.attn_fwd(q, st, k, st, v, strides(T, NH, dv), o, so or strides(T, NH, dv), lse,
                        B, NH, T, dqk, dv, scale, causal, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, B=0) == SHAPE
    assert fwd(lib, T=0) == SHAPE
    assert fwd(lib, NH=-1) == SHAPE
    assert fwd(lib, B=1 << 16, NH=1 << 16, T=4) == SHAPE
    assert fwd(lib, dqk=96, dv=96) == HEADDIM
    assert fwd(lib, dqk=128, dv=64) == HEADDIM
    assert fwd(lib, q=GOOD + 8) == ALIGN
    assert fwd(lib, sq=S(64 * 2 * 64, 64, 2 * 64 + 4)) == STRIDE
    assert fwd(lib, sq=S(-8, 64, 128)) == STRIDE
    assert fwd(lib, sq=S(8, 8, (1 << 24) + 8)) == STRIDE
    assert fwd(lib, scale=float("nan")) == ARG
    assert fwd(lib, scale=float("inf")) == ARG
    assert fwd(lib, scale=0.0) == ARG
    assert fwd(lib, scale=-0.125) == ARG
    assert fwd(lib, causal=2) == ARG
    assert fwd(lib, o=GOOD) == ALIAS               # output overlaps q
    assert fwd(lib, lse=GOOD + 0x300002) == ALIGN   # lse must be 4-byte aligned
    assert fwd(lib, lse=GOOD + 0x200000) == ALIAS   # lse overlaps v


def test_output_rows_must_not_share_elements(lib):
    """An output whose (b, h, t) rows would share elements is rejected (concurrent
    workgroups would write the same bytes); packed outputs pass this rule."""
    T, NH, d = 64, 2, 64
    assert fwd(lib, so=S(T * NH * d, d, 0)) == STRIDE          # every t on one row
    assert fwd(lib, so=S(T * NH * d, 0, NH * d)) == STRIDE     # both heads on one row
    assert fwd(lib, so=S(T * NH * d, d, 8)) == STRIDE          # rows 8 elements apart, d = 64
    assert fwd(lib, so=S(T * NH * d, 32, NH * d)) == STRIDE    # heads 32 apart, d = 64
    assert fwd(lib, B=2, so=S(0, d, NH * d)) == STRIDE         # both batches on one block
    # the same strides with a size-1 dimension are fine (any stride is unused there):
    # validation then goes on and stops at the misaligned lse
    assert fwd(lib, T=1, so=S(NH * d, d, 0), lse=GOOD + 0x300002) == ALIGN
    # a packed (B, T, 3, NH, HS) output slice: strides {T*3*C, HS, 3*C}, C = NH*HS
    C = NH * d
    assert fwd(lib, so=S(T * 3 * C, d, 3 * C), o=GOOD + 0x300000, lse=GOOD + 0x300002 + T * 3 * C * 2) == ALIGN
    assert bwd(lib, sdq=S(T * NH * d, d, 0)) == STRIDE
    assert bwd(lib, sdk=S(T * NH * d, 0, NH * d)) == STRIDE
    assert bwd(lib, sdv=S(T * NH * d, d, 16)) == STRIDE
    assert bwd(lib, sdq=S(T * 3 * C, d, 3 * C), lse=None) == NULL  # packed dQ passes the rule


def bwd(lib, ws=GOOD + 0x900000, ws_bytes=1 << 30, lse=GOOD + 0x400000, stages=7, det=0, dq=GOOD + 0x600000,
        dqk=64, dv=64, T=64, causal=1, scale=0.125, sdq=None, sdk=None, sdv=None):
    st = strides(T, 2, dqk)
    sv = strides(T, 2, dv)
    return lib.attn_bwd_staged(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv, lse,
                               GOOD + 0x500000, sv, dq, sdq or st, GOOD + 0x700000, sdk or st, GOOD + 0x800000,
                               sdv or sv, 1, 2, T, dqk, dv, scale, causal, det, ws, ws_bytes, None, stages)


def test_bwd_validation(lib):
    assert bwd(lib, lse=None) == NULL
    assert bwd(lib, dq=None) == NULL
    assert bwd(lib, ws=None) == WORKSPACE
    assert bwd(lib, ws_bytes=16) == WORKSPACE
    assert bwd(lib, ws=GOOD + 0x900004) == WORKSPACE
    assert bwd(lib, stages=0) == ARG
    assert bwd(lib, stages=8) == ARG
    assert bwd(lib, det=3) == ARG
    assert bwd(lib, dqk=192, dv=192) == HEADDIM
    assert bwd(lib, dq=GOOD) == ALIAS          # dq overlaps q
    assert bwd(lib, ws=GOOD + 0x100000) == ALIAS  # workspace overlaps k
    assert bwd(lib, scale=float("nan")) == ARG
    assert bwd(lib, scale=-1.0) == ARG


def test_workspace_bytes(lib):
    f = lib.attn_bwd_workspace_bytes
    # D and LSE log2(e): 2 x B*NH*Tpad fp32; atomic mode adds B*NH*Tpad*d_qk fp32
    # (Tpad = T rounded up to 128)
    assert f(1, 2, 64, 64, 64, 1) == 2 * 1024
    assert f(1, 2, 64, 64, 64, 0) == 2 * 1024 + 2 * 128 * 64 * 4
    assert f(4, 16, 8192, 128, 128, 0) == 2 * 4 * 16 * 8192 * 4 + 4 * 16 * 8192 * 128 * 4
    assert f(0, 1, 1, 64, 64, 0) == 0
    assert f(1, 2, 64, 64, 64, 2) == 0   # the mode flag is 0 or 1
    assert f(1, 1, 1, 64, 32, 0) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.fwd(x, x, x)


def test_typed_validation(lib):
    """attn_fwd_typed / attn_bwd_typed: an unknown element type is rejected on the host;
    known types reach the same validation as the bf16 entry points."""
    st, sv = strides(64, 2, 64), strides(64, 2, 64)

    def tfwd(dtype, q=GOOD, o=GOOD + 0x300000, lq=None, lk=None, causal=1, window=0, alibi=0):
        return lib.attn_fwd_typed(dtype, q, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, o, sv, None, lq, lk,
                                  1, 2, 64, 64, 64, 0.125, causal, window, alibi, GOOD + 0xb00000, 1 << 20, None)

    def tbwd(dtype, dq=GOOD + 0x600000, stages=7, causal=1, window=0, lq=None, lk=None, alibi=0):
        return lib.attn_bwd_typed(dtype, GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv,
                                  GOOD + 0x400000, GOOD + 0x500000, sv, dq, st, GOOD + 0x700000, st,
                                  GOOD + 0x800000, sv, lq, lk, 1, 2, 64, 64, 64, 0.125, causal, window, alibi, 0,
                                  GOOD + 0x900000, 1 << 30, None, stages)

    for bad in (2, -1, 99):
        assert tfwd(bad) == ARG
        assert tbwd(bad) == ARG
    for dt in (0, 1):
        assert tfwd(dt, q=None) == NULL
        assert tfwd(dt, o=GOOD) == ALIAS
        assert tfwd(dt, lq=GOOD + 0xa00000) == NULL   # one length pointer without the other
        assert tbwd(dt, dq=None) == NULL
        assert tbwd(dt, stages=0) == ARG
        # sliding window: causal only, dense only, never negative
        for f in (tfwd, tbwd):
            assert f(dt, window=-1) == ARG
            assert f(dt, causal=0, window=16) == ARG
            assert f(dt, window=16, lq=GOOD + 0xa00000, lk=GOOD + 0xa00100) == ARG
            # ALiBi: a 0/1 flag, causal only, dense only, not with a window
            assert f(dt, alibi=2) == ARG
            assert f(dt, causal=0, alibi=1) == ARG
            assert f(dt, alibi=1, window=16) == ARG
            assert f(dt, alibi=1, lq=GOOD + 0xa00000, lk=GOOD + 0xa00100) == ARG


def test_decode_validation(lib):
    """attn_fwd_decode: separate query and key row counts, validated on the host."""
    sq, sk = strides(4, 2, 64), strides(64, 2, 64)

    def dec(dtype=0, q=GOOD, o=GOOD + 0x300000, Tq=4, Tk=64, lens=None, scale=0.125):
        return lib.attn_fwd_decode(dtype, q, sq, GOOD + 0x100000, sk, GOOD + 0x200000, sk, o, sq, None, lens,
                                   1, 2, Tq, Tk, 64, 64, scale, None, 0, None)

    assert dec(dtype=5) == ARG
    assert dec(q=None) == NULL
    assert dec(Tq=0) == SHAPE
    assert dec(Tk=0) == SHAPE
    assert dec(scale=0.0) == ARG
    assert dec(o=GOOD + 0x100000) == ALIAS       # output overlaps k
    assert dec(lens=GOOD + 0xa00002) == ALIGN    # lengths must be 4-byte aligned


def test_decode_workspace(lib):
    """Key split of a decode step: none with at least 512 workgroups or a short cache;
    otherwise n chunks of >= 1024 keys, each holding an fp32 partial O and LSE per query
    row and head."""
    f = lib.attn_fwd_decode_workspace_bytes
    assert f(64, 16, 1, 8192, 128, 128) == 0           # 1024 workgroups: no split
    assert f(4, 16, 1, 500, 128, 128) == 0             # a cache shorter than one chunk
    assert f(16, 16, 1, 8192, 128, 128) == 2 * 16 * 16 * 1 * 129 * 4   # 2 chunks of 4096
    assert f(1, 16, 1, 32768, 128, 128) == 32 * 16 * 1 * 129 * 4       # 32 chunks of 1024
    assert f(0, 16, 1, 8192, 128, 128) == 0


def test_binding_checks_every_shape_against_q():
    """The binding derives B, NH, T and d from q; every other tensor must match, or the
    kernels would read or write past it.  Checked before anything reaches the device
    (CPU tensors here, so the shape error has to come first)."""
    import torch

    def t(B=2, T=32, NH=3, d=64):
        return torch.zeros(B, T, NH, d, dtype=torch.bfloat16)

    q = t()
    bad = {
        "fewer key rows": dict(k=t(T=31)),
        "narrower keys": dict(k=t(d=32)),
        "fewer value heads": dict(v=t(NH=2)),
        "fewer value batches": dict(v=t(B=1)),
        "3-D v": dict(v=torch.zeros(2, 32, 64, dtype=torch.bfloat16)),
    }
    for why, kw in bad.items():
        args = dict(k=t(), v=t()) | kw
        with pytest.raises(ValueError, match="must be a 4-D|has \\(B, NH, T, d\\)|expected a 4-D"):
            attn.fwd(q, args["k"], args["v"])
        with pytest.raises(ValueError, match="must be a 4-D|has \\(B, NH, T, d\\)|expected a 4-D"):
            attn.fwd_varlen(q, args["k"], args["v"], torch.zeros(2, dtype=torch.int32),
                            torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="out has"):
        attn.fwd(q, t(), t(), out=t(T=16))
    # backward: every input and every caller-supplied gradient
    ok = dict(k=t(), v=t(), o=t(), do=t())
    lse = torch.zeros(2, 3, 32)
    for name in ("k", "v", "o", "do"):
        args = dict(ok) | {name: t(T=8)}
        with pytest.raises(ValueError, match=f"{name} has"):
            attn.bwd(q, args["k"], args["v"], args["o"], lse, args["do"])
        with pytest.raises(ValueError, match=f"{name} has"):
            attn.bwd_varlen(q, args["k"], args["v"], args["o"], lse, args["do"],
                            torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32))
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError, match=f"{name} has"):
            attn.bwd(q, t(), t(), t(), lse, t(), **{name: t(d=128)})
    # the bhtd layout reads the dimensions in its own order
    qh = torch.zeros(2, 3, 32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k has"):
        attn.fwd(qh, t(), torch.zeros(2, 3, 32, 64, dtype=torch.bfloat16), layout="bhtd")
    # decode: k and v share one cache length; out has the query length
    with pytest.raises(ValueError, match="v has"):
        attn.fwd_decode(t(T=1), t(T=100), t(T=99))
    with pytest.raises(ValueError, match="k has"):
        attn.fwd_decode(t(T=1), t(T=100, d=32), t(T=100))
    with pytest.raises(ValueError, match="out has"):
        attn.fwd_decode(t(T=1), t(T=100), t(T=100), out=t(T=2))
    # shapes right, tensors on the CPU: the device error
    with pytest.raises(ValueError, match="GPU only"):
        attn.fwd(q, t(), t())


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """attn_bwd_noalloc runs on a fixed 64 MiB scratch per GPU: sizes that need more
    workspace are refused before anything is launched or touched."""
    assert lib.attn_bwd_noalloc_max_workspace_bytes() == 64 << 20
    z = S(0, 0, 0)
    args = [GOOD, z] * 4 + [GOOD, GOOD, z] + [GOOD, z] * 3
    # atomic mode at B 4, NH 16, T 8192, d 128 needs 272 MB
    assert lib.attn_bwd_noalloc(*args, 4, 16, 8192, 128, 128, 0.088, 1, 0, None) == WORKSPACE
    # deterministic mode, 2^24 padded rows: 128 MiB
    assert lib.attn_bwd_noalloc(*args, 16, 16, 65536, 128, 128, 0.088, 1, 1, None) == WORKSPACE


def test_blocksparse_validation(lib):
    """attn_fwd_blocksparse / attn_bwd_blocksparse: the map is validated on the host like
    every tensor; the workspace holds the per-item block lists and work lists."""
    st, sv = strides(64, 2, 64), strides(64, 2, 64)
    MAP = GOOD + 0xc00000

    def bfwd(m=MAP, msb=0, msh=0, o=GOOD + 0x300000, ws=GOOD + 0xb00000, ws_bytes=1 << 20):
        return lib.attn_fwd_blocksparse(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, o, sv, None, m, msb, msh,
                                        1, 2, 64, 64, 64, 0.125, 1, ws, ws_bytes, None)

    def bbwd(m=MAP, msb=0, msh=0, dq=GOOD + 0x600000, ws=GOOD + 0x900000, ws_bytes=1 << 20, stages=7):
        return lib.attn_bwd_blocksparse(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv,
                                        GOOD + 0x400000, GOOD + 0x500000, sv, dq, st, GOOD + 0x700000, st,
                                        GOOD + 0x800000, sv, m, msb, msh, 1, 2, 64, 64, 64, 0.125, 1, 1, ws,
                                        ws_bytes, None, stages)

    for f in (bfwd, bbwd):
        assert f(m=None) == NULL
        assert f(msh=-1) == STRIDE
        assert f(ws=None) == WORKSPACE
        assert f(ws_bytes=16) == WORKSPACE
    assert bfwd(o=MAP) == ALIAS            # the output overlaps the map
    assert bbwd(dq=MAP) == ALIAS
    assert bbwd(stages=0) == ARG
    # workspace: per item nb int32 indices, a count and a work-list entry (8 bytes), each
    # part 256-aligned; forward: one item per query block
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    nb = 64  # T = 8192
    items = 4 * 16 * nb
    fw = a256(items * nb * 4) + a256(items * 4) + a256(items * 8)
    assert lib.attn_fwd_blocksparse_workspace_bytes(4, 16, 8192, 128, 128) == fw
    # backward (d = 128: the dQ kernel owns 256 rows, so its items are pairs of query blocks)
    items_dq = 4 * 16 * nb // 2
    dq_lists = a256(items_dq * nb * 4) + a256(items_dq * 4) + a256(items_dq * 8)
    assert lib.attn_bwd_blocksparse_workspace_bytes(4, 16, 8192, 128, 128, 1) == \
        lib.attn_bwd_workspace_bytes(4, 16, 8192, 128, 128, 1) + fw + dq_lists
    assert lib.attn_fwd_blocksparse_workspace_bytes(0, 16, 8192, 128, 128) == 0


def test_binding_blocksparse_map_checks():
    import torch
    q = torch.zeros(2, 300, 3, 64, dtype=torch.bfloat16)
    for m, why in ((torch.zeros(2, 3, 3, 3, dtype=torch.int32), "dtype"),
                   (torch.zeros(2, 3, 2, 3, dtype=torch.uint8), "shape"),
                   (torch.zeros(3, 3, 3, 3, dtype=torch.uint8), "shape"),
                   (torch.zeros(2, 3, 3, 6, dtype=torch.uint8)[..., ::2], "contiguous")):
        with pytest.raises(ValueError):  # wrong map: its dtype, shape or layout
            attn._block_map(m, 2, 3, 300, torch.device("cpu"))
    b, h = attn._block_map(torch.zeros(1, 3, 3, 3, dtype=torch.uint8), 2, 3, 300, torch.device("cpu"))
    assert (b, h) == (0, 9)


def test_keybias_validation(lib):
    st, sv = strides(64, 2, 64), strides(64, 2, 64)
    BIAS, DB = GOOD + 0xc00000, GOOD + 0xd00000

    def kfwd(bias=BIAS, sb=128, sh=64, o=GOOD + 0x300000, ws=GOOD + 0xb00000, ws_bytes=1 << 20):
        return lib.attn_fwd_keybias(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, o, sv, None, bias, sb, sh,
                                    1, 2, 64, 64, 64, 0.125, 1, ws, ws_bytes, None)

    def kbwd(bias=BIAS, dbias=DB, sb=128, sh=64, dq=GOOD + 0x600000, ws=GOOD + 0x900000, ws_bytes=1 << 20):
        return lib.attn_bwd_keybias(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv,
                                    GOOD + 0x400000, GOOD + 0x500000, sv, dq, st, GOOD + 0x700000, st,
                                    GOOD + 0x800000, sv, bias, dbias, sb, sh, 1, 2, 64, 64, 64, 0.125, 1, 1, ws,
                                    ws_bytes, None, 7)

    for f in (kfwd, kbwd):
        assert f(bias=None) == NULL
        assert f(bias=BIAS + 2) == ALIGN
        assert f(sh=-64) == STRIDE
        assert f(ws=None) == WORKSPACE
        assert f(ws_bytes=16) == WORKSPACE
    assert kfwd(o=BIAS) == ALIAS                 # output overlaps the bias
    assert kbwd(dbias=BIAS) == ALIAS             # dbias overlaps the bias
    assert kbwd(dbias=GOOD + 0x100000) == ALIAS  # dbias overlaps k
    assert kbwd(dbias=DB + 2) == ALIGN
    assert kbwd(sh=32) == STRIDE                 # two heads' dbias rows (64 keys) would share elements
    assert kbwd(dq=BIAS) == ALIAS
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert lib.attn_fwd_keybias_workspace_bytes(4, 16, 8192, 128, 128) == a256(4 * 16 * 8192 * 4)
    assert lib.attn_bwd_keybias_workspace_bytes(4, 16, 8192, 128, 128, 1) == \
        lib.attn_bwd_workspace_bytes(4, 16, 8192, 128, 128, 1) + 2 * a256(4 * 16 * 8192 * 4)


def test_fp8_validation(lib):
    s8 = S(64 * 2 * 64, 64, 2 * 64)          # (B, T, NH, d) e4m3, strides in bytes
    so = strides(64, 2, 64)                  # bf16 output

    def f8(q=GOOD, sq=s8, o=GOOD + 0x300000, dqk=64, dv=64, dsq=1.0, ws=GOOD + 0xb00000, ws_bytes=1 << 20,
           causal=1):
        return lib.attn_fwd_fp8(q, sq, GOOD + 0x100000, s8, GOOD + 0x200000, s8, o, so, None, dsq, 1.0, 1.0,
                                1, 2, 64, dqk, dv, 0.125, causal, ws, ws_bytes, None)

    assert f8(q=None) == NULL
    assert f8(q=GOOD + 8) == ALIGN
    assert f8(sq=S(64 * 2 * 64, 64, 2 * 64 + 8)) == STRIDE   # fp8 strides: multiples of 16 bytes
    assert f8(dqk=192, dv=128) == HEADDIM
    assert f8(dqk=128, dv=64) == HEADDIM
    assert f8(dsq=0.0) == ARG
    assert f8(dsq=float("nan")) == ARG
    assert f8(causal=3) == ARG
    assert f8(o=GOOD) == ALIAS
    assert f8(ws=None) == WORKSPACE
    assert f8(ws_bytes=100) == WORKSPACE
    assert f8(ws=GOOD + 0x100000) == ALIAS
    # workspace: the transposed V, d bytes x T rounded up to 64 per head
    assert lib.attn_fwd_fp8_workspace_bytes(4, 16, 8192, 128, 128) == 4 * 16 * 128 * 8192
    assert lib.attn_fwd_fp8_workspace_bytes(1, 2, 100, 64, 64) == (2 * 64 * 128 + 255) // 256 * 256
    assert lib.attn_fwd_fp8_workspace_bytes(1, 2, 100, 192, 128) == 0


def test_dropout_validation(lib):
    st, sv = strides(64, 2, 64), strides(64, 2, 64)
    MASK = GOOD + 0xc00000
    assert lib.attn_dropout_mask_bytes(1, 2, 64) == 2 * 2 * 128 * 16
    assert lib.attn_dropout_mask_bytes(4, 16, 8192) == 2 * 64 * 8192 * 1024
    assert lib.attn_dropout_mask_bytes(0, 2, 64) == 0

    def gen(p=0.1, mask=MASK, nbytes=1 << 20, causal=1, T=64):
        return lib.attn_dropout_mask(p, 1, 0, 1, 2, T, causal, mask, nbytes, None)

    assert gen(p=1.0) == ARG
    assert gen(p=-0.1) == ARG
    assert gen(p=float("nan")) == ARG
    assert gen(causal=2) == ARG
    assert gen(mask=None) == NULL
    assert gen(mask=MASK + 8) == ALIGN
    assert gen(nbytes=100) == WORKSPACE
    assert gen(T=0) == SHAPE

    def dfwd(mask=MASK, p=0.1, o=GOOD + 0x300000):
        return lib.attn_fwd_dropout(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, o, sv, None, mask, p,
                                    1, 2, 64, 64, 64, 0.125, 1, None)

    def dbwd(mask=MASK, p=0.1, dq=GOOD + 0x600000):
        return lib.attn_bwd_dropout(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv,
                                    GOOD + 0x400000, GOOD + 0x500000, sv, dq, st, GOOD + 0x700000, st,
                                    GOOD + 0x800000, sv, mask, p, 1, 2, 64, 64, 64, 0.125, 1, 1, GOOD + 0x900000,
                                    1 << 20, None, 7)

    for f in (dfwd, dbwd):
        assert f(mask=None) == NULL
        assert f(mask=MASK + 8) == ALIGN
        assert f(p=1.5) == ARG
    assert dfwd(o=MASK) == ALIAS
    assert dbwd(dq=MASK) == ALIAS
