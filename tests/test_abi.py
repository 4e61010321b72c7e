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


def bwd(lib, ws=GOOD + 0x900000, ws_bytes=1 << 30, lse=GOOD + 0x400000, stages=7, det=0, dq=GOOD + 0x600000,
        dqk=64, dv=64, T=64, causal=1, scale=0.125):
    st = strides(T, 2, dqk)
    sv = strides(T, 2, dv)
    return lib.attn_bwd_staged(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv, lse,
                               GOOD + 0x500000, sv, dq, st, GOOD + 0x700000, st, GOOD + 0x800000, sv,
                               1, 2, T, dqk, dv, scale, causal, det, ws, ws_bytes, None, stages)


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


def bwd(lib, ws=GOOD + 0x900000, ws_bytes=1 << 30, lse=GOOD + 0x400000, stages=7, det=0, dq=GOOD + 0x600000,
        dqk=64, dv=64, T=64, causal=1, scale=0.125):
    st = strides(T, 2, dqk)
    sv = strides(T, 2, dv)
    return lib.attn_bwd_staged(GOOD, st, GOOD + 0x100000, st, GOOD + 0x200000, sv, GOOD + 0x300000, sv, lse,
                               GOOD + 0x500000, sv, dq, st, GOOD + 0x700000, st, GOOD + 0x800000, sv,
                               1, 2, T, dqk, dv, scale, causal, det, ws, ws_bytes, None, stages)


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
