"""The bench's command line on the CPU: more than one GPU is refused with a message (one
GPU's share is the measured unit), and the FLOP and byte conventions match the
per-configuration sizes."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flop_convention():
    # headline: 2.148e9 unmasked pairs; fwd 2 (d_qk + d_v), bwd 2 (3 d_qk + 2 d_v) flops per pair
    w = workloads.WORKLOADS["headline"]
    assert w.pairs() == 4 * 16 * 8192 * 8193 // 2
    f, b = bench.flops(w)
    assert f == 2 * 256 * w.pairs() and b == 2 * (3 * 128 + 2 * 128) * w.pairs()
    assert abs((f + b) / 1e12 - 3.849) < 1e-3
    # sliding window of 1024 keys: rows i < 1024 see i + 1 keys, the others 1024
    ww = workloads.WORKLOADS["window"]
    assert ww.pairs() == 4 * 16 * (1024 * 1025 // 2 + (8192 - 1024) * 1024)
    # non-causal: every pair
    assert workloads.WORKLOADS["mid_full"].pairs() == 16 * 16 * 2048 * 2048


def test_algorithmic_bytes():
    w = workloads.WORKLOADS["headline"]
    fwd, bwd = bench.alg_bytes(w)
    rows = 4 * 16 * 8192
    assert fwd == rows * (2 * (2 * 128 + 128) + 2 * 128 + 4)          # Q, K, V read; O, LSE written
    assert bwd == rows * (2 * (2 * 128 + 3 * 128) + 12 + 2 * (2 * 128 + 128))


def test_padded_batch_counts():
    """Padded batches: seeded lengths (the first full, the others in [T/8, T], the same on
    every call), and flops and bytes counted over each sequence's own rows only."""
    w = workloads.WORKLOADS["varlen"]
    n = workloads.varlen_lengths(w)
    assert list(n) == list(workloads.varlen_lengths(w)) and len(n) == w.B
    assert n[0] == w.T and all(w.T // 8 <= x <= w.T for x in n)
    pairs = 0
    for x in n:  # causal: a sequence of x rows has x (x + 1) / 2 pairs per head
        pairs += sum(range(1, int(x) + 1))
    assert bench.pairs_of(w) == w.NH * pairs
    f, b = bench.flops(w)
    assert f == 2 * 256 * w.NH * pairs and b == 2 * 640 * w.NH * pairs
    fwd, bwd = bench.alg_bytes(w)
    assert fwd == w.NH * int(sum(n)) * (2 * 384 + 256 + 4)


def test_sources_hash_ignores_comments_only():
    """The traffic figures are keyed to a hash of the kernels' code: comments and line
    layout do not change it, a change to the code does."""
    c = "__global__ void k(float* x) {  // one\n  x[0] = 1.f;  /* two\n three */\n}\n"
    assert bench._code_tokens(c, "c") == bench._code_tokens(
        "__global__ void k(float* x) {\n  // a longer\n  // comment\n  x[0] = 1.f;\n}\n", "c")
    assert bench._code_tokens(c, "c") != bench._code_tokens(c.replace("1.f", "2.f"), "c")
    py = "FLAGS = ['-O3']  # kept\n# a comment line\nX = 1\n"
    assert bench._code_tokens(py, "py") == bench._code_tokens("FLAGS = ['-O3']  # kept\nX = 1\n", "py")
    assert bench._code_tokens(py, "py") != bench._code_tokens(py.replace("-O3", "-O2"), "py")
    assert len(bench.kernel_sources_hash()) == 16
