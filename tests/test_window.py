"""GPU parity of the sliding-window (banded causal) mask: query i sees keys i-W+1 .. i,
the simplest of the block-sparse mask patterns of "深度学习反向传播优化：2-CTA MMA模式与内存访问优化"
sections 5.1 and 5.2, against the fp64 oracle with the same mask.

Windows are chosen to cross tile edges in every way: narrower than one 64-key tile,
not a multiple of the tile, equal to a tile, wider than the sequence (= causal), and
W = 1 (each query sees only its own key).
"""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from tests.gpu_cases import F16_ATOL, F16_RTOL, compare, gpu_inputs, sample_heads, say

pytestmark = pytest.mark.gpu

HEADDIMS = [(64, 64), (128, 128), (192, 128)]


def _run(w, gpu, det, window):
    o, lse = attn.fwd(gpu["q"], gpu["k"], gpu["v"], True, w.scale, window=window)
    dq, dk, dv = attn.bwd(gpu["q"], gpu["k"], gpu["v"], o, lse, gpu["do"], True, w.scale, det, window=window)
    torch.cuda.synchronize()
    return {"o": o.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu(), "lse": lse.cpu()}


def _oracle(w, cpu, window, heads=None):
    from oracle import attn_ref
    if heads is None:
        return attn_ref.attn_ref_bwd(cpu["q"], cpu["k"], cpu["v"], cpu["do"], True, w.scale, window=window)
    return attn_ref.attn_ref_heads(cpu["q"], cpu["k"], cpu["v"], cpu["do"], True, w.scale, heads=heads,
                                   window=window)


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("window", [1, 37, 64, 100, 257, 1000])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_window_small(dims, window, deterministic):
    w = workloads.Workload(f"win{window}_d{dims[0]}x{dims[1]}", 2, 2, 555, dims[0], dims[1], True, 900 + window,
                           window=window)
    say(f"case window {w.name} det={deterministic}")
    cpu, gpu = gpu_inputs(w)
    compare(w, _run(w, gpu, deterministic, window), _oracle(w, cpu, window))


def test_window_fp16_and_large_scores():
    w = workloads.Workload("win_f16", 1, 2, 700, 128, 128, True, 931, window=150)
    say(f"case window fp16 {w.name}")
    cpu, gpu = gpu_inputs(w, dtype=torch.float16)
    compare(w, _run(w, gpu, True, 150), _oracle(w, cpu, 150), tol=(F16_RTOL, F16_ATOL))
    w = workloads.Workload("win_sigma4", 1, 2, 700, 128, 128, True, 937, sigma=4.0, window=90)
    say(f"case window sigma 4 {w.name}")
    cpu, gpu = gpu_inputs(w)
    compare(w, _run(w, gpu, False, 90), _oracle(w, cpu, 90))


def test_window_deterministic_bit_stable():
    w = workloads.Workload("win_det", 2, 2, 900, 128, 128, True, 941, window=200)
    say(f"case window determinism {w.name}")
    _, gpu = gpu_inputs(w)
    first = _run(w, gpu, True, 200)
    for _ in range(3):
        again = _run(w, gpu, True, 200)
        for n in first:
            assert torch.equal(first[n], again[n]), n


def test_window_full_size_sampled():
    """The headline shape under a 1024-key window (the `window` workload of the bench),
    in the bench's launch configuration, sampled heads against the oracle."""
    w = workloads.WORKLOADS["window"]
    heads = sample_heads(w, 2)
    say(f"case window full size heads={heads}")
    cpu, gpu = gpu_inputs(w)
    got = _run(w, gpu, True, w.window)
    del gpu
    compare(w, got, _oracle(w, cpu, w.window, heads=heads), heads=heads)
