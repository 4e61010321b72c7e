"""GPU parity of the ALiBi bias (the use_alibi_mask option among the SDPA options of
"ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" section 1.2): the scaled scores of head h
get -m_h (i - j), m_h = 2^(-8 (h + 1) / NH), under the causal mask; against the fp64
oracle with the same bias.
"""
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import F16_ATOL, F16_RTOL, compare, gpu_inputs, sample_heads, say

pytestmark = pytest.mark.gpu

HEADDIMS = [(64, 64), (128, 128), (192, 128)]


def _run(w, gpu, det):
    o, lse = attn.fwd(gpu["q"], gpu["k"], gpu["v"], True, w.scale, alibi=True)
    dq, dk, dv = attn.bwd(gpu["q"], gpu["k"], gpu["v"], o, lse, gpu["do"], True, w.scale, det, alibi=True)
    torch.cuda.synchronize()
    return {"o": o.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu(), "lse": lse.cpu()}


def _oracle(w, cpu, heads=None):
    if heads is None:
        return attn_ref.attn_ref_bwd(cpu["q"], cpu["k"], cpu["v"], cpu["do"], True, w.scale, alibi=True)
    return attn_ref.attn_ref_heads(cpu["q"], cpu["k"], cpu["v"], cpu["do"], True, w.scale, heads=heads,
                                   alibi=True)


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("T", [1, 129, 555])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_alibi_small(dims, T, deterministic):
    # 8 heads: slopes 1/2 .. 1/256, from sharply local to nearly flat
    w = workloads.Workload(f"alibi_T{T}_d{dims[0]}x{dims[1]}", 1, 8, T, dims[0], dims[1], True, 1000 + T, alibi=True)
    say(f"case alibi {w.name} det={deterministic}")
    cpu, gpu = gpu_inputs(w)
    compare(w, _run(w, gpu, deterministic), _oracle(w, cpu))


def test_alibi_fp16():
    w = workloads.Workload("alibi_f16", 1, 4, 700, 128, 128, True, 1061, alibi=True)
    say(f"case alibi fp16 {w.name}")
    cpu, gpu = gpu_inputs(w, dtype=torch.float16)
    compare(w, _run(w, gpu, True), _oracle(w, cpu), tol=(F16_RTOL, F16_ATOL))


def test_alibi_deterministic_bit_stable():
    w = workloads.Workload("alibi_det", 2, 4, 600, 128, 128, True, 1063, alibi=True)
    say(f"case alibi determinism {w.name}")
    _, gpu = gpu_inputs(w)
    first = _run(w, gpu, True)
    for _ in range(3):
        again = _run(w, gpu, True)
        for n in first:
            assert torch.equal(first[n], again[n]), n


def test_alibi_full_size_sampled():
    """The headline shape with the bias (the `alibi` workload of the bench), in the bench's
    launch configuration; sampled heads, among them head 0 (the steepest slope) and the
    last head (the flattest), against the oracle."""
    w = workloads.WORKLOADS["alibi"]
    heads = sample_heads(w, 2)
    say(f"case alibi full size heads={heads}")
    cpu, gpu = gpu_inputs(w)
    got = _run(w, gpu, True)
    del gpu
    compare(w, got, _oracle(w, cpu, heads=heads), heads=heads)
