"""GPU parity over a seeded random sweep of small problems: batch, heads and sequence length
(1 .. 1100, so every residue of the 64- and 128-row tiles can occur), head widths,
causal or not, the sliding window and ALiBi on causal cases, both dQ modes, bf16 or fp16,
token- or head-major layout, and the input scale.  Every element is compared with the
oracle; the cases are fixed by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import F16_ATOL, F16_RTOL, BF16_ATOL, BF16_RTOL, compare, gpu_inputs, say

pytestmark = pytest.mark.gpu

N_CASES = 40
HEADDIMS = [(64, 64), (128, 128), (192, 128)]


def _cases():
    rng = np.random.default_rng(53100)
    cases = []
    for i in range(N_CASES):
        dims = HEADDIMS[int(rng.integers(3))]
        T = int(rng.integers(1, 1101))
        causal = bool(rng.integers(2))
        kind = int(rng.integers(3)) if causal else 0  # 0 plain, 1 sliding window, 2 ALiBi
        cases.append(dict(
            i=i, dims=dims, T=T, B=int(rng.integers(1, 4)), NH=int(rng.integers(1, 6)), causal=causal,
            window=int(rng.integers(1, T + 65)) if kind == 1 else 0, alibi=kind == 2,
            det=bool(rng.integers(2)), f16=bool(rng.random() < 0.25),
            layout="bhtd" if rng.random() < 0.3 else "bthd", sigma=float((0.5, 1.0, 2.0)[int(rng.integers(3))])))
    return cases


CASES = _cases()


def _name(c):
    return (f"{c['i']}-T{c['T']}-B{c['B']}x{c['NH']}-d{c['dims'][0]}-{'c' if c['causal'] else 'f'}"
            f"{'-w' + str(c['window']) if c['window'] else ''}{'-alibi' if c['alibi'] else ''}"
            f"-{'det' if c['det'] else 'atom'}-{'f16' if c['f16'] else 'bf16'}-{c['layout']}-s{c['sigma']}")


@pytest.mark.parametrize("c", CASES, ids=_name)
def test_random_case(c):
    dqk, dv = c["dims"]
    w = workloads.Workload(f"sweep{c['i']}", c["B"], c["NH"], c["T"], dqk, dv, c["causal"], 53100 + c["i"],
                           sigma=c["sigma"], window=c["window"], alibi=c["alibi"])
    dtype = torch.float16 if c["f16"] else torch.bfloat16
    lay = c["layout"]
    say(f"case sweep {_name(c)}")
    cpu, gpu = gpu_inputs(w, layout=lay, dtype=dtype)
    o, lse = attn.fwd(gpu["q"], gpu["k"], gpu["v"], w.causal, w.scale, layout=lay, window=w.window, alibi=w.alibi)
    dq, dk, dvv = attn.bwd(gpu["q"], gpu["k"], gpu["v"], o, lse, gpu["do"], w.causal, w.scale, c["det"],
                           layout=lay, window=w.window, alibi=w.alibi)
    torch.cuda.synchronize()
    got = {"o": o, "dq": dq, "dk": dk, "dv": dvv}
    if lay == "bhtd":
        got = {n: x.permute(0, 2, 1, 3) for n, x in got.items()}
    got = {n: x.cpu() for n, x in got.items()}
    got["lse"] = lse.cpu()
    ref = attn_ref.attn_ref_bwd(cpu["q"], cpu["k"], cpu["v"], cpu["do"], w.causal, w.scale, window=w.window,
                                alibi=w.alibi)
    tol = (F16_RTOL, F16_ATOL) if c["f16"] else (BF16_RTOL, BF16_ATOL)
    compare(w, got, ref, tol=tol)
