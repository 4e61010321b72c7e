"""Concurrent calls on different streams: the library keeps no state between calls and
its regular entry points share no memory between them, so three different problems run
at the same time on three streams (default priority) must give, bit for bit, what each
gives alone (deterministic dQ mode)."""
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu

PROBLEMS = [
    workloads.Workload("st_a", 2, 4, 1000, 128, 128, True, 701),
    workloads.Workload("st_b", 3, 2, 777, 64, 64, False, 702),
    workloads.Workload("st_c", 1, 3, 1500, 192, 128, True, 703, window=300),
]


def _step(w, x):
    o, lse = attn.fwd(x["q"], x["k"], x["v"], w.causal, w.scale, window=w.window)
    dq, dk, dv = attn.bwd(x["q"], x["k"], x["v"], o, lse, x["do"], w.causal, w.scale, deterministic=True,
                          window=w.window)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_three_streams_match_one_stream_bitwise():
    dev = torch.device("cuda:0")
    inputs = [{n: t.to(dev) for n, t in workloads.make_inputs(w).items() if n in ("q", "k", "v", "do")}
              for w in PROBLEMS]
    say("case streams: each problem alone on the current stream")
    alone = [_step(w, x) for w, x in zip(PROBLEMS, inputs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in PROBLEMS]
    main = torch.cuda.current_stream()
    for rep in range(3):
        say(f"  concurrent round {rep}")
        together = [None] * len(PROBLEMS)
        for i, (w, x, s) in enumerate(zip(PROBLEMS, inputs, streams)):
            s.wait_stream(main)
            with torch.cuda.stream(s):
                together[i] = _step(w, x)
        for s in streams:
            main.wait_stream(s)
        torch.cuda.synchronize()
        for w, a, b in zip(PROBLEMS, alone, together):
            for n in a:
                assert _same(a[n], b[n]), f"{w.name} {n}: concurrent result differs (round {rep})"
