"""d = 64, deterministic mode: one backward call runs the key/value and dQ work in one
launch (when the key/value workgroups number a multiple of 8, plain or causal mask, dense
or padded batches).  It must equal, bit for bit, the backward run as three separate stage calls
(preprocess, key/value kernel, dQ kernel), and match the oracle."""
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import (F16_ATOL, F16_RTOL, BF16_ATOL, BF16_RTOL, check_bf16, compare, gpu_inputs, oracle, say,
                             to_np)

pytestmark = pytest.mark.gpu

# (B, NH, T): ceil(T / 128) * B * NH is a multiple of 8 in each
SHAPES = [(2, 4, 1000), (1, 8, 300), (4, 2, 129), (4, 12, 1024)]


@pytest.mark.parametrize("f16", [False, True], ids=["bf16", "f16"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}xNH{s[1]}xT{s[2]}")
def test_one_call_equals_stage_calls(shape, causal, f16):
    B, NH, T = shape
    assert (T + 127) // 128 * B * NH % 8 == 0
    w = workloads.Workload(f"kvdq_B{B}_NH{NH}_T{T}", B, NH, T, 64, 64, causal, 800 + T + B)
    dtype = torch.float16 if f16 else torch.bfloat16
    say(f"case merged kv+dq {w.name} causal={causal} f16={f16}")
    cpu, gpu = gpu_inputs(w, dtype=dtype)
    q, k, v, do = gpu["q"], gpu["k"], gpu["v"], gpu["do"]
    o, lse = attn.fwd(q, k, v, causal, w.scale)
    one = attn.bwd(q, k, v, o, lse, do, causal, w.scale, deterministic=True)
    ws = torch.empty(attn.workspace_bytes(B, NH, T, 64, 64, True), dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    for stage in (attn.PREPROCESS, attn.MAIN, attn.DQ):
        attn.bwd(q, k, v, o, lse, do, causal, w.scale, deterministic=True, dq=dq, dk=dk, dv=dv, workspace=ws,
                 stages=stage)
    torch.cuda.synchronize()
    for n, a, b in zip(("dq", "dk", "dv"), one, (dq, dk, dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{n}: one call differs from the stage calls"
    got = {"o": o.cpu(), "lse": lse.cpu(), "dq": one[0].cpu(), "dk": one[1].cpu(), "dv": one[2].cpu()}
    compare(w, got, oracle(w, cpu), tol=(F16_RTOL, F16_ATOL) if f16 else (BF16_RTOL, BF16_ATOL))


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_one_call_equals_stage_calls_padded(causal):
    """Padded batches at d = 64: the one-call backward (one launch over both work lists)
    equals the three stage calls bit for bit, and valid rows match the oracle."""
    B, NH, T = 4, 4, 700  # ceil(700 / 128) * 4 * 4 = 96 key/value workgroups
    n = [700, 1, 333, 0]
    w = workloads.Workload("kvdq_padded", B, NH, T, 64, 64, causal, 860)
    say(f"case merged kv+dq padded lengths={n} causal={causal}")
    cpu, gpu = gpu_inputs(w)
    q, k, v, do = gpu["q"], gpu["k"], gpu["v"], gpu["do"]
    lens = torch.tensor(n, dtype=torch.int32, device=q.device)
    o, lse = attn.fwd_varlen(q, k, v, lens, lens, causal, w.scale)
    one = attn.bwd_varlen(q, k, v, o, lse, do, lens, lens, causal, w.scale, deterministic=True)
    ws = torch.empty(int(attn.load().attn_bwd_varlen_workspace_bytes(B, NH, T, 64, 64, 1)), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = (torch.empty_like(x) for x in (q, k, v))
    for stage in (attn.PREPROCESS, attn.MAIN, attn.DQ):
        attn.bwd_varlen(q, k, v, o, lse, do, lens, lens, causal, w.scale, deterministic=True, workspace=ws, dq=dq,
                        dk=dk, dv=dv, stages=stage)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), one, (dq, dk, dv)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: one call differs from the stage calls"
    ref = attn_ref.attn_ref_varlen(cpu["q"], cpu["k"], cpu["v"], cpu["do"], n, n, causal, w.scale)
    for b_ in range(B):
        r = n[b_]
        if r == 0:
            continue
        for name, x in (("o", o), ("dq", one[0]), ("dk", one[1]), ("dv", one[2])):
            check_bf16(f"padded b={b_} {name}", to_np(x[b_, :r]), ref[name][b_, :r])
