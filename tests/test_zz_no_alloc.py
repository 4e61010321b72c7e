"""attn_bwd_noalloc (the backward with the library's fixed per-GPU scratch as its
workspace) against attn_bwd with a caller-owned workspace, both called through ctypes.

Two calls in a row, the second on smaller inputs, so that the second runs on a scratch
array that still holds the first call's contents: deterministic mode must equal attn_bwd
bit for bit, atomic mode within the bf16 tolerance (fp32 atomics add in varying order).
"""
import ctypes

import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from tests.gpu_cases import check_bf16, say, to_np

pytestmark = pytest.mark.gpu


def _st(x):
    return attn.Strides(x.stride(0), x.stride(2), x.stride(1))


def _run(lib, w, deterministic, noalloc):
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = attn.fwd(q, k, v, w.causal, w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    common = (q.data_ptr(), _st(q), k.data_ptr(), _st(k), v.data_ptr(), _st(v), o.data_ptr(), _st(o),
              lse.data_ptr(), do.data_ptr(), _st(do), dq.data_ptr(), _st(dq), dk.data_ptr(), _st(dk),
              dv.data_ptr(), _st(dv), w.B, w.NH, w.T, w.d_qk, w.d_v, ctypes.c_float(w.scale), int(w.causal),
              int(deterministic))
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = lib.attn_bwd_noalloc(*common, stream)
    else:
        nbytes = lib.attn_bwd_workspace_bytes(w.B, w.NH, w.T, w.d_qk, w.d_v, int(deterministic))
        # filled with NaN bytes: a kernel that read workspace it had not written would show
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
        st = lib.attn_bwd(*common, ws.data_ptr(), nbytes, stream)
    assert st == 0, lib.attn_status_string(st)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


CASES = [
    workloads.Workload("noalloc_big", 2, 4, 1000, 128, 128, True, 501),
    workloads.Workload("noalloc_small", 1, 2, 300, 64, 64, True, 502),
]


@pytest.mark.parametrize("deterministic", [True, False], ids=["determ", "atomic"])
def test_noalloc_matches_attn_bwd_on_two_calls(deterministic):
    lib = attn.load()
    assert lib.attn_bwd_noalloc_max_workspace_bytes() == 64 << 20
    for w in CASES:  # second call smaller than the first
        say(f"case noalloc {w.name} det={deterministic}")
        a = _run(lib, w, deterministic, noalloc=True)
        b = _run(lib, w, deterministic, noalloc=False)
        for n, x, y in zip(("dq", "dk", "dv"), a, b):
            if deterministic:
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{w.name} {n} differs"
            else:
                check_bf16(f"{w.name} {n}", to_np(x), to_np(y))
