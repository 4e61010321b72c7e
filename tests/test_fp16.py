"""GPU parity of the fp16 element type (attn_fwd_typed / attn_bwd_typed with
ATTN_DTYPE_F16) against the fp64 oracle.

The pages run attention with 16-bit inputs and outputs and fp32 accumulation, naming
fp16 beside bf16 ("ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" section 1.3).  The
oracle gets the same fp16 values, upcast exactly.  Tolerance (per output tensor):
max|gpu - ref| <= 5e-3 max|ref| + 5e-4 for O, dQ, dK, dV (a quarter of the bf16 bound:
fp16 rounds to 11 significant bits, bf16 to 8); LSE as for bf16.
"""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import (F16_ATOL, F16_RTOL, check_bf16, check_lse, compare, gpu_inputs, oracle, run_gpu,
                             sample_heads, say, to_np)

pytestmark = pytest.mark.gpu

HEADDIMS = [(64, 64), (128, 128), (192, 128)]
TOL = (F16_RTOL, F16_ATOL)
F16 = torch.float16


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", [1, 129, 300])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_fp16_small(dims, T, causal, deterministic):
    w = workloads.Workload(f"f16_T{T}_d{dims[0]}x{dims[1]}", 2 if T < 200 else 1, 3 if T < 200 else 2, T,
                           dims[0], dims[1], causal, 500 + T)
    say(f"case fp16 {w.name} causal={causal} det={deterministic}")
    cpu, gpu = gpu_inputs(w, dtype=F16)
    got = run_gpu(w, gpu, deterministic)
    assert got["o"].dtype == F16 and got["dq"].dtype == F16
    compare(w, got, oracle(w, cpu), tol=TOL)


def test_fp16_packed_and_large_scores():
    """Packed (B, T, 3, NH, HS) QKV in fp16, and N(0, 4^2) inputs (sharply peaked rows)."""
    w = workloads.WORKLOADS["gpt2"].with_(B=1, T=300)
    say(f"case fp16 packed {w.name}")
    cpu, gpu = gpu_inputs(w, dtype=F16)
    compare(w, run_gpu(w, gpu, True), oracle(w, cpu), tol=TOL)
    w = workloads.Workload("f16_sigma4", 1, 2, 333, 128, 128, True, 541, sigma=4.0)
    say(f"case fp16 {w.name}")
    cpu, gpu = gpu_inputs(w, dtype=F16)
    compare(w, run_gpu(w, gpu, False), oracle(w, cpu), tol=TOL)


def test_fp16_deterministic_bit_stable():
    w = workloads.Workload("f16_det", 2, 2, 700, 128, 128, True, 547)
    say(f"case fp16 determinism {w.name}")
    _, gpu = gpu_inputs(w, dtype=F16)
    first = run_gpu(w, gpu, True)
    for _ in range(4):
        again = run_gpu(w, gpu, True)
        for n in first:
            assert torch.equal(first[n], again[n]), n


def test_fp16_varlen():
    B, T, NH, d = 4, 300, 2, 128
    sq, sk = [300, 1, 131, 0], [300, 77, 131, 40]
    say(f"case fp16 varlen {sq} {sk}")
    w = workloads.Workload("f16_varlen", B, NH, T, d, d, True, 553)
    cpu = workloads.make_inputs(w, F16)
    dev = torch.device("cuda:0")
    g = {n: cpu[n].to(dev) for n in ("q", "k", "v", "do")}
    lq = torch.tensor(sq, dtype=torch.int32, device=dev)
    lk = torch.tensor(sk, dtype=torch.int32, device=dev)
    o, lse = attn.fwd_varlen(g["q"], g["k"], g["v"], lq, lk, True, w.scale)
    dq, dk, dv = attn.bwd_varlen(g["q"], g["k"], g["v"], o, lse, g["do"], lq, lk, True, w.scale, True)
    torch.cuda.synchronize()
    ref = attn_ref.attn_ref_varlen(cpu["q"], cpu["k"], cpu["v"], cpu["do"], sq, sk, True, w.scale)
    got = {"o": o, "dq": dq, "dk": dk, "dv": dv}
    for b in range(B):
        rows = sq[b] if sk[b] > 0 else 0
        keys = sk[b] if sq[b] > 0 else 0
        for h in range(NH):
            if rows:
                for n in ("o", "dq"):
                    check_bf16(f"fp16 varlen b={b} h={h} {n}", to_np(got[n][b, :rows, h]), ref[n][b, :rows, h], *TOL)
                check_lse(f"fp16 varlen b={b} h={h} lse", to_np(lse[b, h, :rows]), ref["lse"][b, h, :rows])
            if keys:
                for n in ("dk", "dv"):
                    check_bf16(f"fp16 varlen b={b} h={h} {n}", to_np(got[n][b, :keys, h]), ref[n][b, :keys, h], *TOL)
            assert torch.all(got["o"][b, rows:] == 0) and torch.all(got["dk"][b, keys:] == 0)


@pytest.mark.parametrize("name", ["headline", "asym"])
def test_fp16_full_size_sampled(name):
    """The full-size workloads in fp16, in the launch configuration of the bench
    (deterministic dQ), with every element of sampled (batch, head) pairs compared."""
    w = workloads.WORKLOADS[name]
    heads = sample_heads(w, 2)
    say(f"case fp16 full size {name} heads={heads}")
    cpu, gpu = gpu_inputs(w, dtype=F16)
    got = run_gpu(w, gpu, True)
    del gpu
    compare(w, got, oracle(w, cpu, heads=heads), heads=heads, tol=TOL)
