"""Shared helpers for the GPU parity tests: run the HIP path and the CPU oracle on
the same seeded inputs and compare them element by element.

Tolerances (per output tensor):
  bf16 outputs and gradients (O, dQ, dK, dV): max|gpu - ref| <= 2e-2 * max|ref| + 2e-3
  fp16 outputs and gradients:                 max|gpu - ref| <= 5e-3 * max|ref| + 5e-4
    (fp16 keeps 11 significant bits against bf16's 8, so every rounding of the inputs,
    of P and dS before their products and of the outputs is 4x smaller)
  LSE (fp32):                                 max|gpu - ref| <= 1e-3 * max(1, max|ref|)
"""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref

BF16_RTOL, BF16_ATOL = 2e-2, 2e-3
F16_RTOL, F16_ATOL = 5e-3, 5e-4
LSE_RTOL = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_bound(ref: np.ndarray, rtol: float = BF16_RTOL, atol: float = BF16_ATOL) -> float:
    return rtol * float(np.max(np.abs(ref))) + atol


def check_bf16(name: str, got: np.ndarray, ref: np.ndarray, rtol: float = BF16_RTOL, atol: float = BF16_ATOL):
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in GPU output"
    err = float(np.max(np.abs(got - ref)))
    bound = bf16_bound(ref, rtol, atol)
    assert err <= bound, f"{name}: max err {err:.4e} > bound {bound:.4e}"
    return err / max(bound, 1e-30)


def check_lse(name: str, got: np.ndarray, ref: np.ndarray):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in GPU LSE"
    err = float(np.max(np.abs(got - ref)))
    bound = LSE_RTOL * max(1.0, float(np.max(np.abs(ref))))
    assert err <= bound, f"{name}: max err {err:.4e} > bound {bound:.4e}"
    return err / bound


def to_np(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float64).numpy()


def gpu_inputs(w: workloads.Workload, layout: str = "bthd",
               dtype: torch.dtype = torch.bfloat16) -> Tuple[Dict[str, torch.Tensor], Dict[str, torch.Tensor]]:
    """CPU inputs (B, T, NH, d) for the oracle and their GPU copies in `layout`."""
    cpu = workloads.make_inputs(w, dtype)
    dev = torch.device("cuda:0")
    if w.packed:
        qkv = cpu["qkv"].to(dev)
        gpu = {"qkv": qkv, "q": qkv[:, :, 0], "k": qkv[:, :, 1], "v": qkv[:, :, 2], "do": cpu["do"].to(dev)}
    elif layout == "bhtd":
        gpu = {n: cpu[n].permute(0, 2, 1, 3).contiguous().to(dev) for n in ("q", "k", "v", "do")}
    else:
        gpu = {n: cpu[n].to(dev) for n in ("q", "k", "v", "do")}
    return cpu, gpu


def run_gpu(w: workloads.Workload, gpu: Dict[str, torch.Tensor], deterministic: bool, layout: str = "bthd"):
    """Forward then backward on the GPU; returns host tensors (B, T, NH, d) / (B, NH, T)."""
    if w.packed:
        o, lse = attn.fwd_packed(gpu["qkv"], w.causal, w.scale)
        dqkv = attn.bwd_packed(gpu["qkv"], o, lse, gpu["do"], w.causal, w.scale, deterministic)
        dq, dk, dv = dqkv[:, :, 0], dqkv[:, :, 1], dqkv[:, :, 2]
    else:
        o, lse = attn.fwd(gpu["q"], gpu["k"], gpu["v"], w.causal, w.scale, layout=layout)
        dq, dk, dv = attn.bwd(gpu["q"], gpu["k"], gpu["v"], o, lse, gpu["do"], w.causal, w.scale,
                              deterministic, layout=layout)
    torch.cuda.synchronize()
    out = {"o": o, "dq": dq, "dk": dk, "dv": dv}
    if layout == "bhtd" and not w.packed:
        out = {n: x.permute(0, 2, 1, 3) for n, x in out.items()}
    res = {n: x.to("cpu") for n, x in out.items()}  # bf16 on the host; heads converted on demand
    res["lse"] = lse.to("cpu")
    return res


def compare(w: workloads.Workload, got: Dict[str, np.ndarray], ref, heads=None, tag: str = "",
            tol: Tuple[float, float] = (BF16_RTOL, BF16_ATOL)) -> Dict[str, float]:
    """Element-by-element comparison.  ``ref`` is either the oracle's full result
    (heads=None: every head is compared) or its per-head result {(b, h): {...}}."""
    if heads is None:
        hs = [(b, h) for b in range(w.B) for h in range(w.NH)]
        per = {(b, h): {n: ref[n][b, :, h] for n in ("o", "dq", "dk", "dv")} | {"lse": ref["lse"][b, h]}
               for b, h in hs}
    else:
        hs, per = list(heads), ref
    ratios = {}
    for name in ("o", "dq", "dk", "dv"):
        g = np.stack([to_np(got[name][b, :, h]) for b, h in hs])
        r = np.stack([per[(b, h)][name] for b, h in hs])
        ratios[name] = check_bf16(f"{tag}{w.name} {name}", g, r, *tol)
    g = np.stack([to_np(got["lse"][b, h]) for b, h in hs])
    r = np.stack([per[(b, h)]["lse"] for b, h in hs])
    ratios["lse"] = check_lse(f"{tag}{w.name} lse", g, r)
    return ratios


def oracle(w: workloads.Workload, cpu: Dict[str, torch.Tensor], heads=None):
    if heads is None:
        return attn_ref.attn_ref_bwd(cpu["q"], cpu["k"], cpu["v"], cpu["do"], w.causal, w.scale)
    return attn_ref.attn_ref_heads(cpu["q"], cpu["k"], cpu["v"], cpu["do"], w.causal, w.scale, heads=heads)


def sample_heads(w: workloads.Workload, n: int, seed: int = 0):
    rng = np.random.default_rng(w.seed + seed)
    all_h = [(b, h) for b in range(w.B) for h in range(w.NH)]
    idx = rng.choice(len(all_h), size=min(n, len(all_h)), replace=False)
    # always include the first and the last head
    pick = {all_h[0], all_h[-1]} | {all_h[i] for i in idx}
    return sorted(pick)[: max(n, 2)]
