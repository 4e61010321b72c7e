"""Key bias on the GPU against the fp64 oracle (attn_ref_keybias): S = scale Q K^T +
bias[b, h, key], dbias = sum over queries of dS (summed over shared rows).

Biases are N(0, 2^2) per key with a key-padding part (-1e9 on the last keys of one
batch), per head or shared across batches / heads.
"""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import check_bf16, check_lse, say, to_np

pytestmark = pytest.mark.gpu

HEADDIMS = [(64, 64), (128, 128), (192, 128)]


def _bias(shape, T, seed, pad=True):
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(shape).astype(np.float32) * 2.0
    if pad and T > 8:
        b[-1, :, T - T // 8:] = -1e9  # the last batch row: its last eighth of the keys is padding
    return b


def _run(w, cpu, bias, causal, det, need_dbias=True):
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    bg = torch.from_numpy(bias).to(dev)
    o, lse = attn.fwd_keybias(q, k, v, bg, causal, w.scale)
    dq, dk, dv, db = attn.bwd_keybias(q, k, v, o, lse, do, bg, causal, w.scale, deterministic=det,
                                      need_dbias=need_dbias)
    torch.cuda.synchronize()
    out = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    if db is not None:
        out["dbias"] = db.cpu()
    return out


def _compare(w, got, ref, tag, heads=None):
    hs = heads or [(b, h) for b in range(w.B) for h in range(w.NH)]
    per = ref if heads else {(b, h): {n: ref[n][b, :, h] for n in ("o", "dq", "dk", "dv")} | {"lse": ref["lse"][b, h]}
                             for b, h in hs}
    for name in ("o", "dq", "dk", "dv"):
        g = np.stack([to_np(got[name][b, :, h]) for b, h in hs])
        r = np.stack([per[(b, h)][name] for b, h in hs])
        check_bf16(f"{tag} {name}", g, r)
    g = np.stack([to_np(got["lse"][b, h]) for b, h in hs])
    r = np.stack([per[(b, h)]["lse"] for b, h in hs])
    check_lse(f"{tag} lse", g, r)


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", [1, 129, 300, 555])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_keybias_small(dims, T, causal, deterministic):
    w = workloads.Workload(f"kb_T{T}_d{dims[0]}", 2, 3, T, dims[0], dims[1], causal, 700 + T)
    bias = _bias((2, 3, T), T, 701 + T)
    say(f"case {w.name} causal={causal} det={deterministic}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, bias, causal, deterministic)
    ref = attn_ref.attn_ref_keybias(cpu["q"], cpu["k"], cpu["v"], cpu["do"], bias, causal, w.scale)
    _compare(w, got, ref, w.name)
    check_bf16(f"{w.name} dbias", to_np(got["dbias"]), ref["dbias"])


@pytest.mark.parametrize("shape", [(1, 1), (2, 1), (1, 3)], ids=["shared", "per_batch", "per_head"])
def test_keybias_shared_rows(shape):
    """A bias row shared across batches and/or heads: its gradient sums them."""
    w = workloads.Workload("kb_shared", 2, 3, 333, 128, 128, True, 720)
    bias = _bias((*shape, w.T), w.T, 721)
    say(f"case {w.name} bias shape {bias.shape}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, bias, True, True)
    ref = attn_ref.attn_ref_keybias(cpu["q"], cpu["k"], cpu["v"], cpu["do"], bias, True, w.scale)
    _compare(w, got, ref, w.name)
    assert tuple(got["dbias"].shape) == bias.shape
    check_bf16(f"{w.name} dbias", to_np(got["dbias"]), ref["dbias"])


def test_keybias_sigma4_and_no_dbias():
    """N(0, 4^2) inputs (sharp rows) and the backward without a bias gradient."""
    w = workloads.Workload("kb_sigma4", 1, 2, 700, 128, 128, True, 730, sigma=4.0)
    bias = _bias((1, 2, w.T), w.T, 731)
    say(f"case {w.name}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, bias, True, True, need_dbias=False)
    assert "dbias" not in got
    ref = attn_ref.attn_ref_keybias(cpu["q"], cpu["k"], cpu["v"], cpu["do"], bias, True, w.scale)
    _compare(w, got, ref, w.name)


def test_keybias_deterministic_bit_identical():
    w = workloads.WORKLOADS["keybias"].with_(B=1, NH=4)
    say(f"case determinism {w.name}")
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    bg = torch.from_numpy(workloads.key_bias(w)).to(dev)
    o, lse = attn.fwd_keybias(q, k, v, bg, w.causal, w.scale)
    ref = None
    for run in range(10):
        o2, l2 = attn.fwd_keybias(q, k, v, bg, w.causal, w.scale)
        g = attn.bwd_keybias(q, k, v, o, lse, do, bg, w.causal, w.scale, deterministic=True)
        torch.cuda.synchronize()
        cur = [x.clone() for x in (o2, l2, *g)]
        if ref is None:
            ref = cur
        for n, a, b in zip(("o", "lse", "dq", "dk", "dv", "dbias"), ref, cur):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"{n} differs on run {run}"


@pytest.mark.parametrize("deterministic", [True, False], ids=["determ", "atomic"])
def test_keybias_workload_full_size(deterministic):
    """The bench's key-bias workload (headline shape, causal, a per-head key bias with the
    last keys of odd batches padded) on sampled heads, dbias included."""
    w = workloads.WORKLOADS["keybias"]
    bias = workloads.key_bias(w)
    rng = np.random.default_rng(w.seed)
    heads = sorted({(0, 0), (w.B - 1, w.NH - 1)} | {(int(rng.integers(w.B)), int(rng.integers(w.NH)))})
    say(f"case {w.name} det={deterministic} heads={heads}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, bias, w.causal, deterministic)
    torch.cuda.empty_cache()
    ref = attn_ref.attn_ref_keybias(cpu["q"], cpu["k"], cpu["v"], cpu["do"], bias, w.causal, w.scale, heads=heads)
    _compare(w, got, ref, w.name, heads=heads)
    g = np.stack([to_np(got["dbias"][b, h]) for b, h in heads])
    r = np.stack([ref[hd]["dbias"] for hd in heads])
    check_bf16(f"{w.name} dbias", g, r)
