"""fp8 (e4m3) forward on the GPU against the fp64 oracle (attn_ref_fwd_fp8), which gets
the very same e4m3 codes and descale factors.

Tolerance (derived from the path's one approximation beyond fp32 sums): P is rounded to
e4m3 (3 mantissa bits) before O = P V.  For weights in e4m3's normal range the rounding
moves each weight by at most 2^-4 of itself, and O is a weighted mean of V rows with
weights summing to one, so |dO| <= 2^-4 max|V|; weights in the subnormal range (p < 2^-6 of
a row maximum of at least 1) move by at most 2^-10 each, in random directions, far below
that bound at these sizes.  The bf16 rounding of O adds 2^-8 max|O|.  Hence
  max|O - O_ref| <= 2^-4 max|V| + 2^-8 max|O_ref|       (V: the real, descaled values)
LSE comes from the unrounded fp32 sums: the 16-bit path's bound, 1e-3 max(1, max|LSE|).
"""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import check_lse, say, to_np

pytestmark = pytest.mark.gpu


def _check_o(name, got, ref, vmax):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref)))
    bound = 2.0 ** -4 * vmax + 2.0 ** -8 * float(np.max(np.abs(ref)))
    assert err <= bound, f"{name}: max err {err:.4e} > bound {bound:.4e}"
    say(f"  {name}: err {err:.3e} ({err / bound:.3f} of the bound)")


def _run(w, x, causal, return_lse=True):
    dev = torch.device("cuda:0")
    q8, k8, v8 = (x[n].to(dev) for n in ("q8", "k8", "v8"))
    o, lse = attn.fwd_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], causal, w.scale,
                          return_lse=return_lse)
    torch.cuda.synchronize()
    return o.cpu(), (lse.cpu() if lse is not None else None)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", [1, 64, 129, 300, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_small(d, T, causal):
    w = workloads.Workload(f"fp8_T{T}_d{d}", 2, 3, T, d, d, causal, 800 + T)
    x = workloads.make_fp8_inputs(w)
    say(f"case {w.name} causal={causal}")
    o, lse = _run(w, x, causal)
    ref_o, ref_lse = attn_ref.attn_ref_fwd_fp8(x["q8"].numpy(), x["k8"].numpy(), x["v8"].numpy(), x["descale_q"],
                                               x["descale_k"], x["descale_v"], causal, w.scale)
    vmax = float(np.max(np.abs(attn_ref.e4m3_to_f64(x["v8"].numpy())))) * x["descale_v"]
    _check_o(f"{w.name} o", to_np(o), ref_o, vmax)
    check_lse(f"{w.name} lse", to_np(lse), ref_lse)


def test_fp8_sigma4_and_inference():
    """N(0, 4^2) inputs (sharp rows: the running max is raised mid-row); inference mode
    (no stats) gives the same O bits."""
    w = workloads.Workload("fp8_sigma4", 2, 2, 777, 128, 128, True, 850, sigma=4.0)
    x = workloads.make_fp8_inputs(w)
    say(f"case {w.name}")
    o, lse = _run(w, x, True)
    o2, none = _run(w, x, True, return_lse=False)
    assert none is None and torch.equal(o.view(torch.int16), o2.view(torch.int16))
    ref_o, ref_lse = attn_ref.attn_ref_fwd_fp8(x["q8"].numpy(), x["k8"].numpy(), x["v8"].numpy(), x["descale_q"],
                                               x["descale_k"], x["descale_v"], True, w.scale)
    vmax = float(np.max(np.abs(attn_ref.e4m3_to_f64(x["v8"].numpy())))) * x["descale_v"]
    _check_o(f"{w.name} o", to_np(o), ref_o, vmax)
    check_lse(f"{w.name} lse", to_np(lse), ref_lse)


def test_fp8_headline_full_size():
    """The headline shape (B 4, NH 16, T 8192, d 128, causal) in fp8 on sampled heads, in the
    launch configuration the bench times; the forward is also bit-stable over repeats."""
    w = workloads.WORKLOADS["headline"]
    x = workloads.make_fp8_inputs(w)
    heads = [(0, 0), (1, 7), (3, 15)]
    say(f"case fp8 headline heads={heads}")
    dev = torch.device("cuda:0")
    q8, k8, v8 = (x[n].to(dev) for n in ("q8", "k8", "v8"))
    o, lse = attn.fwd_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], True, w.scale)
    o2, lse2 = attn.fwd_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], True, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    o, lse = o.cpu(), lse.cpu()
    for b, h in heads:
        sl = lambda t: t[b:b + 1, :, h:h + 1].numpy()  # noqa: E731
        ref_o, ref_lse = attn_ref.attn_ref_fwd_fp8(sl(x["q8"]), sl(x["k8"]), sl(x["v8"]), x["descale_q"],
                                                   x["descale_k"], x["descale_v"], True, w.scale)
        vmax = float(np.max(np.abs(attn_ref.e4m3_to_f64(sl(x["v8"]))))) * x["descale_v"]
        _check_o(f"fp8 headline ({b},{h}) o", to_np(o[b:b + 1, :, h:h + 1]), ref_o, vmax)
        check_lse(f"fp8 headline ({b},{h}) lse", to_np(lse[b:b + 1, h:h + 1]), ref_lse)
