"""Dropout on the GPU against the fp64 oracle (attn_ref_dropout).

The keep bits that attn_dropout_mask writes are integer work: both layouts must equal the
oracle's Philox4x32-10 bits exactly.  The attention results are held to the bf16
tolerance; p = 0 must reproduce plain attention, and the deterministic mode must be
bit-stable.

One term is added to the dQ and dK bounds.  The backward takes D_i = sum_k dO_ik O_ik from
the stored bf16 O, which is rounded (relative 2^-8, an 8-bit significand); dS_ij = P_ij (dP_ij - D_i) then
carries P_ij dD_i, so dQ_i moves by at most scale |dD_i| max|K| (the P_ij of a row sum to
one) and dK_j by scale max|dD| max|Q| times the column sum of P, taken at its average, one.
Without dropout O = V exactly where a row has one key, so this residue vanishes where the
reference gradient cancels to zero; with dropout O = V / (1 - p) is rounded there too, and
the reference dQ = 0 of a one-key row (T = 1) is met only to this term:
  |dD| <= 2^-8 max_i sum_k |dO_ik O_ik|.
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


def _bits(buf: np.ndarray, nbh: int, tp: int) -> np.ndarray:
    """(nbh, tp, tp / 8) bytes -> (nbh, tp, tp) bools, bit k of byte c = column 8c + k."""
    return np.unpackbits(buf.reshape(nbh, tp, tp // 8), axis=-1, bitorder="little").astype(bool)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("T", [1, 129, 300])
def test_mask_bits_equal_the_oracle(T, causal):
    B, NH, p, seed, offset = 2, 3, 0.3, 0x0123456789ABCDEF, 12345
    say(f"case dropout mask T={T} causal={causal}")
    m = attn.dropout_mask(p, seed, offset, B, NH, T, causal).cpu().numpy()
    tp = (T + 127) // 128 * 128
    half = B * NH * tp * tp // 8
    rows, cols = _bits(m[:half], B * NH, tp), _bits(m[half:2 * half], B * NH, tp)
    for b in range(B):
        for h in range(NH):
            want = attn_ref.philox_keep(b, h, NH, T, p, seed, offset)
            got_r = rows[b * NH + h, :T, :T]
            got_c = cols[b * NH + h, :T, :T].T
            if causal:  # only the lower triangle is generated (and read)
                tri = np.tril(np.ones((T, T), bool))
                want, got_r, got_c = want[tri], got_r[tri], got_c[tri]
            assert np.array_equal(got_r, want), f"query-major bits of head ({b},{h})"
            assert np.array_equal(got_c, want), f"key-major bits of head ({b},{h})"


def _run(w, cpu, p, seed, offset, causal, det):
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    mask = attn.dropout_mask(p, seed, offset, w.B, w.NH, w.T, causal)
    o, lse = attn.fwd_dropout(q, k, v, mask, p, causal, w.scale)
    dq, dk, dv = attn.bwd_dropout(q, k, v, o, lse, do, mask, p, causal, w.scale, deterministic=det)
    torch.cuda.synchronize()
    return {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


def _compare(w, got, ref, tag, heads=None, cpu=None):
    hs = heads or [(b, h) for b in range(w.B) for h in range(w.NH)]
    per = ref if heads else {(b, h): {n: ref[n][b, :, h] for n in ("o", "dq", "dk", "dv")} | {"lse": ref["lse"][b, h]}
                             for b, h in hs}
    extra = {"o": 0.0, "dv": 0.0, "dq": 0.0, "dk": 0.0}
    if cpu is not None:  # the D-rounding term of the module docstring
        dd = max(float(np.max(np.sum(np.abs(to_np(cpu["do"][b, :, h]) * per[(b, h)]["o"]), axis=-1))) for b, h in hs)
        dd *= 2.0 ** -8
        extra["dq"] = w.scale * dd * float(cpu["k"].float().abs().max())
        extra["dk"] = w.scale * dd * float(cpu["q"].float().abs().max())
    for name in ("o", "dq", "dk", "dv"):
        g = np.stack([to_np(got[name][b, :, h]) for b, h in hs])
        r = np.stack([per[(b, h)][name] for b, h in hs])
        check_bf16(f"{tag} {name}", g, r, atol=2e-3 + extra[name])
    g = np.stack([to_np(got["lse"][b, h]) for b, h in hs])
    r = np.stack([per[(b, h)]["lse"] for b, h in hs])
    check_lse(f"{tag} lse", g, r)


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", [1, 129, 300, 555])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_dropout_small(dims, T, causal, deterministic):
    w = workloads.Workload(f"drop_T{T}_d{dims[0]}", 2, 3, T, dims[0], dims[1], causal, 900 + T)
    p, seed, off = 0.2, 1000 + T, 7
    say(f"case {w.name} causal={causal} det={deterministic}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, p, seed, off, causal, deterministic)
    ref = attn_ref.attn_ref_dropout(cpu["q"], cpu["k"], cpu["v"], cpu["do"], p, seed, off, causal, w.scale)
    _compare(w, got, ref, w.name, cpu=cpu)


@pytest.mark.parametrize("p", [0.0, 0.6])
def test_dropout_rates(p):
    """p = 0 keeps everything (plain attention); a high rate keeps 40 % of the weights."""
    w = workloads.Workload(f"drop_p{p}", 2, 2, 400, 128, 128, True, 930, sigma=2.0)
    say(f"case {w.name}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, p, 77, 0, True, True)
    ref = attn_ref.attn_ref_dropout(cpu["q"], cpu["k"], cpu["v"], cpu["do"], p, 77, 0, True, w.scale)
    _compare(w, got, ref, w.name, cpu=cpu)
    if p == 0.0:
        plain = attn_ref.attn_ref_bwd(cpu["q"], cpu["k"], cpu["v"], cpu["do"], True, w.scale)
        _compare(w, got, plain, w.name + " vs plain")


def test_dropout_deterministic_bit_identical():
    w = workloads.WORKLOADS["dropout"].with_(B=1, NH=4, T=4096)
    say(f"case determinism {w.name}")
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    ref = None
    for run in range(10):
        mask = attn.dropout_mask(workloads.DROPOUT_P, w.seed, 0, w.B, w.NH, w.T, True)
        o, lse = attn.fwd_dropout(q, k, v, mask, workloads.DROPOUT_P, True, w.scale)
        g = attn.bwd_dropout(q, k, v, o, lse, do, mask, workloads.DROPOUT_P, True, w.scale, deterministic=True)
        torch.cuda.synchronize()
        cur = [x.clone() for x in (o, lse, *g)]
        if ref is None:
            ref = cur
        for n, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, cur):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"{n} differs on run {run}"


@pytest.mark.parametrize("deterministic", [True, False], ids=["determ", "atomic"])
def test_dropout_workload_full_size(deterministic):
    """The bench's dropout workload (headline shape, causal, p = 0.1) on sampled heads."""
    w = workloads.WORKLOADS["dropout"]
    heads = [(0, 0), (2, 9), (w.B - 1, w.NH - 1)]
    say(f"case {w.name} det={deterministic} heads={heads}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, workloads.DROPOUT_P, w.seed, 0, True, deterministic)
    torch.cuda.empty_cache()
    ref = attn_ref.attn_ref_dropout(cpu["q"], cpu["k"], cpu["v"], cpu["do"], workloads.DROPOUT_P, w.seed, 0, True,
                                    w.scale, heads=heads)
    _compare(w, got, ref, w.name, heads=heads, cpu=cpu)
