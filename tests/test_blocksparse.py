"""Block-sparse maps on the GPU against the fp64 oracle (attn_ref_blocksparse).

A map marks (query block, key block) pairs of 128 x 128 elements as live or not; element
(i, j) is attended iff its block is live and, when causal, j <= i.  The cases cover maps
per head and shared, rows and key columns with no live block (O = 0, LSE = -inf, zero
gradients), ragged ends, both dQ modes; with an all-live map (or the block-lower
triangle under the causal mask) the block-sparse kernels visit the dense kernels' tiles in
the same order, so their outputs must equal the dense path's bit for bit.
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


def _map(B, NH, T, seed, density=0.5, shared=False):
    nb = (T + 127) // 128
    rng = np.random.default_rng(seed)
    m = (rng.random((1 if shared else B, 1 if shared else NH, nb, nb)) < density).astype(np.uint8)
    if nb > 1 and not shared:
        m[0, 0, nb - 1, :] = 0   # the last query block of head (0, 0) has no key at all
        m[-1, -1, :, 0] = 0      # key block 0 of the last head is attended by no query
    return m


def _run(w, cpu, m, causal, det):
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    mg = torch.from_numpy(m).to(dev)
    o, lse = attn.fwd_blocksparse(q, k, v, mg, causal, w.scale)
    dq, dk, dv = attn.bwd_blocksparse(q, k, v, o, lse, do, mg, causal, w.scale, deterministic=det)
    torch.cuda.synchronize()
    return {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


def _compare(w, got, ref, heads, tag):
    for name in ("o", "dq", "dk", "dv"):
        g = np.stack([to_np(got[name][b, :, h]) for b, h in heads])
        r = np.stack([ref[(b, h)][name] for b, h in heads])
        check_bf16(f"{tag} {name}", g, r)
    g = np.stack([to_np(got["lse"][b, h]) for b, h in heads])
    r = np.stack([ref[(b, h)]["lse"] for b, h in heads])
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), f"{tag}: rows without keys differ (LSE -inf)"
    if fin.any():
        check_lse(f"{tag} lse", g[fin], r[fin])


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("T", [1, 129, 300, 555])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_blocksparse_small(dims, T, causal, deterministic):
    w = workloads.Workload(f"bsp_T{T}_d{dims[0]}", 2, 3, T, dims[0], dims[1], causal, 600 + T)
    m = _map(w.B, w.NH, T, 601 + T)
    say(f"case {w.name} causal={causal} det={deterministic} live={int(m.sum())}/{m.size}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, m, causal, deterministic)
    heads = [(b, h) for b in range(w.B) for h in range(w.NH)]
    ref = attn_ref.attn_ref_blocksparse(cpu["q"], cpu["k"], cpu["v"], cpu["do"], m, causal, w.scale, heads=heads)
    _compare(w, got, ref, heads, w.name)
    if T > 128:  # the planted empty query block and unattended key block
        nb = m.shape[-1]
        assert torch.all(got["o"][0, 128 * (nb - 1):, 0] == 0) and torch.all(got["dq"][0, 128 * (nb - 1):, 0] == 0)
        assert torch.all(torch.isinf(got["lse"][0, 0, 128 * (nb - 1):]))
        assert torch.all(got["dk"][-1, :128, -1] == 0) and torch.all(got["dv"][-1, :128, -1] == 0)


@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_blocksparse_shared_map_sigma4(dims):
    """One map for every head (strides 0), inputs ~ N(0, 4^2) (sharp rows, rescaling)."""
    w = workloads.Workload(f"bsp_shared_d{dims[0]}", 2, 2, 700, dims[0], dims[1], True, 650, sigma=4.0)
    m = _map(1, 1, w.T, 651, density=0.6, shared=True)
    say(f"case {w.name}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, m, True, True)
    heads = [(b, h) for b in range(w.B) for h in range(w.NH)]
    ref = attn_ref.attn_ref_blocksparse(cpu["q"], cpu["k"], cpu["v"], cpu["do"], m, True, w.scale, heads=heads)
    _compare(w, got, ref, heads, w.name)


@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_dense_maps_equal_dense_path_bitwise(dims):
    """All-live map (non-causal) and the block-lower triangle (causal): the same tiles in
    the same order per workgroup as the dense kernels, so bit-identical outputs
    (deterministic mode)."""
    dev = torch.device("cuda:0")
    for causal in (False, True):
        w = workloads.Workload(f"bsp_dense_d{dims[0]}", 2, 2, 1000, dims[0], dims[1], causal, 660)
        say(f"case {w.name} causal={causal}")
        cpu = workloads.make_inputs(w)
        q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
        nb = (w.T + 127) // 128
        m = np.tril(np.ones((nb, nb), np.uint8)) if causal else np.ones((nb, nb), np.uint8)
        mg = torch.from_numpy(m[None, None].copy()).to(dev)
        o1, l1 = attn.fwd_blocksparse(q, k, v, mg, causal, w.scale)
        g1 = attn.bwd_blocksparse(q, k, v, o1, l1, do, mg, causal, w.scale, deterministic=True)
        o2, l2 = attn.fwd(q, k, v, causal, w.scale)
        g2 = attn.bwd(q, k, v, o2, l2, do, causal, w.scale, deterministic=True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "o"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse"
        for n, a, b in zip(("dq", "dk", "dv"), g1, g2):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n


def test_blocksparse_deterministic_bit_identical():
    w = workloads.WORKLOADS["blocksparse"].with_(B=1)
    say(f"case determinism {w.name}")
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    mg = torch.from_numpy(workloads.block_map(w)).to(dev)
    o, lse = attn.fwd_blocksparse(q, k, v, mg, w.causal, w.scale)
    ref = None
    for run in range(10):
        o2, l2 = attn.fwd_blocksparse(q, k, v, mg, w.causal, w.scale)
        g = attn.bwd_blocksparse(q, k, v, o, lse, do, mg, w.causal, w.scale, deterministic=True)
        torch.cuda.synchronize()
        cur = [x.clone() for x in (o2, l2, *g)]
        if ref is None:
            ref = cur
        for n, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, cur):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"{n} differs on run {run}"


@pytest.mark.parametrize("deterministic", [True, False], ids=["determ", "atomic"])
def test_blocksparse_workload_full_size(deterministic):
    """The bench's block-sparse workload (headline shape, causal, local band of 8 blocks
    plus the first block as a global one) on sampled heads."""
    w = workloads.WORKLOADS["blocksparse"]
    m = workloads.block_map(w)
    rng = np.random.default_rng(w.seed)
    heads = sorted({(0, 0), (w.B - 1, w.NH - 1)} | {(int(rng.integers(w.B)), int(rng.integers(w.NH)))})
    say(f"case {w.name} det={deterministic} heads={heads}")
    cpu = workloads.make_inputs(w)
    got = _run(w, cpu, m, w.causal, deterministic)
    torch.cuda.empty_cache()
    ref = attn_ref.attn_ref_blocksparse(cpu["q"], cpu["k"], cpu["v"], cpu["do"], m, w.causal, w.scale, heads=heads)
    _compare(w, got, ref, heads, w.name)
