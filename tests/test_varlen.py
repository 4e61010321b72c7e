"""GPU parity of padded batches (per-batch query and key/value lengths) against the
fp64 oracle: the padding mask with seq_len_q and seq_len_kv among the SDPA options of
"ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析" section 1.2, with the work ordered by
a sorting preprocessing kernel as in "深度学习反向传播优化：2-CTA MMA模式与内存访问优化" section 3.2.

Padding rows of the inputs hold NaN, so any read of them shows up in the outputs.
Valid rows are compared element by element within the bf16 / fp32 tolerances of the
dense tests; padding rows of the outputs must be exactly 0 (LSE exactly -inf).
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


def _inputs(B, T, NH, dqk, dv, seed, seq_q, seq_k):
    w = workloads.Workload("varlen", B, NH, T, dqk, dv, True, seed)
    cpu = workloads.make_inputs(w)
    for b in range(B):  # padding rows: NaN on the GPU side, never read by the oracle
        cpu["q"][b, seq_q[b]:] = float("nan")
        cpu["do"][b, seq_q[b]:] = float("nan")
        cpu["k"][b, seq_k[b]:] = float("nan")
        cpu["v"][b, seq_k[b]:] = float("nan")
    dev = torch.device("cuda:0")
    gpu = {n: cpu[n].to(dev) for n in ("q", "k", "v", "do")}
    lens = (torch.tensor(seq_q, dtype=torch.int32, device=dev), torch.tensor(seq_k, dtype=torch.int32, device=dev))
    return cpu, gpu, lens


def _run(gpu, lens, causal, scale, deterministic):
    o, lse = attn.fwd_varlen(gpu["q"], gpu["k"], gpu["v"], lens[0], lens[1], causal, scale)
    dq, dk, dv = attn.bwd_varlen(gpu["q"], gpu["k"], gpu["v"], o, lse, gpu["do"], lens[0], lens[1], causal, scale,
                                 deterministic)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _compare(name, got, ref, seq_q, seq_k, heads=None):
    B = len(seq_q)
    NH = got["o"].shape[2]
    for b in range(B):
        lq, lk = seq_q[b], seq_k[b]
        rows = lq if lk > 0 else 0          # query rows with at least one key
        keys = lk if lq > 0 else 0          # key rows that some query sees
        hs = range(NH) if heads is None else [h for (bb, h) in heads if bb == b]
        for h in hs:
            g = {n: to_np(got[n][b, :, h]) for n in ("o", "dq", "dk", "dv")}
            g["lse"] = to_np(got["lse"][b, h])
            r = ref(b, h)
            if rows:
                check_bf16(f"{name} b={b} h={h} o", g["o"][:rows], r["o"][:rows])
                check_lse(f"{name} b={b} h={h} lse", g["lse"][:rows], r["lse"][:rows])
                check_bf16(f"{name} b={b} h={h} dq", g["dq"][:rows], r["dq"][:rows])
            if keys:
                check_bf16(f"{name} b={b} h={h} dk", g["dk"][:keys], r["dk"][:keys])
                check_bf16(f"{name} b={b} h={h} dv", g["dv"][:keys], r["dv"][:keys])
            assert np.all(g["o"][rows:] == 0) and np.all(g["dq"][rows:] == 0), f"{name} b={b}: query padding not zero"
            assert np.all(np.isneginf(g["lse"][rows:])), f"{name} b={b}: LSE padding not -inf"
            assert np.all(g["dk"][keys:] == 0) and np.all(g["dv"][keys:] == 0), f"{name} b={b}: key padding not zero"


# lengths: full, ragged, a single row, no keys, no queries, keys longer than queries
SEQ_Q = [300, 1, 131, 64, 0, 257, 45]
SEQ_K = [300, 1, 131, 0, 77, 190, 300]


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_varlen_small(dims, causal, deterministic):
    dqk, dv = dims
    B, T, NH = len(SEQ_Q), 300, 2
    say(f"case varlen small d{dqk}x{dv} causal={causal} det={deterministic}")
    cpu, gpu, lens = _inputs(B, T, NH, dqk, dv, 61, SEQ_Q, SEQ_K)
    scale = 1.0 / np.sqrt(dqk)
    got = _run(gpu, lens, causal, scale, deterministic)
    ref = attn_ref.attn_ref_varlen(cpu["q"], cpu["k"], cpu["v"], cpu["do"], SEQ_Q, SEQ_K, causal, scale)
    _compare(f"varlen d{dqk} causal={causal}", got, lambda b, h: {
        "o": ref["o"][b, :, h], "lse": ref["lse"][b, h], "dq": ref["dq"][b, :, h],
        "dk": ref["dk"][b, :, h], "dv": ref["dv"][b, :, h]}, SEQ_Q, SEQ_K)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_varlen_full_lengths_equal_dense(causal):
    """Every length equal to T: the padded-batch path runs the same per-item arithmetic
    as the dense path, so forward and deterministic backward agree bit for bit."""
    B, T, NH, d = 3, 333, 2, 128
    say(f"case varlen = dense causal={causal}")
    w = workloads.Workload("vd", B, NH, T, d, d, causal, 67)
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    g = {n: cpu[n].to(dev) for n in ("q", "k", "v", "do")}
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    o1, l1 = attn.fwd(g["q"], g["k"], g["v"], causal, w.scale)
    o2, l2 = attn.fwd_varlen(g["q"], g["k"], g["v"], lens, lens, causal, w.scale)
    d1 = attn.bwd(g["q"], g["k"], g["v"], o1, l1, g["do"], causal, w.scale, True)
    d2 = attn.bwd_varlen(g["q"], g["k"], g["v"], o1, l1, g["do"], lens, lens, causal, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(d1, d2):
        assert torch.equal(a, b)


def test_varlen_deterministic_repeats():
    B, T, NH, d = 4, 700, 2, 128
    sq, sk = [700, 513, 64, 1], [700, 600, 700, 5]
    say("case varlen determinism")
    _, gpu, lens = _inputs(B, T, NH, d, d, 71, sq, sk)
    first = _run(gpu, lens, True, 1.0 / np.sqrt(d), True)
    for _ in range(3):
        again = _run(gpu, lens, True, 1.0 / np.sqrt(d), True)
        for n in first:
            assert torch.equal(first[n], again[n]), n


def test_varlen_length_mix_sampled():
    """A batch of 8 causal sequences of mixed lengths up to 2048 (d = 128), the shape of
    a padded training batch; sampled heads against the oracle."""
    B, T, NH, d = 8, 2048, 4, 128
    rng = np.random.default_rng(73)
    sq = [int(x) for x in rng.integers(1, T + 1, size=B)]
    sq[0] = T
    sk = list(sq)
    say(f"case varlen length mix {sq}")
    cpu, gpu, lens = _inputs(B, T, NH, d, d, 79, sq, sk)
    scale = 1.0 / np.sqrt(d)
    got = _run(gpu, lens, True, scale, True)
    heads = [(0, 0), (3, 1), (5, 2), (7, 3)]
    refs = {}
    for b, h in heads:
        lq = sq[b]
        r = attn_ref.head_backward(*(attn_ref.to_f64(cpu[n][b, :lq, h]) for n in ("q", "k", "v", "do")),
                                   scale, True)
        pad = lambda x: np.concatenate([x, np.zeros((T - lq,) + x.shape[1:])])  # noqa: E731
        refs[(b, h)] = {"dq": pad(r[0]), "dk": pad(r[1]), "dv": pad(r[2]), "o": pad(r[3]),
                        "lse": np.concatenate([r[4], np.full(T - lq, -np.inf)])}
    _compare("varlen mix", got, lambda b, h: refs[(b, h)], sq, sk, heads=heads)


@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_varlen_decode_shape(dims):
    """Inference forward of one decode step per sequence: a single query row (or a few)
    against each sequence's own key length, non-causal, without the softmax stats
    (lse = NULL, the inference mode of [SA8 1.2, 1.3]).  O against the oracle; equal bit
    for bit to the same call with stats."""
    dqk, dv = dims
    T, NH = 2500, 3
    sq = [1, 1, 1, 4, 1, 0]
    sk = [2500, 1, 777, 2049, 64, 300]
    B = len(sq)
    say(f"case varlen decode d{dqk}x{dv} seq_q={sq} seq_kv={sk}")
    cpu, gpu, lens = _inputs(B, T, NH, dqk, dv, 83, sq, sk)
    scale = 1.0 / np.sqrt(dqk)
    o_inf, lse_inf = attn.fwd_varlen(gpu["q"], gpu["k"], gpu["v"], lens[0], lens[1], False, scale, return_lse=False)
    o_tr, _ = attn.fwd_varlen(gpu["q"], gpu["k"], gpu["v"], lens[0], lens[1], False, scale)
    torch.cuda.synchronize()
    assert lse_inf is None
    assert torch.equal(o_inf, o_tr)
    ref = attn_ref.attn_ref_varlen(cpu["q"], cpu["k"], cpu["v"], None, sq, sk, False, scale)
    for b in range(B):
        g = to_np(o_inf[b])
        rows = sq[b] if sk[b] > 0 else 0
        for h in range(NH):
            if rows:
                check_bf16(f"decode b={b} h={h} o", g[:rows, h], ref["o"][b, :rows, h])
        assert np.all(g[rows:] == 0), f"decode b={b}: padding rows not zero"


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
def test_varlen_workload_full_size(deterministic):
    """The padded-batch workload the bench times (eight sequences padded to T = 8192,
    lengths from workloads.varlen_lengths), in the same calls, on sampled (b, h) heads:
    the full-length sequence, the shortest and one more, each against the oracle at its
    own length; padding rows must be zero (LSE -inf)."""
    w = workloads.WORKLOADS["varlen"]
    n = [int(x) for x in workloads.varlen_lengths(w)]
    heads = sorted({(0, 0), (int(np.argmin(n)), w.NH - 1), (w.B - 1, 5)})
    say(f"case varlen workload det={deterministic} lengths={n} heads={heads}")
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    gpu = {k: cpu[k].to(dev) for k in ("q", "k", "v", "do")}
    lens = torch.tensor(n, dtype=torch.int32, device=dev)
    got = _run(gpu, (lens, lens), w.causal, w.scale, deterministic)
    del gpu
    refs = {}
    for b, h in heads:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        r = attn_ref.attn_ref_varlen(cpu["q"][sl], cpu["k"][sl], cpu["v"][sl], cpu["do"][sl], n[b:b + 1], n[b:b + 1],
                                     w.causal, w.scale)
        refs[(b, h)] = {"o": r["o"][0, :, 0], "dq": r["dq"][0, :, 0], "dk": r["dk"][0, :, 0], "dv": r["dv"][0, :, 0],
                        "lse": r["lse"][0, 0]}
    _compare("varlen workload", got, lambda b, h: refs[(b, h)], n, n, heads=heads)
