"""GPU parity of the decode-step forward (attn_fwd_decode): Tq query rows per sequence
against that sequence's Tk-row key/value cache (or its first seq_len_kv[b] rows), no
causal mask, in the inference mode of "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析"
sections 1.2-1.3 (no stats) and with stats; against the fp64 oracle's plain definition
on each sequence's rows."""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import F16_ATOL, F16_RTOL, check_bf16, check_lse, say, to_np

pytestmark = pytest.mark.gpu

HEADDIMS = [(64, 64), (128, 128), (192, 128)]


def _case(B, NH, Tq, Tk, dqk, dv, seed, dtype=torch.bfloat16):
    q = workloads._randn((B, Tq, NH, dqk), seed, 1.0, dtype)
    k = workloads._randn((B, Tk, NH, dqk), seed + 1, 1.0, dtype)
    v = workloads._randn((B, Tk, NH, dv), seed + 2, 1.0, dtype)
    return q, k, v


def _check(q, k, v, lens, got_o, got_lse, scale, tol):
    B, Tq, NH, _ = q.shape
    for b in range(B):
        L = lens[b]
        for h in range(NH):
            g = to_np(got_o[b, :, h])
            if L == 0:
                assert np.all(g == 0), f"b={b}: no keys, O not zero"
                if got_lse is not None:
                    assert np.all(np.isneginf(to_np(got_lse[b, h]))), f"b={b}: no keys, LSE not -inf"
                continue
            o, lse = attn_ref.head_forward(attn_ref.to_f64(q[b, :, h]), attn_ref.to_f64(k[b, :L, h]),
                                           attn_ref.to_f64(v[b, :L, h]), scale, False)
            check_bf16(f"decode b={b} h={h} o", g, o, *tol)
            if got_lse is not None:
                check_lse(f"decode b={b} h={h} lse", to_np(got_lse[b, h]), lse)


@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 2500), (4, 100), (33, 777), (130, 300)])
@pytest.mark.parametrize("dims", HEADDIMS, ids=lambda d: f"d{d[0]}x{d[1]}")
def test_decode(dims, Tq, Tk):
    dqk, dv = dims
    B, NH = 4, 3
    say(f"case decode d{dqk}x{dv} Tq={Tq} Tk={Tk}")
    q, k, v = _case(B, NH, Tq, Tk, dqk, dv, 1100 + Tq + Tk)
    dev = torch.device("cuda:0")
    lens = [Tk, max(1, Tk // 3), 0, min(Tk, 65)]
    gq, gk, gv = q.to(dev), k.to(dev), v.to(dev)
    lk = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = 1.0 / np.sqrt(dqk)
    o_inf, none = attn.fwd_decode(gq, gk, gv, lk, scale)
    o_tr, lse = attn.fwd_decode(gq, gk, gv, lk, scale, return_lse=True)
    o_all, _ = attn.fwd_decode(gq, gk, gv, None, scale)
    torch.cuda.synchronize()
    assert none is None and torch.equal(o_inf, o_tr)
    _check(q, k, v, lens, o_tr, lse, scale, (2e-2, 2e-3))
    _check(q, k, v, [Tk] * B, o_all, None, scale, (2e-2, 2e-3))


def test_decode_fp16_and_bhtd():
    B, NH, Tq, Tk, d = 2, 4, 1, 3000, 128
    say("case decode fp16 bhtd")
    q, k, v = _case(B, NH, Tq, Tk, d, d, 1177, torch.float16)
    dev = torch.device("cuda:0")
    perm = lambda x: x.permute(0, 2, 1, 3).contiguous().to(dev)  # noqa: E731
    o, lse = attn.fwd_decode(perm(q), perm(k), perm(v), None, 1.0 / np.sqrt(d), return_lse=True, layout="bhtd")
    torch.cuda.synchronize()
    _check(q, k, v, [Tk] * B, o.permute(0, 2, 1, 3), lse, 1.0 / np.sqrt(d), (F16_RTOL, F16_ATOL))


@pytest.mark.parametrize("Tq", [1, 3])
def test_decode_key_split(Tq):
    """Few (b, h) pairs and a long cache: the keys are split into chunks of >= 1024 (here
    20 chunks) whose partial results are merged; caches of 20000, 5000, 1 and 1025 rows
    leave different chunks empty."""
    B, NH, Tk, d = 4, 2, 20000, 128
    say(f"case decode key split Tq={Tq}")
    q, k, v = _case(B, NH, Tq, Tk, d, d, 1201 + Tq)
    dev = torch.device("cuda:0")
    lens = [Tk, 5000, 1, 1025]
    lk = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = 1.0 / np.sqrt(d)
    o, lse = attn.fwd_decode(q.to(dev), k.to(dev), v.to(dev), lk, scale, return_lse=True)
    torch.cuda.synchronize()
    assert attn.load().attn_fwd_decode_workspace_bytes(B, NH, Tq, Tk, d, d) > 0
    _check(q, k, v, lens, o, lse, scale, (2e-2, 2e-3))
