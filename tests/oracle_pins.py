"""Pins for the CPU oracle: checks against facts that the pages and the mathematics
fix, not against the oracle's own formulas.

Every pin takes ``ref``, an object with the oracle's public functions
(attn_ref_fwd, attn_ref_bwd, attn_ref_bwd_loop), so that the same pins can be run
against copies of the oracle with a planted mistake (test_oracle.py checks that
each planted mistake trips at least one pin).

Pages cited:
  [SA8] "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析", sections 1.2 (padding mask,
        seq_len_q, seq_len_kv; ALiBi mask), 2.1, 2.2, A.1-A.3.
  [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化", sections 5.1, 5.2 (causal and
        block-sparse mask patterns).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

import workloads

TINY = workloads.WORKLOADS["tiny"]


def _inputs(B, T, NH, dqk, dv, seed, sigma=1.0):
    w = workloads.Workload("pin", B, NH, T, dqk, dv, True, seed, sigma=sigma)
    x = workloads.make_inputs(w)
    return [x[n].to(torch.float64).numpy() for n in ("q", "k", "v", "do")]


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    bound = rtol * max(np.max(np.abs(b)) if b.size else 0.0, 1e-300) + atol
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= bound, f"{what}: max err {err:.3e} > {bound:.3e}"


# ---------------------------------------------------------------------------------
# 1. Central finite differences of f(Q, K, V) = sum(O * dO)       [SA8 2.1 chain rule]
# ---------------------------------------------------------------------------------
def pin_finite_differences(ref, causal: bool, T: int = 16, h: float = 1e-5):
    """dQ, dK, dV of the oracle equal central differences of sum(O * dO).

    Tiny shape (B=1, NH=2, d=64) at T=16, float64; every input element is perturbed.
    """
    q, k, v, do = _inputs(1, T, 2, TINY.d_qk, TINY.d_v, TINY.seed)
    scale = 1.0 / math.sqrt(q.shape[-1])
    g = ref.attn_ref_bwd(q, k, v, do, causal, scale)

    def f(qq, kk, vv):
        o, _ = ref.attn_ref_fwd(qq, kk, vv, causal, scale)
        return float(np.sum(o * do))

    for name, x, grad in (("dq", q, g["dq"]), ("dk", k, g["dk"]), ("dv", v, g["dv"])):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = [q, k, v]; args_m = [q, k, v]
            pos = {"dq": 0, "dk": 1, "dv": 2}[name]
            args_p[pos] = xp; args_m[pos] = xm
            fd[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(grad, fd, rtol=1e-6, atol=1e-9, what=f"finite differences {name} causal={causal}")


# ---------------------------------------------------------------------------------
# 2. Matrix form against the Jacobian loop form                    [SA8 2.2, A.3]
# ---------------------------------------------------------------------------------
def pin_loop_form(ref, causal: bool, T: int = 23, dqk: int = 16, dv: int = 24):
    q, k, v, do = _inputs(1, T, 2, dqk, dv, 777)
    scale = 0.37
    g = ref.attn_ref_bwd(q, k, v, do, causal, scale)
    dq, dk, dv_, o, lse = ref.attn_ref_bwd_loop(q, k, v, do, causal, scale)
    for name, a, b in (("o", g["o"], o), ("lse", g["lse"], lse), ("dq", g["dq"], dq),
                       ("dk", g["dk"], dk), ("dv", g["dv"], dv_)):
        _close(a, b, rtol=1e-12, what=f"loop form {name} causal={causal}")


# ---------------------------------------------------------------------------------
# 3. Softmax invariants                                             [SA8 2.1]
# ---------------------------------------------------------------------------------
def pin_softmax_invariants(ref, causal: bool, T: int = 40):
    """With V = I (d_v = T), O is P itself: rows sum to 1, entries are >= 0, and
    under the causal mask P_ij = 0 for j > i.  With dO = I as well, dV = P^T dO = P^T
    (the closed form dV = P^T dO).  D = (dP * P) 1 equals rowsum(dO * O)."""
    q, k, _, _ = _inputs(1, T, 2, 32, 32, 4242, sigma=1.5)
    eye = np.broadcast_to(np.eye(T)[None, :, None, :], (1, T, 2, T)).copy()
    scale = 1.0 / math.sqrt(32)
    g = ref.attn_ref_bwd(q, k, eye, eye, causal, scale)
    P = g["o"]                                   # (1, T, 2, T): row t, key j
    _close(P.sum(axis=-1), np.ones((1, T, 2)), rtol=1e-13, what="rows of P sum to 1")
    assert np.all(P >= 0.0), "P has negative entries"
    if causal:
        mask = np.triu(np.ones((T, T), dtype=bool), 1)
        assert np.all(P[0, :, 0][mask] == 0.0) and np.all(P[0, :, 1][mask] == 0.0), \
            "causal P has weight above the diagonal"
    # dV = P^T dO with dO = I:  dV[j, :] = P[:, j]
    for h in range(2):
        _close(g["dv"][0, :, h], P[0, :, h].T, rtol=1e-13, what="dV = P^T dO")
    # D identity on a random dO
    q, k, v, do = _inputs(2, T, 3, 16, 8, 99)
    g = ref.attn_ref_bwd(q, k, v, do, causal, 0.5)
    D2 = np.einsum("btnd,btnd->bnt", do, g["o"])
    _close(g["D"], D2, rtol=1e-12, what="D = rowsum(dP*P) = rowsum(dO*O)")


def pin_shift_invariance(ref, causal: bool, T: int = 29):
    """K -> K + 1 c^T adds the same constant to every allowed key of a row of S, so
    P, O, LSE - scale <q_i, c> and dV are unchanged, and dQ is unchanged because
    each row of dS sums to zero (rowsum(dS) = 0)."""
    q, k, v, do = _inputs(1, T, 2, 16, 16, 31337)
    c = np.linspace(-1.0, 2.0, 16)
    scale = 0.25
    g0 = ref.attn_ref_bwd(q, k, v, do, causal, scale)
    g1 = ref.attn_ref_bwd(q, k + c, v, do, causal, scale)
    _close(g1["o"], g0["o"], rtol=1e-12, what="shift: O")
    _close(g1["dv"], g0["dv"], rtol=1e-12, what="shift: dV")
    _close(g1["dq"], g0["dq"], rtol=1e-10, atol=1e-13, what="shift: dQ (rowsum dS = 0)")
    shift = scale * np.einsum("btnd,d->bnt", q, c)
    _close(g1["lse"] - shift, g0["lse"], rtol=1e-12, what="shift: LSE")


# ---------------------------------------------------------------------------------
# 4. Closed forms and special cases
# ---------------------------------------------------------------------------------
def pin_zero_queries(ref, causal: bool, T: int = 37):
    """Q = 0 makes every score 0: P is uniform over the allowed keys, so O_i is the
    mean of V over those keys and LSE_i = ln(count)."""
    _, k, v, do = _inputs(1, T, 2, 16, 12, 5)
    q = np.zeros_like(k)
    o, lse = ref.attn_ref_fwd(q, k, v, causal, 0.3)
    cnt = np.arange(1, T + 1) if causal else np.full(T, T)
    if causal:
        mean = np.cumsum(v, axis=1) / cnt[None, :, None, None]
    else:
        mean = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    _close(o, mean, rtol=1e-13, what="Q=0: O = mean of allowed V")
    _close(lse, np.broadcast_to(np.log(cnt)[None, None, :], lse.shape), rtol=1e-13,
           what="Q=0: LSE = ln(count)")


def pin_single_token(ref, causal: bool):
    """T = 1: P = [1], so O = V, LSE = scale <q, k>, dV = dO, dQ = dK = 0."""
    q, k, v, do = _inputs(2, 1, 3, 16, 8, 11)
    g = ref.attn_ref_bwd(q, k, v, do, causal, 0.7)
    _close(g["o"], v, rtol=1e-15, what="T=1: O = V")
    _close(g["lse"], 0.7 * np.einsum("btnd,btnd->bnt", q, k), rtol=1e-14, what="T=1: LSE")
    _close(g["dv"], do, rtol=1e-15, what="T=1: dV = dO")
    assert np.max(np.abs(g["dq"])) <= 1e-14 and np.max(np.abs(g["dk"])) <= 1e-14, "T=1: dQ, dK != 0"


def pin_causal_first_row(ref, T: int = 19):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale <q_0, k_0>, dQ_0 = 0."""
    q, k, v, do = _inputs(1, T, 2, 16, 16, 12)
    g = ref.attn_ref_bwd(q, k, v, do, True, 0.4)
    _close(g["o"][:, 0], v[:, 0], rtol=1e-15, what="causal row 0: O")
    _close(g["lse"][:, :, 0], 0.4 * np.einsum("bnd,bnd->bn", q[:, 0], k[:, 0]), rtol=1e-14,
           what="causal row 0: LSE")
    assert np.max(np.abs(g["dq"][:, 0])) <= 1e-14, "causal row 0: dQ != 0"


def pin_two_keys_closed_form(ref):
    """T = 2, d = 1, no mask: softmax over two scores is the logistic function,
    P_i0 = sigma(s_i0 - s_i1) with sigma(x) = 1 / (1 + e^-x), so
      O_i   = v_1 + (v_0 - v_1) sigma(a q_i),        a = scale (k_0 - k_1)
      LSE_i = s_i1 + ln(1 + e^(s_i0 - s_i1))
      dQ_i  = dO_i (v_0 - v_1) sigma'(a q_i) a,       sigma' = sigma (1 - sigma)
      dV_j  = sum_i P_ij dO_i.
    Values chosen by hand; everything below is that closed form, evaluated directly."""
    q = np.array([0.5, -1.25]).reshape(1, 2, 1, 1)
    k = np.array([2.0, -0.75]).reshape(1, 2, 1, 1)
    v = np.array([3.0, -1.0]).reshape(1, 2, 1, 1)
    do = np.array([0.25, 2.0]).reshape(1, 2, 1, 1)
    scale = 0.8
    g = ref.attn_ref_bwd(q, k, v, do, False, scale)
    qs, ks, vs, ds = q.ravel(), k.ravel(), v.ravel(), do.ravel()
    a = scale * (ks[0] - ks[1])
    sig = 1.0 / (1.0 + np.exp(-a * qs))
    o = vs[1] + (vs[0] - vs[1]) * sig
    s0, s1 = scale * qs * ks[0], scale * qs * ks[1]
    lse = s1 + np.log1p(np.exp(s0 - s1))
    dq = ds * (vs[0] - vs[1]) * sig * (1 - sig) * a
    P = np.stack([sig, 1 - sig], axis=1)         # P[i, j]
    dv = P.T @ ds
    # dK_j = sum_i dS_ij scale q_i with dS_i0 = -dS_i1 = sig (1 - sig) (v_0 - v_1) dO_i
    dS0 = sig * (1 - sig) * (vs[0] - vs[1]) * ds
    dk = np.array([np.sum(dS0 * scale * qs), -np.sum(dS0 * scale * qs)])
    _close(g["o"].ravel(), o, rtol=1e-15, what="two keys: O")
    _close(g["lse"].ravel(), lse, rtol=1e-15, what="two keys: LSE")
    _close(g["dq"].ravel(), dq, rtol=1e-14, what="two keys: dQ")
    _close(g["dk"].ravel(), dk, rtol=1e-14, what="two keys: dK")
    _close(g["dv"].ravel(), dv, rtol=1e-15, what="two keys: dV")


def pin_worked_example(ref, case: str):
    """The hand-worked three-token example of tests/golden/worked_example.json: Q = I,
    scale = 1 and K chosen so that exp(S) is a small integer matrix, which makes P, O,
    dV, D and dS exact rationals (worked out by hand in the file) and LSE the log of
    an integer."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_example.json")
    with open(path) as fh:
        ex = json.load(fh)
    want = ex["cases"][case]
    frac = lambda m: np.array([[float(Fraction(x)) for x in row] for row in m]) if isinstance(m[0], list) \
        else np.array([float(Fraction(x)) for x in m])
    a = np.array(ex["a"], dtype=np.float64)
    q = np.eye(3).reshape(1, 3, 1, 3)
    k = np.log(a).T.reshape(1, 3, 1, 3)             # K[j][c] = ln a[c][j]
    v = np.array(ex["v"], dtype=np.float64).reshape(1, 3, 1, 2)
    do = np.array(ex["do"], dtype=np.float64).reshape(1, 3, 1, 2)
    g = ref.attn_ref_bwd(q, k, v, do, case == "causal", 1.0)
    ds = frac(want["ds"])
    _close(g["o"][0, :, 0], frac(want["o"]), rtol=1e-15, atol=1e-15, what=f"worked {case}: O")
    _close(g["lse"][0, 0], np.log(np.array(want["lse_ln_of"], dtype=np.float64)), rtol=1e-15, atol=1e-15,
           what=f"worked {case}: LSE")
    _close(g["dv"][0, :, 0], frac(want["dv"]), rtol=1e-15, atol=1e-15, what=f"worked {case}: dV")
    _close(g["dk"][0, :, 0], ds.T, rtol=1e-14, atol=1e-15, what=f"worked {case}: dK")
    # dQ[i][c] = sum_j dS[i][j] ln a[c][j], from the hand-derived dS
    _close(g["dq"][0, :, 0], ds @ np.log(a).T, rtol=1e-14, atol=1e-15, what=f"worked {case}: dQ")
    # the forward alone gives the same O and LSE
    o, lse = ref.attn_ref_fwd(q, k, v, case == "causal", 1.0)
    _close(o[0, :, 0], frac(want["o"]), rtol=1e-15, atol=1e-15, what=f"worked {case}: forward O")
    _close(lse[0, 0], np.log(np.array(want["lse_ln_of"], dtype=np.float64)), rtol=1e-15, atol=1e-15,
           what=f"worked {case}: forward LSE")


# ---------------------------------------------------------------------------------
# 5. Library cross-check: torch float64 autograd through softmax(scale Q K^T) V
# ---------------------------------------------------------------------------------
def pin_torch_autograd(ref, causal: bool, B=2, T=37, NH=3, dqk=16, dv=24):
    q, k, v, do = _inputs(B, T, NH, dqk, dv, 2024)
    scale = 1.0 / math.sqrt(dqk)
    g = ref.attn_ref_bwd(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = torch.einsum("bind,bjnd->bnij", tq, tk) * scale
    if causal:
        s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bnij,bjnd->bind", p, tv)
    lse = torch.logsumexp(s, dim=-1)
    o.backward(torch.tensor(do))
    for name, a, b in (("o", g["o"], o.detach()), ("lse", g["lse"], lse.detach()),
                       ("dq", g["dq"], tq.grad), ("dk", g["dk"], tk.grad), ("dv", g["dv"], tv.grad)):
        _close(a, b.numpy(), rtol=1e-12, what=f"torch autograd {name} causal={causal}")


# ---------------------------------------------------------------------------------
# 6. Padded batches: the padding mask with seq_len_q / seq_len_kv   [SA8 1.2]
# ---------------------------------------------------------------------------------
def _check_varlen_padding(r, seq_q, seq_k, what):
    """Padding query rows: O = 0, LSE = -inf, dQ = 0; padding key rows: dK = dV = 0;
    a batch with no keys: O = 0, LSE = -inf everywhere."""
    B, T = r["o"].shape[:2]
    for b in range(B):
        lq, lk = int(seq_q[b]), int(seq_k[b])
        empty = lq if lk > 0 else 0
        assert np.all(r["o"][b, empty:] == 0), f"{what}: O padding b={b}"
        assert np.all(np.isneginf(r["lse"][b, :, empty:])), f"{what}: LSE padding b={b}"
        assert np.all(np.isfinite(r["lse"][b, :, :empty])), f"{what}: LSE rows b={b}"
        if "dq" in r:
            assert np.all(r["dq"][b, empty:] == 0), f"{what}: dQ padding b={b}"
            kept = lk if lq > 0 else 0
            assert np.all(r["dk"][b, kept:] == 0) and np.all(r["dv"][b, kept:] == 0), f"{what}: dK/dV padding b={b}"


def pin_varlen_full_length(ref, causal: bool):
    """Every length equal to T: the padded-batch result is the dense one."""
    q, k, v, do = _inputs(2, 21, 2, 16, 24, 31)
    g = ref.attn_ref_bwd(q, k, v, do, causal, 0.4)
    r = ref.attn_ref_varlen(q, k, v, do, [21, 21], [21, 21], causal, 0.4)
    for name in ("o", "lse", "dq", "dk", "dv"):
        _close(r[name], g[name], rtol=1e-12, what=f"varlen full length {name} causal={causal}")


VARLEN_Q = [9, 4, 6, 0, 9]
VARLEN_K = [5, 9, 0, 3, 9]


def pin_varlen_loops(ref, causal: bool):
    """Forward of padded batches (query and key lengths differ, one batch without keys,
    one without queries) by scalar loops over (i, j): for i < Lq_b the allowed keys are
    j < Lk_b (and j <= i under the causal mask); O_i = sum_j e^(s_ij - m_i) v_j /
    sum_j e^(s_ij - m_i), LSE_i = m_i + ln sum_j e^(s_ij - m_i)."""
    q, k, v, _ = _inputs(5, 9, 2, 4, 3, 41)
    scale = 0.7
    r = ref.attn_ref_varlen(q, k, v, None, VARLEN_Q, VARLEN_K, causal, scale)
    _check_varlen_padding(r, VARLEN_Q, VARLEN_K, f"varlen loops causal={causal}")
    for b in range(5):
        for h in range(2):
            for i in range(VARLEN_Q[b]):
                js = [j for j in range(VARLEN_K[b]) if not (causal and j > i)]
                if not js:
                    continue
                s_ = [scale * sum(q[b, i, h, c] * k[b, j, h, c] for c in range(4)) for j in js]
                m = max(s_)
                e = [math.exp(x - m) for x in s_]
                tot = math.fsum(e)
                o = [math.fsum(e[n] * v[b, j, h, c] for n, j in enumerate(js)) / tot for c in range(3)]
                _close(r["o"][b, i, h], o, rtol=1e-13, what=f"varlen loops O b={b} i={i}")
                _close([r["lse"][b, h, i]], [m + math.log(tot)], rtol=1e-14, what=f"varlen loops LSE b={b} i={i}")


def pin_varlen_padding_ignored(ref, causal: bool):
    """Rows past the lengths are never read: NaN there changes nothing."""
    q, k, v, do = _inputs(5, 9, 2, 4, 3, 43)
    a = ref.attn_ref_varlen(q, k, v, do, VARLEN_Q, VARLEN_K, causal)
    q2, k2, v2, do2 = (x.copy() for x in (q, k, v, do))
    for b in range(5):
        q2[b, VARLEN_Q[b]:] = np.nan
        do2[b, VARLEN_Q[b]:] = np.nan
        k2[b, VARLEN_K[b]:] = np.nan
        v2[b, VARLEN_K[b]:] = np.nan
    c = ref.attn_ref_varlen(q2, k2, v2, do2, VARLEN_Q, VARLEN_K, causal)
    _check_varlen_padding(c, VARLEN_Q, VARLEN_K, f"varlen NaN padding causal={causal}")
    for name in ("o", "dq", "dk", "dv"):
        np.testing.assert_array_equal(a[name], c[name], err_msg=f"varlen NaN padding {name}")
    np.testing.assert_array_equal(a["lse"], c["lse"])


def pin_varlen_finite_differences(ref, causal: bool, h: float = 1e-6):
    """dQ, dK, dV of padded batches with different query and key lengths equal central
    differences of sum(O * dO) over every input element (padding included, where the
    derivative is zero)."""
    q, k, v, do = _inputs(2, 6, 1, 3, 2, 47)
    sq, sk = [6, 3], [4, 6]
    g = ref.attn_ref_varlen(q, k, v, do, sq, sk, causal, 0.6)

    def f(qq, kk, vv):
        return float(np.sum(ref.attn_ref_varlen(qq, kk, vv, None, sq, sk, causal, 0.6)["o"] * do))

    for pos, name in enumerate(("dq", "dk", "dv")):
        x = (q, k, v)[pos]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p, args_m = [q, k, v], [q, k, v]
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p[pos], args_m[pos] = xp, xm
            fd[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(g[name], fd, rtol=1e-6, atol=1e-9, what=f"varlen finite differences {name} causal={causal}")


def pin_varlen_zero_queries(ref, causal: bool):
    """Q = 0: O_i is the mean of V over the allowed keys and LSE_i = ln(count), with
    count = min(i + 1, Lk) under the causal mask and Lk otherwise."""
    _, k, v, _ = _inputs(5, 9, 2, 4, 3, 53)
    q = np.zeros((5, 9, 2, 4))
    r = ref.attn_ref_varlen(q, k, v, None, VARLEN_Q, VARLEN_K, causal)
    for b in range(5):
        lk = VARLEN_K[b]
        if lk == 0:
            continue
        for i in range(VARLEN_Q[b]):
            n = min(i + 1, lk) if causal else lk
            _close(r["o"][b, i], v[b, :n].mean(axis=0), rtol=1e-14, what=f"varlen zero queries O b={b} i={i}")
            _close(r["lse"][b, :, i], np.full(2, math.log(n)), rtol=1e-14, atol=1e-15,
                   what=f"varlen zero queries LSE b={b} i={i}")


# ---------------------------------------------------------------------------------
# Sliding-window (banded causal) mask: query i sees keys i-W+1 .. i.  A mask pattern of
# the block-sparse family of [2CTA 5.1, 5.2]; pinned by reductions and closed forms.
# ---------------------------------------------------------------------------------
def pin_window_wide_is_causal(ref):
    """A window at least T wide masks nothing beyond the causal mask."""
    q, k, v, do = _inputs(2, 21, 2, 16, 24, 861)
    a = ref.attn_ref_bwd(q, k, v, do, True)
    for W in (21, 40):
        b = ref.attn_ref_bwd(q, k, v, do, True, window=W)
        for n in ("o", "lse", "dq", "dk", "dv"):
            _close(b[n], a[n], rtol=1e-15, atol=1e-15, what=f"window {W} = causal {n}")


def pin_window_one(ref):
    """W = 1: every query sees only its own key, so P = I: O = V, LSE_i = scale <q_i, k_i>,
    dV = dO, and dS = 0 (a softmax over one entry has zero derivative): dQ = dK = 0."""
    q, k, v, do = _inputs(1, 17, 2, 16, 24, 863)
    scale = 0.37
    r = ref.attn_ref_bwd(q, k, v, do, True, scale, window=1)
    _close(r["o"], v, rtol=1e-15, what="window 1 O")
    _close(r["dv"], do, rtol=1e-15, what="window 1 dV")
    _close(r["lse"], scale * np.einsum("bthd,bthd->bht", q, k), rtol=1e-14, what="window 1 LSE")
    assert np.max(np.abs(r["dq"])) < 1e-13 and np.max(np.abs(r["dk"])) < 1e-13, "window 1: dQ, dK not zero"


def pin_window_zero_queries(ref):
    """Q = 0: P is uniform over the W most recent keys: O_i = mean of V rows
    max(0, i-W+1) .. i, LSE_i = ln(min(i + 1, W))."""
    _, k, v, _ = _inputs(1, 30, 2, 16, 24, 865)
    q = np.zeros_like(k)
    for W in (1, 4, 7):
        o, lse = ref.attn_ref_fwd(q, k, v, True, window=W)
        for i in range(30):
            lo = max(0, i - W + 1)
            _close(o[0, i], v[0, lo:i + 1].mean(axis=0), rtol=1e-14, what=f"window {W} zero queries O row {i}")
            _close(lse[0, :, i], np.full(2, math.log(i + 1 - lo)), rtol=1e-14, atol=1e-15,
                   what=f"window {W} zero queries LSE row {i}")


def pin_window_loops(ref):
    """Matrix form against the scalar loop nest, with the window in the loop bounds."""
    q, k, v, do = _inputs(2, 23, 2, 16, 24, 867)
    for W in (2, 5, 11):
        dq, dk, dv, o, lse = ref.attn_ref_bwd_loop(q, k, v, do, True, window=W)
        r = ref.attn_ref_bwd(q, k, v, do, True, window=W)
        for n, x in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o), ("lse", lse)):
            _close(r[n], x, rtol=1e-12, atol=1e-14, what=f"window {W} loop form {n}")


def pin_window_finite_differences(ref, h: float = 1e-6):
    """dQ, dK, dV under the window equal central differences of sum(O * dO)."""
    q, k, v, do = _inputs(1, 12, 1, 8, 8, 869)
    W = 4
    r = ref.attn_ref_bwd(q, k, v, do, True, window=W)

    def f(qq, kk, vv):
        return float(np.sum(ref.attn_ref_fwd(qq, kk, vv, True, window=W)[0] * do))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            args_m = [xm if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(r[name], g, rtol=1e-6, atol=1e-8, what=f"window finite differences {name}")


# ---------------------------------------------------------------------------------
# ALiBi bias (use_alibi_mask of [SA8 1.2]): S_ij -= m_h (i - j) under the causal mask.
# ---------------------------------------------------------------------------------
def pin_alibi_slopes(ref):
    """The linear-bias slopes for 8 heads are 1/2, 1/4, ..., 1/256; for 16 heads the
    sequence 2^-0.5, 2^-1, ..., 2^-8."""
    _close(ref.alibi_slopes(8), [1 / 2 ** (h + 1) for h in range(8)], rtol=1e-15, what="alibi slopes NH=8")
    _close(ref.alibi_slopes(16), [2 ** (-(h + 1) / 2) for h in range(16)], rtol=1e-15, what="alibi slopes NH=16")


def pin_alibi_zero_queries(ref):
    """Q = 0: row i weighs key i - d by r^d with r = e^(-m_h), so O_i = sum_d r^d V_(i-d) / Z_i
    and LSE_i = ln Z_i with the geometric sum Z_i = (1 - r^(i+1)) / (1 - r)."""
    _, k, v, _ = _inputs(1, 25, 4, 16, 24, 871)
    q = np.zeros_like(k)
    o, lse = ref.attn_ref_fwd(q, k, v, True, alibi=True)
    for h in range(4):
        r = math.exp(-(2.0 ** (-8.0 * (h + 1) / 4)))
        for i in range(25):
            z = (1 - r ** (i + 1)) / (1 - r)
            num = sum(r ** d * v[0, i - d, h] for d in range(i + 1))
            _close(o[0, i, h], num / z, rtol=1e-13, what=f"alibi zero queries O h={h} row {i}")
            _close(lse[0, h, i], math.log(z), rtol=1e-13, atol=1e-15, what=f"alibi zero queries LSE h={h} row {i}")


def pin_alibi_loops(ref):
    """Matrix form against the scalar loop nest with the bias in the scores."""
    q, k, v, do = _inputs(2, 23, 4, 16, 24, 873)
    dq, dk, dv, o, lse = ref.attn_ref_bwd_loop(q, k, v, do, True, alibi=True)
    r = ref.attn_ref_bwd(q, k, v, do, True, alibi=True)
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o), ("lse", lse)):
        _close(r[n], x, rtol=1e-12, atol=1e-14, what=f"alibi loop form {n}")


def pin_alibi_finite_differences(ref, h: float = 1e-6):
    """dQ, dK, dV with the bias equal central differences of sum(O * dO): the bias is a
    constant, so it changes P but adds no gradient term."""
    q, k, v, do = _inputs(1, 12, 2, 8, 8, 875)
    r = ref.attn_ref_bwd(q, k, v, do, True, alibi=True)

    def f(qq, kk, vv):
        return float(np.sum(ref.attn_ref_fwd(qq, kk, vv, True, alibi=True)[0] * do))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            args_m = [xm if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(r[name], g, rtol=1e-6, atol=1e-8, what=f"alibi finite differences {name}")


# ---------------------------------------------------------------------------------
# Block-sparse map (the block-sparse mask pattern of [2CTA 5.1, 5.2]): element (i, j)
# allowed iff map[i // block, j // block] != 0, ANDed with the causal mask.  The pins use
# small blocks so that short sequences span several of them.
# ---------------------------------------------------------------------------------
def _bs_map(B, NH, nb, seed, density=0.5):
    rng = np.random.default_rng(seed)
    return (rng.random((B, NH, nb, nb)) < density).astype(np.uint8)


def pin_blocksparse_all_ones_is_dense(ref):
    """A map with every block live masks nothing: dense (and, with the causal mask,
    causal) attention exactly."""
    q, k, v, do = _inputs(2, 37, 2, 16, 24, 881)
    for causal in (False, True):
        a = ref.attn_ref_bwd(q, k, v, do, causal)
        b = ref.attn_ref_blocksparse(q, k, v, do, np.ones((1, 1, 5, 5), np.uint8), causal, block=8)
        for n in ("o", "lse", "dq", "dk", "dv"):
            _close(b[n], a[n], rtol=1e-15, atol=1e-15, what=f"all-ones map causal={causal} {n}")


def pin_blocksparse_lower_triangle_is_causal(ref):
    """Without the causal flag, a block-lower-triangular map lets the keys of a query's
    own block through (up to the block's end), so it differs from causal attention; with
    the flag it equals causal attention.  Blocks above the diagonal hold nothing the causal
    mask allows, so removing them changes nothing."""
    q, k, v, do = _inputs(1, 40, 2, 16, 16, 883)
    tri = np.tril(np.ones((5, 5), np.uint8))[None, None]
    a = ref.attn_ref_bwd(q, k, v, do, True)
    b = ref.attn_ref_blocksparse(q, k, v, do, tri, True, block=8)
    for n in ("o", "lse", "dq", "dk", "dv"):
        _close(b[n], a[n], rtol=1e-15, atol=1e-15, what=f"lower-triangular map + causal {n}")
    c = ref.attn_ref_blocksparse(q, k, v, do, tri, False, block=8)
    assert np.max(np.abs(c["o"] - a["o"])) > 1e-3, "lower-triangular map without the causal flag equals causal"
    # row 7 (last of block 0) sees keys 0..7 either way; row 0 sees keys 0..7 only without it
    _close(c["o"][:, 7], a["o"][:, 7], rtol=1e-14, what="row 7 of block 0")


def pin_blocksparse_band_is_block_window(ref):
    """A band of w blocks on and below the diagonal, with the causal mask, lets query i see
    keys from the start of block i // b - w + 1 up to i: the element mask written out
    directly through the loop form's predicate."""
    q, k, v, do = _inputs(1, 45, 2, 8, 8, 885)
    b, nb, w = 6, 8, 3
    band = np.array([[1 if 0 <= r - c < w else 0 for c in range(nb)] for r in range(nb)], np.uint8)[None, None]
    dq, dk, dv, o, lse = ref.attn_ref_bwd_loop(
        q, k, v, do, True, allowed=lambda bb, hh, t, t2: t2 >= b * max(0, t // b - w + 1))
    r = ref.attn_ref_blocksparse(q, k, v, do, band, True, block=b)
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o), ("lse", lse)):
        _close(r[n], x, rtol=1e-12, atol=1e-14, what=f"band map loop form {n}")


def pin_blocksparse_random_map_loops(ref):
    """A random per-head map, causal and not, against the scalar loop nest with the map
    read element by element (map[b, h, t // block, t2 // block]); rows and key columns
    left with no live block are among the cases (the map has empty rows)."""
    q, k, v, do = _inputs(2, 27, 3, 8, 16, 887)
    blk = 4
    m = _bs_map(2, 3, 7, 888, density=0.45)
    m[0, 1, 2, :] = 0  # rows 8..11 of head (0, 1): no key at all
    m[1, 2, :, 3] = 0  # keys 12..15 of head (1, 2): seen by no query
    for causal in (False, True):
        dq, dk, dv, o, lse = ref.attn_ref_bwd_loop(
            q, k, v, do, causal, allowed=lambda bb, hh, t, t2: m[bb, hh, t // blk, t2 // blk] != 0)
        r = ref.attn_ref_blocksparse(q, k, v, do, m, causal, block=blk)
        for n, x in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o)):
            _close(r[n], x, rtol=1e-12, atol=1e-14, what=f"random map causal={causal} loop form {n}")
        fin = np.isfinite(lse)
        assert np.array_equal(fin, np.isfinite(r["lse"])), "rows without keys differ"
        _close(r["lse"][fin], lse[fin], rtol=1e-12, atol=1e-14, what=f"random map causal={causal} lse")
    r = ref.attn_ref_blocksparse(q, k, v, do, m, False, block=blk)
    assert np.all(r["o"][0, 8:12, 1] == 0) and np.all(r["lse"][0, 1, 8:12] == -np.inf), "empty rows: O, LSE"
    assert np.all(r["dq"][0, 8:12, 1] == 0), "empty rows: dQ"
    assert np.all(r["dk"][1, 12:16, 2] == 0) and np.all(r["dv"][1, 12:16, 2] == 0), "unseen keys: dK, dV"


def pin_blocksparse_zero_queries(ref):
    """Q = 0: P is uniform over the allowed keys: O_i is the mean of the V rows in the live
    blocks of row i's block (up to i when causal), LSE_i = ln(count)."""
    _, k, v, _ = _inputs(1, 30, 2, 16, 24, 889)
    q = np.zeros_like(k)
    blk = 5
    m = _bs_map(1, 1, 6, 890, density=0.6)
    m[0, 0, np.arange(6), np.arange(6)] = 1  # every row keeps its own block
    for causal in (False, True):
        r = ref.attn_ref_blocksparse(q, k, v, None, m, causal, block=blk)
        for i in range(30):
            keys = [j for j in range(30) if m[0, 0, i // blk, j // blk] and (not causal or j <= i)]
            _close(r["o"][0, i], v[0, keys].mean(axis=0), rtol=1e-14, what=f"map zero queries O row {i}")
            _close(r["lse"][0, :, i], np.full(2, math.log(len(keys))), rtol=1e-14, atol=1e-15,
                   what=f"map zero queries LSE row {i}")


def pin_blocksparse_finite_differences(ref, h: float = 1e-6):
    """dQ, dK, dV under a map (with an empty row block) equal central differences of
    sum(O * dO)."""
    q, k, v, do = _inputs(1, 12, 1, 8, 8, 891)
    m = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 0]], np.uint8)[None, None]
    r = ref.attn_ref_blocksparse(q, k, v, do, m, False, block=4)

    def f(qq, kk, vv):
        return float(np.sum(ref.attn_ref_blocksparse(qq, kk, vv, None, m, False, block=4)["o"] * do))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            args_m = [xm if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(r[name], g, rtol=1e-6, atol=1e-8, what=f"map finite differences {name}")


# ---------------------------------------------------------------------------------
# Key bias (the `bias` option of [SA8 1.2], read as a per-key bias broadcast over the
# queries): S_ij += bias_j; dbias_j = sum_i dS_ij.
# ---------------------------------------------------------------------------------
def _bias(B, NH, T, seed, sd=1.0):
    return np.random.default_rng(seed).standard_normal((B, NH, T)) * sd


def pin_keybias_zero_is_plain(ref):
    """A zero bias changes nothing, and dbias = sum over queries of dS sums to zero over
    the keys of each head (every row of dS sums to zero)."""
    q, k, v, do = _inputs(2, 29, 2, 16, 24, 901)
    for causal in (False, True):
        a = ref.attn_ref_bwd(q, k, v, do, causal)
        b = ref.attn_ref_keybias(q, k, v, do, np.zeros((2, 2, 29)), causal)
        for n in ("o", "lse", "dq", "dk", "dv"):
            _close(b[n], a[n], rtol=1e-15, atol=1e-15, what=f"zero bias causal={causal} {n}")
        _close(b["dbias"].sum(axis=2), np.zeros((2, 2)), rtol=0, atol=1e-12, what="sum of dbias over keys")


def pin_keybias_constant_shift(ref):
    """A bias equal for every key shifts each row of S by one constant: P, O and the
    gradients do not change, LSE moves by that constant (non-causal)."""
    q, k, v, do = _inputs(1, 31, 2, 16, 16, 903)
    a = ref.attn_ref_bwd(q, k, v, do, False)
    b = ref.attn_ref_keybias(q, k, v, do, np.full((1, 2, 31), 2.5), False)
    for n in ("o", "dq", "dk", "dv"):
        _close(b[n], a[n], rtol=1e-12, atol=1e-14, what=f"constant bias {n}")
    _close(b["lse"], a["lse"] + 2.5, rtol=1e-14, what="constant bias LSE")


def pin_keybias_loops(ref):
    """Matrix form against the scalar loop nest with the bias in preatt, dbias included,
    causal and not, per head and shared."""
    q, k, v, do = _inputs(2, 21, 3, 8, 16, 905)
    for shape in ((2, 3, 21), (1, 1, 21)):
        bias = _bias(*shape, 906, sd=2.0)
        for causal in (False, True):
            dq, dk, dv, o, lse, dbias = ref.attn_ref_bwd_loop(
                q, k, v, do, causal, key_bias=lambda b, h, t2: bias[b % shape[0], h % shape[1], t2])
            r = ref.attn_ref_keybias(q, k, v, do, bias, causal)
            for n, x in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o), ("lse", lse)):
                _close(r[n], x, rtol=1e-12, atol=1e-14, what=f"bias {shape} causal={causal} loop form {n}")
            want = dbias.sum(axis=(0, 1), keepdims=True) if shape[0] == 1 else dbias
            _close(r["dbias"], want, rtol=1e-12, atol=1e-14, what=f"bias {shape} causal={causal} dbias")


def pin_keybias_padding(ref):
    """A key-padding bias (0 on the first L keys, -1e9 on the rest) equals attention over
    the first L keys only; the padded keys get exactly zero dK, dV and dbias."""
    q, k, v, do = _inputs(1, 24, 2, 16, 16, 907)
    L = 17
    bias = np.zeros((1, 1, 24))
    bias[..., L:] = -1e9
    r = ref.attn_ref_keybias(q, k, v, do, bias, False)
    for h in range(2):
        o, lse = ref.head_forward(q[0, :, h], k[0, :L, h], v[0, :L, h], 1 / 4, False)
        _close(r["o"][0, :, h], o, rtol=1e-14, what="padding bias O")
        _close(r["lse"][0, h], lse, rtol=1e-14, what="padding bias LSE")
        g = ref.head_backward(q[0, :, h], k[0, :L, h], v[0, :L, h], do[0, :, h], 1 / 4, False)
        _close(r["dq"][0, :, h], g[0], rtol=1e-13, atol=1e-15, what="padding bias dQ")
        _close(r["dk"][0, :L, h], g[1], rtol=1e-13, atol=1e-15, what="padding bias dK")
    assert np.all(r["dk"][0, L:] == 0) and np.all(r["dv"][0, L:] == 0) and np.all(r["dbias"][..., L:] == 0)


def pin_keybias_finite_differences(ref, h: float = 1e-6):
    """dbias (and dQ, dK, dV) equal central differences of sum(O * dO)."""
    q, k, v, do = _inputs(1, 10, 2, 8, 8, 909)
    bias = _bias(1, 2, 10, 910)
    r = ref.attn_ref_keybias(q, k, v, do, bias, True)

    def f(qq, kk, vv, bb):
        return float(np.sum(ref.attn_ref_keybias(qq, kk, vv, None, bb, True)["o"] * do))

    ins = (("dq", q), ("dk", k), ("dv", v), ("dbias", bias))
    for name, x in ins:
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if n == name else y for n, y in ins]
            args_m = [xm if n == name else y for n, y in ins]
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(r[name], g, rtol=1e-6, atol=1e-8, what=f"bias finite differences {name}")


# ---------------------------------------------------------------------------------
# fp8 (e4m3) inputs: the decoder of the 8-bit format, and the forward on decoded inputs.
# ---------------------------------------------------------------------------------
def pin_e4m3_code_points(ref):
    """Code points fixed by the format: 0 and -0, the smallest subnormal 2^-9, the largest
    subnormal 7/8 * 2^-6, the smallest normal 2^-6, 1, 1.125 (one mantissa step), 2, the
    largest finite 448 (and its negative), NaN; positive codes increase monotonically."""
    d = ref.e4m3_to_f64
    pts = {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6, 0x08: 2.0 ** -6, 0x38: 1.0,
           0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in pts.items():
        assert d([c])[0] == v, f"e4m3 code {c:#x}: {d([c])[0]} != {v}"
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0]), "e4m3 NaN codes"
    pos = d(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0), "positive codes not increasing"


def pin_e4m3_library(ref):
    """Every code against torch's float8_e4m3fn (an independent implementation of the
    same format)."""
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ref.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(lib)), "NaN codes differ"
    ok = ~np.isnan(lib)
    assert np.array_equal(got[ok], lib[ok]), "e4m3 decode differs from the library"


def pin_fp8_forward_zero_queries(ref):
    """fp8 codes with descales: Q = 0 gives O_i = descale_v * mean of the decoded V rows up
    to i (causal) and LSE_i = ln(i + 1), whatever descale_q and descale_k are."""
    rng = np.random.default_rng(911)
    k8 = rng.integers(0, 0x7F, size=(1, 21, 2, 16), dtype=np.uint8)
    v8 = rng.integers(0, 0xFF, size=(1, 21, 2, 16), dtype=np.uint8)
    v8[(v8 & 0x7F) == 0x7F] = 0x38  # no NaN codes
    q8 = np.zeros_like(k8)
    o, lse = ref.attn_ref_fwd_fp8(q8, k8, v8, 3.0, 0.5, 0.25, True)
    vd = ref.e4m3_to_f64(v8) * 0.25
    for i in range(21):
        _close(o[0, i], vd[0, :i + 1].mean(axis=0), rtol=1e-14, atol=1e-300, what=f"fp8 zero queries O row {i}")
    _close(lse[0], np.log(np.arange(1, 22))[None, :].repeat(2, 0), rtol=1e-14, atol=1e-15, what="fp8 LSE")


# ---------------------------------------------------------------------------------
# Dropout (the dropout option of [SA8 1.2]): Philox4x32-10 keep masks and inverted
# dropout on the attention weights.
# ---------------------------------------------------------------------------------
def pin_philox_known_answers(ref):
    """The published known-answer vectors of Philox4x32-10 (Random123's test vectors)."""
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in kat:
        got = ref.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
        assert tuple(int(x) for x in got) == want, f"Philox4x32-10 {ctr}: {[hex(int(x)) for x in got]}"


def _philox_scalar(ctr, key):
    """Philox4x32-10 on Python integers: a second implementation for the keep-mask pin."""
    c, k = list(ctr), list(key)
    for r in range(10):
        if r:
            k = [(k[0] + 0x9E3779B9) & 0xFFFFFFFF, (k[1] + 0xBB67AE85) & 0xFFFFFFFF]
        a, b = 0xD2511F53 * c[0], 0xCD9E8D57 * c[2]
        c = [(b >> 32) ^ c[1] ^ k[0], b & 0xFFFFFFFF, (a >> 32) ^ c[3] ^ k[1], a & 0xFFFFFFFF]
    return c


def pin_keep_mask_element_by_element(ref):
    """The keep mask against its definition evaluated one element at a time: element (i, j)
    of head (b, h) is kept iff 16-bit value j % 8 of Philox4x32-10 at counter
    (j // 8, i, b NH + h, offset), key (seed low, seed high) is >= round(p 65536)."""
    NH, T, p, seed, offset = 3, 37, 0.3, 0x0123456789ABCDEF, 77
    thr = int(np.floor(p * 65536 + 0.5))
    rng = np.random.default_rng(5)
    for b, h in ((0, 0), (1, 2)):
        m = ref.philox_keep(b, h, NH, T, p, seed, offset)
        for _ in range(60):
            i, j = int(rng.integers(T)), int(rng.integers(T))
            x = _philox_scalar((j // 8, i, b * NH + h, offset), (seed & 0xFFFFFFFF, seed >> 32))
            u = (x[(j % 8) // 2] >> (16 * (j % 2))) & 0xFFFF
            assert bool(m[i, j]) == (u >= thr), f"keep mask ({b},{h},{i},{j})"


def pin_keep_fraction(ref):
    """Kept fraction of a large mask within five standard deviations of 1 - p."""
    for p in (0.1, 0.5, 0.9):
        m = np.concatenate([ref.philox_keep(0, h, 4, 256, p, 1234, 5) for h in range(4)])
        n = m.size
        assert abs(m.mean() - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n), f"keep fraction at p={p}: {m.mean()}"
    assert ref.philox_keep(0, 0, 1, 64, 0.0, 1, 0).all(), "p = 0 keeps everything"


def pin_dropout_zero_is_plain(ref):
    """p = 0 keeps every weight: plain attention, exactly."""
    q, k, v, do = _inputs(2, 23, 2, 16, 24, 921)
    for causal in (False, True):
        a = ref.attn_ref_bwd(q, k, v, do, causal)
        b = ref.attn_ref_dropout(q, k, v, do, 0.0, 99, 0, causal)
        for n in ("o", "lse", "dq", "dk", "dv"):
            _close(b[n], a[n], rtol=1e-15, atol=1e-15, what=f"dropout p=0 causal={causal} {n}")


def pin_dropout_loops(ref):
    """Matrix form against the scalar loop nest with the keep mask in the value path."""
    q, k, v, do = _inputs(2, 19, 2, 8, 16, 923)
    p, seed, off = 0.35, 0xDEADBEEF12345, 3
    masks = {(b, h): ref.philox_keep(b, h, 2, 19, p, seed, off) for b in range(2) for h in range(2)}
    for causal in (False, True):
        dq, dk, dv, o, lse = ref.attn_ref_bwd_loop(q, k, v, do, causal, keep=lambda b, h, t, t2: masks[(b, h)][t, t2],
                                                  p_drop=p)
        r = ref.attn_ref_dropout(q, k, v, do, p, seed, off, causal)
        for n, x in (("dq", dq), ("dk", dk), ("dv", dv), ("o", o), ("lse", lse)):
            _close(r[n], x, rtol=1e-12, atol=1e-14, what=f"dropout causal={causal} loop form {n}")


def pin_dropout_finite_differences(ref, h: float = 1e-6):
    """With the mask held fixed, dQ, dK, dV equal central differences of sum(O * dO)."""
    q, k, v, do = _inputs(1, 12, 1, 8, 8, 925)
    p, seed, off = 0.4, 42, 9
    r = ref.attn_ref_dropout(q, k, v, do, p, seed, off, True)

    def f(qq, kk, vv):
        return float(np.sum(ref.attn_ref_dropout(qq, kk, vv, do, p, seed, off, True)["o"] * do))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            args_m = [xm if n == name else y for n, y in (("dq", q), ("dk", k), ("dv", v))]
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
        _close(r[name], g, rtol=1e-6, atol=1e-8, what=f"dropout finite differences {name}")


ALL_PINS = [
    ("finite_differences_causal", lambda r: pin_finite_differences(r, True)),
    ("finite_differences_full", lambda r: pin_finite_differences(r, False)),
    ("loop_form_causal", lambda r: pin_loop_form(r, True)),
    ("loop_form_full", lambda r: pin_loop_form(r, False)),
    ("softmax_invariants_causal", lambda r: pin_softmax_invariants(r, True)),
    ("softmax_invariants_full", lambda r: pin_softmax_invariants(r, False)),
    ("shift_invariance_causal", lambda r: pin_shift_invariance(r, True)),
    ("shift_invariance_full", lambda r: pin_shift_invariance(r, False)),
    ("zero_queries_causal", lambda r: pin_zero_queries(r, True)),
    ("zero_queries_full", lambda r: pin_zero_queries(r, False)),
    ("single_token_causal", lambda r: pin_single_token(r, True)),
    ("single_token_full", lambda r: pin_single_token(r, False)),
    ("causal_first_row", pin_causal_first_row),
    ("two_keys_closed_form", pin_two_keys_closed_form),
    ("worked_example_full", lambda r: pin_worked_example(r, "full")),
    ("worked_example_causal", lambda r: pin_worked_example(r, "causal")),
    ("torch_autograd_causal", lambda r: pin_torch_autograd(r, True)),
    ("torch_autograd_full", lambda r: pin_torch_autograd(r, False)),
    ("varlen_full_length_causal", lambda r: pin_varlen_full_length(r, True)),
    ("varlen_full_length_full", lambda r: pin_varlen_full_length(r, False)),
    ("varlen_loops_causal", lambda r: pin_varlen_loops(r, True)),
    ("varlen_loops_full", lambda r: pin_varlen_loops(r, False)),
    ("varlen_padding_ignored_causal", lambda r: pin_varlen_padding_ignored(r, True)),
    ("varlen_padding_ignored_full", lambda r: pin_varlen_padding_ignored(r, False)),
    ("varlen_zero_queries_causal", lambda r: pin_varlen_zero_queries(r, True)),
    ("varlen_zero_queries_full", lambda r: pin_varlen_zero_queries(r, False)),
    ("finite_differences_varlen_causal", lambda r: pin_varlen_finite_differences(r, True)),
    ("finite_differences_varlen_full", lambda r: pin_varlen_finite_differences(r, False)),
    ("window_wide_is_causal", pin_window_wide_is_causal),
    ("window_one", pin_window_one),
    ("window_zero_queries", pin_window_zero_queries),
    ("window_loops", pin_window_loops),
    ("finite_differences_window", pin_window_finite_differences),
    ("blocksparse_all_ones_is_dense", pin_blocksparse_all_ones_is_dense),
    ("blocksparse_lower_triangle_is_causal", pin_blocksparse_lower_triangle_is_causal),
    ("blocksparse_band_is_block_window", pin_blocksparse_band_is_block_window),
    ("blocksparse_random_map_loops", pin_blocksparse_random_map_loops),
    ("blocksparse_zero_queries", pin_blocksparse_zero_queries),
    ("finite_differences_blocksparse", pin_blocksparse_finite_differences),
    ("keybias_zero_is_plain", pin_keybias_zero_is_plain),
    ("keybias_constant_shift", pin_keybias_constant_shift),
    ("keybias_loops", pin_keybias_loops),
    ("keybias_padding", pin_keybias_padding),
    ("finite_differences_keybias", pin_keybias_finite_differences),
    ("e4m3_code_points", pin_e4m3_code_points),
    ("e4m3_library", pin_e4m3_library),
    ("fp8_forward_zero_queries", pin_fp8_forward_zero_queries),
    ("philox_known_answers", pin_philox_known_answers),
    ("keep_mask_element_by_element", pin_keep_mask_element_by_element),
    ("keep_fraction", pin_keep_fraction),
    ("dropout_zero_is_plain", pin_dropout_zero_is_plain),
    ("dropout_loops", pin_dropout_loops),
    ("finite_differences_dropout", pin_dropout_finite_differences),
    ("alibi_slopes", pin_alibi_slopes),
    ("alibi_zero_queries", pin_alibi_zero_queries),
    ("alibi_loops", pin_alibi_loops),
    ("finite_differences_alibi", pin_alibi_finite_differences),
]
