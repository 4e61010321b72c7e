"""Plain fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module.  The GPU library never calls it and shares
no code with it.

Pages cited (by title and section):
  [SA8]  "ops(8)：self-attention 的 CUDA 实现及优化 (下) - 深度分析"
         section 2.1 (matrix-product and softmax derivatives, the attention backward
         chain), section 2.2 (CPU reference loop nest), Appendix A.1-A.3 (formula sheet).
  [FAT]  "FlashAttention Triton实现中的内存访问模式优化与寄存器分配策略"
         section 2.2 (one program per query block; running max and running sum).
  [2CTA] "深度学习反向传播优化：2-CTA MMA模式与内存访问优化"
         sections 5.1, 5.2 (mask patterns, causal and block-sparse, as modules).

What is computed (the plain definition, S and P materialised, float64 throughout):
  forward   S = scale * Q K^T                      [SA8 2.1, A.1]
            causal: S[i, j] = -inf for key j > query i (the loop bound t2 <= t of
            the CPU reference in [SA8 2.2]; top-left aligned, T_q == T_k)
            P = softmax(S) row by row                [SA8 2.1, A.1]
            sliding window (causal only, window W >= 1): additionally S[i, j] = -inf
            for i - j >= W, so query i sees keys i-W+1 .. i — a banded mask, the
            simplest of the block-sparse mask patterns of [2CTA 5.1, 5.2]
            ALiBi (causal only; the use_alibi_mask option of [SA8 1.2]): additionally
            S[i, j] -= m_h (i - j) with the head slopes m_h = 2^(-8 (h+1) / NH) of the
            linear-bias scheme (the page names the option but not its slopes; this
            geometric sequence is the reading taken)
            block-sparse mask (the block-sparse pattern of [2CTA 5.1, 5.2], composed
            with the causal mask as an independent module): a map M over
            (query block, key block) pairs of `block` x `block` elements;
            additionally S[i, j] = -inf where M[i // block, j // block] == 0.  The
            pages give no format; this map, ANDed with the causal mask, is the
            reading taken.  A row left with no allowed key gets P = 0, O = 0,
            LSE = -inf and zero gradients (the logsumexp of an empty set)
            dropout (the `dropout` option of [SA8 1.2], whose form the page does not
            give; inverted dropout on the attention weights is the reading taken):
            O = (P * Z) V / (1 - p) with the keep mask Z of philox_keep, the LSE from the
            undropped P; backward dV = (P * Z)^T dO / (1 - p), dP = (dO V^T) * Z / (1 - p)
            key bias (the `bias` option among the SDPA options of [SA8 1.2], whose
            shape the page does not give; a per-key bias broadcast over the queries
            is the reading taken): additionally S[i, j] += bias[j] (finite values;
            a large negative value masks a key)
            O = P V                                  [SA8 2.1, A.1]
            LSE_i = m_i + ln(sum_j exp(S_ij - m_i)),  m_i = max_j S_ij
            (the pages' "softmax stats" [SA8 1.2, 1.3] are never defined; this
            natural-log logsumexp is the reading taken)
  backward  dV = P^T dO                              [SA8 2.1 step 1, A.2]
            dP = dO V^T                              [SA8 2.1 step 2, A.2]
            dS = P * (dP - (dP * P) 1)               [SA8 2.1 step 3, A.2]
            dQ = scale * dS K                        [SA8 2.1 step 4, A.2]
            dK = scale * dS^T Q                      [SA8 2.1 step 5, A.2]
            dbias[j] = sum_i dS[i, j]  (S is linear in the bias with slope 1; summed
            further over the heads and batches that share one bias row)

Layout: every tensor argument is (B, T, NH, d) (token-major, heads inside), the layout
of the pages' output O; LSE is (B, NH, T).  Inputs may be numpy arrays or torch
tensors of any float dtype; they are converted exactly to float64.

Memory: for long sequences the per-head work is split into blocks of query rows.
Each block still forms complete rows of S and P, and the sums over query rows that
make up dV and dK are added block after block, so the arithmetic is the definition
above with its sum over queries split into consecutive parts.  Under the causal mask
the columns past a block's last query are left out: their P entries are exactly zero.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "to_f64",
    "head_forward",
    "head_backward",
    "attn_ref_fwd",
    "attn_ref_bwd",
    "attn_ref_heads",
    "attn_ref_varlen",
    "attn_ref_blocksparse",
    "attn_ref_keybias",
    "attn_ref_fwd_fp8",
    "e4m3_to_f64",
    "philox4x32_10",
    "philox_keep",
    "dropout_threshold",
    "attn_ref_dropout",
    "attn_ref_bwd_loop",
    "alibi_slopes",
]


def to_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a (CPU or GPU) torch tensor to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only reached when a torch tensor is passed

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, row0: int, window: int = 0,
            slope: float = 0.0) -> np.ndarray:
    """S = scale * Q K^T for query rows row0 .. row0+len(q)-1 against all given keys,
    with the causal mask (key index > query index -> -inf), when window > 0 the
    sliding-window mask (query index - key index >= window -> -inf), and when slope > 0
    the linear bias -slope * (query index - key index)."""
    S = scale * (q @ k.T)
    if causal:
        qi = np.arange(row0, row0 + q.shape[0])[:, None]
        kj = np.arange(k.shape[0])[None, :]
        if slope:
            S = S - slope * (qi - kj)
        S = np.where(kj > qi, -np.inf, S)
        if window > 0:
            S = np.where(qi - kj >= window, -np.inf, S)
    return S


def alibi_slopes(NH: int) -> np.ndarray:
    """Head slopes of the linear-bias (ALiBi) mask: m_h = 2^(-8 (h + 1) / NH)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / NH) for h in range(NH)])


def _check_window(causal: bool, window: int, slope: float = 0.0):
    if window < 0 or (window > 0 and not causal):
        raise ValueError("a sliding window needs the causal mask and window >= 1 (0 = none)")
    if slope < 0 or (slope > 0 and not causal):
        raise ValueError("the ALiBi bias needs the causal mask and a slope > 0")


def _softmax_rows(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise softmax and natural-log logsumexp, shifted by the row maximum."""
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def _softmax_rows_or_empty(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """_softmax_rows on the rows holding at least one allowed key; a row with none gets
    P = 0 and LSE = -inf."""
    empty = np.all(S == -np.inf, axis=1)
    if not empty.any():
        return _softmax_rows(S)
    P = np.zeros_like(S)
    lse = np.full(S.shape[0], -np.inf)
    if (~empty).any():
        P[~empty], lse[~empty] = _softmax_rows(S[~empty])
    return P, lse


def _block_allowed(block_map: Optional[np.ndarray], block: int, r0: int, r1: int, nk: int):
    """Element mask of query rows r0 .. r1-1 against keys 0 .. nk-1 from a block map:
    element (i, j) is allowed iff block_map[i // block, j // block] != 0.  None: no map."""
    if block_map is None:
        return None
    qi = np.arange(r0, r1) // block
    kj = np.arange(nk) // block
    return np.asarray(block_map)[qi[:, None], kj[None, :]] != 0


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                 block_rows: Optional[int] = None, window: int = 0,
                 slope: float = 0.0, block_map: Optional[np.ndarray] = None,
                 block: int = 128, key_bias: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """One head: q (T, d_qk), k (Tk, d_qk), v (Tk, d_v) float64 -> O (T, d_v), LSE (T,).
    Tk >= 1 may differ from T (padded batches); the causal mask stays top-left.
    block_map: (ceil(T / block), ceil(Tk / block)) block-sparse map or None."""
    _check_window(causal, window, slope)
    T, Tk = q.shape[0], k.shape[0]
    br = T if block_rows is None else block_rows
    O = np.empty((T, v.shape[1]))
    lse = np.empty(T)
    for r0 in range(0, T, br):
        r1 = min(T, r0 + br)
        nk = min(r1, Tk) if causal else Tk  # keys past the last query are all masked
        S = _scores(q[r0:r1], k[:nk], scale, causal, r0, window, slope)
        if key_bias is not None:
            S = S + key_bias[None, :nk]
        allowed = _block_allowed(block_map, block, r0, r1, nk)
        if allowed is not None:
            S = np.where(allowed, S, -np.inf)
        P, lse[r0:r1] = _softmax_rows_or_empty(S)
        O[r0:r1] = P @ v[:nk]
    return O, lse


def head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                  causal: bool, block_rows: Optional[int] = None, window: int = 0, slope: float = 0.0,
                  block_map: Optional[np.ndarray] = None, block: int = 128,
                  key_bias: Optional[np.ndarray] = None, keep: Optional[np.ndarray] = None, p_drop: float = 0.0):
    """One head: returns dQ, dK, dV and also O, LSE and D = (dP * P) 1 (all float64).
    q, do have T rows, k, v have Tk >= 1 rows (Tk may differ from T).  The bias is a
    constant of the inputs: it changes P but adds no term to the gradients; neither does
    the block map (a row with no allowed key has P = 0 and gets zero gradients).  With a
    key bias (Tk,) the result also holds dbias (Tk,) = sum over queries of dS, as an
    eighth entry.  keep (T, Tk) bool: dropout with probability p_drop, the kept weights
    scaled by 1 / (1 - p_drop) (O and the gradients; LSE and D as without it)."""
    _check_window(causal, window, slope)
    T, Tk = q.shape[0], k.shape[0]
    br = T if block_rows is None else block_rows
    O = np.empty((T, v.shape[1]))
    lse = np.empty(T)
    D = np.empty(T)
    dQ = np.empty_like(q)
    dbias = np.zeros(Tk)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for r0 in range(0, T, br):
        r1 = min(T, r0 + br)
        nk = min(r1, Tk) if causal else Tk
        S = _scores(q[r0:r1], k[:nk], scale, causal, r0, window, slope)
        if key_bias is not None:
            S = S + key_bias[None, :nk]
        allowed = _block_allowed(block_map, block, r0, r1, nk)
        if allowed is not None:
            S = np.where(allowed, S, -np.inf)
        P, lse[r0:r1] = _softmax_rows_or_empty(S)
        Pk = P if keep is None else P * (keep[r0:r1, :nk] / (1.0 - p_drop))  # weights after dropout
        O[r0:r1] = Pk @ v[:nk]
        dV[:nk] += Pk.T @ do[r0:r1]                     # dV = P^T dO
        dP = do[r0:r1] @ v[:nk].T                       # dP = dO V^T
        if keep is not None:
            dP = dP * (keep[r0:r1, :nk] / (1.0 - p_drop))  # through the dropout
        Dr = (dP * P).sum(axis=1)                       # (dP * P) 1
        dS = P * (dP - Dr[:, None])                     # dS = P * (dP - (dP * P) 1)
        dQ[r0:r1] = scale * (dS @ k[:nk])               # dQ = dS K / sqrt(d_k)
        dK[:nk] += scale * (dS.T @ q[r0:r1])            # dK = dS^T Q / sqrt(d_k)
        D[r0:r1] = Dr
        if key_bias is not None:
            dbias[:nk] += dS.sum(axis=0)                # dbias_j = sum_i dS_ij
    if key_bias is not None:
        return dQ, dK, dV, O, lse, D, dbias
    return dQ, dK, dV, O, lse, D


def _block_rows(T: int, width: int) -> int:
    # keep each block's S/P/dP/dS at a few hundred MB
    return max(1, min(T, (1 << 25) // max(T, 1) // max(1, width // 64)))


def attn_ref_fwd(q, k, v, causal: bool, scale: Optional[float] = None, window: int = 0, alibi: bool = False):
    """Forward over (B, T, NH, d) tensors.  Returns O (B, T, NH, d_v) and LSE (B, NH, T)
    in float64."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, T, NH, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    slopes = alibi_slopes(NH) if alibi else np.zeros(NH)
    O = np.empty((B, T, NH, v.shape[3]))
    lse = np.empty((B, NH, T))
    br = _block_rows(T, dqk)
    for b in range(B):
        for h in range(NH):
            O[b, :, h], lse[b, h] = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal, br, window,
                                                 slopes[h])
    return O, lse


def attn_ref_bwd(q, k, v, do, causal: bool, scale: Optional[float] = None, window: int = 0, alibi: bool = False):
    """Backward over (B, T, NH, d) tensors.  Returns a dict with dq, dk, dv
    (B, T, NH, d), o (B, T, NH, d_v), lse and D (B, NH, T), all float64."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, T, NH, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    slopes = alibi_slopes(NH) if alibi else np.zeros(NH)
    out = {
        "dq": np.empty((B, T, NH, dqk)),
        "dk": np.empty((B, T, NH, dqk)),
        "dv": np.empty((B, T, NH, v.shape[3])),
        "o": np.empty((B, T, NH, v.shape[3])),
        "lse": np.empty((B, NH, T)),
        "D": np.empty((B, NH, T)),
    }
    br = _block_rows(T, dqk)
    for b in range(B):
        for h in range(NH):
            r = head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal, br, window, slopes[h])
            for name, x in zip(("dq", "dk", "dv", "o"), r[:4]):
                out[name][b, :, h] = x
            out["lse"][b, h], out["D"][b, h] = r[4], r[5]
    return out


def attn_ref_heads(q, k, v, do, causal: bool, scale: Optional[float] = None,
                   heads: Sequence[Tuple[int, int]] = (), window: int = 0, alibi: bool = False):
    """Forward and backward of selected (b, h) heads of (B, T, NH, d) tensors; only
    those heads are converted to float64.  Returns {(b, h): {"dq", "dk", "dv", "o":
    (T, d) arrays, "lse", "D": (T,) arrays}}."""
    dqk = q.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    T = q.shape[1]
    br = _block_rows(T, dqk)
    slopes = alibi_slopes(q.shape[2]) if alibi else np.zeros(q.shape[2])
    res = {}
    for b, h in heads:
        b, h = int(b), int(h)
        qh, kh, vh, dh = (np.ascontiguousarray(to_f64(x[b, :, h])) for x in (q, k, v, do))
        r = head_backward(qh, kh, vh, dh, scale, causal, br, window, slopes[h])
        res[(b, h)] = dict(zip(("dq", "dk", "dv", "o", "lse", "D"), r))
    return res


def attn_ref_blocksparse(q, k, v, do, block_map, causal: bool, scale: Optional[float] = None, block: int = 128,
                         heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Block-sparse attention over (B, T, NH, d) tensors.  block_map is indexed
    [b, h, query block, key block] (any of its two leading dimensions may have size 1,
    which broadcasts) with ceil(T / block) blocks along each of the last two; element
    (i, j) of head (b, h) is allowed iff block_map[b, h, i // block, j // block] != 0 and,
    when causal, j <= i.  do may be None (forward only).  Returns the dict of
    attn_ref_bwd (o, lse, dq, dk, dv, D) for every head, or for the selected `heads`
    {(b, h): {...}} as attn_ref_heads does."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    do = None if do is None else to_f64(do)
    B, T, NH, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    bm = np.asarray(block_map)
    nb = (T + block - 1) // block
    if bm.ndim != 4 or bm.shape[0] not in (1, B) or bm.shape[1] not in (1, NH) or bm.shape[2:] != (nb, nb):
        raise ValueError(f"block_map must be (B or 1, NH or 1, {nb}, {nb}), got {bm.shape}")
    br = _block_rows(T, dqk)

    def one(b, h):
        m = bm[b if bm.shape[0] > 1 else 0, h if bm.shape[1] > 1 else 0]
        if do is None:
            o, lse = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal, br, block_map=m, block=block)
            return {"o": o, "lse": lse}
        r = head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal, br, block_map=m,
                          block=block)
        return dict(zip(("dq", "dk", "dv", "o", "lse", "D"), r))

    if heads is not None:
        return {(int(b), int(h)): one(int(b), int(h)) for b, h in heads}
    out = {"o": np.empty((B, T, NH, v.shape[3])), "lse": np.empty((B, NH, T))}
    if do is not None:
        out.update(dq=np.empty((B, T, NH, dqk)), dk=np.empty((B, T, NH, dqk)), dv=np.empty((B, T, NH, v.shape[3])),
                   D=np.empty((B, NH, T)))
    for b in range(B):
        for h in range(NH):
            r = one(b, h)
            for name, x in r.items():
                if name in ("lse", "D"):
                    out[name][b, h] = x
                else:
                    out[name][b, :, h] = x
    return out


def attn_ref_keybias(q, k, v, do, bias, causal: bool, scale: Optional[float] = None,
                     heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Attention with a key bias over (B, T, NH, d) tensors: S = scale Q K^T + bias, the
    bias indexed [b, h, j] with any of its two leading dimensions of size 1 (shared by
    the batches / heads).  do may be None (forward only).  Returns the dict of
    attn_ref_bwd plus "dbias" of the bias's own shape: sum over queries of dS, summed over
    the batches and heads that share a bias row.  With `heads`, only those heads, as
    {(b, h): {...}} with each head's own (T,) dbias contribution."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    do = None if do is None else to_f64(do)
    bias = to_f64(bias)
    B, T, NH, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    if bias.ndim != 3 or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, NH) or bias.shape[2] != T:
        raise ValueError(f"bias must be (B or 1, NH or 1, {T}), got {bias.shape}")
    br = _block_rows(T, dqk)

    def one(b, h):
        kb = bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]
        if do is None:
            o, lse = head_forward(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal, br, key_bias=kb)
            return {"o": o, "lse": lse}
        r = head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal, br, key_bias=kb)
        return dict(zip(("dq", "dk", "dv", "o", "lse", "D", "dbias"), r))

    if heads is not None:
        return {(int(b), int(h)): one(int(b), int(h)) for b, h in heads}
    out = {"o": np.empty((B, T, NH, v.shape[3])), "lse": np.empty((B, NH, T))}
    if do is not None:
        out.update(dq=np.empty((B, T, NH, dqk)), dk=np.empty((B, T, NH, dqk)), dv=np.empty((B, T, NH, v.shape[3])),
                   D=np.empty((B, NH, T)), dbias=np.zeros(bias.shape))
    for b in range(B):
        for h in range(NH):
            r = one(b, h)
            for name, x in r.items():
                if name in ("lse", "D"):
                    out[name][b, h] = x
                elif name == "dbias":
                    out["dbias"][b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0] += x
                else:
                    out[name][b, :, h] = x
    return out


def e4m3_to_f64(codes) -> np.ndarray:
    """Decodes 8-bit floating-point codes of the e4m3 format (1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 is subnormal, m / 8 * 2^-6; the code
    with every exponent and mantissa bit set is NaN; there is no infinity; largest finite
    value 448) to float64, exactly."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def attn_ref_fwd_fp8(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, causal: bool,
                     scale: Optional[float] = None):
    """Forward on fp8 (e4m3) inputs with per-tensor descale factors: the real inputs are
    descale * decode(code), and the result is the plain definition (attn_ref_fwd) on them,
    in float64.  q8, k8, v8 are (B, T, NH, d) uint8 code arrays.  P is not rounded here:
    the GPU's rounding of P to e4m3 is an error of the kernel, bounded in its tolerance."""
    q = e4m3_to_f64(q8) * descale_q
    k = e4m3_to_f64(k8) * descale_k
    v = e4m3_to_f64(v8) * descale_v
    return attn_ref_fwd(q, k, v, causal, scale)


# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2,
# 3", SC'11): a 128-bit counter and a 64-bit key; ten rounds of two 32x32 -> 64-bit
# multiplications, the key bumped by the Weyl constants before every round but the first.
PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85


def philox4x32_10(ctr, key) -> np.ndarray:
    """ctr: (..., 4) integers < 2^32, key: two integers < 2^32 -> (..., 4) uint32."""
    c = [np.asarray(ctr, dtype=np.uint64)[..., i] for i in range(4)]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(PHILOX_W1)) & mask
        p0 = np.uint64(PHILOX_M0) * c[0]
        p1 = np.uint64(PHILOX_M1) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & mask, (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & mask]
    return np.stack(c, axis=-1).astype(np.uint32)


def dropout_threshold(p_drop: float) -> int:
    """A weight is kept when its 16-bit random value is >= this (p quantised to 1/65536)."""
    if not 0.0 <= p_drop < 1.0:
        raise ValueError("the dropout probability must be in [0, 1)")
    return min(65536, int(np.floor(p_drop * 65536.0 + 0.5)))


def philox_keep(b: int, h: int, NH: int, T: int, p_drop: float, seed: int, offset: int) -> np.ndarray:
    """Keep mask (T, T) of head (b, h): element (i, j) takes 16-bit value j % 8 of the
    Philox4x32-10 output at counter (j // 8, i, b * NH + h, offset), key (seed mod 2^32,
    seed // 2^32): output word (j % 8) // 2, low half for even j, high half for odd j; it is
    kept iff that value >= dropout_threshold(p_drop)."""
    i = np.arange(T, dtype=np.uint64)[:, None]
    g = (np.arange((T + 7) // 8, dtype=np.uint64))[None, :]
    ctr = np.stack(np.broadcast_arrays(g, i, np.uint64(b * NH + h), np.uint64(offset & 0xFFFFFFFF)), axis=-1)
    x = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))  # (T, ngroups, 4)
    u = np.empty((T, x.shape[1], 8), dtype=np.uint32)
    for e in range(8):
        u[:, :, e] = (x[:, :, e // 2] >> (16 * (e % 2))) & 0xFFFF
    return (u.reshape(T, -1)[:, :T] >= dropout_threshold(p_drop))


def attn_ref_dropout(q, k, v, do, p_drop: float, seed: int, offset: int, causal: bool,
                     scale: Optional[float] = None, heads: Optional[Sequence[Tuple[int, int]]] = None):
    """Attention with dropout on the weights over (B, T, NH, d) tensors, the keep mask of
    each head from philox_keep.  Returns the dict of attn_ref_bwd (o, lse, dq, dk, dv, D),
    or for the selected `heads` {(b, h): {...}}."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, T, NH, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    br = _block_rows(T, dqk)

    def one(b, h):
        keep = philox_keep(b, h, NH, T, p_drop, seed, offset)
        r = head_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal, br, keep=keep,
                          p_drop=p_drop)
        return dict(zip(("dq", "dk", "dv", "o", "lse", "D"), r))

    if heads is not None:
        return {(int(b), int(h)): one(int(b), int(h)) for b, h in heads}
    out = {"dq": np.empty((B, T, NH, dqk)), "dk": np.empty((B, T, NH, dqk)), "dv": np.empty((B, T, NH, v.shape[3])),
           "o": np.empty((B, T, NH, v.shape[3])), "lse": np.empty((B, NH, T)), "D": np.empty((B, NH, T))}
    for b in range(B):
        for h in range(NH):
            for name, x in one(b, h).items():
                if name in ("lse", "D"):
                    out[name][b, h] = x
                else:
                    out[name][b, :, h] = x
    return out


def attn_ref_varlen(q, k, v, do, seq_q, seq_k, causal: bool, scale: Optional[float] = None):
    """Padded batches: the padding mask with per-batch lengths seq_len_q and seq_len_kv
    among the SDPA options of [SA8 1.2].  Batch b uses query rows 0 .. seq_q[b]-1 and
    key/value rows 0 .. seq_k[b]-1 of its (T, NH, d) slices; everything past them is
    padding and never read.  Within a batch the result is the plain definition above on
    the unpadded rows (causal: key j allowed for query i iff j <= i, top-left).

    Readings where the page is silent: padding query rows get O = 0, LSE = -inf and
    dQ = 0; padding key rows get dK = dV = 0; a query with no allowed key (seq_k[b] = 0)
    gets O = 0, LSE = -inf (the logsumexp of an empty set) and zero gradients.
    do may be None (forward only).  Returns a dict o, lse (and dq, dk, dv), float64,
    in the (B, T, NH, d) / (B, NH, T) layouts.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    do = None if do is None else to_f64(do)
    B, T, NH, dqk = q.shape
    dv_w = v.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    out = {"o": np.zeros((B, T, NH, dv_w)), "lse": np.full((B, NH, T), -np.inf)}
    if do is not None:
        out.update(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v))
    for b in range(B):
        lq, lk = int(seq_q[b]), int(seq_k[b])
        if lq == 0 or lk == 0:
            continue
        for h in range(NH):
            qh, kh, vh = q[b, :lq, h], k[b, :lk, h], v[b, :lk, h]
            if do is None:
                out["o"][b, :lq, h], out["lse"][b, h, :lq] = head_forward(qh, kh, vh, scale, causal)
                continue
            dq, dk, dv, o, lse, _ = head_backward(qh, kh, vh, do[b, :lq, h], scale, causal)
            out["o"][b, :lq, h], out["lse"][b, h, :lq] = o, lse
            out["dq"][b, :lq, h], out["dk"][b, :lk, h], out["dv"][b, :lk, h] = dq, dk, dv
    return out


def attn_ref_bwd_loop(q, k, v, do, causal: bool, scale: Optional[float] = None, window: int = 0,
                      alibi: bool = False, allowed=None, key_bias=None, keep=None, p_drop: float = 0.0):
    """Independent loop formulation for small T (T <= 64), written from the softmax
    Jacobian dy_i/dx_j = y_i (delta_ij - y_j) [SA8 2.1, A.3] and the per-(b, t, h)
    loop nest of the CPU reference in [SA8 2.2]:

      for each (b, t, h):
        att[t2]      = softmax over t2 (t2 <= t when causal; also t2 > t - window
                       when window > 0) of scale * <q_t, k_t2> - m_h (t - t2)
                       (m_h = 0 without the ALiBi bias)
        datt[t2]     = <v_t2, do_t>                       (gradient w.r.t. att)
        dv_t2       += att[t2] * do_t
        dpreatt[t3]  = scale * sum_t2 att[t2] (delta(t2, t3) - att[t3]) datt[t2]
        dq_t        += sum_t2 dpreatt[t2] k_t2
        dk_t2       += dpreatt[t2] q_t

    The scale sits inside dpreatt, so dq and dk take no second factor.  It does not
    share a line with head_forward/head_backward and serves to pin them.
    allowed: None, or a predicate allowed(b, h, t, t2) -> bool; keys it refuses are
    left out of the row like keys outside the window (a row with no key left gets
    att = 0, o = 0, lse = -inf and no gradient).
    key_bias: None, or a function key_bias(b, h, t2) added to preatt[t2]; the gradient
    with respect to it is dpreatt / scale (preatt is scale * q.k plus the bias), summed
    into dbias[b, h, t2], returned as a sixth value.
    keep: None, or a predicate keep(b, h, t, t2) -> bool: dropout, the value path uses
    att[t2] * z[t2] with z = keep / (1 - p_drop) (o and dv), and the gradient w.r.t. att
    is datt[t2] * z[t2].
    Returns dq, dk, dv, o (B, T, NH, d) and lse (B, NH, T) in float64.
    """
    _check_window(causal, window, 1.0 if alibi else 0.0)
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    B, T, NH, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    slopes = alibi_slopes(NH) if alibi else np.zeros(NH)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros((B, T, NH, v.shape[3]))
    lse = np.zeros((B, NH, T))
    dbias = np.zeros((B, NH, T))
    for b in range(B):
        for t in range(T):
            for h in range(NH):
                last = t + 1 if causal else T
                first = max(0, t - window + 1) if window > 0 else 0
                # forward row by loops: preatt, max, exp, sum, normalise (keys before
                # `first` get -inf scores: exp gives exactly 0, so they add nothing)
                pre = [scale * float(np.dot(q[b, t, h], k[b, t2, h])) - slopes[h] * (t - t2)
                       + (key_bias(b, h, t2) if key_bias is not None else 0.0)
                       if t2 >= first and (allowed is None or allowed(b, h, t, t2)) else -math.inf
                       for t2 in range(last)]
                mx = max(pre)
                if mx == -math.inf:  # no key left in this row
                    lse[b, h, t] = -math.inf
                    continue
                ex = [np.exp(p - mx) for p in pre]
                tot = sum(ex)
                att = [e / tot for e in ex]
                lse[b, h, t] = mx + np.log(tot)
                z = [1.0 if keep is None else (1.0 / (1.0 - p_drop) if keep(b, h, t, t2) else 0.0)
                     for t2 in range(last)]
                for t2 in range(last):
                    o[b, t, h] += att[t2] * z[t2] * v[b, t2, h]
                # backward through O = (att z) . V
                datt = [float(np.dot(v[b, t2, h], do[b, t, h])) * z[t2] for t2 in range(last)]
                for t2 in range(last):
                    dv[b, t2, h] += att[t2] * z[t2] * do[b, t, h]
                # backward through the softmax by its Jacobian
                dpre = [0.0] * last
                for t2 in range(last):
                    for t3 in range(last):
                        ind = 1.0 if t2 == t3 else 0.0
                        dpre[t3] += scale * att[t2] * (ind - att[t3]) * datt[t2]
                # backward through preatt = scale * q . k (+ bias)
                for t2 in range(last):
                    dq[b, t, h] += dpre[t2] * k[b, t2, h]
                    dk[b, t2, h] += dpre[t2] * q[b, t, h]
                    dbias[b, h, t2] += dpre[t2] / scale
    if key_bias is not None:
        return dq, dk, dv, o, lse, dbias
    return dq, dk, dv, o, lse
