"""Seeded synthetic attention workloads, shared by the tests, the bench and the smoke check.

This module only draws random inputs and describes shapes.  It holds none of the
attention arithmetic: both the GPU library and the CPU oracle receive the very same
bf16 tensors that it produces.

The pages measure on no dataset.  The FlashAttention-4 backward page ("2-CTA MMA mode
and memory-access optimisation", section 4.1) sweeps head dims 64/128/(192,128),
sequence lengths 1K-32K and keeps the total token count at 32K; the self-attention
CUDA page (section 1.3) uses a GPT-2 style packed (B, T, 3, NH, HS) QKV input.  The
configurations below stand in for those sweeps.

Recipe (every workload):
  * values are float32 standard normals from ``torch.Generator().manual_seed(seed + k)``,
    multiplied by sigma, then rounded to bfloat16 (round-to-nearest-even), or to
    float16 for the fp16 element type;
  * k = 0, 1, 2, 3 draw Q, K, V, dO in that order (separate layout), or
    k = 0 draws the packed QKV block and k = 1 draws dO (packed layout);
  * sigma is a standard deviation (the GPT-2 case uses 0.5 for QKV, 1 for dO).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    NH: int
    T: int
    d_qk: int
    d_v: int
    causal: bool
    seed: int
    sigma: float = 1.0       # std of Q, K, V
    sigma_do: float = 1.0    # std of dO
    packed: bool = False     # Q, K, V are views of one (B, T, 3, NH, HS) tensor
    window: int = 0          # causal sliding window: query i sees keys i-window+1 .. i (0 = none)
    alibi: bool = False      # causal ALiBi bias -m_h (i - j), m_h = 2^(-8 (h+1) / NH)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    def pairs(self) -> int:
        """Unmasked (query, key) pairs over all heads."""
        T, W = self.T, self.window
        if self.causal and 0 < W < T:  # rows i < W see i + 1 keys, the others W
            per_head = W * (W + 1) // 2 + (T - W) * W
        else:
            per_head = T * (T + 1) // 2 if self.causal else T * T
        return self.B * self.NH * per_head

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 2, 128, 64, 64, True, 53001),
    "gpt2": Workload("gpt2", 4, 12, 1024, 64, 64, True, 53002, sigma=0.5, packed=True),
    "mid_causal": Workload("mid_causal", 16, 16, 2048, 128, 128, True, 53003),
    "mid_full": Workload("mid_full", 16, 16, 2048, 128, 128, False, 53003),
    "long": Workload("long", 1, 16, 32768, 128, 128, True, 53004),
    "asym": Workload("asym", 4, 16, 8192, 192, 128, True, 53005),
    "headline": Workload("headline", 4, 16, 8192, 128, 128, True, 53006),
    # the headline shape under a 1024-key sliding window (local attention)
    "window": Workload("window", 4, 16, 8192, 128, 128, True, 53007, window=1024),
    # the headline shape with the ALiBi bias
    "alibi": Workload("alibi", 4, 16, 8192, 128, 128, True, 53008, alibi=True),
    # one decode step (inference forward, no stats): one query row per sequence against
    # an 8192-row key/value cache, non-causal
    "decode": Workload("decode", 16, 16, 8192, 128, 128, False, 53009),
    # the headline shape under a block-sparse map (see block_map): causal, each query
    # block sees the 8 most recent key blocks (1024 keys) and the first one
    "blocksparse": Workload("blocksparse", 4, 16, 8192, 128, 128, True, 53010),
    # the headline shape with a per-head key bias (see key_bias)
    "keybias": Workload("keybias", 4, 16, 8192, 128, 128, True, 53011),
    # the headline shape with dropout on the attention weights, p = DROPOUT_P, the
    # generator seeded with the workload's seed, counter offset 0
    "dropout": Workload("dropout", 4, 16, 8192, 128, 128, True, 53012),
    # padded batches: eight sequences padded to T = 8192 (the headline's width and length),
    # each of its own length (see varlen_lengths), causal
    "varlen": Workload("varlen", 8, 16, 8192, 128, 128, True, 53015),
    # tensors past 4 GiB (element offsets past 2^31, byte offsets past 2^32): many causal
    # sequences (the batch offset grows large) ...
    "big_batch": Workload("big_batch", 576, 16, 2048, 128, 128, True, 53013),
    # ... and one long sequence under a sliding window (the row offset grows large; the
    # last query block is ragged)
    "big_rows": Workload("big_rows", 1, 16, (1 << 20) + 77, 128, 128, True, 53014, window=256),
}

DROPOUT_P = 0.1

BS_BLOCK = 128


def block_map(w: Workload):
    """The block-sparse map of a workload, uint8 (1, 1, nb, nb), one map for every head:
    query block r sees key blocks r - 7 .. r (a local band) and block 0 (a global block).
    Combined with the causal mask inside the diagonal block."""
    import numpy as np

    nb = (w.T + BS_BLOCK - 1) // BS_BLOCK
    r = np.arange(nb)[:, None]
    c = np.arange(nb)[None, :]
    return (((r - c >= 0) & (r - c < 8)) | (c == 0)).astype(np.uint8)[None, None]


def block_map_pairs(w: Workload, m) -> int:
    """Attended (query, key) pairs of a block-sparse workload, counted element by element
    over one head's map times B * NH (maps are shared across heads here)."""
    import numpy as np

    T = w.T
    nb = m.shape[-1]
    total = 0
    for qb in range(nb):
        rows = np.arange(qb * BS_BLOCK, min(T, (qb + 1) * BS_BLOCK))
        for kb in np.nonzero(m[0, 0, qb])[0]:
            k0, k1 = kb * BS_BLOCK, min(T, (kb + 1) * BS_BLOCK)
            if w.causal:
                total += int(np.clip(rows + 1 - k0, 0, k1 - k0).sum())
            else:
                total += len(rows) * (k1 - k0)
    return total * w.B * w.NH


def varlen_lengths(w: Workload):
    """Per-sequence lengths of a padded-batch workload, int32 (B,): the first sequence is
    full (T rows), the others uniform in [T / 8, T] from numpy's default_rng(seed)."""
    import numpy as np

    rng = np.random.default_rng(w.seed)
    n = rng.integers(w.T // 8, w.T + 1, size=w.B).astype(np.int32)
    n[0] = w.T
    return n


def _randn(shape, seed: int, sigma: float, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * sigma).to(dtype)


def make_device_inputs(w: Workload, device, dtype: torch.dtype = torch.bfloat16) -> Dict[str, torch.Tensor]:
    """q, k, v, do of shape (B, T, NH, d) drawn directly in device memory, for workloads
    too large to draw on the host: float32 standard normals from a device generator
    (``torch.Generator(device).manual_seed(seed + k)``, k = 0, 1, 2, 3 for Q, K, V, dO),
    times sigma, rounded to `dtype`.  A test copies the rows it checks to the host, so
    both sides still see the very same values."""
    B, T, NH = w.B, w.T, w.NH
    out = {}
    for k, (name, d, sigma) in enumerate((("q", w.d_qk, w.sigma), ("k", w.d_qk, w.sigma), ("v", w.d_v, w.sigma),
                                          ("do", w.d_v, w.sigma_do))):
        g = torch.Generator(device=device).manual_seed(w.seed + k)
        x = torch.empty((B, T, NH, d), dtype=dtype, device=device)
        flat = x.view(-1)
        step = 1 << 28  # draw in chunks: the float32 draw is twice the size of the result
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            flat[i:i + n] = (torch.randn(n, generator=g, dtype=torch.float32, device=device) * sigma).to(dtype)
        out[name] = x
    return out


def make_inputs(w: Workload, dtype: torch.dtype = torch.bfloat16) -> Dict[str, torch.Tensor]:
    """CPU tensors of element type `dtype` (bf16 or fp16) for one workload.

    Returns q, k, v of shape (B, T, NH, d) (possibly strided views of a packed block,
    which is then also returned as ``qkv``) and do of shape (B, T, NH, d_v).
    """
    B, T, NH = w.B, w.T, w.NH
    if w.packed:
        if w.d_qk != w.d_v:
            raise ValueError("packed QKV needs d_qk == d_v")
        qkv = _randn((B, T, 3, NH, w.d_qk), w.seed + 0, w.sigma, dtype)
        do = _randn((B, T, NH, w.d_v), w.seed + 1, w.sigma_do, dtype)
        return {"qkv": qkv, "q": qkv[:, :, 0], "k": qkv[:, :, 1], "v": qkv[:, :, 2], "do": do}
    q = _randn((B, T, NH, w.d_qk), w.seed + 0, w.sigma, dtype)
    k = _randn((B, T, NH, w.d_qk), w.seed + 1, w.sigma, dtype)
    v = _randn((B, T, NH, w.d_v), w.seed + 2, w.sigma, dtype)
    do = _randn((B, T, NH, w.d_v), w.seed + 3, w.sigma_do, dtype)
    return {"q": q, "k": k, "v": v, "do": do}


def key_bias(w: Workload):
    """The key bias of a workload, float32 (B, NH, T): N(0, 1) per (b, h, key) from seed
    w.seed + 10, and in the odd batches the last quarter of the keys padded with -1e9."""
    g = torch.Generator().manual_seed(w.seed + 10)
    b = torch.randn((w.B, w.NH, w.T), generator=g, dtype=torch.float32)
    b[1::2, :, w.T - w.T // 4:] = -1e9
    return b.numpy()


E4M3_MAX = 448.0


def make_fp8_inputs(w: Workload):
    """fp8 (e4m3) inputs of a workload: the same float32 normals as make_inputs (Q, K, V from
    seeds w.seed + 0, 1, 2), each tensor scaled by one descale factor max|x| / 448 so that
    its largest value maps to the largest e4m3 value, and rounded to e4m3 (nearest even,
    torch's float8_e4m3fn conversion).  Returns uint8 codes q8, k8, v8 (B, T, NH, d) and the
    descale factors."""
    B, T, NH = w.B, w.T, w.NH
    out = {}
    for name, k, d in (("q", 0, w.d_qk), ("k", 1, w.d_qk), ("v", 2, w.d_v)):
        g = torch.Generator().manual_seed(w.seed + k)
        x = torch.randn((B, T, NH, d), generator=g, dtype=torch.float32) * w.sigma
        ds = float(x.abs().max()) / E4M3_MAX
        out[name + "8"] = (x / ds).to(torch.float8_e4m3fn).view(torch.uint8)
        out["descale_" + name] = ds
    return out
