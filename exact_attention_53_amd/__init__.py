"""Fused exact attention (forward + backward) for AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/attn53.h`` (library
``libattn53.so``, built in-tree by ``exact_attention_53_amd._build``).  The binding
only marshals arguments: it takes device pointers and strides from torch tensors,
allocates outputs and the workspace with torch, and passes torch's current HIP
stream.  Every step of the computation runs in the library's HIP kernels; there is
no fallback path, and a missing library raises.

Element type: bf16, or fp16 (the same dtype for every 16-bit tensor of a call; bf16
calls go through attn_fwd / attn_bwd / *_varlen, fp16 calls through attn_fwd_typed /
attn_bwd_typed).

Tensor layout: 4-D tensors in (B, T, NH, d) order by default (``layout="bthd"``,
the layout of the pages' output O), or (B, NH, T, d) (``layout="bhtd"``); any strides
whose last one is 1 and whose others are multiples of 8 elements.  Packed QKV blocks
(B, T, 3, NH, HS) are accepted through ``qkv[:, :, 0]`` etc. or ``fwd_packed``.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "AttnError", "lib_path", "load", "fwd", "fwd_packed", "bwd", "bwd_packed",
    "workspace_bytes", "fwd_varlen", "bwd_varlen", "fwd_decode", "bwd_noalloc", "fwd_blocksparse", "bwd_blocksparse", "BS_BLOCK",
    "fwd_keybias", "bwd_keybias", "fwd_fp8", "dropout_mask", "fwd_dropout", "bwd_dropout", "PREPROCESS", "MAIN", "DQ", "ALL_STAGES", "version",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libattn53.so")

PREPROCESS, MAIN, DQ, ALL_STAGES = 1, 2, 4, 7


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attn53 status {status}: {message}")
        self.status = status


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("t", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads libattn53.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing: build it with `python -m exact_attention_53_amd._build`")
    lib = ctypes.CDLL(lib_path)
    vp, S, i, f, sz = ctypes.c_void_p, Strides, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i]
    lib.attn_version.restype = i
    lib.attn_version.argtypes = []
    lib.attn_fwd.restype = i
    lib.attn_fwd.argtypes = [vp, S, vp, S, vp, S, vp, S, vp, i, i, i, i, i, f, i, vp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    bwd_args = [vp, S, vp, S, vp, S, vp, S, vp, vp, S, vp, S, vp, S, vp, S,
                i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd.argtypes = bwd_args
    lib.attn_bwd_staged.restype = i
    lib.attn_bwd_staged.argtypes = bwd_args + [ctypes.c_uint]
    lib.attn_fwd_varlen_workspace_bytes.restype = sz
    lib.attn_fwd_varlen_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fwd_varlen.argtypes = [vp, S, vp, S, vp, S, vp, S, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_bwd_varlen_workspace_bytes.restype = sz
    lib.attn_bwd_varlen_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_bwd_varlen.restype = i
    lib.attn_bwd_varlen.argtypes = bwd_args[:17] + [vp, vp] + bwd_args[17:]
    lib.attn_fwd_typed.restype = i
    lib.attn_fwd_typed.argtypes = [i, vp, S, vp, S, vp, S, vp, S, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.attn_fwd_decode.restype = i
    lib.attn_fwd_decode.argtypes = [i, vp, S, vp, S, vp, S, vp, S, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    lib.attn_fwd_decode_workspace_bytes.restype = sz
    lib.attn_fwd_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_bwd_typed.restype = i
    lib.attn_bwd_typed.argtypes = [i] + bwd_args[:17] + [vp, vp] + bwd_args[17:24] + [i, i] + bwd_args[24:] + [ctypes.c_uint]
    lib.attn_fwd_blocksparse_workspace_bytes.restype = sz
    lib.attn_fwd_blocksparse_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_blocksparse_workspace_bytes.restype = sz
    lib.attn_bwd_blocksparse_workspace_bytes.argtypes = [i, i, i, i, i, i]
    i64 = ctypes.c_int64
    lib.attn_fwd_blocksparse.restype = i
    lib.attn_fwd_blocksparse.argtypes = [vp, S, vp, S, vp, S, vp, S, vp, vp, i64, i64, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_bwd_blocksparse.restype = i
    lib.attn_bwd_blocksparse.argtypes = bwd_args[:17] + [vp, i64, i64] + bwd_args[17:] + [ctypes.c_uint]
    lib.attn_fwd_keybias_workspace_bytes.restype = sz
    lib.attn_fwd_keybias_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd_keybias_workspace_bytes.restype = sz
    lib.attn_bwd_keybias_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_fwd_keybias.restype = i
    lib.attn_fwd_keybias.argtypes = [vp, S, vp, S, vp, S, vp, S, vp, vp, i64, i64, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_bwd_keybias.restype = i
    lib.attn_bwd_keybias.argtypes = bwd_args[:17] + [vp, vp, i64, i64] + bwd_args[17:] + [ctypes.c_uint]
    lib.attn_fwd_fp8_workspace_bytes.restype = sz
    lib.attn_fwd_fp8_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_fwd_fp8.restype = i
    lib.attn_fwd_fp8.argtypes = [vp, S, vp, S, vp, S, vp, S, vp, f, f, f, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_dropout_mask_bytes.restype = sz
    lib.attn_dropout_mask_bytes.argtypes = [i, i, i]
    lib.attn_dropout_mask.restype = i
    lib.attn_dropout_mask.argtypes = [f, ctypes.c_uint64, ctypes.c_uint32, i, i, i, i, vp, sz, vp]
    lib.attn_fwd_dropout.restype = i
    lib.attn_fwd_dropout.argtypes = [vp, S, vp, S, vp, S, vp, S, vp, vp, f, i, i, i, i, i, f, i, vp]
    lib.attn_bwd_dropout.restype = i
    lib.attn_bwd_dropout.argtypes = bwd_args[:17] + [vp, f] + bwd_args[17:] + [ctypes.c_uint]
    lib.attn_bwd_noalloc.restype = i
    lib.attn_bwd_noalloc.argtypes = bwd_args[:25] + [vp]
    lib.attn_bwd_noalloc_max_workspace_bytes.restype = sz
    lib.attn_bwd_noalloc_max_workspace_bytes.argtypes = []
    _lib = lib
    return lib


def version() -> int:
    return load().attn_version()


def _check(status: int):
    if status != 0:
        raise AttnError(status, load().attn_status_string(status).decode())


def _strides(x: torch.Tensor, layout: str) -> Strides:
    if x.dim() != 4:
        raise ValueError(f"expected a 4-D tensor, got shape {tuple(x.shape)}")
    if x.stride(3) != 1:
        raise ValueError("the head-dim stride must be 1")
    if layout == "bthd":
        return Strides(x.stride(0), x.stride(2), x.stride(1))
    if layout == "bhtd":
        return Strides(x.stride(0), x.stride(1), x.stride(2))
    raise ValueError(f"layout must be 'bthd' or 'bhtd', not {layout!r}")


def _dims(x: torch.Tensor, layout: str) -> Tuple[int, int, int, int]:
    if x.dim() != 4:
        raise ValueError(f"expected a 4-D tensor, got shape {tuple(x.shape)}")
    if layout not in ("bthd", "bhtd"):
        raise ValueError(f"layout must be 'bthd' or 'bhtd', not {layout!r}")
    B, a, c, d = x.shape
    return (B, c, a, d) if layout == "bthd" else (B, a, c, d)  # -> B, NH, T, d


_DTYPE_CODE = {torch.bfloat16: 0, torch.float16: 1}  # attn_dtype of the C ABI


def _need(x: torch.Tensor, name: str, dev: torch.device, dtype: torch.dtype = torch.bfloat16):
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (the dtype of q), got {x.dtype}")
    if x.device != dev:
        raise ValueError(f"{name} is on {x.device}, expected {dev}")


def _shape(x: torch.Tensor, name: str, layout: str, B: int, NH: int, T: int, d: int):
    """Checks that x is the 4-D (B, NH, T, d) tensor (in `layout` order) that the call
    needs: the C ABI sees only pointers and strides, so a smaller tensor would be read or
    written past its end."""
    if x.dim() != 4:
        raise ValueError(f"{name} must be a 4-D tensor, got shape {tuple(x.shape)}")
    got = _dims(x, layout)
    if got != (B, NH, T, d):
        raise ValueError(f"{name} has (B, NH, T, d) = {got}, expected {(B, NH, T, d)}")


def _check_workspace(ws: Optional[torch.Tensor], dev: torch.device):
    """A caller's workspace must be device memory of the call's GPU (its size is checked by
    the library, which returns ATTN_ERR_WORKSPACE when it is too small)."""
    if ws is not None and (ws.device != dev or not ws.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")


def _on_gpu(fn: str, dev: torch.device):
    if dev.type != "cuda":
        raise ValueError(f"{fn} runs on the GPU only; got a CPU tensor")


def _elem(q: torch.Tensor) -> torch.dtype:
    if q.dtype not in _DTYPE_CODE:
        raise TypeError(f"q must be bfloat16 or float16, got {q.dtype}")
    return q.dtype


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
        scale: Optional[float] = None, return_lse: bool = True, layout: str = "bthd",
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, window: int = 0,
        alibi: bool = False):
    """Exact attention forward.  Returns (o, lse); lse is None when return_lse is False
    (inference mode: the kernel skips the stats).  window > 0 (causal only): query i sees
    keys i-window+1 .. i.  alibi (causal only): linear bias -m_h (i - j) on the scaled
    scores, m_h = 2^(-8 (h+1) / NH)."""
    B, NH, T, dqk = _dims(q, layout)
    dv = v.shape[-1]
    _shape(k, "k", layout, B, NH, T, dqk)
    _shape(v, "v", layout, B, NH, T, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, T, dv)
    dev = q.device
    _on_gpu("fwd", dev)
    lib = load()
    et = _elem(q)
    for n, x in (("q", q), ("k", k), ("v", v)):
        _need(x, n, dev, et)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, T, NH, dv) if layout == "bthd" else (B, NH, T, dv)
        out = torch.empty(shape, dtype=et, device=dev)
    _need(out, "out", dev, et)
    if return_lse and lse is None:
        lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev):
        raise ValueError("lse must be a contiguous float32 (B, NH, T) tensor on the device of q")
    tensors = (q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
               v.data_ptr(), _strides(v, layout), out.data_ptr(), _strides(out, layout),
               lse.data_ptr() if return_lse else None)
    with torch.cuda.device(dev):
        if et == torch.bfloat16 and window == 0 and not alibi:
            _check(lib.attn_fwd(*tensors, B, NH, T, dqk, dv, float(scale), int(bool(causal)), _stream(dev)))
        else:
            _check(lib.attn_fwd_typed(_DTYPE_CODE[et], *tensors, None, None, B, NH, T, dqk, dv, float(scale),
                                      int(bool(causal)), int(window), int(bool(alibi)), None, 0, _stream(dev)))
    return out, (lse if return_lse else None)


def fwd_packed(qkv: torch.Tensor, causal: bool = True, scale: Optional[float] = None, return_lse: bool = True):
    """Forward on a packed (B, T, 3, NH, HS) QKV block; o is (B, T, NH, HS)."""
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise ValueError("qkv must have shape (B, T, 3, NH, HS)")
    return fwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], causal, scale, return_lse)


def workspace_bytes(B: int, NH: int, T: int, d_qk: int, d_v: int, deterministic: bool) -> int:
    return int(load().attn_bwd_workspace_bytes(B, NH, T, d_qk, d_v, int(bool(deterministic))))


def bwd(q, k, v, o, lse, do, causal: bool = True, scale: Optional[float] = None,
        deterministic: bool = False, layout: str = "bthd", dq=None, dk=None, dv=None,
        workspace: Optional[torch.Tensor] = None, stages: int = ALL_STAGES, window: int = 0,
        alibi: bool = False):
    """Exact attention backward.  Returns (dq, dk, dv).  window, alibi: the forward's
    sliding window (0 = none) and ALiBi flag."""
    B, NH, T, dqk = _dims(q, layout)
    dvd = v.shape[-1]
    for n, x, d in (("k", k, dqk), ("v", v, dvd), ("o", o, dvd), ("do", do, dvd), ("dq", dq, dqk), ("dk", dk, dqk),
                    ("dv", dv, dvd)):
        if x is not None:
            _shape(x, n, layout, B, NH, T, d)
    dev = q.device
    _on_gpu("bwd", dev)
    lib = load()
    et = _elem(q)
    for n, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(x, n, dev, et)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev:
        raise ValueError("lse must be the forward's contiguous float32 (B, NH, T) stats, on the device of q")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    need = workspace_bytes(B, NH, T, dqk, dvd, deterministic)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(x, n, dev, et)
    tensors = (q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
               v.data_ptr(), _strides(v, layout), o.data_ptr(), _strides(o, layout),
               lse.data_ptr(), do.data_ptr(), _strides(do, layout),
               dq.data_ptr(), _strides(dq, layout), dk.data_ptr(), _strides(dk, layout),
               dv.data_ptr(), _strides(dv, layout))
    dims = (B, NH, T, dqk, dvd, float(scale), int(bool(causal)))
    rest = (int(bool(deterministic)), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream(dev), int(stages))
    with torch.cuda.device(dev):
        if et == torch.bfloat16 and window == 0 and not alibi:
            _check(lib.attn_bwd_staged(*tensors, *dims, *rest))
        else:
            _check(lib.attn_bwd_typed(_DTYPE_CODE[et], *tensors, None, None, *dims, int(window), int(bool(alibi)),
                                      *rest))
    return dq, dk, dv


BS_BLOCK = 128  # block-sparse maps: elements per block along each side


def _block_map(block_map: torch.Tensor, B: int, NH: int, T: int, dev: torch.device):
    """Checks a (B or 1, NH or 1, nb, nb) uint8 map and returns its (b, h) strides (0 where
    the map is shared)."""
    nb = (T + BS_BLOCK - 1) // BS_BLOCK
    if block_map.dtype != torch.uint8 or block_map.dim() != 4:
        raise ValueError("block_map must be a 4-D uint8 tensor (B or 1, NH or 1, nb, nb)")
    Bm, Hm, r, c = block_map.shape
    if Bm not in (1, B) or Hm not in (1, NH) or (r, c) != (nb, nb):
        raise ValueError(f"block_map has shape {tuple(block_map.shape)}, expected (B or 1, NH or 1, {nb}, {nb})")
    if block_map.stride(3) != 1 or block_map.stride(2) != nb:
        raise ValueError("each (nb, nb) map must be contiguous and row-major")
    if block_map.device != dev:
        raise ValueError(f"block_map is on {block_map.device}, expected {dev}")
    return (block_map.stride(0) if Bm > 1 else 0), (block_map.stride(1) if Hm > 1 else 0)


def fwd_blocksparse(q, k, v, block_map: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
                    return_lse: bool = True, layout: str = "bthd", out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Block-sparse forward (bf16): element (i, j) is attended iff block_map[b, h, i // 128,
    j // 128] != 0 and, when causal, j <= i.  block_map is uint8 (B or 1, NH or 1, nb, nb) on
    the device, nb = ceil(T / 128).  Rows with no key get O = 0, LSE = -inf.  Returns (o, lse)."""
    B, NH, T, dqk = _dims(q, layout)
    dv = v.shape[-1]
    _shape(k, "k", layout, B, NH, T, dqk)
    _shape(v, "v", layout, B, NH, T, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, T, dv)
    dev = q.device
    _on_gpu("fwd_blocksparse", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v)):
        _need(x, n, dev, torch.bfloat16)
    msb, msh = _block_map(block_map, B, NH, T, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, T, NH, dv) if layout == "bthd" else (B, NH, T, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", dev, torch.bfloat16)
    if return_lse and lse is None:
        lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev):
        raise ValueError("lse must be a contiguous float32 (B, NH, T) tensor on the device of q")
    need = int(lib.attn_fwd_blocksparse_workspace_bytes(B, NH, T, dqk, dv))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_fwd_blocksparse(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                        v.data_ptr(), _strides(v, layout), out.data_ptr(), _strides(out, layout),
                                        lse.data_ptr() if return_lse else None, block_map.data_ptr(), msb, msh,
                                        B, NH, T, dqk, dv, float(scale), int(bool(causal)), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, (lse if return_lse else None)


def bwd_blocksparse(q, k, v, o, lse, do, block_map: torch.Tensor, causal: bool = False,
                    scale: Optional[float] = None, deterministic: bool = False, layout: str = "bthd",
                    dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None, stages: int = ALL_STAGES):
    """Block-sparse backward (bf16) with the forward's map and causal flag.  Returns
    (dq, dk, dv); rows without keys get dQ = 0, keys no query attends dK = dV = 0."""
    B, NH, T, dqk = _dims(q, layout)
    dvd = v.shape[-1]
    for n, x, d in (("k", k, dqk), ("v", v, dvd), ("o", o, dvd), ("do", do, dvd), ("dq", dq, dqk), ("dk", dk, dqk),
                    ("dv", dv, dvd)):
        if x is not None:
            _shape(x, n, layout, B, NH, T, d)
    dev = q.device
    _on_gpu("bwd_blocksparse", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(x, n, dev, torch.bfloat16)
    msb, msh = _block_map(block_map, B, NH, T, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev:
        raise ValueError("lse must be the forward's contiguous float32 (B, NH, T) stats, on the device of q")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(x, n, dev, torch.bfloat16)
    need = int(lib.attn_bwd_blocksparse_workspace_bytes(B, NH, T, dqk, dvd, int(bool(deterministic))))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_bwd_blocksparse(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                        v.data_ptr(), _strides(v, layout), o.data_ptr(), _strides(o, layout),
                                        lse.data_ptr(), do.data_ptr(), _strides(do, layout),
                                        dq.data_ptr(), _strides(dq, layout), dk.data_ptr(), _strides(dk, layout),
                                        dv.data_ptr(), _strides(dv, layout), block_map.data_ptr(), msb, msh,
                                        B, NH, T, dqk, dvd, float(scale), int(bool(causal)), int(bool(deterministic)),
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        _stream(dev), int(stages)))
    return dq, dk, dv


def _key_bias(bias: torch.Tensor, B: int, NH: int, T: int, dev: torch.device):
    """Checks a (B or 1, NH or 1, T) float32 key bias and returns its (b, h) element strides
    (0 where it is shared)."""
    if bias.dtype != torch.float32 or bias.dim() != 3:
        raise ValueError("bias must be a 3-D float32 tensor (B or 1, NH or 1, T)")
    Bb, Hb, Tb = bias.shape
    if Bb not in (1, B) or Hb not in (1, NH) or Tb != T:
        raise ValueError(f"bias has shape {tuple(bias.shape)}, expected (B or 1, NH or 1, {T})")
    if bias.stride(2) != 1:
        raise ValueError("bias must be contiguous along the keys")
    if bias.device != dev:
        raise ValueError(f"bias is on {bias.device}, expected {dev}")
    return (bias.stride(0) if Bb > 1 else 0), (bias.stride(1) if Hb > 1 else 0)


def fwd_keybias(q, k, v, bias: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
                return_lse: bool = True, layout: str = "bthd", out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Forward with a key bias (bf16): S = scale Q K^T + bias[b, h, key], bias float32
    (B or 1, NH or 1, T) on the device, finite values (mask a key with a large negative
    value).  Returns (o, lse)."""
    B, NH, T, dqk = _dims(q, layout)
    dv = v.shape[-1]
    _shape(k, "k", layout, B, NH, T, dqk)
    _shape(v, "v", layout, B, NH, T, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, T, dv)
    dev = q.device
    _on_gpu("fwd_keybias", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v)):
        _need(x, n, dev, torch.bfloat16)
    sb, sh = _key_bias(bias, B, NH, T, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, T, NH, dv) if layout == "bthd" else (B, NH, T, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", dev, torch.bfloat16)
    if return_lse and lse is None:
        lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev):
        raise ValueError("lse must be a contiguous float32 (B, NH, T) tensor on the device of q")
    need = int(lib.attn_fwd_keybias_workspace_bytes(B, NH, T, dqk, dv))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_fwd_keybias(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                    v.data_ptr(), _strides(v, layout), out.data_ptr(), _strides(out, layout),
                                    lse.data_ptr() if return_lse else None, bias.data_ptr(), sb, sh,
                                    B, NH, T, dqk, dv, float(scale), int(bool(causal)), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, (lse if return_lse else None)


def bwd_keybias(q, k, v, o, lse, do, bias: torch.Tensor, causal: bool = False, scale: Optional[float] = None,
                deterministic: bool = False, layout: str = "bthd", dq=None, dk=None, dv=None,
                dbias: Optional[torch.Tensor] = None, need_dbias: bool = True,
                workspace: Optional[torch.Tensor] = None, stages: int = ALL_STAGES):
    """Backward with the forward's key bias (bf16).  Returns (dq, dk, dv, dbias); dbias has
    the bias's shape (summed over the batches / heads that share a row), None when
    need_dbias is False."""
    B, NH, T, dqk = _dims(q, layout)
    dvd = v.shape[-1]
    for n, x, d in (("k", k, dqk), ("v", v, dvd), ("o", o, dvd), ("do", do, dvd), ("dq", dq, dqk), ("dk", dk, dqk),
                    ("dv", dv, dvd)):
        if x is not None:
            _shape(x, n, layout, B, NH, T, d)
    dev = q.device
    _on_gpu("bwd_keybias", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(x, n, dev, torch.bfloat16)
    sb, sh = _key_bias(bias, B, NH, T, dev)
    if need_dbias:
        if dbias is None:
            dbias = torch.empty_strided(bias.shape, bias.stride(), dtype=torch.float32, device=dev)
        if dbias.shape != bias.shape or dbias.stride() != bias.stride() or dbias.dtype != torch.float32:
            raise ValueError("dbias must be float32 with the bias's shape and strides")
    else:
        dbias = None
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev:
        raise ValueError("lse must be the forward's contiguous float32 (B, NH, T) stats, on the device of q")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(x, n, dev, torch.bfloat16)
    need = int(lib.attn_bwd_keybias_workspace_bytes(B, NH, T, dqk, dvd, int(bool(deterministic))))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_bwd_keybias(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                    v.data_ptr(), _strides(v, layout), o.data_ptr(), _strides(o, layout),
                                    lse.data_ptr(), do.data_ptr(), _strides(do, layout),
                                    dq.data_ptr(), _strides(dq, layout), dk.data_ptr(), _strides(dk, layout),
                                    dv.data_ptr(), _strides(dv, layout), bias.data_ptr(),
                                    dbias.data_ptr() if dbias is not None else None, sb, sh,
                                    B, NH, T, dqk, dvd, float(scale), int(bool(causal)), int(bool(deterministic)),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream(dev), int(stages)))
    return dq, dk, dv, dbias


_FP8_TYPES = (torch.uint8, torch.float8_e4m3fn)


def fwd_fp8(q, k, v, descale_q: float, descale_k: float, descale_v: float, causal: bool = True,
            scale: Optional[float] = None, return_lse: bool = True, layout: str = "bthd",
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None):
    """Forward on fp8 e4m3 inputs (torch.float8_e4m3fn, or uint8 holding the codes) with
    per-tensor descale factors: the real inputs are descale_x * x.  d_qk = d_v in {64, 128}.
    Returns (o, lse), o in bf16."""
    B, NH, T, dqk = _dims(q, layout)
    dv = v.shape[-1]
    _shape(k, "k", layout, B, NH, T, dqk)
    _shape(v, "v", layout, B, NH, T, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, T, dv)
    dev = q.device
    _on_gpu("fwd_fp8", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype not in _FP8_TYPES:
            raise TypeError(f"{n} must hold e4m3 codes (float8_e4m3fn or uint8), got {x.dtype}")
        if x.device != dev:
            raise ValueError(f"{n} is on {x.device}, expected {dev}")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, T, NH, dv) if layout == "bthd" else (B, NH, T, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", dev, torch.bfloat16)
    if return_lse and lse is None:
        lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev):
        raise ValueError("lse must be a contiguous float32 (B, NH, T) tensor on the device of q")
    need = int(lib.attn_fwd_fp8_workspace_bytes(B, NH, T, dqk, dv))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_fwd_fp8(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                v.data_ptr(), _strides(v, layout), out.data_ptr(), _strides(out, layout),
                                lse.data_ptr() if return_lse else None, float(descale_q), float(descale_k),
                                float(descale_v), B, NH, T, dqk, dv, float(scale), int(bool(causal)),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, (lse if return_lse else None)


def dropout_mask(p_drop: float, seed: int, offset: int, B: int, NH: int, T: int, causal: bool = True,
                 device=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The keep bits of dropout with probability p_drop for one step (Philox4x32-10 at
    counter (key / 8, query, b * NH + h, offset), key seed): a uint8 buffer of both bit
    layouts, to be passed to fwd_dropout and bwd_dropout."""
    lib = load()
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    _on_gpu("dropout_mask", dev)
    need = int(lib.attn_dropout_mask_bytes(B, NH, T))
    if need == 0:
        raise ValueError("invalid sizes for a dropout mask")
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=dev)
    if out.dtype != torch.uint8 or out.device != dev or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 buffer on {dev}")
    with torch.cuda.device(dev):
        _check(lib.attn_dropout_mask(float(p_drop), int(seed) & (2 ** 64 - 1), int(offset) & 0xFFFFFFFF, B, NH, T,
                                     int(bool(causal)), out.data_ptr(), out.numel(), _stream(dev)))
    return out


def _dropout_mask_arg(lib, mask: torch.Tensor, B: int, NH: int, T: int, dev: torch.device):
    if (mask.dtype != torch.uint8 or mask.device != dev or not mask.is_contiguous()
            or mask.numel() < int(lib.attn_dropout_mask_bytes(B, NH, T))):
        raise ValueError("mask must be the contiguous uint8 buffer from dropout_mask for these sizes, on q's device")


def fwd_dropout(q, k, v, mask: torch.Tensor, p_drop: float, causal: bool = True, scale: Optional[float] = None,
                return_lse: bool = True, layout: str = "bthd", out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None):
    """Forward with dropout on the attention weights (bf16), the keep bits from dropout_mask
    (same p_drop, causal flag and sizes).  Returns (o, lse); LSE is that of the undropped
    weights."""
    B, NH, T, dqk = _dims(q, layout)
    dv = v.shape[-1]
    _shape(k, "k", layout, B, NH, T, dqk)
    _shape(v, "v", layout, B, NH, T, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, T, dv)
    dev = q.device
    _on_gpu("fwd_dropout", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v)):
        _need(x, n, dev, torch.bfloat16)
    _dropout_mask_arg(lib, mask, B, NH, T, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, T, NH, dv) if layout == "bthd" else (B, NH, T, dv)
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", dev, torch.bfloat16)
    if return_lse and lse is None:
        lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev):
        raise ValueError("lse must be a contiguous float32 (B, NH, T) tensor on the device of q")
    with torch.cuda.device(dev):
        _check(lib.attn_fwd_dropout(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                    v.data_ptr(), _strides(v, layout), out.data_ptr(), _strides(out, layout),
                                    lse.data_ptr() if return_lse else None, mask.data_ptr(), float(p_drop),
                                    B, NH, T, dqk, dv, float(scale), int(bool(causal)), _stream(dev)))
    return out, (lse if return_lse else None)


def bwd_dropout(q, k, v, o, lse, do, mask: torch.Tensor, p_drop: float, causal: bool = True,
                scale: Optional[float] = None, deterministic: bool = False, layout: str = "bthd",
                dq=None, dk=None, dv=None, workspace: Optional[torch.Tensor] = None, stages: int = ALL_STAGES):
    """Backward with the forward's dropout mask and p_drop (bf16).  Returns (dq, dk, dv)."""
    B, NH, T, dqk = _dims(q, layout)
    dvd = v.shape[-1]
    for n, x, d in (("k", k, dqk), ("v", v, dvd), ("o", o, dvd), ("do", do, dvd), ("dq", dq, dqk), ("dk", dk, dqk),
                    ("dv", dv, dvd)):
        if x is not None:
            _shape(x, n, layout, B, NH, T, d)
    dev = q.device
    _on_gpu("bwd_dropout", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(x, n, dev, torch.bfloat16)
    _dropout_mask_arg(lib, mask, B, NH, T, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev:
        raise ValueError("lse must be the forward's contiguous float32 (B, NH, T) stats, on the device of q")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(x, n, dev, torch.bfloat16)
    need = workspace_bytes(B, NH, T, dqk, dvd, deterministic)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_bwd_dropout(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                    v.data_ptr(), _strides(v, layout), o.data_ptr(), _strides(o, layout),
                                    lse.data_ptr(), do.data_ptr(), _strides(do, layout),
                                    dq.data_ptr(), _strides(dq, layout), dk.data_ptr(), _strides(dk, layout),
                                    dv.data_ptr(), _strides(dv, layout), mask.data_ptr(), float(p_drop),
                                    B, NH, T, dqk, dvd, float(scale), int(bool(causal)), int(bool(deterministic)),
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream(dev), int(stages)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, causal: bool = True, scale: Optional[float] = None,
                deterministic: bool = False, layout: str = "bthd"):
    """attn_bwd_noalloc: the backward into caller-supplied dq, dk, dv with the library's
    fixed per-GPU scratch as its workspace (nothing is allocated, by torch or the
    library).  Calls that overlap in time on one GPU race; raises AttnError when the sizes
    need more scratch than the library holds."""
    B, NH, T, dqk = _dims(q, layout)
    dvd = v.shape[-1]
    for n, x, d in (("k", k, dqk), ("v", v, dvd), ("o", o, dvd), ("do", do, dvd), ("dq", dq, dqk), ("dk", dk, dqk),
                    ("dv", dv, dvd)):
        _shape(x, n, layout, B, NH, T, d)
    dev = q.device
    _on_gpu("bwd_noalloc", dev)
    lib = load()
    for n, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(x, n, dev, torch.bfloat16)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev:
        raise ValueError("lse must be the forward's contiguous float32 (B, NH, T) stats, on the device of q")
    with torch.cuda.device(dev):
        _check(lib.attn_bwd_noalloc(q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
                                    v.data_ptr(), _strides(v, layout), o.data_ptr(), _strides(o, layout),
                                    lse.data_ptr(), do.data_ptr(), _strides(do, layout),
                                    dq.data_ptr(), _strides(dq, layout), dk.data_ptr(), _strides(dk, layout),
                                    dv.data_ptr(), _strides(dv, layout), B, NH, T, dqk, dvd, float(scale),
                                    int(bool(causal)), int(bool(deterministic)), _stream(dev)))
    return dq, dk, dv


def bwd_packed(qkv, o, lse, do, causal: bool = True, scale: Optional[float] = None,
               deterministic: bool = False, dqkv: Optional[torch.Tensor] = None, workspace=None):
    """Backward on a packed (B, T, 3, NH, HS) QKV block; returns dqkv of the same layout."""
    if dqkv is None:
        dqkv = torch.empty_like(qkv, memory_format=torch.contiguous_format)
    bwd(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], o, lse, do, causal, scale, deterministic,
        dq=dqkv[:, :, 0], dk=dqkv[:, :, 1], dv=dqkv[:, :, 2], workspace=workspace)
    return dqkv


def fwd_decode(q, k, v, seq_len_kv: Optional[torch.Tensor] = None, scale: Optional[float] = None,
               return_lse: bool = False, layout: str = "bthd", out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None):
    """Decode-step forward: the Tq query rows of each sequence attend to all rows of its
    key/value cache (Tk rows, or seq_len_kv[b] of them), no causal mask.  q is
    (B, Tq, NH, d_qk), k and v (B, Tk, NH, d).  Returns (o, lse); lse is None unless
    return_lse (the inference mode skips the stats)."""
    B, NH, Tq, dqk = _dims(q, layout)
    if k.dim() != 4:
        raise ValueError(f"k must be a 4-D tensor, got shape {tuple(k.shape)}")
    Tk, dv = _dims(k, layout)[2], v.shape[-1]
    _shape(k, "k", layout, B, NH, Tk, dqk)
    _shape(v, "v", layout, B, NH, Tk, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, Tq, dv)
    dev = q.device
    _on_gpu("fwd_decode", dev)
    lib = load()
    et = _elem(q)
    for n, x in (("q", q), ("k", k), ("v", v)):
        _need(x, n, dev, et)
    if seq_len_kv is not None:
        _lengths(seq_len_kv, "seq_len_kv", B, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, Tq, NH, dv) if layout == "bthd" else (B, NH, Tq, dv)
        out = torch.empty(shape, dtype=et, device=dev)
    _need(out, "out", dev, et)
    lse = torch.empty((B, NH, Tq), dtype=torch.float32, device=dev) if return_lse else None
    need = int(lib.attn_fwd_decode_workspace_bytes(B, NH, Tq, Tk, dqk, dv))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    with torch.cuda.device(dev):
        _check(lib.attn_fwd_decode(_DTYPE_CODE[et], q.data_ptr(), _strides(q, layout), k.data_ptr(),
                                   _strides(k, layout), v.data_ptr(), _strides(v, layout), out.data_ptr(),
                                   _strides(out, layout), lse.data_ptr() if return_lse else None,
                                   seq_len_kv.data_ptr() if seq_len_kv is not None else None,
                                   B, NH, Tq, Tk, dqk, dv, float(scale),
                                   workspace.data_ptr() if workspace is not None else None,
                                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                   _stream(dev)))
    return out, lse


def _lengths(x: torch.Tensor, name: str, B: int, dev: torch.device) -> torch.Tensor:
    if x.dtype != torch.int32 or x.dim() != 1 or x.numel() != B or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of B = {B} lengths")
    if x.device != dev:
        raise ValueError(f"{name} is on {x.device}, expected {dev}")
    return x


def fwd_varlen(q, k, v, seq_len_q: torch.Tensor, seq_len_kv: torch.Tensor, causal: bool = True,
               scale: Optional[float] = None, return_lse: bool = True, layout: str = "bthd",
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None):
    """Forward on padded batches: batch b uses the first seq_len_q[b] query rows and the
    first seq_len_kv[b] key/value rows (int32 device tensors of B lengths); padding rows
    of o are written as 0 and of lse as -inf.  Returns (o, lse)."""
    B, NH, T, dqk = _dims(q, layout)
    dv = v.shape[-1]
    _shape(k, "k", layout, B, NH, T, dqk)
    _shape(v, "v", layout, B, NH, T, dv)
    if out is not None:
        _shape(out, "out", layout, B, NH, T, dv)
    dev = q.device
    _on_gpu("fwd_varlen", dev)
    lib = load()
    et = _elem(q)
    for n, x in (("q", q), ("k", k), ("v", v)):
        _need(x, n, dev, et)
    _lengths(seq_len_q, "seq_len_q", B, dev)
    _lengths(seq_len_kv, "seq_len_kv", B, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if out is None:
        shape = (B, T, NH, dv) if layout == "bthd" else (B, NH, T, dv)
        out = torch.empty(shape, dtype=et, device=dev)
    _need(out, "out", dev, et)
    if return_lse and lse is None:
        lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev):
        raise ValueError("lse must be a contiguous float32 (B, NH, T) tensor on the device of q")
    need = int(lib.attn_fwd_varlen_workspace_bytes(B, NH, T, dqk, dv))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    args = (q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
            v.data_ptr(), _strides(v, layout), out.data_ptr(), _strides(out, layout),
            lse.data_ptr() if return_lse else None, seq_len_q.data_ptr(), seq_len_kv.data_ptr(),
            B, NH, T, dqk, dv, float(scale), int(bool(causal)),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(dev))
    with torch.cuda.device(dev):
        if et == torch.bfloat16:
            _check(lib.attn_fwd_varlen(*args))
        else:
            _check(lib.attn_fwd_typed(_DTYPE_CODE[et], *args[:18], 0, 0, *args[18:]))
    return out, (lse if return_lse else None)


def bwd_varlen(q, k, v, o, lse, do, seq_len_q: torch.Tensor, seq_len_kv: torch.Tensor, causal: bool = True,
               scale: Optional[float] = None, deterministic: bool = False, layout: str = "bthd",
               workspace: Optional[torch.Tensor] = None, dq=None, dk=None, dv=None, stages: int = ALL_STAGES):
    """Backward on padded batches (see fwd_varlen).  Returns (dq, dk, dv); padding rows
    are written as 0.  stages: as in bwd."""
    B, NH, T, dqk = _dims(q, layout)
    dvd = v.shape[-1]
    for n, x, d in (("k", k, dqk), ("v", v, dvd), ("o", o, dvd), ("do", do, dvd), ("dq", dq, dqk), ("dk", dk, dqk),
                    ("dv", dv, dvd)):
        if x is not None:
            _shape(x, n, layout, B, NH, T, d)
    dev = q.device
    _on_gpu("bwd_varlen", dev)
    lib = load()
    et = _elem(q)
    for n, x in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _need(x, n, dev, et)
    _lengths(seq_len_q, "seq_len_q", B, dev)
    _lengths(seq_len_kv, "seq_len_kv", B, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * NH * T or lse.device != dev:
        raise ValueError("lse must be the forward's contiguous float32 (B, NH, T) stats, on the device of q")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(x, n, dev, et)
    need = int(lib.attn_bwd_varlen_workspace_bytes(B, NH, T, dqk, dvd, int(bool(deterministic))))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, dev)
    args = (q.data_ptr(), _strides(q, layout), k.data_ptr(), _strides(k, layout),
            v.data_ptr(), _strides(v, layout), o.data_ptr(), _strides(o, layout),
            lse.data_ptr(), do.data_ptr(), _strides(do, layout),
            dq.data_ptr(), _strides(dq, layout), dk.data_ptr(), _strides(dk, layout),
            dv.data_ptr(), _strides(dv, layout), seq_len_q.data_ptr(), seq_len_kv.data_ptr(),
            B, NH, T, dqk, dvd, float(scale), int(bool(causal)), int(bool(deterministic)),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(dev))
    with torch.cuda.device(dev):
        if et == torch.bfloat16 and stages == ALL_STAGES:
            _check(lib.attn_bwd_varlen(*args))
        else:
            _check(lib.attn_bwd_typed(_DTYPE_CODE[et], *args[:26], 0, 0, *args[26:], int(stages)))
    return dq, dk, dv
