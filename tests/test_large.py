"""GPU parity on tensors past 4 GiB: every element and byte offset beyond 32 bits.

Both workloads are drawn in device memory (workloads.make_device_inputs); the rows a
check needs are copied to the host for the oracle.

* big_batch (NH 16, T 2048, causal; d 128 at B 576, as well as d 64 at B 1152 and
  d (192, 128) at B 384; 4.5 GiB per q tensor): the causal kernels of each head width,
  with batch offsets past 2^32 bytes.  Whole heads of the first and the last sequence
  are compared, in both dQ modes.
* big_rows (B 1, NH 16, T 2^20 + 77, d 128, 256-key sliding window; 4 GiB per tensor):
  row offsets past 2^32 bytes and a ragged last query block.  A windowed row sees only
  the 255 keys before it, so the oracle runs on a slice that starts 255 rows before the
  rows compared: on the slice the mask is the same (it depends on i - j only), rows from
  slice index 255 on have their whole window, and a key from that index on receives
  gradient only from rows that do.  O, LSE and dQ are compared on those rows, dK and dV
  on those keys, at the end of the sequence; and on the first rows, where every window
  is whole (dK and dV there only on keys whose rows all lie in the slice).
"""
import numpy as np
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from oracle import attn_ref
from tests.gpu_cases import check_bf16, check_lse, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _free_gib() -> float:
    free, _ = torch.cuda.mem_get_info(DEV)
    return free / 2**30


def _need_gib(w, deterministic: bool) -> float:
    elems = w.B * w.T * w.NH * w.d_qk
    ws = 0 if deterministic else elems * 4  # atomic mode: fp32 dQ accumulator
    return (8 * elems * 2 + ws + 2 * w.B * w.NH * w.T * 4) / 2**30 + 4


def _run(w, gpu, deterministic: bool):
    o, lse = attn.fwd(gpu["q"], gpu["k"], gpu["v"], w.causal, w.scale, window=w.window)
    dq, dk, dv = attn.bwd(gpu["q"], gpu["k"], gpu["v"], o, lse, gpu["do"], w.causal, w.scale, deterministic,
                          window=w.window)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _check(tag, got, ref, rows=slice(None), keys=slice(None)):
    """got: GPU tensors of one head, (T, d) / (T,); ref: oracle result of the same rows.
    O, LSE and dQ are compared on `rows`, dK and dV on `keys`."""
    dq, dk, dv, o, lse = ref[:5]
    for name, r, sel in (("o", o, rows), ("dq", dq, rows), ("dk", dk, keys), ("dv", dv, keys)):
        check_bf16(f"{tag} {name}", to_np(got[name])[sel], r[sel])
    check_lse(f"{tag} lse", to_np(got["lse"])[rows], lse[rows])


# head widths of the three kernel families; B sized so that q passes 4 GiB
BIG_DIMS = {(64, 64): 1152, (128, 128): 576, (192, 128): 384}


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
@pytest.mark.parametrize("dims", list(BIG_DIMS), ids=lambda d: f"d{d[0]}x{d[1]}")
def test_big_batch(dims, deterministic):
    w = workloads.WORKLOADS["big_batch"].with_(B=BIG_DIMS[dims], d_qk=dims[0], d_v=dims[1])
    assert w.B * w.T * w.NH * w.d_qk * 2 > 4 * 2**30
    if _free_gib() < _need_gib(w, deterministic):
        pytest.skip(f"needs {_need_gib(w, deterministic):.0f} GiB of free device memory")
    say(f"case big_batch B={w.B} d={dims} det={deterministic}: drawing inputs")
    gpu = workloads.make_device_inputs(w, DEV)
    say("  fwd + bwd")
    out = _run(w, gpu, deterministic)
    for b, h in ((0, 0), (w.B - 1, w.NH - 1), (w.B - 1, 3)):
        say(f"  head b={b} h={h}")
        x = {n: to_np(gpu[n][b, :, h]) for n in ("q", "k", "v", "do")}
        ref = attn_ref.head_backward(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal)
        got = {n: out[n][b, :, h] for n in ("o", "dq", "dk", "dv")}
        got["lse"] = out["lse"][b, h]
        _check(f"big_batch det={deterministic} ({b},{h})", got, ref)
    del gpu, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("deterministic", [False, True], ids=["atomic", "determ"])
def test_big_rows_window(deterministic):
    w = workloads.WORKLOADS["big_rows"]
    W, T = w.window, w.T
    assert w.B * T * w.NH * w.d_qk * 2 > 4 * 2**30 and T % 128 != 0
    if _free_gib() < _need_gib(w, deterministic):
        pytest.skip(f"needs {_need_gib(w, deterministic):.0f} GiB of free device memory")
    say(f"case big_rows det={deterministic}: drawing inputs")
    gpu = workloads.make_device_inputs(w, DEV)
    say("  fwd + bwd")
    out = _run(w, gpu, deterministic)
    R = 400  # rows compared per slice
    for h in (0, w.NH - 1):
        # The first R rows: the slice starts at row 0, where every window is whole; its
        # keys past R - W also take gradient from rows after the slice, so dK and dV are
        # compared on keys 0 .. R - W only.  The last R rows, with the W - 1 rows before
        # them: every row and key from slice index W - 1 on is complete.
        for s0, rows, keys in ((0, slice(0, R), slice(0, R - W + 1)),
                               (T - R - (W - 1), slice(W - 1, None), slice(W - 1, None))):
            say(f"  head h={h} slice from row {s0}")
            sl = slice(s0, s0 + R + (W - 1) if s0 else R)
            x = {n: to_np(gpu[n][0, sl, h]) for n in ("q", "k", "v", "do")}
            ref = attn_ref.head_backward(x["q"], x["k"], x["v"], x["do"], w.scale, True, window=W)
            got = {n: out[n][0, sl, h] for n in ("o", "dq", "dk", "dv")}
            got["lse"] = out["lse"][0, h, sl]
            _check(f"big_rows det={deterministic} h={h} from row {s0}", got, ref, rows=rows, keys=keys)
    del gpu, out
    torch.cuda.empty_cache()
