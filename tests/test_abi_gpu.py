"""The two core entry points, attn_fwd and attn_bwd, called through ctypes directly
(not through the binding's staged or typed paths), against the CPU oracle.

attn_bwd runs every backward stage in one call; it must equal three attn_bwd_staged
calls bit for bit in the deterministic mode.
"""
import ctypes

import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from tests.gpu_cases import compare, oracle, say

pytestmark = pytest.mark.gpu


def _st(x):
    # (B, T, NH, d) tensor -> element strides along b, h, t
    return attn.Strides(x.stride(0), x.stride(2), x.stride(1))


@pytest.mark.parametrize("deterministic", [0, 1], ids=["atomic", "determ"])
@pytest.mark.parametrize("dims,T,causal", [((64, 64), 200, 1), ((128, 128), 333, 1), ((128, 128), 256, 0),
                                           ((192, 128), 129, 1)])
def test_core_entry_points_direct(dims, T, causal, deterministic):
    dqk, dv = dims
    w = workloads.Workload(f"abi_T{T}_d{dqk}", 2, 3, T, dqk, dv, bool(causal), 400 + T)
    say(f"case direct ABI {w.name} causal={causal} det={deterministic}")
    lib = attn.load()
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    B, NH = w.B, w.NH
    o = torch.empty(B, T, NH, dv, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, NH, T, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.attn_fwd(q.data_ptr(), _st(q), k.data_ptr(), _st(k), v.data_ptr(), _st(v), o.data_ptr(), _st(o),
                      lse.data_ptr(), B, NH, T, dqk, dv, ctypes.c_float(w.scale), causal, stream)
    assert st == 0, lib.attn_status_string(st)
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dvv = torch.empty_like(v)
    nbytes = lib.attn_bwd_workspace_bytes(B, NH, T, dqk, dv, deterministic)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = lib.attn_bwd(q.data_ptr(), _st(q), k.data_ptr(), _st(k), v.data_ptr(), _st(v), o.data_ptr(), _st(o),
                      lse.data_ptr(), do.data_ptr(), _st(do), dq.data_ptr(), _st(dq), dk.data_ptr(), _st(dk),
                      dvv.data_ptr(), _st(dvv), B, NH, T, dqk, dv, ctypes.c_float(w.scale), causal, deterministic,
                      ws.data_ptr(), nbytes, stream)
    assert st == 0, lib.attn_status_string(st)
    torch.cuda.synchronize()
    got = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dvv.cpu()}
    compare(w, got, oracle(w, cpu))
    if deterministic:
        dq2, dk2, dv2 = attn.bwd(q, k, v, o, lse, do, bool(causal), w.scale, deterministic=True)
        torch.cuda.synchronize()
        for n, a, b in (("dq", dq, dq2), ("dk", dk, dk2), ("dv", dvv, dv2)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"attn_bwd vs staged: {n} differs"


def _in_layout(x_bthd, layout, dev):
    """A (B, T, NH, d) view of a copy of x held in memory in `layout`: "bthd", "bhtd",
    "hbtd" (heads outermost) or "pad" (token-major with 64 extra elements per row)."""
    B, T, NH, d = x_bthd.shape
    if layout == "pad":
        buf = torch.zeros(B, T, NH * d + 64, dtype=x_bthd.dtype, device=dev)
        view = buf[:, :, :NH * d].view(B, T, NH, d)
        view.copy_(x_bthd.to(dev))
        return view
    order = {"bthd": (0, 1, 2, 3), "bhtd": (0, 2, 1, 3), "hbtd": (2, 0, 1, 3)}[layout]
    inv = [order.index(i) for i in range(4)]
    return x_bthd.permute(*order).contiguous().to(dev).permute(*inv)


@pytest.mark.parametrize("deterministic", [0, 1], ids=["atomic", "determ"])
@pytest.mark.parametrize("dims,causal", [((128, 128), 1), ((128, 128), 0), ((192, 128), 1)])
def test_core_entry_points_mixed_strides(dims, causal, deterministic):
    """Every tensor in a memory layout of its own: the kernels take each one's (b, h, t)
    strides from the call, as the ABI states."""
    dqk, dv = dims
    T = 300
    w = workloads.Workload(f"mixed_T{T}_d{dqk}", 2, 3, T, dqk, dv, bool(causal), 500 + dqk)
    say(f"case mixed strides {w.name} causal={causal} det={deterministic}")
    lib = attn.load()
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    B, NH = w.B, w.NH
    q = _in_layout(cpu["q"], "bthd", dev)
    k = _in_layout(cpu["k"], "bhtd", dev)
    v = _in_layout(cpu["v"], "pad", dev)
    do = _in_layout(cpu["do"], "bhtd", dev)
    zeros = lambda d, lay: _in_layout(torch.zeros(B, T, NH, d, dtype=torch.bfloat16), lay, dev)
    o, dq, dk, dvv = zeros(dv, "hbtd"), zeros(dqk, "bhtd"), zeros(dqk, "pad"), zeros(dv, "hbtd")
    assert len({x.stride() for x in (q, k, v, o)}) == 4  # four different memory layouts
    lse = torch.empty(B, NH, T, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.attn_fwd(q.data_ptr(), _st(q), k.data_ptr(), _st(k), v.data_ptr(), _st(v), o.data_ptr(), _st(o),
                      lse.data_ptr(), B, NH, T, dqk, dv, ctypes.c_float(w.scale), causal, stream)
    assert st == 0, lib.attn_status_string(st)
    nbytes = lib.attn_bwd_workspace_bytes(B, NH, T, dqk, dv, deterministic)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    st = lib.attn_bwd(q.data_ptr(), _st(q), k.data_ptr(), _st(k), v.data_ptr(), _st(v), o.data_ptr(), _st(o),
                      lse.data_ptr(), do.data_ptr(), _st(do), dq.data_ptr(), _st(dq), dk.data_ptr(), _st(dk),
                      dvv.data_ptr(), _st(dvv), B, NH, T, dqk, dv, ctypes.c_float(w.scale), causal, deterministic,
                      ws.data_ptr(), nbytes, stream)
    assert st == 0, lib.attn_status_string(st)
    torch.cuda.synchronize()
    got = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dvv.cpu()}
    compare(w, got, oracle(w, cpu))


def test_binding_rejects_bad_dropout_buffers():
    """The keep-bit buffer is read (and written by dropout_mask) as plain bytes from its
    first address: a host buffer, another element type or a strided view is refused
    before any launch."""
    w = workloads.Workload("drop_bufs", 1, 2, 128, 64, 64, True, 78)
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    need = int(attn.load().attn_dropout_mask_bytes(1, 2, 128))
    for bad in (torch.empty(need, dtype=torch.uint8), torch.empty(need, dtype=torch.float32, device=dev),
                torch.empty(2 * need, dtype=torch.uint8, device=dev)[::2]):
        with pytest.raises(ValueError):
            attn.dropout_mask(0.1, 1, 0, 1, 2, 128, True, device=dev, out=bad)
    mask = attn.dropout_mask(0.1, 1, 0, 1, 2, 128, True, device=dev)
    strided = torch.empty(2 * mask.numel(), dtype=torch.uint8, device=dev)[::2]
    strided.copy_(mask)
    o, lse = attn.fwd_dropout(q, k, v, mask, 0.1, True, w.scale)
    for bad in (mask.cpu(), strided):
        with pytest.raises(ValueError):
            attn.fwd_dropout(q, k, v, bad, 0.1, True, w.scale)
        with pytest.raises(ValueError):
            attn.bwd_dropout(q, k, v, o, lse, do, bad, 0.1, True, w.scale)
    torch.cuda.synchronize()


def test_binding_rejects_host_lse_and_workspace():
    """The library sees only pointers: an lse or workspace left in host memory would be
    handed to the kernels as a device address.  The binding refuses both before any
    launch."""
    w = workloads.Workload("host_bufs", 1, 2, 128, 64, 64, True, 77)
    cpu = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = attn.fwd(q, k, v, True, w.scale)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse.cpu(), do, True, w.scale)
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, True, w.scale, lse=torch.empty(1, 2, 128, dtype=torch.float32))
    need = attn.workspace_bytes(1, 2, 128, 64, 64, True)
    with pytest.raises(ValueError):
        attn.bwd(q, k, v, o, lse, do, True, w.scale, deterministic=True, workspace=torch.empty(need, dtype=torch.uint8))
    torch.cuda.synchronize()
