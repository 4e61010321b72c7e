"""The forward and backward captured in a HIP graph and replayed.

The library launches kernels only (no allocation, memset or synchronisation), so a
caller can capture a whole training step.  The graph is replayed several times, with the
program's own eager work and synchronisations between the replays, and every replay
must reproduce the eager result: bit for bit in the deterministic mode, within the bf16
tolerance in the atomic one (its dQ sums in no fixed order).
"""
import pytest
import torch

import exact_attention_53_amd as attn
import workloads
from tests.gpu_cases import check_bf16, say, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("deterministic", [True, False], ids=["determ", "atomic"])
# the last case: B * NH * ceil(T / 128) = 32, so at d = 64 the deterministic backward's
# key/value and dQ work run as one launch inside the graph
@pytest.mark.parametrize("dims,T,NH", [((128, 128), 333, 3), ((64, 64), 256, 3), ((64, 64), 512, 4)])
def test_graph_replays_match_eager(dims, T, NH, deterministic):
    dqk, dv_ = dims
    w = workloads.Workload(f"graph_T{T}_d{dqk}_NH{NH}", 2, NH, T, dqk, dv_, True, 600 + T)
    say(f"case graph {w.name} det={deterministic}")
    dev = torch.device("cuda:0")
    cpu = workloads.make_inputs(w)
    q, k, v, do = (cpu[n].to(dev) for n in ("q", "k", "v", "do"))
    B, NH = w.B, w.NH
    o = torch.empty(B, T, NH, dv_, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, NH, T, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(attn.workspace_bytes(B, NH, T, dqk, dv_, deterministic), dtype=torch.uint8, device=dev)

    def step():
        attn.fwd(q, k, v, True, w.scale, out=o, lse=lse)
        attn.bwd(q, k, v, o, lse, do, True, w.scale, deterministic, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for x in (o, lse, dq, dk, dv):  # eager work between the replays
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(("o", "lse", "dq", "dk", "dv"), eager, (o, lse, dq, dk, dv)):
            if deterministic or n in ("o", "lse"):
                assert torch.equal(a, b), f"replay {rep}: {n} differs from the eager result"
            else:
                check_bf16(f"replay {rep} {n}", to_np(b), to_np(a))
    del graph
    torch.cuda.synchronize()
