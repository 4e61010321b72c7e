"""Throughput of the fused exact-attention path (forward + backward) on one MI355X.

A step is one forward and one backward pass (every stage of the hot path) over one
batch of synthetic input already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--dq-mode deterministic|atomic] [--no-cpu-baseline] [--cold]

FLOP convention: per unmasked (query, key) pair and head, the forward counts
2 (d_qk + d_v) (S = QK^T, O = PV) and the backward 2 (3 d_qk + 2 d_v) (S recomputed,
dQ, dK over d_qk; dP, dV over d_v).  Exp, max and elementwise work are not counted.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attention fwd+bwd TFLOP/s (bf16) and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0


# HBM traffic per launch on the headline workload (B4 NH16 T8192 d128 causal,
# deterministic dQ), from two rocprofv3 --pmc passes over `bench.py --steps 1 --warmup 0
# --no-cpu-baseline --no-extras`: FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch.  They are scaled by
# what the same counters read for a streaming kernel of known size (`bench.py
# --copy-calibration 1024`, 1 GiB read and 1 GiB written per launch): FETCH_SIZE read
# 524294.5 KiB there, WRITE_SIZE 1048576 KiB.  The figures hold only for the kernel
# sources they were taken on, identified by a hash of their code; any change to the code
# (not to its comments) makes them null.
TRAFFIC_SOURCES = "8bbb21248f275bfa"
TRAFFIC_KIB = {  # kernel: (FETCH_SIZE, WRITE_SIZE) per dispatch
    "attn_fwd": (1173027.5, 133181.59375),
    "bwd_preprocess": (132232.375, 4369.375),
    "bwd_kv": (1267532.875, 262144.0),
    "bwd_dq": (812033.3125, 131072.0),
}
FETCH_SCALE = 1048576.0 / 524294.5
WRITE_SCALE = 1048576.0 / 1048576.0


def _code_tokens(text: str, lang: str) -> bytes:
    """The code of a source file without its comments, as whitespace-separated tokens, so
    that editing a comment or re-wrapping lines leaves the hash unchanged."""
    import re
    if lang == "c":
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
    else:  # Python: whole-line comments only (a '#' inside a string stays)
        text = re.sub(r"(?m)^\s*#[^\n]*$", " ", text)
    return " ".join(text.split()).encode()


def kernel_sources_hash() -> str:
    """Hash of the code the kernels are built from: the HIP sources and headers and the
    build script (whose flags shape the code), comments and layout aside."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_53_amd", "csrc")
    build = os.path.join(ROOT, "exact_attention_53_amd", "_build.py")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))) + [build]:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_tokens(fh.read(), "py" if f.endswith(".py") else "c"))
    return h.hexdigest()[:16]


def hbm_traffic(kernel: str, w, dq_mode: str, dtype: str = "bf16"):
    """Measured HBM bytes per launch of `kernel`, or None where no measurement of the
    current sources on this workload exists."""
    if w.name != "headline" or dq_mode != "deterministic" or dtype != "bf16" or kernel not in TRAFFIC_KIB:
        return None
    if kernel_sources_hash() != TRAFFIC_SOURCES:
        return None
    fetch, write = TRAFFIC_KIB[kernel]
    return round((fetch * FETCH_SCALE + write * WRITE_SCALE) * 1024.0)


def pairs_of(w):
    """Attended (query, key) pairs over all heads (block-sparse: counted from the map;
    padded batches: from each sequence's own length)."""
    import workloads
    if w.name == "blocksparse":
        return workloads.block_map_pairs(w, workloads.block_map(w))
    if w.name == "varlen":
        return w.NH * sum(int(n) * (int(n) + 1) // 2 if w.causal else int(n) ** 2 for n in workloads.varlen_lengths(w))
    return w.pairs()


def flops(w):
    pairs = pairs_of(w)
    return 2.0 * (w.d_qk + w.d_v) * pairs, 2.0 * (3 * w.d_qk + 2 * w.d_v) * pairs


def alg_bytes(w):
    """HBM bytes the method must move (each tensor read or written once): the forward
    reads Q, K, V and writes O and LSE; the backward reads Q, K, V, O, dO and LSE and writes
    dQ, dK, dV (D is its own intermediate: written and read once, 8 bytes per row)."""
    import workloads
    rows = w.NH * int(workloads.varlen_lengths(w).sum()) if w.name == "varlen" else w.B * w.NH * w.T
    fwd = rows * (2 * (2 * w.d_qk + w.d_v) + 2 * w.d_v + 4)
    bwd = rows * (2 * (2 * w.d_qk + 3 * w.d_v) + 4 + 8 + 2 * (2 * w.d_qk + w.d_v))
    return float(fwd), float(bwd)


def cpu_baseline(w, seconds_budget: float = 20.0):
    """Times the CPU oracle (numpy float64) on a bounded sample of the same workload:
    complete forward + backward of whole (b, h) heads."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads
    from oracle import attn_ref

    cpu = workloads.make_inputs(w)
    lengths = workloads.varlen_lengths(w) if w.name == "varlen" else None

    def head_flops(b):
        if lengths is None:
            return sum(flops(w.with_(B=1, NH=1)))
        n = int(lengths[b])
        return 2.0 * (4 * w.d_qk + 3 * w.d_v) * (n * (n + 1) // 2 if w.causal else n * n)

    flops_done = 0.0
    done, t_total, heads = 0, 0.0, []
    all_heads = [(b, h) for b in range(w.B) for h in range(w.NH)]
    while done < len(all_heads) and t_total < seconds_budget * 0.5:
        hd = all_heads[done]
        t0 = time.perf_counter()
        if w.name == "dropout":
            attn_ref.attn_ref_dropout(cpu["q"], cpu["k"], cpu["v"], cpu["do"], workloads.DROPOUT_P, w.seed, 0, w.causal,
                                      w.scale, heads=[hd])
        elif w.name == "keybias":
            attn_ref.attn_ref_keybias(cpu["q"], cpu["k"], cpu["v"], cpu["do"], workloads.key_bias(w), w.causal,
                                      w.scale, heads=[hd])
        elif w.name == "blocksparse":
            attn_ref.attn_ref_blocksparse(cpu["q"], cpu["k"], cpu["v"], cpu["do"], workloads.block_map(w), w.causal,
                                          w.scale, heads=[hd])
        elif lengths is not None:  # one sequence, one head, at its own length
            b_, h_ = hd
            sl = (slice(b_, b_ + 1), slice(None), slice(h_, h_ + 1))
            n = lengths[b_:b_ + 1]
            attn_ref.attn_ref_varlen(cpu["q"][sl], cpu["k"][sl], cpu["v"][sl], cpu["do"][sl], n, n, w.causal, w.scale)
        else:
            attn_ref.attn_ref_heads(cpu["q"], cpu["k"], cpu["v"], cpu["do"], w.causal, w.scale, heads=[hd],
                                    window=w.window, alibi=w.alibi)
        t_total += time.perf_counter() - t0
        flops_done += head_flops(hd[0])
        heads.append(hd)
        done += 1
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max((i.get("num_threads", 1) for i in blas), default=1)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": flops_done / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(all_heads)} (b,h) heads of the {w.name} workload, full forward+backward "
                  f"per head in numpy float64 ({t_total:.1f} s)",
        "host": {"cpu": cpu_model, "affinity": len(os.sched_getaffinity(0)), "numpy": np.__version__,
                 "blas": ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas)},
    }


POWER_SECONDS = 5.0


def sustained_clock_power(run_step, ms_step: float, dev, value: float, keep: str = ""):
    """Runs steps back to back for about POWER_SECONDS while power_sampler.py (a child
    process of its own, started before the loop) records the GPU's shader clock and
    power.  Returns the means over the loop (its first second left out), the throughput of
    that loop, and the fraction of the bf16 MFMA peak at the clock observed (the spec peak
    scaled by observed clock / 2400 MHz).  None when the amdgpu kernel driver's metrics are unreadable."""
    import subprocess
    import tempfile

    import torch

    try:
        pr = torch.cuda.get_device_properties(dev)
        bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0"
    except Exception as e:  # noqa: BLE001
        return {"error": f"no PCI address: {e}"}
    out = tempfile.NamedTemporaryFile(prefix="power_", suffix=".jsonl", delete=False).name
    sampler = subprocess.Popen([sys.executable, os.path.join(ROOT, "power_sampler.py"), "--bdf", bdf, "--out", out],
                               stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    try:
        time.sleep(1.0)  # the sampler's import and first reads
        if sampler.poll() is not None:
            return {"error": "sampler exited: " + sampler.stderr.read().decode()[-300:]}
        n = max(1, int(POWER_SECONDS * 1e3 / max(ms_step, 1e-3)))
        torch.cuda.synchronize()
        t0 = time.time()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            run_step()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.time()
        ms = e0.elapsed_time(e1) / n
    finally:
        sampler.terminate()
        try:
            sampler.wait(timeout=10)
        except subprocess.TimeoutExpired:
            sampler.kill()
    rows = []
    with open(out) as f:
        for line in f:
            r = json.loads(line)
            if "t" in r and t0 + 1.0 <= r["t"] <= t1:
                rows.append(r)
    # the firmware refreshes its metrics about once a second: keep the first sighting of
    # each refresh (its host time is the refresh time to within one sampling period)
    snaps, seen = [], set()
    for r in rows:
        key = r.get("fw_ts")
        if key is None or key not in seen:
            seen.add(key)
            snaps.append(r)
    if keep:
        import shutil
        shutil.move(out, keep)
    else:
        os.unlink(out)

    def mean(key):
        vals = [r[key] for r in rows if r.get(key) is not None]
        return sum(vals) / len(vals) if vals else None

    def smean(key):
        vals = [r[key] for r in snaps if r.get(key) is not None]
        return sum(vals) / len(vals) if vals else None

    def delta(key, a, b):
        return b[key] - a[key] if a.get(key) is not None and b.get(key) is not None else None

    clk = smean("gfxclk_mhz")
    ppt = thm = None
    if len(snaps) >= 2:
        dacc = delta("acc", snaps[0], snaps[-1])
        if dacc:
            dp, dt_ = delta("ppt_acc", snaps[0], snaps[-1]), delta("thm_acc", snaps[0], snaps[-1])
            ppt = dp / dacc if dp is not None else None
            thm = dt_ / dacc if dt_ is not None else None
    sustained = value * ms_step / ms
    res = {
        "seconds": round(t1 - t0, 2), "steps": n, "samples": len(rows), "refreshes": len(snaps),
        "ms_per_step": round(ms, 4), "tflops": round(sustained, 1),
        "gfxclk_mhz_mean": round(clk, 1) if clk else None,
        "gfxclk_mhz_min": min((r["gfxclk_mhz"] for r in snaps if r.get("gfxclk_mhz")), default=None),
        "power_w_mean": round(smean("power_w"), 1) if smean("power_w") else None,
        "ppt_limit_residency": round(ppt, 3) if ppt is not None else None,
        "thermal_limit_residency": round(thm, 3) if thm is not None else None,
        "temp_c_max": max((r["temp_c"] for r in rows if r.get("temp_c") is not None), default=None),
        "throttle_status": sorted({str(r.get("throttle")) for r in rows}),
    }
    if clk:
        res["frac_of_peak_at_observed_clock"] = round(sustained / (PEAK_BF16_TFLOPS * clk / 2400.0), 4)
    return res


def decode_bench(args, w):
    """One decode step per sequence: the inference forward (no stats) of one query row
    against each sequence's w.T-row key/value cache (attn_fwd_decode).  HBM-bound:
    reported as the K, V, Q and O bytes moved per second against the 8 TB/s peak."""
    import torch

    import exact_attention_53_amd as attn
    import workloads

    dev = torch.device("cuda:0")
    B, T, NH = w.B, w.T, w.NH
    et = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    k = workloads._randn((B, T, NH, w.d_qk), w.seed + 1, w.sigma, et)
    v = workloads._randn((B, T, NH, w.d_v), w.seed + 2, w.sigma, et)
    q = workloads._randn((B, 1, NH, w.d_qk), w.seed + 0, w.sigma, et)
    lay = args.layout
    if lay == "bhtd":  # head-major cache: each head's keys contiguous
        k, v, q = (x.permute(0, 2, 1, 3).contiguous() for x in (k, v, q))
    k, v, q = k.to(dev), v.to(dev), q.to(dev)
    o = torch.empty((B, 1, NH, w.d_v) if lay == "bthd" else (B, NH, 1, w.d_v), dtype=et, device=dev)
    for _ in range(args.warmup):
        attn.fwd_decode(q, k, v, None, w.scale, out=o, layout=lay)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        attn.fwd_decode(q, k, v, None, w.scale, out=o, layout=lay)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    moved = B * NH * (T * (w.d_qk + w.d_v) * 2 + (w.d_qk + w.d_v) * 2)  # K, V read; q read, o written
    gbs = moved / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "decode attention forward HBM GB/s", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"decode: B={B} NH={NH} one query row against {T} keys, d={w.d_qk}, non-causal, "
                               f"no stats, {lay.upper()} cache", "B": B, "NH": NH, "T_kv": T, "d": w.d_qk,
                   "layout": lay},
        "tflops": round(2.0 * (w.d_qk + w.d_v) * B * NH * T / (ms * 1e-3) / 1e12, 2),
        "roofline": {"kernel": "attn_fwd (decode)", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
    }), flush=True)


PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA: twice the bf16 rate


def fp8_bench(args, w):
    """The fp8 (e4m3) forward alone (its transpose of V included): forward TFLOP/s against
    the dense fp8 MFMA peak, with the bf16 forward of the same workload timed beside it."""
    import torch

    import exact_attention_53_amd as attn
    import workloads

    dev = torch.device("cuda:0")
    x = workloads.make_fp8_inputs(w)
    q8, k8, v8 = (x[n].to(dev) for n in ("q8", "k8", "v8"))
    B, T, NH = w.B, w.T, w.NH
    o = torch.empty((B, T, NH, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    ws = torch.empty(attn.load().attn_fwd_fp8_workspace_bytes(B, NH, T, w.d_qk, w.d_v), dtype=torch.uint8,
                     device=dev)

    def run():
        attn.fwd_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], w.causal, w.scale, out=o, lse=lse,
                     workspace=ws)

    def timeit(fn, n):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timeit(run, args.steps)
    cpu = workloads.make_inputs(w)
    qb, kb, vb = (cpu[n].to(dev) for n in ("q", "k", "v"))
    del cpu
    ms_bf16 = timeit(lambda: attn.fwd(qb, kb, vb, w.causal, w.scale, out=o, lse=lse), args.steps)
    f_fwd = flops(w)[0]
    tf = f_fwd / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "causal attention fwd TFLOP/s (fp8 e4m3 inputs) and % of MI355X fp8 MFMA peak", "value": round(tf, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "config": {"workload": f"{w.name} forward only, fp8 e4m3 Q/K/V with per-tensor descales, bf16 O: B={B} NH={NH} "
                               f"T={T} d={w.d_qk} {'causal' if w.causal else 'non-causal'}",
                   "B": B, "NH": NH, "T": T, "d_qk": w.d_qk, "d_v": w.d_v, "causal": w.causal},
        "pct_of_peak": round(100.0 * tf / PEAK_FP8_TFLOPS, 2),
        "bf16_fwd_same_workload": {"ms": round(ms_bf16, 4), "tflops": round(f_fwd / (ms_bf16 * 1e-3) / 1e12, 2)},
        "speedup_over_bf16_fwd": round(ms_bf16 / ms, 3),
        "roofline": {"kernel": "attn_fwd_fp8", "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None},
    }), flush=True)


def copy_calibration(mib: int):
    """A streaming kernel of known size: an elementwise negation that reads and writes
    exactly mib MiB per launch (a kernel, unlike a DMA copy, is seen by the counters).
    The FETCH_SIZE / WRITE_SIZE counters of these launches give the factor that turns
    the counters of the attention kernels into bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--dq-mode", choices=["deterministic", "atomic"], default="deterministic",
                    help="dQ summed in a fixed order without atomics (default) or by fp32 atomics")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other-dQ-mode timing and the sustained clock/power window")
    ap.add_argument("--power-seconds", type=float, default=5.0,
                    help="length of the sustained loop timed beside the clock/power sampler")
    ap.add_argument("--power-log", default="", help="keep the sampler's samples (JSON lines) in this file")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="only time the CPU oracle on a bounded sample of the workload (no GPU use)")
    ap.add_argument("--dtype", choices=["bf16", "f16", "fp8"], default="bf16",
                    help="element type of Q, K, V, O and the gradients (the metric is quoted for bf16); fp8: the "
                         "e4m3 forward alone")
    ap.add_argument("--layout", choices=["bthd", "bhtd"], default="bthd",
                    help="decode workload only: the key/value cache token-major (B, T, NH, d) or head-major "
                         "(B, NH, T, d)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed (no host launch "
                         "overhead between the kernels); reported as graph_* beside the eager figures")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB buffer before every step (evicts the 256 MB last-level cache); "
                         "the step time is then the sum of the kernel intervals, without the eviction")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the known-size "
                         "kernel that scales the HBM byte counters)")
    args = ap.parse_args()
    global POWER_SECONDS
    POWER_SECONDS = args.power_seconds
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} given): attention shards over "
              f"(batch, head) pairs with no communication, so each GPU runs its share as this "
              f"one-GPU workload", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.cpu_baseline_only:
        import workloads
        w = workloads.WORKLOADS[args.workload]
        print(json.dumps({"workload": w.name, "cpu_baseline": cpu_baseline(w)}), flush=True)
        return

    import torch

    import exact_attention_53_amd as attn
    import workloads

    w = workloads.WORKLOADS[args.workload]
    if w.name == "decode":
        decode_bench(args, w)
        return
    if args.dtype == "fp8":
        fp8_bench(args, w)
        return
    dev = torch.device("cuda:0")
    et = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    cpu = workloads.make_inputs(w, et)
    if w.packed:
        qkv = cpu["qkv"].to(dev)
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    else:
        q, k, v = (cpu[n].to(dev) for n in ("q", "k", "v"))
    do = cpu["do"].to(dev)
    del cpu
    B, T, NH = w.B, w.T, w.NH
    o = torch.empty((B, T, NH, w.d_v), dtype=et, device=dev)
    lse = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, NH, w.d_qk), dtype=et, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty((B, T, NH, w.d_v), dtype=et, device=dev)
    det = args.dq_mode == "deterministic"
    workspaces = {}

    def workspace(mode_det):
        if mode_det not in workspaces:
            lib = attn.load()
            if w.name == "blocksparse":
                nbytes = lib.attn_bwd_blocksparse_workspace_bytes(B, NH, T, w.d_qk, w.d_v, int(mode_det))
            elif w.name == "keybias":
                nbytes = lib.attn_bwd_keybias_workspace_bytes(B, NH, T, w.d_qk, w.d_v, int(mode_det))
            elif w.name == "varlen":
                nbytes = lib.attn_bwd_varlen_workspace_bytes(B, NH, T, w.d_qk, w.d_v, int(mode_det))
            else:
                nbytes = attn.workspace_bytes(B, NH, T, w.d_qk, w.d_v, mode_det)
            workspaces[mode_det] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return workspaces[mode_det]

    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev) if args.cold else None

    bsp = w.name == "blocksparse"
    kbw = w.name == "keybias"
    drw = w.name == "dropout"
    vl = w.name == "varlen"
    if vl:  # per-sequence lengths on the device; the forward's work list in its own workspace
        seqs = torch.from_numpy(workloads.varlen_lengths(w)).to(dev)
        fws = torch.empty(max(1, attn.load().attn_fwd_varlen_workspace_bytes(B, NH, T, w.d_qk, w.d_v)),
                          dtype=torch.uint8, device=dev)
    if drw:  # the keep bits are drawn inside every timed step (before the forward)
        dmask = attn.dropout_mask(workloads.DROPOUT_P, w.seed, 0, B, NH, T, w.causal, device=dev)
    if kbw:
        kbias = torch.from_numpy(workloads.key_bias(w)).to(dev)
        dbias = torch.empty_like(kbias)
        fws = torch.empty(attn.load().attn_fwd_keybias_workspace_bytes(B, NH, T, w.d_qk, w.d_v), dtype=torch.uint8,
                          device=dev)
    if bsp:
        bmap = torch.from_numpy(workloads.block_map(w)).to(dev)
        fws = torch.empty(attn.load().attn_fwd_blocksparse_workspace_bytes(B, NH, T, w.d_qk, w.d_v), dtype=torch.uint8,
                          device=dev)

    def fwd_call():
        if drw:
            attn.dropout_mask(workloads.DROPOUT_P, w.seed, 0, B, NH, T, w.causal, device=dev, out=dmask)
            attn.fwd_dropout(q, k, v, dmask, workloads.DROPOUT_P, w.causal, w.scale, out=o, lse=lse)
        elif kbw:
            attn.fwd_keybias(q, k, v, kbias, w.causal, w.scale, out=o, lse=lse, workspace=fws)
        elif bsp:
            attn.fwd_blocksparse(q, k, v, bmap, w.causal, w.scale, out=o, lse=lse, workspace=fws)
        elif vl:
            attn.fwd_varlen(q, k, v, seqs, seqs, w.causal, w.scale, out=o, lse=lse, workspace=fws)
        else:
            attn.fwd(q, k, v, w.causal, w.scale, out=o, lse=lse, window=w.window, alibi=w.alibi)

    def bwd_call(mode_det, ws, stages):
        if drw:
            attn.bwd_dropout(q, k, v, o, lse, do, dmask, workloads.DROPOUT_P, w.causal, w.scale, mode_det, dq=dq, dk=dk,
                             dv=dv, workspace=ws, stages=stages)
        elif kbw:
            attn.bwd_keybias(q, k, v, o, lse, do, kbias, w.causal, w.scale, mode_det, dq=dq, dk=dk, dv=dv,
                             dbias=dbias, workspace=ws, stages=stages)
        elif bsp:
            attn.bwd_blocksparse(q, k, v, o, lse, do, bmap, w.causal, w.scale, mode_det, dq=dq, dk=dk, dv=dv,
                                 workspace=ws, stages=stages)
        elif vl:
            attn.bwd_varlen(q, k, v, o, lse, do, seqs, seqs, w.causal, w.scale, mode_det, workspace=ws, dq=dq, dk=dk,
                            dv=dv, stages=stages)
        else:
            attn.bwd(q, k, v, o, lse, do, w.causal, w.scale, mode_det, dq=dq, dk=dk, dv=dv, workspace=ws,
                     stages=stages, window=w.window, alibi=w.alibi)

    def step(ev=None, mode_det=det, split=False):
        """One forward and one backward.  The backward is one call, as a user makes it (at
        d = 64 in deterministic mode the key/value and dQ work then share one launch), or,
        with split, its three stages as three calls with events between them, for the
        per-kernel times."""
        ws = workspace(mode_det)
        if flush is not None:
            flush.fill_(1.0)
        if ev is not None:
            ev[0].record()
        fwd_call()
        if ev is not None:
            ev[1].record()
        if not split:
            bwd_call(mode_det, ws, attn.ALL_STAGES)
            if ev is not None:
                ev[4].record()
            return
        bwd_call(mode_det, ws, attn.PREPROCESS)
        if ev is not None:
            ev[2].record()
        bwd_call(mode_det, ws, attn.MAIN)
        if ev is not None:
            ev[3].record()
        bwd_call(mode_det, ws, attn.DQ)
        if ev is not None:
            ev[4].record()

    def timed(n, mode_det, split):
        """n steps bracketed by events; returns (ms per step, ms of the forward and of the
        backward call, or with split of the forward and each backward stage, wall s)."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        start.record()
        for i in range(n):
            step(evs[i], mode_det, split)
        end.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall

        def avg(a, b):
            return sum(e[a].elapsed_time(e[b]) for e in evs) / n

        parts = (avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)) if split else (avg(0, 1), avg(1, 4))
        return start.elapsed_time(end) / n, parts, t_wall

    def measure(n, mode_det):
        """The timed steps (one backward call each) and, in a second loop of as many steps,
        the per-kernel split."""
        ms, (t_f, t_b), wall = timed(n, mode_det, False)
        step(mode_det=mode_det, split=True)
        _, per_kernel, _ = timed(n, mode_det, True)
        if args.cold:  # the eviction between steps is not part of the step
            ms = t_f + t_b
        return ms, t_f, t_b, per_kernel, wall

    for _ in range(args.warmup):
        step()
    ms_step, t_fwd_call, t_bwd_call, (t_fwd, t_pre, t_main, t_dq), t_wall = measure(args.steps, det)
    f_fwd, f_bwd = flops(w)
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    # Algorithmic flops carried by each kernel (recomputation is not counted): the
    # key/value kernel forms S, dP, dV, dK (and, in atomic mode, the dQ products); the
    # deterministic dQ kernel contributes the dQ product only.
    pairs = pairs_of(w)
    f_dq = 2.0 * w.d_qk * pairs
    f_main = f_bwd if not det else f_bwd - f_dq
    kernels = {
        "attn_fwd": {"ms": t_fwd, "flops": f_fwd},
        "bwd_preprocess": {"ms": t_pre, "flops": 0.0},
        "bwd_kv": {"ms": t_main, "flops": f_main},
        "bwd_dq" if det else "bwd_dq_convert": {"ms": t_dq, "flops": f_dq if det else 0.0},
    }
    for k_ in kernels.values():
        k_["tflops"] = k_["flops"] / (k_["ms"] * 1e-3) / 1e12 if k_["ms"] > 0 else 0.0
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    achieved = kernels[dom]["tflops"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={B} NH={NH} T={T} d_qk={w.d_qk} d_v={w.d_v} "
                        f"{'causal' if w.causal else 'non-causal'}"
                        f"{f' window {w.window}' if w.window else ''}{' ALiBi' if w.alibi else ''}"
                        f"{' block-sparse map (local band of 8 blocks + block 0)' if w.name == 'blocksparse' else ''}"
                        f"{' per-head key bias with dbias' if w.name == 'keybias' else ''}"
                        f"{f' dropout p={workloads.DROPOUT_P} (Philox keep bits drawn each step)' if w.name == 'dropout' else ''}"
                        f"{f' padded batch, sequence lengths {list(map(int, workloads.varlen_lengths(w)))}' if vl else ''}, "
                        f"{'packed QKV' if w.packed else 'BTHD'}, "
                        f"dQ mode {args.dq_mode}",
            "B": B, "NH": NH, "T": T, "d_qk": w.d_qk, "d_v": w.d_v, "causal": w.causal, "window": w.window, "alibi": w.alibi,
            "dq_mode": args.dq_mode,
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(f_fwd / (t_fwd_call * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / (t_bwd_call * 1e-3) / 1e12, 2),
        "fwd_ms": round(t_fwd_call, 4),
        "bwd_ms": round(t_bwd_call, 4),
        "kernels_ms": {n: round(v["ms"], 4) for n, v in kernels.items()},
        "kernels_tflops": {n: round(v["tflops"], 1) for n, v in kernels.items() if v["flops"] > 0},
        "alg_gbs": {"fwd": round(alg_bytes(w)[0] / (t_fwd_call * 1e-3) / 1e9, 1),
                    "bwd": round(alg_bytes(w)[1] / (t_bwd_call * 1e-3) / 1e9, 1)},
        "cache": "cold (1 GiB written before each step)" if args.cold else "warm",
        "wall_s_timed": round(t_wall, 3),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": hbm_traffic(dom, w, args.dq_mode, args.dtype),
            "traffic_unit": "bytes per launch",
        },
    }
    if args.graph and not args.cold:
        # One step (the forward and the backward call) captured in a HIP graph on a side
        # stream, then replayed: the same kernels, launched without the binding's host work
        # in between, which bounds short steps (the GPT-2 shape) rather than the kernels.
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step()
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_graph = g0.elapsed_time(g1) / args.steps
        line["graph_ms_per_step"] = round(ms_graph, 4)
        line["graph_value"] = round((f_fwd + f_bwd) / (ms_graph * 1e-3) / 1e12, 2)
        del graph
    if not args.cold and not args.no_extras:
        # The other dQ mode on the same inputs, a few steps: the atomic mode's extra time
        # in the key/value kernel (its partial dQ products and fp32 atomics) as a share of
        # its step, the analogue of the atomic-add share of total time.
        step(mode_det=not det)
        n_alt = max(3, min(10, args.steps))
        ms_alt, _, _, k_alt, _ = measure(n_alt, not det)
        ms_det, ms_atom = (ms_step, ms_alt) if det else (ms_alt, ms_step)
        kv_det, kv_atom = (t_main, k_alt[2]) if det else (k_alt[2], t_main)
        line["dq_modes"] = {
            "other_mode": "atomic" if det else "deterministic",
            "other_ms_per_step": round(ms_alt, 4),
            "other_kernels_ms": dict(zip(("attn_fwd", "bwd_preprocess", "bwd_kv",
                                          "bwd_dq_convert" if det else "bwd_dq"), (round(x, 4) for x in k_alt))),
            "atomic_over_deterministic_step_time": round(ms_atom / ms_det, 3),
            "atomic_share_of_atomic_step": round(max(0.0, kv_atom - kv_det) / ms_atom, 3),
        }
        line["clock_power"] = sustained_clock_power(lambda: step(), ms_step, dev, value, args.power_log)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
