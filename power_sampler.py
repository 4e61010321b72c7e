"""Samples one GPU's shader clock, socket power, power-limit residency and temperature while
another process runs, and writes one JSON object per sample to a file.

  python power_sampler.py --bdf 0000:xx:00.0 --out samples.jsonl [--period 0.02]

Started by ``bench.py`` as a child process of its own before a sustained timed loop
and stopped (SIGTERM) after it, so the clock and power the kernels actually ran at can
be set beside the throughput.  It only reads the driver's metrics (amdsmi): it never
touches the GPU's compute queues.

Each line: {"t": host time (s), "gfxclk_mhz": current shader clock (the mean over the
XCDs where the driver reports one per XCD), "power_w": current socket power, "temp_c": hotspot temperature,
"throttle": the driver's throttle status word, "fw_ts": the metrics table's firmware
timestamp, "acc" / "ppt_acc" / "thm_acc": the firmware's sample counter and its counts
of samples at the package power limit and at the thermal limit}.  The first line is
{"metrics_keys": [...]} (what the driver reports, for the record).
"""
from __future__ import annotations

import argparse
import json
import signal
import sys
import time


def _num(x):
    try:
        v = float(x)
    except (TypeError, ValueError):
        return None
    # the driver reports unsupported fields as all-ones words
    return None if v in (0xFFFF, 0xFFFFFFFF, 0xFFFFFFFFFFFFFFFF) else v


def _mean(xs):
    vals = [v for v in (_num(x) for x in xs) if v is not None and v > 0]
    return sum(vals) / len(vals) if vals else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--bdf", required=True, help="PCI address of the GPU, domain:bus:device.function")
    ap.add_argument("--out", required=True)
    ap.add_argument("--period", type=float, default=0.02, help="seconds between samples")
    args = ap.parse_args()

    import amdsmi

    stop = {"now": False}
    signal.signal(signal.SIGTERM, lambda *_: stop.update(now=True))
    amdsmi.amdsmi_init()
    try:
        want = args.bdf.lower()
        handle = None
        for h in amdsmi.amdsmi_get_processor_handles():
            if amdsmi.amdsmi_get_gpu_device_bdf(h).lower() == want:
                handle = h
                break
        if handle is None:
            raise SystemExit(f"power_sampler: no GPU at {args.bdf}")
        with open(args.out, "w") as f:
            first = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            f.write(json.dumps({"metrics_keys": sorted(first)}) + "\n")
            f.flush()
            while not stop["now"]:
                t = time.time()
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clk = m.get("current_gfxclks")
                clk = _mean(clk) if isinstance(clk, (list, tuple)) else _num(m.get("current_gfxclk"))
                f.write(json.dumps({
                    "t": t,
                    "gfxclk_mhz": clk,
                    "power_w": _num(m.get("current_socket_power")),
                    "temp_c": _num(m.get("temperature_hotspot")),
                    "throttle": m.get("throttle_status"),
                    # the firmware refreshes the metrics table about once a second: its
                    # timestamp tells the refreshes apart; the residency accumulators count
                    # firmware samples spent at the package power limit (ppt) or the thermal
                    # limit, accumulation_counter all firmware samples
                    "fw_ts": _num(m.get("firmware_timestamp")),
                    "acc": _num(m.get("accumulation_counter")),
                    "ppt_acc": _num(m.get("ppt_residency_acc")),
                    "thm_acc": _num(m.get("socket_thm_residency_acc")),
                }) + "\n")
                f.flush()
                time.sleep(args.period)
    finally:
        amdsmi.amdsmi_shut_down()


if __name__ == "__main__":
    sys.exit(main())
