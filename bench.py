"""Benchmark: causal prefill attention TFLOP/s, FP8 and BF16, S=32K, head dim 128.

One step is one pass of the whole path over one batch of seeded synthetic
input: an FP8 e4m3 forward (B=1, H=32, S=32768, D=128, Gaussian, per-tensor
scales) followed by a BF16 forward of the same shape, each one launch of the
HIP library on torch's current stream, inputs already resident in HBM.

FLOPs use the causal count B*H*S^2*(Dqk+Dv) (the visible half of the score
matrix, two matrix products of 2 flop per multiply-add); the figure under the
literal 2*B*H*S^2*(Dqk+Dv) formula is printed beside it. Peaks are MI355X's
published dense matrix-core figures: 5.0 PFLOP/s FP8, 2.5 PFLOP/s BF16.

Before the warmup steps, steps run back to back for a few seconds untimed
(--settle-seconds) so that the timed ones run at the sustained, power-limited
clock rather than the idle boost. The GPU clock is sampled (driver metrics
through amdsmi, or sysfs) while the timed steps run and reported beside them, with the mean kernel time of the
first and the last quarter of the timed launches. After the timed steps each
path also runs alone under a sustained load (4 s untimed, then about 2 s
timed, clock sampled), and the other full-size workloads (the MLA-shaped and
the peaked GQA FP8 prefills) and one GPU's share under 8-way head parallelism
are timed as extra fields, outside the step.

Prints one JSON line. --gpus above 1 is refused: the benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attn TFLOP/s, FP8 & BF16, S=32K hd128; % of MFMA peak"
PEAK = {"fp8": 5033.2, "bf16": 2516.6}  # TFLOP/s: 256 CU * 4 SIMD * {2048, 1024} flop/clk * 2.4 GHz
PATHS = ["fp8_mha_s32k", "bf16_mha_s32k"]
# the pages' own FP8 figures on these workloads (context, other builds)
PAGES_TFLOPS = {"fp8_mha_s32k": 2672.0, "fp8_mla_s32k": 2464.0}
# the other full-size workloads, timed after the benchmark step (not part of it)
OTHER_CONFIGS = ["fp8_mla_s32k", "fp8_gqa_s16k_peaked"]


# Sources whose text defines each kernel's code and launch: a stored HBM
# traffic figure is used only while their hash matches the one recorded with it.
_COMMON_SOURCES = ["include/fp8_bf16_causal.h", "fp8_bf16_causal_amd/csrc/attn_params.h",
                   "fp8_bf16_causal_amd/csrc/attn_common.h", "fp8_bf16_causal_amd/csrc/attn_launch.h",
                   "fp8_bf16_causal_amd/csrc/attn_api.cpp", "fp8_bf16_causal_amd/build.py"]
KERNEL_SOURCES = {
    "fp8": _COMMON_SOURCES + ["fp8_bf16_causal_amd/csrc/attn_fwd_fp8.hip"],
    "bf16": _COMMON_SOURCES + ["fp8_bf16_causal_amd/csrc/attn_fwd_bf16.hip"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_s32k_hbm_traffic.txt")
CLOCK_FILE = os.path.join(ROOT, "profiles", "attn_fwd_s32k_mfma_clock_lds.txt")


def _code_text(path):
    """A source file without its comments and blank lines (C/C++ `//` and
    `/* */` comments, Python `#` comments; these files hold no comment marker
    inside a string), so that editing a comment keeps the hash."""
    import re

    with open(path, encoding="utf-8") as f:
        text = f.read()
    if path.endswith(".py"):
        text = re.sub(r"#[^\n]*", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    lines = (ln.strip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def sources_sha256(kind):
    """Hash of the code (comments left out) of the files a kernel is built from."""
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        h.update(rel.encode() + b"\0" + _code_text(os.path.join(ROOT, rel)).encode() + b"\0")
    return h.hexdigest()


def profiled_line(path, workload, kind):
    """The key=value fields of the line for `workload` in a committed profile
    summary, if it was taken on the current kernel sources."""
    try:
        with open(path) as f:
            lines = [ln.split() for ln in f if ln.startswith("workload=")]
    except OSError:
        return None
    sha = sources_sha256(kind)
    for fields in lines:
        kv = dict(x.split("=", 1) for x in fields)
        if kv.get("workload") == workload and kv.get("sources_sha256") == sha:
            return kv
    return None


def measured_traffic(workload, kind):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (copy-calibrated), or None if it is missing or was taken on
    other kernel sources."""
    kv = profiled_line(TRAFFIC_FILE, workload, kind)
    return int(kv["traffic_bytes"]) if kv else None


def time_quant_prologue(steps, warmup):
    """The FP8 quantize prologue (attn_quantize_e4m3) on the 32K benchmark's
    query tensor as BF16 (32768 x 32 x 128), plain and with the Hadamard
    rotation: HBM-bound, 5 algorithmic bytes per element (two reads of the
    BF16 input, since the per-tensor amax precedes every code, and one byte
    written)."""
    import torch

    import fp8_bf16_causal_amd as fbc

    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((32768, 32, 128), generator=g, device="cuda").to(torch.bfloat16)
    n = x.numel()
    # the C-ABI call with its outputs allocated once, as a serving loop would
    # make it (the Python wrapper allocates fresh outputs on every call)
    y = torch.empty(n, dtype=torch.uint8, device="cuda")
    sc = torch.empty(2, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {"workload": "query tensor of fp8_mha_s32k as BF16, 32768 x 32 x 128", "bytes_per_element": 5,
           "peak_GBps": 8000.0, "call": "attn_quantize_e4m3, outputs allocated once"}

    def call(had):
        rc = fbc.attn_quantize_e4m3(x.data_ptr(), y.data_ptr(), sc.data_ptr(), 32768 * 32, 128, had, stream)
        if rc != fbc.ATTN_OK:
            raise RuntimeError(fbc.attn_strerror(rc))

    for had in (False, True):
        for _ in range(warmup):
            call(int(had))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call(int(had))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbs = 5.0 * n / (ms * 1e-3) / 1e9
        key = "hadamard" if had else "plain"
        res[key] = {"ms": round(ms, 4), "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / 8000.0, 4)}
    return res



def time_fp8_from_bf16(inp, steps=20, warmup=10):
    """FP8 prefill from BF16 activations end to end, on the BF16 benchmark's
    inputs (1 x 32K x 32 x 128): flash_attn_fp8_func, i.e. three quantize
    calls (Q and K with the Hadamard rotation) and the FP8 attention on the
    factors they leave on the device, against the BF16 attention on the same
    tensors. The two are timed alternately, median of `steps` each."""
    import torch

    import fp8_bf16_causal_amd as fbc

    p = inp.shape
    out = torch.empty((p["B"], p["S"], p["Hq"], p["Dv"]), dtype=torch.bfloat16, device="cuda")
    runs = {"fp8_chain": lambda: fbc.flash_attn_fp8_func(inp.q, inp.k, inp.v, inp.scale, out=out),
            "bf16": lambda: fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True, out=out)}
    for _ in range(warmup):
        for f in runs.values():
            f()
    torch.cuda.synchronize()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for k in runs}
    for s in range(steps):
        for k, f in runs.items():
            ev[k][s][0].record()
            f()
            ev[k][s][1].record()
    torch.cuda.synchronize()
    med = {k: sorted(a.elapsed_time(b) for a, b in v)[steps // 2] for k, v in ev.items()}
    del out
    return {"workload": "bf16_mha_s32k tensors; FP8 path = quantize Q, K (rotated) and V, then FP8 attention "
                        "on device factors (flash_attn_fp8_func)",
            "fp8_chain_ms_median": round(med["fp8_chain"], 4), "bf16_attention_ms_median": round(med["bf16"], 4),
            "speedup_vs_bf16": round(med["bf16"] / med["fp8_chain"], 3)}

# One GPU's share of each workload under 8-way tensor parallelism over heads
# (each GPU takes 1/8 of the KV heads with their query heads; no exchange).
TP_SHARES = [("fp8_mha_s32k", dict(Hq=4, Hkv=4)), ("bf16_mha_s32k", dict(Hq=4, Hkv=4)),
             ("fp8_gqa_s16k_peaked", dict(Hq=4, Hkv=1)), ("fp8_mla_s32k", dict(Hq=2, Hkv=2))]
N_CU, N_XCD, BQ, BK = 256, 8, 256, 128


def balance_bound(B, Hq, Hkv, S):
    """Upper bound on the fraction of the chip a causal grid can keep busy:
    mean CU load / largest CU load when the workgroups, in launch order, go
    round-robin to the 8 XCDs and, within one, each to the CU that frees
    first (one workgroup per CU at a time). A workgroup's load is its number
    of 128-key tiles. The launch order is the kernels' own: heaviest query
    blocks first over all heads, or, when B*Hkv is a multiple of 8, one KV
    head's blocks per XCD, heaviest first."""
    import heapq

    nqb = (S + BQ - 1) // BQ
    G = Hq // Hkv
    nkv = B * Hkv

    def tiles(qb):
        return (min(qb * BQ + BQ, S) + BK - 1) // BK

    order = []
    if nkv % N_XCD == 0:
        per_head = G * nqb
        for bid in range(B * Hq * nqb):
            slot = bid // N_XCD
            order.append(tiles(nqb - 1 - (slot % per_head) // G))
    else:
        for bid in range(B * Hq * nqb):
            order.append(tiles(nqb - 1 - bid // (nkv * G)))
    cus = [[0] * (N_CU // N_XCD) for _ in range(N_XCD)]
    for bid, w in enumerate(order):
        heap = cus[bid % N_XCD]
        heapq.heapreplace(heap, heap[0] + w)
    total = sum(order)
    return total / N_CU / max(max(h) for h in cus)


def time_tp_shares(full_paths, steps=20, warmup=20):
    """The kernels at one GPU's share of each workload under 8-way tensor
    parallelism (1/8 of the heads): small grids, where the causal imbalance
    between query blocks decides how much of the chip stays busy."""
    import torch

    import fp8_bf16_causal_amd as fbc
    from fp8_bf16_causal_amd import synth

    res = []
    for name, ov in TP_SHARES:
        inp = synth.make_config(name, device="cuda", **ov)
        p = inp.shape
        out = torch.empty((p["B"], p["S"], p["Hq"], p["Dv"]), dtype=torch.bfloat16, device="cuda")
        dq, dk, dv = inp.descale
        for _ in range(warmup):
            fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                                descale_q=dq, descale_k=dk, descale_v=dv, out=out)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record()
            fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                                descale_q=dq, descale_k=dk, descale_v=dv, out=out)
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[steps // 2]
        tf = causal_flops(p) / (ms * 1e-3) / 1e12
        nwg = p["B"] * p["Hq"] * ((p["S"] + BQ - 1) // BQ)
        row = {"workload": name, "share": "1/8 of the heads", "B": p["B"], "Hq": p["Hq"], "Hkv": p["Hkv"],
               "S": p["S"], "Dqk": p["Dqk"], "workgroups": nwg, "kernel_ms_median": round(ms, 4),
               "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK[inp.dtype], 4),
               "balance_bound": round(balance_bound(p["B"], p["Hq"], p["Hkv"], p["S"]), 4)}
        if name in full_paths:
            row["vs_full_shape"] = round(tf / full_paths[name]["tflops"], 4)
        res.append(row)
        del inp, out
    torch.cuda.empty_cache()
    return res


def time_other_configs(steps=20, warmup=20):
    """The kernels on the other full-size workloads: the MLA-shaped FP8
    prefill (head dim 192/128, H=16, S=32K) and the GQA FP8 prefill with
    peaked scores (Hq=32, Hkv=8, S=16K). Median of `steps` launches, each
    bracketed by events on the launch stream."""
    import torch

    import fp8_bf16_causal_amd as fbc
    from fp8_bf16_causal_amd import synth

    res = {}
    for name in OTHER_CONFIGS:
        inp = synth.make_config(name, device="cuda")
        p = inp.shape
        out = torch.empty((p["B"], p["S"], p["Hq"], p["Dv"]), dtype=torch.bfloat16, device="cuda")
        dq, dk, dv = inp.descale
        for _ in range(warmup):
            fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                                descale_q=dq, descale_k=dk, descale_v=dv, out=out)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in ev:
            a.record()
            fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                                descale_q=dq, descale_k=dk, descale_v=dv, out=out)
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[steps // 2]
        tf = causal_flops(p) / (ms * 1e-3) / 1e12
        row = {"B": p["B"], "Hq": p["Hq"], "Hkv": p["Hkv"], "S": p["S"], "Dqk": p["Dqk"], "Dv": p["Dv"],
               "kernel_ms_median": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK[inp.dtype], 4)}
        if name in PAGES_TFLOPS:
            row["pages_tflops"] = PAGES_TFLOPS[name]
            row["ratio_to_pages"] = round(tf / PAGES_TFLOPS[name], 3)
        res[name] = row
        del inp, out
    torch.cuda.empty_cache()
    return res


def _power_file():
    """The board's socket-power sensor (hwmon power1_input, microwatts), if the
    driver exposes one."""
    import glob

    files = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
    return files[0] if files else None


class ClockSampler:
    """Samples the GPU's current graphics clock from a reader thread while
    kernels run (every `period` s): the mean over the 8 XCDs' current gfxclk
    from the driver's metrics table through amdsmi, else amdsmi's single GFX
    clock, else the current line of sysfs pp_dpm_sclk. File and library reads
    only; nothing is sent to the GPU's queues."""

    def __init__(self, period=0.01):
        import threading

        self.period, self.samples, self.source = period, [], None
        self._stop = threading.Event()
        self._thread = None
        self._read = self._pick_source()

    def _pick_source(self):
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]

            def metrics():
                v = amdsmi.amdsmi_get_gpu_metrics_info(h).get("current_gfxclk")
                v = [x for x in (v if isinstance(v, list) else [v]) if isinstance(x, (int, float)) and 0 < x < 10000]
                return sum(v) / len(v) if v else None

            if metrics() is not None:
                self.source = "amdsmi gpu_metrics current_gfxclk (mean over XCDs)"
                return metrics

            def clock():
                return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"])

            clock()
            self.source = "amdsmi clock_info GFX"
            return clock
        except Exception:
            pass
        import glob
        import re

        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if files:
            def sysfs():
                with open(files[0]) as f:
                    for ln in f:
                        if ln.rstrip().endswith("*"):
                            m = re.search(r"(\d+)\s*Mhz", ln, re.I)
                            return float(m.group(1)) if m else None
                return None

            self.source = files[0]
            return sysfs
        return None

    def _loop(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except Exception:
                v = None
            if v:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        import threading

        if self._read:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def mean_mhz(self):
        return round(sum(self.samples) / len(self.samples), 1) if self.samples else None


def sustained(inputs, launch, seconds_warm, seconds_timed):
    """Each path alone, back to back: `seconds_warm` of untimed launches so the
    clock settles under the power limit, then about `seconds_timed` of timed
    launches (events on the launch stream around the whole loop) with the
    clock sampled meanwhile."""
    import torch

    res = {}
    for n in inputs:
        p = inputs[n].shape
        kind = inputs[n].dtype
        ck = ClockSampler()  # set up before the launches: no idle gap in front of the timed ones
        launch(n)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        k = 0
        while time.perf_counter() - t0 < seconds_warm:
            for _ in range(10):
                launch(n)
            torch.cuda.synchronize()
            k += 10
        per = (time.perf_counter() - t0) / k
        reps = max(10, int(seconds_timed / per))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with ck:
            e0.record()
            for _ in range(reps):
                launch(n)
            e1.record()
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = causal_flops(p) / (ms * 1e-3) / 1e12
        mhz = ck.mean_mhz()
        res[n] = {"warm_s": seconds_warm, "launches_timed": reps, "kernel_ms_mean": round(ms, 4),
                  "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK[kind], 4), "sclk_mhz": mhz,
                  "clock_samples": len(ck.samples),
                  "frac_of_peak_at_clock": None if not mhz else round(tf / (PEAK[kind] * mhz / 2400.0), 4)}
        if n in PAGES_TFLOPS:
            res[n]["ratio_to_pages"] = round(tf / PAGES_TFLOPS[n], 3)
    return res


def energy_study(seconds):
    """Sustained throughput, board power and energy efficiency of the FP8 and
    BF16 kernels on Gaussian and peaked operands of the same 32K shape (the
    pages report that the clock, and so the speed, depends on the operand
    values). Board power: hwmon power1_input sampled every 5 ms by a reader
    thread while the launches run (file reads only). Each case first runs for
    `seconds` untimed, then about `seconds` timed."""
    import threading

    import torch

    import fp8_bf16_causal_amd as fbc
    from fp8_bf16_causal_amd import synth

    pf = _power_file()

    def read_w():
        with open(pf) as f:
            return int(f.read()) / 1e6

    def sample(stop, out):
        while not stop.is_set():
            out.append(read_w())
            time.sleep(0.005)

    idle = None
    if pf:
        vals = []
        for _ in range(50):
            vals.append(read_w())
            time.sleep(0.01)
        idle = sum(vals) / len(vals)
    res = {"power_sensor": pf, "idle_W": None if idle is None else round(idle, 1), "cases": []}
    for name, structure in (("fp8_mha_s32k", "gaussian"), ("fp8_mha_s32k", "peaked"), ("bf16_mha_s32k", "gaussian"),
                            ("bf16_mha_s32k", "peaked")):
        inp = synth.make_config(name, device="cuda", structure=structure)
        p = inp.shape
        out = torch.empty((p["B"], p["S"], p["Hq"], p["Dv"]), dtype=torch.bfloat16, device="cuda")
        dq, dk, dv = inp.descale

        def launch():
            fbc.flash_attn_func(inp.q, inp.k, inp.v, inp.scale, causal=True,
                                descale_q=dq, descale_k=dk, descale_v=dv, out=out)

        launch()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_warm = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                launch()
            torch.cuda.synchronize()
            n_warm += 10
        per = (time.perf_counter() - t0) / n_warm
        n = max(10, int(seconds / per))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        watts, stop = [], threading.Event()
        th = threading.Thread(target=sample, args=(stop, watts)) if pf else None
        if th:
            th.start()
        e0.record()
        for _ in range(n):
            launch()
        e1.record()
        torch.cuda.synchronize()
        stop.set()
        if th:
            th.join()
        ms = e0.elapsed_time(e1) / n
        tf = causal_flops(p) / (ms * 1e-3) / 1e12
        w = sum(watts) / len(watts) if watts else None
        res["cases"].append({"workload": name, "structure": structure, "launches": 1 + n_warm + n, "timed": n,
                             "ms": round(ms, 4), "tflops": round(tf, 1),
                             "board_W": None if w is None else round(w, 1), "power_samples": len(watts),
                             "tflop_per_J": None if w is None else round(tf / w, 3)})
        print(json.dumps({"energy_case": res["cases"][-1]}), flush=True)
        del inp, out
        torch.cuda.empty_cache()
    return res


def causal_flops(p):
    return float(p["B"]) * p["Hq"] * p["S"] * p["S"] * (p["Dqk"] + p["Dv"])


def cpu_baseline(inputs, budget_rows, threads):
    """The fp64 oracle, as it stands, on a bounded sample of rows of the same
    workload, on the host cores."""
    import numpy as np

    import oracle
    from fp8_bf16_causal_amd import synth

    total_flop, total_s, parts = 0.0, 0.0, []
    for name, inp in inputs.items():
        p = inp.shape
        rng = np.random.default_rng(2024)
        n = budget_rows
        rows = np.stack([np.zeros(n, dtype=np.int64), rng.integers(0, p["Hq"], n), rng.integers(0, p["S"], n)], 1)
        q, k, v = synth.raw_codes(inp.q), synth.raw_codes(inp.k), synth.raw_codes(inp.v)
        dt = oracle.BF16 if inp.dtype == "bf16" else oracle.FP8_E4M3
        dq, dk, dv = inp.descale
        t0 = time.perf_counter()
        oracle.attention(q, k, v, dt, inp.scale, dq, dk, dv, rows=rows, nthreads=threads)
        dt_s = time.perf_counter() - t0
        flop = float(np.sum(rows[:, 2] + 1)) * 2.0 * (p["Dqk"] + p["Dv"])
        total_flop += flop
        total_s += dt_s
        parts.append(f"{n} random (head, row) pairs of {name}")
    return {"value": total_flop / total_s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(parts) + f"; {total_s:.1f} s of fp64 oracle time, causal flops of the sampled rows"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the timed ones")
    ap.add_argument("--settle-seconds", type=float, default=4.0,
                    help="back-to-back untimed steps for this long before the warmup steps, so that the timed steps "
                         "run at the sustained (power-limited) clock")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=65536, help="rows per path in the CPU-baseline sample (about 15 s of oracle time on 16 cores)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy (a known byte count for HBM counters)")
    ap.add_argument("--paths", default=",".join(PATHS))
    ap.add_argument("--no-quant", action="store_true", help="skip the FP8 quantize-prologue timing")
    ap.add_argument("--quant-only", action="store_true", help="time only the FP8 quantize prologue")
    ap.add_argument("--energy", action="store_true",
                    help="sustained speed, board power and TFLOP/J on Gaussian vs peaked operands (not a bench line)")
    ap.add_argument("--energy-seconds", type=float, default=4.0, help="untimed and timed seconds per energy case")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the timing of the other full-size workloads (MLA shape, peaked GQA)")
    ap.add_argument("--no-shares", action="store_true",
                    help="skip the timing of one GPU's share under 8-way tensor parallelism")
    ap.add_argument("--no-sustained", action="store_true",
                    help="skip the sustained-clock timing of each path (4 s warm, 2 s timed, clock sampled)")
    ap.add_argument("--sustained-seconds", type=float, default=4.0, help="warm seconds per path in the sustained timing")
    ap.add_argument("--fp8-flags", type=int, default=0,
                    help="ATTN_FLAG_* bits for the FP8 launches (1 exact P, 2 no block scaling): ablations only")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only (there is no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_bf16_causal_amd as fbc
    from fp8_bf16_causal_amd import synth

    fbc._lib.load()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.energy:
        print(json.dumps({"energy_study": energy_study(args.energy_seconds)}), flush=True)
        return
    if args.quant_only:
        print(json.dumps({"quantize_prologue": time_quant_prologue(args.steps, min(args.warmup, 20))}), flush=True)
        return
    names = args.paths.split(",")
    inputs = {n: synth.make_config(n, device="cuda") for n in names}
    outs = {n: torch.empty((i.shape["B"], i.shape["S"], i.shape["Hq"], i.shape["Dv"]), dtype=torch.bfloat16,
                           device="cuda") for n, i in inputs.items()}

    def launch(n):
        i = inputs[n]
        dq, dk, dv = i.descale
        ab = dict(exact_p=bool(args.fp8_flags & 1), block_scale=not (args.fp8_flags & 2)) if i.dtype == "fp8" else {}
        fbc.flash_attn_func(i.q, i.k, i.v, i.scale, causal=True,
                            descale_q=dq, descale_k=dk, descale_v=dv, out=outs[n], **ab)

    # everything the timed region needs is set up before the settle and warmup
    # launches, so that the GPU does not idle (and boost its clock) in front
    # of the timed steps
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
          for n in names}
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clock = ClockSampler()

    # settle the clock: the kernels drive the board to its power limit within
    # seconds, and the clock drops from its idle boost to the sustained one
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for n in names:
            launch(n)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        for n in names:
            launch(n)
    torch.cuda.synchronize()

    # timed region: K steps, each kernel bracketed by events on the launch stream
    with clock:
        start.record()
        for s in range(args.steps):
            for n in names:
                ev[n][s][0].record()
                launch(n)
                ev[n][s][1].record()
        stop.record()
        torch.cuda.synchronize()
    sclk_run = clock.mean_mhz()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    paths, flop_step, ideal_s = {}, 0.0, 0.0
    for n in names:
        p = inputs[n].shape
        kind = inputs[n].dtype
        ms = [a.elapsed_time(b) for a, b in ev[n]]
        avg = sum(ms) / len(ms)
        f = causal_flops(p)
        flop_step += f
        ideal_s += f / (PEAK[kind] * 1e12)
        tf = f / (avg * 1e-3) / 1e12
        med = sorted(ms)[len(ms) // 2]
        paths[n] = {"kernel_ms_avg": round(avg, 4), "kernel_ms_median": round(med, 4), "kernel_ms_min": round(min(ms), 4),
                    "tflops": round(tf, 1), "tflops_literal_2x": round(2 * tf, 1),
                    "peak_tflops": PEAK[kind], "frac_of_peak": round(tf / PEAK[kind], 4)}
        q = max(1, len(ms) // 4)
        paths[n]["kernel_ms_first_quarter"] = round(sum(ms[:q]) / q, 4)
        paths[n]["kernel_ms_last_quarter"] = round(sum(ms[-q:]) / q, 4)
        if sclk_run:  # the clock sampled during these timed steps (both paths alternate)
            paths[n]["frac_of_peak_at_run_clock"] = round(tf / (PEAK[kind] * sclk_run / 2400.0), 4)
        ck = profiled_line(CLOCK_FILE, n, kind)
        if ck:  # figures of the same kernel in the committed rocprofv3 counter run (another run)
            paths[n]["profile_sclk_mhz"] = float(ck["sclk_mhz"])
            paths[n]["profile_mfma_busy"] = float(ck["mfma_busy"])
        if n in PAGES_TFLOPS:
            paths[n]["pages_tflops"] = PAGES_TFLOPS[n]
            paths[n]["ratio_to_pages"] = round(tf / PAGES_TFLOPS[n], 3)

    value = flop_step / (ms_per_step * 1e-3) / 1e12
    dom = max(names, key=lambda n: paths[n]["kernel_ms_avg"])
    dom_kind = inputs[dom].dtype
    roofline = {"bound": "mfma", "achieved": paths[dom]["tflops"], "peak": PEAK[dom_kind], "unit": "TFLOP/s",
                "frac": paths[dom]["frac_of_peak"], "traffic": measured_traffic(dom, dom_kind), "kernel": dom}
    for n in names:
        paths[n]["hbm_traffic_bytes"] = measured_traffic(n, inputs[n].dtype)
    if args.fp8_flags:
        # an ablation of the FP8 softmax: not the method's number, not comparable with the pages' figure
        for n in names:
            paths[n].pop("pages_tflops", None)
            paths[n].pop("ratio_to_pages", None)
    cfg = {"workload": "+".join(names), "B": 1, "H": 32, "S": 32768, "Dqk": 128, "Dv": 128,
           "input": "Gaussian N(0,1), seeds 3 (fp8) and 4 (bf16), per-tensor e4m3 scales",
           "flop_count": "causal B*H*S^2*(Dqk+Dv)"}
    line = {"metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "+".join(sorted({inputs[n].dtype for n in names})), "data": "synthetic",
            "config": cfg, "frac_of_peak": round(ideal_s / (ms_per_step * 1e-3), 4),
            "clock_settle_s": args.settle_seconds, "sclk_mhz_run": sclk_run, "sclk_source": clock.source,
            "sclk_samples_run": len(clock.samples),
            "paths": paths, "roofline": roofline}
    if args.fp8_flags:
        line["fp8_flags"] = args.fp8_flags
    if not args.no_sustained:
        line["sustained"] = sustained(inputs, launch, args.sustained_seconds, 2.0)
    if not args.no_others and not args.fp8_flags:
        line["other_configs"] = time_other_configs()
    if not args.no_shares and not args.fp8_flags:
        line["tp8_shares"] = time_tp_shares({**paths, **line.get("other_configs", {})})
    if not args.no_quant and not args.fp8_flags:
        line["quantize_prologue"] = time_quant_prologue(50, 10)
        if "bf16_mha_s32k" in inputs:
            line["fp8_from_bf16"] = time_fp8_from_bf16(inputs["bf16_mha_s32k"])
    if not args.no_cpu_baseline:
        threads = min(int(os.environ.get("OMP_NUM_THREADS", "16")), os.cpu_count() or 1, 16)
        line["cpu_baseline"] = cpu_baseline(inputs, args.cpu_rows, threads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
