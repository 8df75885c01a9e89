#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

One step is one pass over the whole hot path on seeded synthetic bf16 inputs already resident
in HBM:
  * prefill (attn_fwd, causal, d=128): B=1, H=8, N=16384 (the headline workload: causal
    prefill at N >= 4096), then B=4, H=16, N=4096 (the longest sequence of the N 512-4096 sweep)
    and B=2, H=16, N=2048;
  * decode:  attn_decode_splitkv (split kernel + combine kernel) on B=8, Hq=32, Hkv=8, Nk=8192,
             d=128, n_splits=16, once with Nq=1 and once with Nq=4.  Four distinct K/V buffer sets
             (4 x 268 MB) are rotated so the 256 MB MALL cannot serve repeated reads.

Before the W warm-up steps the parts run round-robin for --settle-s seconds (default 1): an idle
MI355X takes a large fraction of a second to raise its clock, far longer than a few warm-up
steps of this hot path.  The timed region then runs exactly K steps, grouped by part: part j's K launches run back to back in
a few brackets (4 when K >= 4), each bracket between one pair of HIP events recorded on the
stream the library launches on (torch's current stream), and the device is synchronised between
parts.  Per-launch event pairs were avoided because each adds about 5 us of marker overhead.  The
calls are marshalled once before the timed region so that host-side overhead cannot leave the GPU
idle inside a bracket.  The printed JSON line carries:
  value         TFLOPS of the headline prefill (4*B*H*N^2*d / 2 for causal, over the mean time
                per launch of all K launches);
  prefill_extra the same for the other two prefill workloads;
  decode        HBM GB/s of each split + combine pair over the algorithmic bytes (K and V once,
                Q, O, LSE), for Nq=1 and Nq=4;
  roofline      the headline prefill kernel against the bf16 dense MFMA peak (each extra
                workload and decode pair carries its own: MFMA, or 8 TB/s HBM);
  min_ms, median_ms  the fastest and the median bracket of each part (mean per launch);
  device       the device name, compute units and ROCm version;
  clock         the shader clock under each part's load: a spin kernel of known cycle count
                timed beside an untimed repetition of the part (null when it did not overlap);
  cpu_baseline  the CPU fp64 oracle timed on a bounded sample of each workload.

Options: --sweep prints one extra line per prefill/decode workload; --extras prints one line per
variant with per-batch key lengths or an additive bias (see ``extras``); --bwd prints one line per
backward workload (see ``backward``); --only runs a single workload for profiler runs (a name
ending in ":bwd" runs its backward); --copy-bytes runs a plain device copy for counter
calibration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("causal bf16 attn fwd TFLOPS (% MFMA peak); decode split-KV HBM GB/s (% peak)")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
HEADLINE = "long_causal_b1h8n16384"
PREFILL_EXTRA = ("sweep_n4096_b4_causal", "prefill_causal_b2h16n2048")
DECODE = ("decode_gqa_nq1", "decode_gqa_nq4")
BRACKETS = 4
KV_SETS = 4
PROFILES = os.path.join(ROOT, "profiles")
MFMA_BUSY_MAX = 0.9  # largest matrix-core busy fraction a clock reading may imply
CSRC = os.path.join(ROOT, "scaled_dot_product_fa2_amd", "csrc")


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "prefill": ("fwd_bf16.hip", "fa_device.h"),
    "decode": ("decode.hip", "fa_device.h"),
}


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when the summary is
    missing or was taken on a different kernel source than the one built now."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get("kernels", {}).get(f"{kind}:{workload}")
    if not entry or entry.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kind]):
        return None
    return entry.get("hbm_bytes_per_launch")


def algorithmic_bytes(w, n_kv_reads=1):
    kv = 2 * w.B * w.Hkv * w.Nk * w.d * 2 * n_kv_reads
    qo = 2 * w.B * w.Hq * w.Nq * w.d * 2
    return kv + qo + w.B * w.Hq * w.Nq * 4


def ensure_built():
    from scaled_dot_product_fa2_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        from scaled_dot_product_fa2_amd import build

        build.build()
    return binding.load()


class Prefill:
    def __init__(self, w, torch, fa, I, seqlens_k=None, bias=None):
        self.w, self.torch, self.fa = w, torch, fa
        x = w.draw()
        self.q, self.k, self.v = (I.to_device(a, "bf16") for a in (x.q, x.k, x.v))
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
        self.call = fa.prepare_fwd(self.q, self.k, self.v, self.out, self.lse, causal=w.causal,
                                   seqlens_k=seqlens_k, bias=bias)

    def __call__(self, i):
        self.call()

    def flops(self):
        return self.w.flops()


class Decode:
    def __init__(self, w, torch, fa, I, kv_sets, seqlens_k=None, bias=None):
        self.w, self.torch, self.fa = w, torch, fa
        self.kv = []
        for s in range(len(kv_sets)):
            self.kv.append(kv_sets[s])
        x = I.draw_qkv(w.seed, w.B, w.Hq, w.Hkv, w.Nq, 1, w.d)  # only Q is drawn here
        self.q = I.to_device(x.q, "bf16")
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
        need = fa.attn_decode_workspace_bytes(w.B, w.Hq, w.Nq, w.d, w.n_splits)
        self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        self.calls = [fa.prepare_decode(self.q, k, v, w.n_splits, self.out, self.lse, self.ws,
                                        causal=w.causal, seqlens_k=seqlens_k, bias=bias)
                      for k, v in self.kv]

    def __call__(self, i):
        self.calls[i % len(self.calls)]()


def decode_kv_sets(torch, I, w, n):
    sets = []
    for s in range(n):
        x = I.draw_qkv(w.seed + 100 * s, w.B, w.Hq, w.Hkv, 1, w.Nk, w.d)
        sets.append((I.to_device(x.k, "bf16"), I.to_device(x.v, "bf16")))
    return sets


def clock_during(torch, part, steps, part_ms):
    """The shader clock while `part` runs, from a separate, untimed repetition of its `steps`
    launches: once the first launch is done, a spin kernel that waits a known number of
    shader-clock cycles runs beside the others on a second stream (one wave, next to the part's
    waves), and HIP events on that stream time it.
    The estimate counts only when the spin ended before the part did (so it ran under the load
    throughout); otherwise it is reported as null.  Returns (MHz or None, spin ms, part ms)."""
    cycles = int(max(part_ms * (steps - 1), 0.2) * 1e-3 * 0.5 * 1.0e9)  # half the rest at 1 GHz
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    first = torch.cuda.Event()
    m0.record()
    for i in range(steps):
        part(i)
        if i == 0:
            first.record()
            # the spin starts once the part's first launch is done, i.e. under the load of the
            # following launches
            side.wait_event(first)
            with torch.cuda.stream(side):
                e0.record(side)
                torch.cuda._sleep(cycles)
                e1.record(side)
    m1.record()
    torch.cuda.synchronize()
    spin_ms, run_ms = e0.elapsed_time(e1), m0.elapsed_time(m1)
    inside = m0.elapsed_time(e1) <= run_ms
    mhz = round(cycles / (spin_ms * 1e3), 1) if inside and spin_ms > 0 else None
    return mhz, round(spin_ms, 4), round(run_ms, 4)


def settle(torch, parts, seconds):
    """Run the parts round-robin for `seconds` of wall time before the warm-up steps: an idle
    GPU takes a large fraction of a second to raise its clock (a 5-step warm-up of this hot path
    is ~5 ms), so without this the first parts would be timed while the clock still ramps."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for p in parts:
            p(n)
        n += 1
        torch.cuda.synchronize()
    return n


def _bracket_sizes(steps, brackets):
    n = max(1, min(brackets, steps))
    return [steps // n + (1 if r < steps % n else 0) for r in range(n)]


def time_parts(torch, parts, names, steps, warmup, brackets=BRACKETS, settle_s=0.0, clock=False):
    """Run the parts for `settle_s` seconds (see ``settle``), then `warmup` untimed steps, then
    exactly `steps` steps grouped by part: part j runs its `steps` launches back to back, split
    into up to `brackets` brackets that each sit between one pair of events on the current
    stream; the device is synchronised between parts.  (An event pair around every single
    launch adds about 5 us of marker overhead on this stack, which would inflate each kernel's
    time.)  With `clock`, each part is then repeated once, untimed, beside a spin kernel that
    measures the shader clock under that load (``clock_during``).  Returns (wall ms per step,
    {name: stats}) with stats holding the mean per launch over all `steps` launches, the min /
    median of the bracket means and the clock."""
    settle_steps = settle(torch, parts, settle_s) if settle_s > 0 else 0
    for i in range(warmup):
        for p in parts:
            p(i)
    torch.cuda.synchronize()
    sizes = _bracket_sizes(steps, brackets)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in sizes] for _ in parts]
    torch.cuda.synchronize()
    t_all = time.perf_counter()
    for j, p in enumerate(parts):
        i = 0
        for r, n in enumerate(sizes):
            evs[j][r][0].record()
            for _ in range(n):
                p(i)
                i += 1
            evs[j][r][1].record()
        torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_all) * 1e3 / steps
    stats = {}
    for j, name in enumerate(names):
        tot = [evs[j][r][0].elapsed_time(evs[j][r][1]) for r in range(len(sizes))]
        per = [t / n for t, n in zip(tot, sizes)]
        stats[name] = {"mean_ms": sum(tot) / steps, "min_ms": min(per),
                       "median_ms": statistics.median(per), "brackets": len(sizes),
                       "settle_steps": settle_steps}
    if clock:
        for j, name in enumerate(names):
            mhz, spin_ms, run_ms = clock_during(torch, parts[j], steps, stats[name]["mean_ms"])
            stats[name]["clock"] = {"mhz": mhz, "spin_ms": spin_ms, "part_ms": run_ms}
    return wall_ms, stats


def time_steps(torch, parts, steps, warmup):
    """time_parts without names: (wall ms per step, [mean ms per launch of each part])."""
    names = [f"part{j}" for j in range(len(parts))]
    wall, st = time_parts(torch, parts, names, steps, warmup)
    return wall, [st[n]["mean_ms"] for n in names]


def oracle_cores():
    """Threads for the CPU baseline: every core this process may run on, at most 16 (the host
    CPU share a one-GPU job is granted on the GPU machines, whatever the node's core count)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(w, seconds: float, cores: int):
    """The CPU fp64 oracle, unmodified, on a bounded sample of the workload: tasks of (batch,
    query head, up to 1024 query rows), each the oracle's row function on that slice, run on
    `cores` threads with single-threaded BLAS, for about `seconds` of wall time.  Returns the
    rate scaled to the whole workload (TFLOPS in the FLOP convention for prefill, GB/s of
    algorithmic bytes for decode) and a description of the sample."""
    import concurrent.futures

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    x = w.draw()
    q, k, v = x.as_f64()
    scale = float(np.float32(w.scale))
    G = w.Hq // w.Hkv
    chunk = min(1024, w.Nq)
    tasks = [(b, h, r0) for r0 in range(0, w.Nq, chunk) for b in range(w.B) for h in range(w.Hq)]

    def one(t):
        b, h, r0 = t
        rows = np.arange(r0, min(w.Nq, r0 + chunk))
        A.attention_rows_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                              v[b:b + 1, h // G:h // G + 1], scale, w.causal, rows)
        return len(rows)

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        one(tasks[0])
        per_task = time.perf_counter() - t0
        want = max(cores, int(seconds * cores / max(per_task, 1e-6)))
        # spread the sample over the tensor: every stride-th task
        stride = max(1, len(tasks) // want)
        sample = tasks[::stride][:want]
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as ex:
            rows = sum(ex.map(one, sample))
        wall = time.perf_counter() - t0
    share = rows / (w.B * w.Hq * w.Nq)
    if w.n_splits:
        rate, unit = algorithmic_bytes(w) * share / wall / 1e9, "GB/s"
    else:
        rate, unit = w.flops() * share / wall / 1e12, "TFLOPS"
    what = (f"{len(sample)} of {len(tasks)} (batch, head, {chunk}-row) tasks of {w.name} "
            f"({100 * share:.2f}% of its rows), numpy fp64, {wall:.1f} s wall on {cores} threads")
    return {"value": round(rate, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": what}


class Backward:
    """attn_bwd on a workload's inputs, after one forward call that provides out and LSE."""

    def __init__(self, w, torch, fa, I, seqlens_k=None, bias=None):
        x = w.draw()
        self.q, self.k, self.v = (I.to_device(a, "bf16") for a in (x.q, x.k, x.v))
        self.dout = I.to_device(I.draw_grad(w.seed + 1, (w.B, w.Hq, w.Nq, w.d)), "bf16")
        self.out, self.lse = fa.attn_fwd_ex(self.q, self.k, self.v, causal=w.causal,
                                            seqlens_k=seqlens_k, bias=bias)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
        ws = torch.empty(max(fa.attn_bwd_workspace_bytes(w.B, w.Hq, w.Nq), 16), dtype=torch.uint8,
                         device="cuda")
        self.ws = ws
        self.call = fa.prepare_bwd(self.q, self.k, self.v, self.out, self.lse, self.dout, self.dq,
                                   self.dk, self.dv, ws, causal=w.causal, seqlens_k=seqlens_k,
                                   bias=bias)

    def __call__(self, i):
        self.call()


def bwd_flops(w):
    """Backward FLOP convention: the five products of the gradient (dV, dP, dQ, dK and the
    recomputed S) at 2*Nq*Nk*d each, i.e. 2.5x the forward's, halved when causal; the kernels
    recompute S and dP once more (seven products executed)."""
    return 2.5 * w.flops()


def backward(torch, fab, I, W, steps, warmup, names=("prefill_causal_b2h16n2048",
                                                      "sweep_n4096_b4_causal",
                                                      "long_causal_b1h8n16384")):
    rows = []
    for name in names:
        w = W[name]
        part = Backward(w, torch, fab, I)
        _, (ms,) = time_steps(torch, [part], steps, warmup)
        tf = bwd_flops(w) / (ms * 1e-3) / 1e12
        line = {"backward": name, "mean_ms": round(ms, 5), "TFLOPS": round(tf, 1),
                "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}
        rows.append(line)
        print(json.dumps(line), flush=True)
        del part
        torch.cuda.empty_cache()
    # the backward of the forward extras on the B2 H16 N2048 causal workload: an ALiBi bias
    # [1, H, N, N] (FLOPs as without it), and key lengths (FLOPs over the visible pairs)
    w = W["prefill_causal_b2h16n2048"]
    bias = I.to_device(I.draw_bias(1001, 1, w.Hq, w.Nq, w.Nk, "alibi"), "bf16")
    L = I.draw_seqlens(1010, w.B, w.Nk, edges=False)
    lens = torch.as_tensor(L, device="cuda")
    vis_flops = 2.5 * sum(4.0 * w.Hq * w.d * visible_pairs(w.Nq, int(l), w.causal) for l in L)
    for tag, kw, flops in (("bias_1x16_alibi", {"bias": bias}, bwd_flops(w)),
                           ("varlen_" + "_".join(str(int(x)) for x in L), {"seqlens_k": lens},
                            vis_flops)):
        part = Backward(w, torch, fab, I, **kw)
        _, (ms,) = time_steps(torch, [part], steps, warmup)
        tf = flops / (ms * 1e-3) / 1e12
        line = {"backward": w.name, "extra": tag, "mean_ms": round(ms, 5), "TFLOPS": round(tf, 1),
                "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}
        rows.append(line)
        print(json.dumps(line), flush=True)
        del part
    return rows


def visible_pairs(Nq, L, causal):
    """(query, key) pairs a row block attends to with L keys, causal mask aligned to the end."""
    if not causal:
        return Nq * L
    return sum(max(0, min(L, i + L - Nq + 1)) for i in range(Nq))


def extras(torch, fab, I, W, steps, warmup, kv):
    """One line per variant with the optional inputs, each timed like the main parts:
      * prefill with a bias shared by the batch ([1, H, N, N], an ALiBi-style distance penalty)
        and with a bias per (batch, head) ([B, H, N, N], which must stream from HBM);
      * prefill with a length mix (per-batch key counts uniform in [1, N]); its TFLOPS count
        only the visible (query, key) pairs of each element;
      * decode (Nq=1 and Nq=4) with a length mix over the 8192-key capacity (GB/s over the K/V
        rows that exist) and with a per-head bias [1, Hq, Nq, Nk] (its bytes counted)."""
    w = W["prefill_causal_b2h16n2048"]
    rows = []

    def prefill_line(name, part, flops, extra_bytes):
        _, (ms,) = time_steps(torch, [part], steps, warmup)
        tf = flops / (ms * 1e-3) / 1e12
        line = {"extra": name, "workload": w.name, "mean_ms": round(ms, 5), "TFLOPS": round(tf, 1),
                "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}
        if extra_bytes:
            line["bias_bytes"] = extra_bytes
            line["bias_GBps"] = round(extra_bytes / (ms * 1e-3) / 1e9, 1)
        rows.append(line)
        print(json.dumps(line), flush=True)

    for bb, kind in ((1, "alibi"), (w.B, "normal")):
        bits = I.draw_bias(1000 + bb, bb, w.Hq, w.Nq, w.Nk, kind)
        bias = I.to_device(bits, "bf16")
        prefill_line(f"bias_{bb}x{w.Hq}_{kind}", Prefill(w, torch, fab, I, bias=bias), w.flops(),
                     bits.size * 2)
        del bias
    L = I.draw_seqlens(1010, w.B, w.Nk, edges=False)
    flops = sum(4.0 * w.Hq * w.d * visible_pairs(w.Nq, int(l), w.causal) for l in L)
    lens = torch.as_tensor(L, device="cuda")
    prefill_line(f"varlen_{'_'.join(str(int(x)) for x in L)}",
                 Prefill(w, torch, fab, I, seqlens_k=lens), flops, 0)

    for name in DECODE:
        wd = W[name]
        L = I.draw_seqlens(1020, wd.B, wd.Nk, edges=False)
        lens = torch.as_tensor(L, device="cuda")
        bits = I.draw_bias(1030, 1, wd.Hq, wd.Nq, wd.Nk, "alibi")
        bias = I.to_device(bits, "bf16")
        qo = 2 * wd.B * wd.Hq * wd.Nq * wd.d * 2 + wd.B * wd.Hq * wd.Nq * 4
        for tag, kw, nbytes in (
                ("varlen", {"seqlens_k": lens}, 2 * int(L.sum()) * wd.Hkv * wd.d * 2 + qo),
                ("bias", {"bias": bias}, algorithmic_bytes(wd) + bits.size * 2)):
            part = Decode(wd, torch, fab, I, kv, **kw)
            _, (ms,) = time_steps(torch, [part], steps, warmup)
            gbps = nbytes / (ms * 1e-3) / 1e9
            line = {"extra": tag, "workload": name, "mean_ms": round(ms, 5),
                    "algorithmic_bytes": nbytes, "GBps": round(gbps, 1),
                    "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}
            if tag == "varlen":
                line["seqlens_k"] = [int(x) for x in L]
            rows.append(line)
            print(json.dumps(line), flush=True)
    return rows


def roofline_mfma(flops, ms, traffic):
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic}


def roofline_hbm(nbytes, ms, traffic):
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic}


def checked_clock(clk, tflops):
    """A spin wave that shares a SIMD with busy, raised-priority waves can be issued late and so
    overshoot its cycle count, which reads as too low a clock.  The prefill kernel keeps its
    matrix cores busy 0.58-0.68 of the cycles (SQ counters), so a reading under which the measured
    rate would need them busy more than MFMA_BUSY_MAX of the cycles is withdrawn."""
    if clk.get("mhz") is not None and tflops is not None:
        floor = tflops / (PEAK_BF16_TFLOPS * MFMA_BUSY_MAX) * 2400.0
        if clk["mhz"] < floor:
            return {**clk, "mhz": None, "mhz_read": clk["mhz"],
                    "note": f"spin starved: the measured rate needs at least {floor:.0f} MHz"}
    return clk


def device_record(torch):
    p = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count, "rocm": rocm,
            "hip_runtime": torch.version.hip}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sweep", action="store_true", help="also print one line per workload")
    ap.add_argument("--extras", action="store_true",
                    help="also print one line per key-length / bias variant")
    ap.add_argument("--bwd", action="store_true", help="also print one line per backward workload")
    ap.add_argument("--only", default=None, help="run only this workload (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed steps before the warm-up, so the clock has ramped")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="CPU oracle wall seconds per reported workload")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="run a plain device-to-device copy of this many bytes and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU sharding "
                                   "is design only", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from scaled_dot_product_fa2_amd import inputs as I

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no HIP device visible"}))
        sys.exit(1)

    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": args.steps}))
        return

    fa = ensure_built()
    from scaled_dot_product_fa2_amd import binding as fab

    W = I.WORKLOADS
    if args.only:
        name, _, kind = args.only.partition(":")
        w = W[name]
        if kind == "bwd":
            part = Backward(w, torch, fab, I)
            wall, (ms,) = time_steps(torch, [part], args.steps, args.warmup)
            print(json.dumps({"workload": args.only, "mean_ms": round(ms, 5), "steps": args.steps}))
            return
        if w.n_splits:
            part = Decode(w, torch, fab, I, decode_kv_sets(torch, I, w, KV_SETS))
        else:
            part = Prefill(w, torch, fab, I)
        wall, (ms,) = time_steps(torch, [part], args.steps, args.warmup)
        print(json.dumps({"workload": args.only, "mean_ms": round(ms, 5), "steps": args.steps}))
        return

    prefill_names = (HEADLINE, *PREFILL_EXTRA)
    prefills = [Prefill(W[n], torch, fab, I) for n in prefill_names]
    kv = decode_kv_sets(torch, I, W[DECODE[0]], KV_SETS)
    decodes = [Decode(W[n], torch, fab, I, kv) for n in DECODE]
    names = (*prefill_names, *DECODE)
    torch.cuda.synchronize()
    wall_ms, st = time_parts(torch, [*prefills, *decodes], names, args.steps, args.warmup,
                             settle_s=args.settle_s, clock=True)

    def r5(x):
        return round(x, 5)

    def prefill_obj(name):
        w, t = W[name], st[name]
        tf = w.flops() / (t["mean_ms"] * 1e-3) / 1e12
        return {"value": round(tf, 2), "unit": "TFLOPS", "mean_ms": r5(t["mean_ms"]),
                "min_ms": r5(t["min_ms"]), "median_ms": r5(t["median_ms"]),
                "shape": {"B": w.B, "H": w.Hq, "N": w.Nq, "d": w.d, "causal": w.causal},
                "roofline": roofline_mfma(w.flops(), t["mean_ms"],
                                          measured_traffic("prefill", name)),
                "clock": checked_clock(t["clock"], tf)}

    head = prefill_obj(HEADLINE)
    decode_obj = {}
    for name in DECODE:
        wd, t = W[name], st[name]
        nbytes = algorithmic_bytes(wd)
        decode_obj[name] = {
            "value": round(nbytes / (t["mean_ms"] * 1e-3) / 1e9, 1), "unit": "GB/s",
            "mean_ms": r5(t["mean_ms"]), "min_ms": r5(t["min_ms"]),
            "median_ms": r5(t["median_ms"]), "algorithmic_bytes": nbytes,
            "roofline": roofline_hbm(nbytes, t["mean_ms"], measured_traffic("decode", name)),
            "clock": t["clock"],
        }
    w = W[HEADLINE]
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r5(wall_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE,
                   "prefill": head["shape"],
                   "step_also_runs": [*PREFILL_EXTRA, *DECODE],
                   "decode": {"B": 8, "Hq": 32, "Hkv": 8, "Nq": [1, 4], "Nk": 8192, "d": 128,
                              "n_splits": 16, "kv_buffer_sets": KV_SETS},
                   "timing": f"{args.steps} launches per part in "
                             f"{len(_bracket_sizes(args.steps, BRACKETS))} event brackets, after "
                             f"{args.settle_s:g} s of settling and {args.warmup} warm-up steps",
                   "settle_steps": st[HEADLINE]["settle_steps"]},
        "prefill_mean_ms": head["mean_ms"],
        "prefill_min_ms": head["min_ms"],
        "prefill_median_ms": head["median_ms"],
        "roofline": head["roofline"],
        "clock": head["clock"],
        "prefill_extra": {n: prefill_obj(n) for n in PREFILL_EXTRA},
        "decode": decode_obj,
        "device": device_record(torch),
    }
    if not args.no_cpu_baseline:
        cores = oracle_cores()
        per = {n: cpu_baseline(W[n], args.cpu_seconds, cores) for n in names}
        line["cpu_baseline"] = {**per[HEADLINE],
                                "per_workload": {n: per[n] for n in names if n != HEADLINE}}
    print(json.dumps(line), flush=True)

    if args.extras:
        extras(torch, fab, I, W, args.steps, args.warmup, kv)

    if args.bwd:
        backward(torch, fab, I, W, args.steps, args.warmup)

    if args.sweep:
        for name, wk in W.items():
            if wk.dtype != "bf16" or name in names:
                continue
            if wk.n_splits:
                continue
            part = Prefill(wk, torch, fab, I)
            _, (ms,) = time_steps(torch, [part], args.steps, args.warmup)
            tf = wk.flops() / (ms * 1e-3) / 1e12
            print(json.dumps({"workload": name, "mean_ms": round(ms, 5),
                              "TFLOPS": round(tf, 1),
                              "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
            del part
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
