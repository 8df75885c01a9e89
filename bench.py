#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

One step is one pass over the whole hot path on seeded synthetic bf16 inputs already resident
in HBM:
  * prefill: attn_fwd on B=2, H=16, N=2048, d=128, causal (the headline workload);
  * decode:  attn_decode_splitkv (split kernel + combine kernel) on B=8, Hq=32, Hkv=8, Nk=8192,
             d=128, n_splits=16, once with Nq=1 and once with Nq=4.  Four distinct K/V buffer sets
             (4 x 268 MB) are rotated so the 256 MB MALL cannot serve repeated reads.

The timed region runs exactly K steps, grouped by part: the K prefill launches back to back, then
the K decode (Nq=1) calls, then the K decode (Nq=4) calls, each group between one pair of HIP
events recorded on the stream the library launches on (torch's current stream).  Per-launch event
pairs were avoided because each adds about 5 us of marker overhead.  The calls are marshalled once
before the timed region so that host-side overhead cannot leave the GPU idle inside a bracket.  The printed JSON line carries:
  value      prefill TFLOPS (4*B*H*N^2*d / 2 for causal, over the prefill kernel's mean time);
  decode     HBM GB/s of the split + combine pair over the algorithmic bytes (K and V once, Q, O,
             LSE), for Nq=1 and Nq=4;
  roofline   the prefill kernel against the bf16 dense MFMA peak (and decode against 8 TB/s);
  cpu_baseline  the CPU fp64 oracle timed on a bounded sample of the prefill workload.

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
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("causal bf16 attn fwd TFLOPS (% MFMA peak); decode split-KV HBM GB/s (% peak)")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
HEADLINE = "prefill_causal_b2h16n2048"
DECODE = ("decode_gqa_nq1", "decode_gqa_nq4")
KV_SETS = 4
PROFILES = os.path.join(ROOT, "profiles")
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


def time_steps(torch, parts, steps, warmup):
    """Run warmup untimed steps, then exactly `steps` steps.  The timed region is grouped by part:
    part j runs its `steps` launches back to back between one pair of events on the current
    stream, then part j+1 follows.  (An event pair around every single launch adds about 5 us of
    marker overhead per bracket on this stack, which would inflate each kernel's time.)
    Returns (wall ms per step, [mean ms per launch of each part])."""
    for i in range(warmup):
        for p in parts:
            p(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in parts]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j, p in enumerate(parts):
        ev[j][0].record()
        for i in range(steps):
            p(i)
        ev[j][1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    means = [ev[j][0].elapsed_time(ev[j][1]) / steps for j in range(len(parts))]
    return wall_ms, means


def cpu_baseline(w, target_s: float):
    """The CPU fp64 oracle, unmodified, over a bounded sample of (batch, head) slices of the
    workload, one slice per worker thread with single-threaded BLAS."""
    import concurrent.futures

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    x = w.draw()
    q, k, v = x.as_f64()
    scale = float(np.float32(w.scale))
    slices = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    cores = max(1, min(16, len(os.sched_getaffinity(0))))

    def one(bh):
        b, h = bh
        hk = h // (w.Hq // w.Hkv)
        A.attention_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1],
                         scale, w.causal)

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        one(slices[0])
        per_slice = time.perf_counter() - t0
        # about target_s seconds of CPU work: a prefix of the slices when one pass is longer,
        # else whole passes over every slice
        want = max(1, round(target_s / max(per_slice, 1e-6)))
        if want >= len(slices):
            passes = max(1, want // len(slices))
            sample = slices * passes
            what = f"{passes} pass(es) over all {len(slices)} (batch, head) slices"
        else:
            sample = slices[:max(cores, want)]
            what = f"{len(sample)} of {len(slices)} (batch, head) slices"
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as ex:
            list(ex.map(one, sample))
        wall = time.perf_counter() - t0
    flops = w.flops() * len(sample) / len(slices)
    return {"value": round(flops / wall / 1e12, 6), "unit": "TFLOPS", "cores": cores,
            "kind": "oracle",
            "sample": f"{what} of {w.name}, all rows of each, numpy fp64, {wall:.1f} s wall on "
                      f"{cores} threads"}


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
    w = W[HEADLINE]
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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

    prefill = Prefill(W[HEADLINE], torch, fab, I)
    kv = decode_kv_sets(torch, I, W[DECODE[0]], KV_SETS)
    decodes = [Decode(W[n], torch, fab, I, kv) for n in DECODE]
    torch.cuda.synchronize()
    wall_ms, means = time_steps(torch, [prefill, *decodes], args.steps, args.warmup)
    pre_ms, dec_ms = means[0], means[1:]

    w = W[HEADLINE]
    tflops = w.flops() / (pre_ms * 1e-3) / 1e12
    decode_obj = {}
    for name, ms in zip(DECODE, dec_ms):
        wd = W[name]
        nbytes = algorithmic_bytes(wd)
        decode_obj[name] = {
            "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "mean_ms": round(ms, 5),
            "algorithmic_bytes": nbytes,
            "roofline": roofline_hbm(nbytes, ms, measured_traffic("decode", name)),
        }
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{HEADLINE} + {DECODE[0]} + {DECODE[1]}",
                   "prefill": {"B": w.B, "H": w.Hq, "N": w.Nq, "d": w.d, "causal": w.causal},
                   "decode": {"B": 8, "Hq": 32, "Hkv": 8, "Nq": [1, 4], "Nk": 8192, "d": 128,
                              "n_splits": 16, "kv_buffer_sets": KV_SETS}},
        "prefill_mean_ms": round(pre_ms, 5),
        "roofline": roofline_mfma(w.flops(), pre_ms, measured_traffic("prefill", HEADLINE)),
        "decode": decode_obj,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)

    if args.extras:
        extras(torch, fab, I, W, args.steps, args.warmup, kv)

    if args.bwd:
        backward(torch, fab, I, W, args.steps, args.warmup)

    if args.sweep:
        for name, wk in W.items():
            if wk.dtype != "bf16" or name == HEADLINE:
                continue
            if wk.n_splits:
                part = decodes[DECODE.index(name)] if name in DECODE else None
                if part is None:
                    continue
                _, (ms,) = time_steps(torch, [part], args.steps, args.warmup)
                nbytes = algorithmic_bytes(wk)
                print(json.dumps({"workload": name, "mean_ms": round(ms, 5),
                                  "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}),
                      flush=True)
            else:
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
