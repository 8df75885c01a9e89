"""Helpers for the GPU parity tests: upload seeded inputs, run the C ABI through the binding,
and compare against the CPU fp64 oracle element by element."""
from __future__ import annotations

import concurrent.futures
import os
import sys

import numpy as np

from scaled_dot_product_fa2_amd import inputs as I

# Tolerances (fixed by the target: bf16 inputs max-abs 2e-2 / mean-abs 2e-3; fp32 inputs 1e-4;
# logsumexp 1e-3 on every configuration).
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4
F32_MEAN_ABS = 1e-4
LSE_MAX_ABS = 1e-3


def say(msg: str):
    """Name the case before each GPU step (flushed, so a fault still shows which case ran)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_f64(t) -> np.ndarray:
    import torch

    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return I.bf16_bits_to_f32(bits).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def upload(x: I.QKV, device="cuda"):
    return (I.to_device(x.q, x.dtype, device), I.to_device(x.k, x.dtype, device),
            I.to_device(x.v, x.dtype, device))


def compare(out, lse, O_ref, lse_ref, max_abs, mean_abs, lse_tol=LSE_MAX_ABS, what=""):
    """Element-wise comparison; returns (max_abs_err, mean_abs_err, lse_max_err)."""
    out = np.asarray(out, np.float64)
    O_ref = np.asarray(O_ref, np.float64)
    assert out.shape == O_ref.shape, f"{what}: shape {out.shape} vs {O_ref.shape}"
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - O_ref)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    lerr = 0.0
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        ref_inf = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse), ref_inf), f"{what}: -inf pattern of lse differs"
        assert np.all(np.isfinite(lse[~ref_inf])), f"{what}: non-finite lse"
        if (~ref_inf).any():
            lerr = float(np.abs(lse[~ref_inf] - lse_ref[~ref_inf]).max())
    say(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} lse_max={lerr:.3e}")
    assert mx <= max_abs, f"{what}: max abs error {mx} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean abs error {mean} > {mean_abs}"
    assert lerr <= lse_tol, f"{what}: lse error {lerr} > {lse_tol}"
    return mx, mean, lerr


def sample_rows(Nq: int, n_random: int = 16, seed: int = 0) -> np.ndarray:
    """Rows at both ends, around Q-tile boundaries and at seeded random positions."""
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, Nq // 2, Nq - 129, Nq - 128, Nq - 65,
             Nq - 64, Nq - 2, Nq - 1]
    rnd = np.random.default_rng(seed).integers(0, Nq, size=n_random)
    rows = np.array(sorted({int(r) for r in list(fixed) + list(rnd) if 0 <= r < Nq}))
    return rows


def oracle_threads() -> int:
    """Worker threads for the oracle: the host cores this process may run on, at most 16 (the
    CPU share a one-GPU machine grants a job)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_full(q, k, v, scale: float, causal: bool, row_chunk: int = 2048):
    """The oracle's O and LSE over every element of a (large) problem, computed as independent
    tasks of (batch, query head, row chunk) on a thread pool with single-threaded BLAS per task.

    Each task is ``attention_rows_fp64`` on that slice's K/V head and those query positions (the
    oracle's own row function, whose rows are exact rows of the full result: the causal mask uses
    each row's true position), so nothing here changes what the oracle computes."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A

    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    tasks = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, Nq, row_chunk)]

    def one(task):
        b, h, r0 = task
        rows = np.arange(r0, min(Nq, r0 + row_chunk))
        o, l = A.attention_rows_fp64(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                                     v[b:b + 1, h // G:h // G + 1], scale, causal, rows)
        out[b, h, rows] = o[0, 0]
        lse[b, h, rows] = l[0, 0]

    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=oracle_threads()) as ex:
            list(ex.map(one, tasks))
    return out, lse
