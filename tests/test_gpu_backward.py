"""GPU parity of the backward pass (attn_bwd) against the CPU fp64 oracle's gradients.

The forward runs on the GPU first (its bf16 output and fp32 logsumexp are the backward's
inputs, as in training); the oracle differentiates the definition from the same bf16 q, k, v and
dout.  Every call goes through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, compare, say, to_f64, upload  # noqa: E402
from oracle import attention as A  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu

# Tolerances relative to the largest reference gradient of each tensor.  The kernels round P and
# dS to bf16 for the matrix cores (relative 2^-9 each), take D from the bf16 forward output and
# store bf16 gradients (another 2^-9); with sums over hundreds of terms the elementwise error
# stays a small multiple of 2^-9 of the largest entry.
GRAD_MAX_REL = 2e-2    # max |gpu - ref| / max |ref|
GRAD_MEAN_REL = 2e-3   # mean |gpu - ref| / max |ref|
# A gradient that is exactly zero (one key: the softmax is constant, so dq = dk = 0) is compared
# on an absolute scale instead: P and D carry fp32/bf16 rounding, so the GPU's value is tiny,
# not zero.
GRAD_FLOOR = 2.0 ** -10


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


def _s32(d):
    return float(np.float32(1.0 / np.sqrt(d)))


def _check(name, got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    scale = max(float(np.abs(ref).max(initial=0.0)), GRAD_FLOOR)
    err = np.abs(got - ref)
    mx, mean = float(err.max(initial=0.0)) / scale, (float(err.mean()) / scale if err.size else 0.0)
    say(f"  {name}: max|ref|={scale:.3e} max_rel={mx:.3e} mean_rel={mean:.3e}")
    assert mx <= GRAD_MAX_REL, f"{name}: max error {mx} of max|ref| > {GRAD_MAX_REL}"
    assert mean <= GRAD_MEAN_REL, f"{name}: mean error {mean} of max|ref| > {GRAD_MEAN_REL}"


def _run(B, Hq, Hkv, Nq, Nk, causal, seed, d=128):
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(seed + 1, (B, Hq, Nq, d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    s32 = _s32(d)
    say(f"backward B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} causal={causal} seed={seed}")
    out, lse = fa.attn_fwd(q, k, v, causal=causal, scale=s32)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=causal, scale=s32)
    torch.cuda.synchronize()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    rq, rk, rv = A.attention_backward_fp64(*x.as_f64(), g, s32, causal)
    return (to_f64(dq), to_f64(dk), to_f64(dv)), (rq, rk, rv), (q, k, v, out, lse, dout)


# (B, Hq, Hkv, Nq, Nk, causal): one and several 64/128-row blocks with ragged tails, GQA groups of
# 1, 2 and 4, Nq != Nk both ways (the first rows without any key), a single key, non-causal
CASES = [
    (1, 2, 2, 128, 128, True),
    (2, 4, 2, 200, 200, True),
    (1, 4, 1, 257, 257, False),
    (1, 2, 1, 130, 300, True),
    (1, 2, 2, 300, 130, True),
    (2, 2, 2, 77, 1, True),
    (1, 8, 2, 64, 512, False),
    (2, 8, 8, 384, 384, True),
]
# head dimension 64: the same kinds of shapes
CASES64 = [
    (1, 2, 2, 128, 128, True),
    (2, 4, 2, 200, 333, True),
    (1, 4, 1, 257, 130, False),
    (2, 2, 2, 77, 1, True),
    (1, 8, 4, 300, 300, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_{}".format(
    *c[:5], "causal" if c[5] else "full"))
def test_backward_matches_oracle(case):
    B, Hq, Hkv, Nq, Nk, causal = case
    got, ref, _ = _run(B, Hq, Hkv, Nq, Nk, causal, seed=4000 + Nq + 3 * Nk)
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, a, r)


@pytest.mark.parametrize("case", CASES64, ids=lambda c: "d64_B{}_Hq{}_Hkv{}_Nq{}_Nk{}_{}".format(
    *c[:5], "causal" if c[5] else "full"))
def test_backward_head_dim_64(case):
    B, Hq, Hkv, Nq, Nk, causal = case
    got, ref, _ = _run(B, Hq, Hkv, Nq, Nk, causal, seed=4500 + Nq + 3 * Nk, d=64)
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, a, r)


def test_backward_long_causal():
    # B=1, H=4, N=1024, causal: 16 key blocks of 64 per query block, 8 query blocks per key block
    got, ref, _ = _run(1, 4, 4, 1024, 1024, True, seed=4100)
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, a, r)


def test_backward_bench_shape_sampled_heads():
    # the launch the backward benchmark times (B2 H16 N2048 causal, all heads in one call); the
    # oracle differentiates four whole (batch, head) slices of it
    w = I.WORKLOADS["prefill_causal_b2h16n2048"]
    x = w.draw()
    g_bits = I.draw_grad(w.seed + 4300, (w.B, w.Hq, w.Nq, w.d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    s32 = _s32(w.d)
    say("backward B2 H16 N2048 causal, sampled heads")
    out, lse = fa.attn_fwd(q, k, v, causal=True, scale=s32)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=True, scale=s32)
    torch.cuda.synchronize()
    got = [to_f64(t) for t in (dq, dk, dv)]
    qf, kf, vf = x.as_f64()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    for b, hh in ((0, 0), (0, 15), (1, 7), (1, 12)):
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        ref = A.attention_backward_fp64(qf[sl], kf[sl], vf[sl], g[sl], s32, True)
        for name, a, r in zip(("dq", "dk", "dv"), got, ref):
            _check(f"{name}[{b},{hh}]", a[sl], r)


def test_backward_deterministic_and_fully_written():
    got, _, (q, k, v, out, lse, dout) = _run(2, 4, 2, 200, 333, True, seed=4200)
    s32 = _s32(128)
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    fa.attn_bwd(q, k, v, out, lse, dout, causal=True, scale=s32, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), got):
        assert not bool(torch.isnan(a.float()).any()), f"{name} not fully written"
        assert np.array_equal(to_f64(a), b), f"{name} differs between two identical calls"


@pytest.mark.parametrize("scale", [2.0 ** -32, 2.0 ** -10, 0.5, 2.0])
def test_backward_at_other_scales(scale):
    # the row terms -LSE / scale and the exponent argument (S - LSE / scale) * scale * log2e at
    # scales from the accepted floor (near-uniform softmax) to sharply peaked rows
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 200, 260, 128
    x = I.draw_qkv(4400, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(4401, (B, Hq, Nq, d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    s32 = float(np.float32(scale))
    say(f"backward at scale {s32!r}")
    out, lse = fa.attn_fwd(q, k, v, causal=True, scale=s32)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=True, scale=s32)
    torch.cuda.synchronize()
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), s32, True)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"forward at scale {s32!r}")
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    rq, rk, rv = A.attention_backward_fp64(*x.as_f64(), g, s32, True)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), (rq, rk, rv)):
        _check(name, to_f64(a), r)


def test_backward_workspace_holds_the_documented_row_terms():
    # the workspace contract: fp32 -D [B, Hq, Nq], then -lse / scale [B, Hq, Nq] (-inf for rows
    # whose lse is -inf); Nq > Nk causal gives such rows (the first Nq - Nk rows see no key)
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 2, 300, 130, 128
    _, _, (q, k, v, out, lse, dout) = _run(B, Hq, Hkv, Nq, Nk, True, seed=4300)
    s32 = _s32(d)
    ws = torch.full((fa.attn_bwd_workspace_bytes(B, Hq, Nq),), 0x7f, dtype=torch.uint8,
                    device="cuda")
    fa.attn_bwd(q, k, v, out, lse, dout, causal=True, scale=s32, workspace=ws)
    torch.cuda.synchronize()
    rows = B * Hq * Nq
    terms = ws.view(torch.float32).cpu().numpy().astype(np.float64)
    dn, ln = terms[:rows], terms[rows:2 * rows]
    o, g = to_f64(out).reshape(rows, d), to_f64(dout).reshape(rows, d)
    dref = (o * g).sum(axis=1)
    bound = 1e-6 * np.maximum(np.abs(o * g).sum(axis=1), 1e-30)
    assert np.all(np.abs(dn + dref) <= bound), float(np.abs(dn + dref).max())
    l32 = lse.cpu().numpy().reshape(rows)
    dead = np.isneginf(l32)
    assert dead.sum() == B * Hq * (Nq - Nk)
    assert np.all(np.isneginf(ln[dead]))
    lref = (-l32[~dead].astype(np.float32) / np.float32(s32)).astype(np.float64)
    ulp = np.spacing(np.abs(lref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(ln[~dead] - lref) <= ulp)


def test_backward_without_query_rows_zeroes_dk_dv():
    say("backward Nq=0")
    k = torch.ones((1, 2, 70, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    out, dout = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    fa.attn_bwd(q, k, k.clone(), out, lse, dout, causal=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert bool((dk.float() == 0).all()) and bool((dv.float() == 0).all())


def test_backward_rejects_other_head_dims():
    q = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 2, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.AttentionError, match="head dimension"):
        fa.attn_bwd(q, q, q, q, lse, q)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_without_keys_zeroes_dq(d):
    # Nk = 0: every row has no visible key (forward: out = 0, lse = -inf), so no gradient flows
    say(f"backward Nk=0 d={d}")
    x = I.draw_qkv(4600 + d, 2, 4, 2, 70, 0, d)
    q, k, v = upload(x)
    dout = I.to_device(I.draw_grad(4601 + d, (2, 4, 70, d)), "bf16")
    out, lse = fa.attn_fwd(q, k, v, causal=True)
    dq = torch.full_like(q, float("nan"))
    fa.attn_bwd(q, k, v, out, lse, dout, causal=True, dq=dq)
    torch.cuda.synchronize()
    assert bool((lse == -float("inf")).all())
    assert bool((dq.float() == 0).all())


# per-batch key lengths (attn_bwd_ex): (B, Hq, Hkv, Nq, Nk capacity, d, causal, lengths) with
# lengths 0, 1, ragged, whole 128-key tiles and the capacity; Nq above a length (rows without a
# key); GQA; head dims 128 and 64
VARLEN = [
    (4, 4, 2, 130, 300, 128, True, [0, 1, 257, 300]),
    (3, 2, 1, 200, 200, 64, False, [64, 199, 128]),
    (2, 8, 2, 64, 520, 128, True, [520, 130]),
    (4, 2, 2, 300, 130, 128, True, [130, 0, 77, 128]),
    (2, 8, 2, 150, 333, 64, True, [333, 200]),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_cap{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_backward_with_key_lengths(case):
    B, Hq, Hkv, Nq, Nk, d, causal, L = case
    seed = 4800 + Nq + 7 * Nk + d
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(seed + 1, (B, Hq, Nq, d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    lens = torch.as_tensor(np.asarray(L, np.int32), device="cuda")
    s32 = _s32(d)
    say(f"backward with lengths {case}")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=causal, scale=s32, seqlens_k=lens)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.attn_bwd(q, k, v, out, lse, dout, causal=causal, scale=s32, dq=dq, dk=dk, dv=dv,
                seqlens_k=lens)
    torch.cuda.synchronize()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    ref = A.attention_backward_fp64(*x.as_f64(), g, s32, causal, seqlens_k=L)
    got = [to_f64(t) for t in (dq, dk, dv)]
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, a, r)
    for b, Lb in enumerate(L):  # rows of K/V past the length: exactly zero, and written
        assert np.all(got[1][b, :, Lb:] == 0) and np.all(got[2][b, :, Lb:] == 0), f"b={b}"
        if Lb == 0:
            assert np.all(got[0][b] == 0), f"b={b}: no key, dq must be 0"


def test_backward_with_lengths_matches_truncated_tensors():
    # one element, 333 of 520 keys: bit-identical to the plain backward on K/V cut to 333 keys
    B, Hq, Hkv, Nq, Nk, Lb, d = 1, 4, 2, 200, 520, 333, 128
    x = I.draw_qkv(4900, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    dout = I.to_device(I.draw_grad(4901, (B, Hq, Nq, d)), "bf16")
    lens = torch.full((1,), Lb, dtype=torch.int32, device="cuda")
    say("backward with lengths vs truncated K/V")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=True, seqlens_k=lens)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=True, seqlens_k=lens)
    kt, vt = k[:, :, :Lb].contiguous(), v[:, :, :Lb].contiguous()
    out_t, lse_t = fa.attn_fwd(q, kt, vt, causal=True)
    dq_t, dk_t, dv_t = fa.attn_bwd(q, kt, vt, out_t, lse_t, dout, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_t.view(torch.int16))
    assert torch.equal(dq.view(torch.int16), dq_t.view(torch.int16))
    assert torch.equal(dk[:, :, :Lb].view(torch.int16), dk_t.view(torch.int16))
    assert torch.equal(dv[:, :, :Lb].view(torch.int16), dv_t.view(torch.int16))
    assert bool((dk[:, :, Lb:].float() == 0).all()) and bool((dv[:, :, Lb:].float() == 0).all())


# additive bias (attn_bwd_ex): (B, Hq, Hkv, Nq, Nk, d, causal, bias batch, bias heads, kind,
# -inf fraction, lengths or None); Nk a multiple of 4 as the bias layout requires
BIASED = [
    (2, 4, 2, 130, 300, 128, True, 2, 4, "normal", 0.1, None),
    (1, 4, 1, 257, 128, 128, False, 1, 4, "alibi", 0.0, None),
    (3, 2, 2, 200, 200, 64, True, 1, 1, "normal", 0.0, [200, 0, 77]),
    (2, 8, 2, 64, 520, 128, True, 2, 1, "alibi", 0.0, [520, 131]),
    (2, 2, 1, 300, 132, 64, False, 2, 2, "normal", 0.2, [100, 132]),
]


@pytest.mark.parametrize("case", BIASED, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_bias{}x{}_{}".format(
    *c[:6], "causal" if c[6] else "full", c[7], c[8], c[9]))
def test_backward_with_bias(case):
    B, Hq, Hkv, Nq, Nk, d, causal, Bb, Hb, kind, masked, L = case
    seed = 5100 + Nq + 3 * Nk + d
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(seed + 1, (B, Hq, Nq, d))
    bias_bits = I.draw_bias(seed + 2, Bb, Hb, Nq, Nk, kind, masked_frac=masked)
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    bias = I.to_device(bias_bits, "bf16")
    lens = None if L is None else torch.as_tensor(np.asarray(L, np.int32), device="cuda")
    s32 = _s32(d)
    say(f"backward with bias {case}")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=causal, scale=s32, seqlens_k=lens, bias=bias)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
    fa.attn_bwd(q, k, v, out, lse, dout, causal=causal, scale=s32, dq=dq, dk=dk, dv=dv,
                seqlens_k=lens, bias=bias)
    torch.cuda.synchronize()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    ref = A.attention_backward_fp64(*x.as_f64(), g, s32, causal, seqlens_k=L,
                                    bias=I.bf16_bits_to_f32(bias_bits).astype(np.float64))
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _check(name, to_f64(a), r)
