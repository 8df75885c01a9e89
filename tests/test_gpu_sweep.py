"""Seeded sweep of small random shapes through every entry point, each against the CPU oracle.

The shapes are drawn from one seeded generator (batch 1-3, 1-4 K/V heads, GQA groups of 1-4,
query and key lengths 1-400 in any ratio, head dimension 64 or 128, causal or not, split counts
up to the key length), so the hand-picked edge cases elsewhere are complemented by shapes nobody
chose: ragged tails in every position, Nq far above and below Nk, splits shorter than a block."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, compare, say, to_f64, upload  # noqa: E402
from oracle import attention as A  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu

GRAD_MAX_REL, GRAD_MEAN_REL, GRAD_FLOOR = 2e-2, 2e-3, 2.0 ** -10


def _shapes(seed, n, d_choices=(64, 128)):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.integers(1, 5))
        out.append((int(rng.integers(1, 4)), Hkv * int(rng.integers(1, 5)), Hkv,
                    int(rng.integers(1, 401)), int(rng.integers(1, 401)),
                    int(rng.choice(d_choices)), bool(rng.integers(0, 2))))
    return out


FWD = _shapes(9100, 24)
DEC = _shapes(9200, 16)
BWD = _shapes(9300, 12)


def _ids(c):
    return "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}".format(*c[:6], "causal" if c[6] else "full")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


def _s32(d):
    return float(np.float32(1.0 / np.sqrt(d)))


@pytest.mark.parametrize("case", FWD, ids=_ids)
def test_forward_and_routing(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    seed = 9100 + 7 * Nq + Nk
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    say(f"sweep forward {case}")
    out, lse = fa.attn_fwd(q, k, v, causal=causal, scale=_s32(d))
    # the routing entry point: split-KV below 32 query rows, the prefill kernel above
    out2, lse2, _ = fa.attn_forward(q, k, v, causal=causal, scale=_s32(d))
    torch.cuda.synchronize()
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), _s32(d), causal)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=str(case))
    compare(to_f64(out2), to_f64(lse2), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"attn_forward {case}")


@pytest.mark.parametrize("case", DEC, ids=_ids)
def test_decode_splits(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    Nq = 1 + Nq % 8  # decode: a few query rows against the keys
    rng = np.random.default_rng(9200 + Nk)
    n_splits = int(rng.integers(1, min(Nk, 40) + 1))
    seed = 9200 + 5 * Nq + Nk
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    say(f"sweep decode {case[:3]} Nq={Nq} Nk={Nk} d={d} causal={causal} splits={n_splits}")
    out, lse, _ = fa.attn_decode_splitkv(q, k, v, n_splits, causal=causal, scale=_s32(d))
    torch.cuda.synchronize()
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), _s32(d), causal)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"decode {case} splits={n_splits}")


@pytest.mark.parametrize("case", BWD, ids=_ids)
def test_backward(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    seed = 9300 + 3 * Nq + Nk
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(seed + 1, (B, Hq, Nq, d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    say(f"sweep backward {case}")
    out, lse = fa.attn_fwd(q, k, v, causal=causal, scale=_s32(d))
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=causal, scale=_s32(d))
    torch.cuda.synchronize()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    ref = A.attention_backward_fp64(*x.as_f64(), g, _s32(d), causal)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        a = to_f64(a)
        scale = max(float(np.abs(r).max(initial=0.0)), GRAD_FLOOR)
        err = np.abs(a - r)
        assert np.all(np.isfinite(a)), name
        assert float(err.max()) / scale <= GRAD_MAX_REL, f"{name} {case}"
        assert float(err.mean()) / scale <= GRAD_MEAN_REL, f"{name} {case}"


def _extras_draw(case, seed):
    """Random per-batch key lengths and a random bias of a random broadcast shape for a case."""
    B, Hq, Hkv, Nq, Nk, d, causal = case
    rng = np.random.default_rng(seed)
    L = I.draw_seqlens(seed + 1, B, Nk, edges=False) if rng.integers(0, 2) else None
    bias_bits = None
    if rng.integers(0, 3):  # two cases in three carry a bias
        Bb = B if rng.integers(0, 2) else 1
        Hb = Hq if rng.integers(0, 2) else 1
        kind = "alibi" if rng.integers(0, 3) == 0 else "normal"
        bias_bits = I.draw_bias(seed + 2, Bb, Hb, Nq, Nk, kind, std=float(rng.choice([1.0, 4.0])),
                                masked_frac=float(rng.choice([0.0, 0.1])))
    return L, bias_bits


def _extras_case(c, nq_max=None):
    # bias rows are 8-byte groups of four keys: Nk a multiple of 4
    B, Hq, Hkv, Nq, Nk, d, causal = c
    if nq_max is not None:
        Nq = 1 + Nq % nq_max
    return (B, Hq, Hkv, Nq, max(4, Nk - Nk % 4), d, causal)


FWD_EX = [_extras_case(c) for c in _shapes(9400, 16)]
DEC_EX = [_extras_case(c, 8) for c in _shapes(9500, 12)]


def _ref(x, s32, causal, L, bias_bits):
    return A.attention_fp64(*x.as_f64(), s32, causal, seqlens_k=L,
                            bias=None if bias_bits is None else
                            I.bf16_bits_to_f32(bias_bits).astype(np.float64))


def _dev_extras(L, bias_bits):
    return (None if L is None else torch.as_tensor(np.asarray(L, np.int32), device="cuda"),
            None if bias_bits is None else I.to_device(bias_bits, "bf16"))


@pytest.mark.parametrize("case", FWD_EX, ids=_ids)
def test_forward_with_extras(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    seed = 9400 + 11 * Nq + Nk
    L, bias_bits = _extras_draw(case, seed)
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    sl, bias = _dev_extras(L, bias_bits)
    say(f"sweep forward_ex {case} lens={None if L is None else list(L)} "
        f"bias={None if bias_bits is None else bias_bits.shape}")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=causal, scale=_s32(d), seqlens_k=sl, bias=bias)
    out2, lse2, _ = fa.attn_forward(q, k, v, causal=causal, scale=_s32(d), seqlens_k=sl, bias=bias)
    torch.cuda.synchronize()
    O_ref, lse_ref = _ref(x, _s32(d), causal, L, bias_bits)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=str(case))
    compare(to_f64(out2), to_f64(lse2), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"attn_forward {case}")


@pytest.mark.parametrize("case", DEC_EX, ids=_ids)
def test_decode_with_extras(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    seed = 9500 + 13 * Nq + Nk
    L, bias_bits = _extras_draw(case, seed)
    n_splits = int(np.random.default_rng(seed).integers(1, min(Nk, 40) + 1))
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    sl, bias = _dev_extras(L, bias_bits)
    say(f"sweep decode_ex {case} splits={n_splits} lens={None if L is None else list(L)} "
        f"bias={None if bias_bits is None else bias_bits.shape}")
    out, lse, _ = fa.attn_decode_splitkv_ex(q, k, v, n_splits, causal=causal, scale=_s32(d),
                                            seqlens_k=sl, bias=bias)
    torch.cuda.synchronize()
    O_ref, lse_ref = _ref(x, _s32(d), causal, L, bias_bits)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"decode_ex {case} splits={n_splits}")


BWD_EX = _shapes(9600, 8)


@pytest.mark.parametrize("case", BWD_EX, ids=_ids)
def test_backward_with_key_lengths(case):
    # the forward with random per-batch key lengths, then its backward (attn_bwd_ex)
    B, Hq, Hkv, Nq, Nk, d, causal = case
    seed = 9600 + 5 * Nq + Nk
    L = I.draw_seqlens(seed + 2, B, Nk, edges=True)
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(seed + 1, (B, Hq, Nq, d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    lens = torch.as_tensor(np.asarray(L, np.int32), device="cuda")
    say(f"sweep backward with lengths {case} lens={list(L)}")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=causal, scale=_s32(d), seqlens_k=lens)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=causal, scale=_s32(d),
                             seqlens_k=lens)
    torch.cuda.synchronize()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    ref = A.attention_backward_fp64(*x.as_f64(), g, _s32(d), causal, seqlens_k=L)
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        a = to_f64(a)
        scale = max(float(np.abs(r).max(initial=0.0)), GRAD_FLOOR)
        err = np.abs(a - r)
        assert np.all(np.isfinite(a)), name
        assert float(err.max()) / scale <= GRAD_MAX_REL, f"{name} {case}"
        assert float(err.mean()) / scale <= GRAD_MEAN_REL, f"{name} {case}"


BWD_BIAS = [_extras_case(c) for c in _shapes(9700, 8)]


@pytest.mark.parametrize("case", BWD_BIAS, ids=_ids)
def test_backward_with_extras(case):
    # the forward with random key lengths and / or a random bias, then its backward
    B, Hq, Hkv, Nq, Nk, d, causal = case
    seed = 9700 + 11 * Nq + Nk
    L, bias_bits = _extras_draw(case, seed)
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    g_bits = I.draw_grad(seed + 1, (B, Hq, Nq, d))
    q, k, v = upload(x)
    dout = I.to_device(g_bits, "bf16")
    sl, bias = _dev_extras(L, bias_bits)
    say(f"sweep backward_ex {case} lens={None if L is None else list(L)} "
        f"bias={None if bias_bits is None else bias_bits.shape}")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=causal, scale=_s32(d), seqlens_k=sl, bias=bias)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=causal, scale=_s32(d),
                             seqlens_k=sl, bias=bias)
    torch.cuda.synchronize()
    g = I.bf16_bits_to_f32(g_bits).astype(np.float64)
    ref = A.attention_backward_fp64(
        *x.as_f64(), g, _s32(d), causal, seqlens_k=L,
        bias=None if bias_bits is None else I.bf16_bits_to_f32(bias_bits).astype(np.float64))
    for name, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        a = to_f64(a)
        scale = max(float(np.abs(r).max(initial=0.0)), GRAD_FLOOR)
        err = np.abs(a - r)
        assert np.all(np.isfinite(a)), name
        assert float(err.max()) / scale <= GRAD_MAX_REL, f"{name} {case}"
        assert float(err.mean()) / scale <= GRAD_MEAN_REL, f"{name} {case}"
