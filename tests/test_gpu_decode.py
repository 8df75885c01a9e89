"""GPU parity of the split-KV decode path (attn_decode_splitkv: split kernel + combine kernel)
against the CPU fp64 oracle, including the per-split partials and (max, sum) metadata left in the
workspace, which are checked against the oracle's split model."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, compare, say, to_f64, upload  # noqa: E402
from oracle import attention as A  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu

PARTIAL_MAX_ABS = 2e-2  # partials are fp32 sums of bf16-rounded probabilities times bf16 V
META_M_MAX_ABS = 1e-4   # local max of scaled scores (fp32 dot products of bf16 inputs)
META_L_REL = 1e-2       # local sums of exp (fp32 exp2 of rounded scores)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


def _scale32(d):
    return float(np.float32(1.0 / np.sqrt(d)))


def _run(B, Hq, Hkv, Nq, Nk, d, causal, S, seed):
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    s32 = _scale32(d)
    say(f"decode B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} S={S} seed={seed}")
    out, lse, ws = fa.attn_decode_splitkv(q, k, v, S, causal=causal, scale=s32)
    torch.cuda.synchronize()
    return x, s32, out, lse, ws


def _workspace(ws, B, Hq, Nq, S, d):
    f = ws.view(torch.float32)
    n = B * Hq * Nq * S
    O_s = f[: n * d].view(B, Hq, Nq, S, d)
    ml = f[n * d: n * d + 2 * n].view(B, Hq, Nq, S, 2)
    return to_f64(O_s), to_f64(ml[..., 0]), to_f64(ml[..., 1])


def _check_partials(x, s32, causal, S, ws, B, Hq, Nq, d):
    O_s, m_s, l_s = _workspace(ws, B, Hq, Nq, S, d)
    rO, rm, rl = A.splitkv_partials_fp64(*x.as_f64(), s32, causal, S)
    empty = rl == 0
    assert np.array_equal(l_s == 0, empty), "empty-split pattern differs"
    assert np.all(np.isneginf(m_s[empty])) and np.all(O_s[empty] == 0)
    full = ~empty
    if full.any():
        assert np.abs(m_s[full] - rm[full]).max() <= META_M_MAX_ABS
        assert (np.abs(l_s[full] - rl[full]) / rl[full]).max() <= META_L_REL
        assert np.abs(O_s[full] - rO[full]).max() <= PARTIAL_MAX_ABS


@pytest.mark.parametrize("name", ["decode_gqa_nq1", "decode_gqa_nq4"])
def test_config_decode_gqa(name):
    w = I.WORKLOADS[name]
    x, s32, out, lse, ws = _run(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, w.n_splits, w.seed)
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), s32, w.causal)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=name)
    # the partials of two (batch, KV head) groups against the oracle's split model
    for b, hkv in ((0, 0), (w.B - 1, w.Hkv - 1)):
        G = w.Hq // w.Hkv
        sub = I.QKV(q=x.q[b:b + 1, hkv * G:(hkv + 1) * G], k=x.k[b:b + 1, hkv:hkv + 1],
                    v=x.v[b:b + 1, hkv:hkv + 1], dtype="bf16")
        f = ws.view(torch.float32)
        n = w.B * w.Hq * w.Nq * w.n_splits
        O_s = f[: n * w.d].view(w.B, w.Hq, w.Nq, w.n_splits, w.d)[b:b + 1, hkv * G:(hkv + 1) * G]
        ml = f[n * w.d: n * w.d + 2 * n].view(w.B, w.Hq, w.Nq, w.n_splits, 2)[
            b:b + 1, hkv * G:(hkv + 1) * G]
        packed = torch.cat([O_s.reshape(-1), ml.reshape(-1)]).contiguous().view(torch.uint8)
        _check_partials(sub, s32, w.causal, w.n_splits, packed, 1, G, w.Nq, w.d)


# (B, Hq, Hkv, Nq, Nk, d, causal, n_splits): ragged split lengths, one key per split, more than
# 32 query rows per KV head (two row groups), non-causal, Nq > Nk (rows and splits with no
# visible key), head dim 64, GQA ratios 1, 4 and 8; (batch, KV head) pair counts that are
# multiples of 8 (the XCD-grouped mapping of both kernels) with two row groups and with ragged ones;
# grids of 1024 workgroups or more with at least 8 query rows per KV head (one wave per split):
# head dim 64 with ragged splits, 9 pairs (not a multiple of 8) with two row groups in two rounds
# of workgroups, splits past the end of the keys (L = 5, so the last splits are empty), and more
# query rows than keys (row 0 sees no key).
EDGE_CASES = [
    (2, 8, 2, 1, 1000, 128, True, 3),
    (1, 4, 4, 1, 33, 64, True, 33),
    (1, 8, 1, 8, 513, 128, True, 16),
    (2, 4, 2, 4, 100, 128, False, 1),
    (1, 4, 1, 5, 4, 128, True, 4),
    (1, 2, 2, 3, 257, 64, True, 7),
    (1, 32, 8, 4, 8192, 128, True, 16),
    (1, 8, 8, 1, 70, 128, False, 70),
    (2, 64, 4, 2, 300, 64, True, 5),
    (4, 12, 4, 3, 200, 128, False, 6),
    (4, 8, 4, 4, 3000, 64, True, 64),
    (3, 12, 3, 5, 2000, 128, False, 128),
    (2, 16, 2, 1, 1030, 128, True, 257),
    (128, 8, 4, 4, 3, 64, True, 3),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_S{}".format(
    *c[:6], "causal" if c[6] else "full", c[7]))
def test_edge_shapes(case):
    B, Hq, Hkv, Nq, Nk, d, causal, S = case
    x, s32, out, lse, ws = _run(B, Hq, Hkv, Nq, Nk, d, causal, S, seed=3000 + Nk + S)
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), s32, causal)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=str(case))
    _check_partials(x, s32, causal, S, ws, B, Hq, Nq, d)


def test_decode_equals_prefill_rows():
    # decode rows are the last Nq rows of a square causal prefill over the same keys
    B, Hq, Hkv, Nk, d, Nq = 2, 8, 2, 700, 128, 4
    x = I.draw_qkv(41, B, Hq, Hkv, Nk, Nk, d)
    q, k, v = upload(x)
    say("decode vs prefill rows")
    full, lse_full = fa.attn_fwd(q, k, v, causal=True)
    dec, lse_dec, _ = fa.attn_decode_splitkv(q[:, :, Nk - Nq:].contiguous(), k, v, 9, causal=True)
    torch.cuda.synchronize()
    assert np.abs(to_f64(dec) - to_f64(full[:, :, Nk - Nq:])).max() <= 2 * BF16_MAX_ABS
    assert np.abs(to_f64(lse_dec) - to_f64(lse_full[:, :, Nk - Nq:])).max() <= 2e-3


def test_deterministic_and_workspace_reuse():
    x = I.draw_qkv(42, 2, 8, 2, 4, 1500, 128)
    q, k, v = upload(x)
    say("decode determinism / workspace reuse / poison")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((2, 8, 4), float("nan"), device=q.device)
    need = fa.attn_decode_workspace_bytes(2, 8, 4, 128, 16)
    ws = torch.full((need // 4,), float("nan"), device=q.device).view(torch.uint8)
    fa.attn_decode_splitkv(q, k, v, 16, out=out, lse=lse, workspace=ws)
    out2, lse2, _ = fa.attn_decode_splitkv(q, k, v, 16)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out.float()).any()) and not bool(torch.isnan(lse).any())
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


@pytest.mark.parametrize("B", [2, 256], ids=["four_wave", "one_wave"])
def test_decode_without_keys(B):
    # Nk = 0 (one split): no row sees a key, so O = 0, LSE = -inf and the split's metadata is
    # (-inf, 0); B = 256 gives 1024 split workgroups of 8 rows each (one wave per split)
    Hq, Hkv, Nq, d = 8, 4, 4, 128
    say(f"decode Nk=0 B={B}")
    q = I.to_device(I.draw_qkv(4700 + B, B, Hq, Hkv, Nq, 1, d).q, "bf16")
    k = torch.empty((B, Hkv, 0, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), device="cuda")
    out, lse, ws = fa.attn_decode_splitkv(q, k, k, 1, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out.float() == 0).all()) and bool((lse == -float("inf")).all())
    O_s, m_s, l_s = _workspace(ws, B, Hq, Nq, 1, d)
    assert np.all(O_s == 0) and np.all(np.isneginf(m_s)) and np.all(l_s == 0)


def test_invalid_decode_arguments():
    q = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 10, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.AttentionError, match="n_splits"):
        fa.attn_decode_splitkv(q, k, k, 11)
    with pytest.raises(fa.AttentionError, match="n_splits"):
        fa.attn_decode_splitkv(q, k, k, 0)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.AttentionError, match="workspace"):
        fa.attn_decode_splitkv(q, k, k, 2, workspace=small)
