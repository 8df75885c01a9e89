"""GPU parity of the prefill forward (attn_fwd, attn_fwd_f32) against the CPU fp64 oracle.

Every workload is compared on full tensors: every element of O and LSE, including the N 512-4096
sweep and the B1 H8 N16384 causal workload at their full launch sizes (the oracle runs there as
independent (batch, head, row chunk) tasks on the host cores).  Sampled rows of the same launches
are checked as well.  Every call goes through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, F32_MEAN_ABS, compare,  # noqa: E402
                         oracle_full, sample_rows, say, to_f64, upload)
from oracle import attention as A  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


def _scale32(scale, d):
    """The float32 scale both sides use (0 means 1/sqrt(d))."""
    return float(np.float32(scale if scale else 1.0 / np.sqrt(d)))


def _run_full(B, Hq, Hkv, Nq, Nk, d, causal, seed, dtype="bf16", scale=0.0):
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d, dtype)
    q, k, v = upload(x)
    s32 = _scale32(scale, d)
    say(f"prefill {dtype} B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} seed={seed}")
    fn = fa.attn_fwd if dtype == "bf16" else fa.attn_fwd_f32
    out, lse = fn(q, k, v, causal=causal, scale=s32)
    torch.cuda.synchronize()
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), s32, causal)
    return x, to_f64(out), to_f64(lse), O_ref, lse_ref


def test_config_tiny_causal_f32():
    w = I.WORKLOADS["tiny_causal_f32"]
    _, out, lse, O_ref, lse_ref = _run_full(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, w.seed,
                                            "f32", w.scale)
    compare(out, lse, O_ref, lse_ref, F32_MAX_ABS, F32_MEAN_ABS, what=w.name)


def test_config_prefill_causal_b2h16n2048_full():
    w = I.WORKLOADS["prefill_causal_b2h16n2048"]
    x, out, lse, O_ref, lse_ref = _run_full(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.causal, w.seed,
                                            "bf16", w.scale)
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=w.name)
    # causal row 0 sees only key 0: p = 1, l = 1, so the bf16 output is v_0 bit for bit
    v0 = I.bf16_bits_to_f32(x.v[:, :, 0]).astype(np.float64)
    assert np.array_equal(out[:, :, 0], v0), "row 0 is not v_0 bit-exactly"


def _full_size(name):
    """The workload at its real launch size, compared on every element with the oracle."""
    w = I.WORKLOADS[name]
    x = w.draw()
    q, k, v = upload(x)
    say(f"{name}: full-size launch, full tensors")
    s32 = _scale32(w.scale, w.d)
    out, lse = fa.attn_fwd(q, k, v, causal=w.causal, scale=s32)
    torch.cuda.synchronize()
    out64, lse64 = to_f64(out), to_f64(lse)
    del q, k, v, out, lse
    O_ref, lse_ref = oracle_full(*x.as_f64(), s32, w.causal)
    compare(out64, lse64, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=f"{name} full")
    if w.causal:
        v0 = I.bf16_bits_to_f32(x.v[:, :, 0]).astype(np.float64)
        assert np.array_equal(out64[:, :, 0], v0), "row 0 is not v_0 bit-exactly"


@pytest.mark.parametrize("name", [n for n in I.WORKLOADS if n.startswith("sweep_")])
def test_config_sweep_full(name):
    _full_size(name)


def test_config_long_causal_b1h8n16384_full():
    _full_size("long_causal_b1h8n16384")


def _sampled(name, n_random=16):
    w = I.WORKLOADS[name]
    x = w.draw()
    q, k, v = upload(x)
    say(f"{name}: full-size launch, sampled rows")
    s32 = _scale32(w.scale, w.d)
    out, lse = fa.attn_fwd(q, k, v, causal=w.causal, scale=s32)
    torch.cuda.synchronize()
    rows = sample_rows(w.Nq, n_random, seed=w.seed)
    outs = to_f64(out[:, :, torch.as_tensor(rows, device=out.device)])
    lses = to_f64(lse[:, :, torch.as_tensor(rows, device=out.device)])
    O_ref, lse_ref = A.attention_rows_fp64(*x.as_f64(), s32, w.causal, rows)
    compare(outs, lses, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=f"{name} sampled rows")


def test_config_long_causal_b1h8n16384_sampled():
    # tile boundaries and seeded rows of the long workload, through the oracle's single-pass
    # row function (an extra to the full-tensor test above)
    _sampled("long_causal_b1h8n16384", n_random=24)


# (B, Hq, Hkv, Nq, Nk, d, causal): ragged tails, one-row and one-key problems, Nq != Nk in both
# directions (Nq > Nk leaves the first rows with no visible key), GQA, head dim 64, and grids of
# one and of several rounds of workgroups.
EDGE_CASES = [
    (1, 2, 2, 1, 1, 128, True),
    (1, 2, 2, 77, 77, 128, True),
    (2, 3, 3, 200, 200, 64, False),
    (1, 2, 1, 1000, 1000, 128, True),
    (1, 4, 2, 129, 300, 128, True),
    (1, 2, 2, 300, 129, 128, True),
    (1, 8, 2, 256, 256, 64, True),
    (3, 2, 2, 130, 70, 128, False),
    (1, 2, 2, 65, 63, 64, True),
    (2, 16, 4, 384, 384, 128, False),
    # grids of more than 512 workgroups (more than one round of two per CU), full-tensor
    (4, 64, 16, 300, 300, 64, True),
    (4, 64, 64, 200, 333, 128, False),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_edge_shapes_bf16(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    _, out, lse, O_ref, lse_ref = _run_full(B, Hq, Hkv, Nq, Nk, d, causal, seed=1000 + Nq + Nk)
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=str(case))


@pytest.mark.parametrize("case", [(1, 2, 2, 77, 77, 128, True), (2, 4, 2, 130, 300, 64, True),
                                  (1, 2, 2, 200, 100, 128, False)])
def test_edge_shapes_f32(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    _, out, lse, O_ref, lse_ref = _run_full(B, Hq, Hkv, Nq, Nk, d, causal, seed=2000 + Nq, dtype="f32")
    compare(out, lse, O_ref, lse_ref, F32_MAX_ABS, F32_MEAN_ABS, what=str(case))


def test_no_keys_gives_zero_rows_and_neg_inf_lse():
    x = I.draw_qkv(7, 1, 2, 2, 64, 0, 128)
    q, k, v = upload(x)
    say("prefill Nk=0")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, 2, 64), float("nan"), device=q.device)
    fa.attn_fwd(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out.float() == 0).all()) and bool(torch.isneginf(lse).all())


def test_empty_problems_are_no_ops():
    say("prefill empty problems")
    for shape_q, shape_k in (((0, 2, 16, 64), (0, 2, 16, 64)), ((1, 2, 0, 64), (1, 2, 16, 64))):
        q = torch.empty(shape_q, dtype=torch.bfloat16, device="cuda")
        k = torch.empty(shape_k, dtype=torch.bfloat16, device="cuda")
        out, lse = fa.attn_fwd(q, k, k.clone(), causal=True)
        assert out.shape == q.shape and lse.shape == q.shape[:3]


def test_every_output_written_deterministic_and_stream_ordered():
    x = I.draw_qkv(11, 2, 4, 2, 333, 333, 128)
    q, k, v = upload(x)
    say("prefill poison / determinism / side stream")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((2, 4, 333), float("nan"), device=q.device)
    fa.attn_fwd(q, k, v, causal=True, out=out, lse=lse)
    out2, lse2 = fa.attn_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out3, lse3 = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(out.float()).any()) and not bool(torch.isnan(lse).any())
    for o, l in ((out2, lse2), (out3, lse3)):
        assert torch.equal(out.view(torch.int16), o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l.view(torch.int32))


def test_default_scale_and_explicit_scale_agree():
    x = I.draw_qkv(12, 1, 2, 2, 150, 150, 64)
    q, k, v = upload(x)
    say("prefill scale 0 vs 1/sqrt(d)")
    a, la = fa.attn_fwd(q, k, v, causal=True, scale=0.0)
    b, lb = fa.attn_fwd(q, k, v, causal=True, scale=1.0 / 8.0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    c, lc = fa.attn_fwd(q, k, v, causal=True, scale=0.3)
    torch.cuda.synchronize()
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), _scale32(0.3, 64), True)
    compare(to_f64(c), to_f64(lc), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what="scale 0.3")


def test_invalid_arguments_raise_before_launch():
    q = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.AttentionError, match="head dimension"):
        fa.attn_fwd(q, q, q)
    q = torch.zeros((1, 3, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.AttentionError, match="multiple"):
        fa.attn_fwd(q, k, k)
    with pytest.raises(fa.AttentionError, match="scale"):
        fa.attn_fwd(k, k, k, scale=float("nan"))


def test_binding_rejects_mismatched_outputs():
    # caller-supplied outputs, gradients and workspaces must match what the kernels write; the
    # binding refuses anything else before a launch
    q = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    bad_out = torch.empty((1, 2, 32, 128), dtype=torch.bfloat16, device="cuda")
    bad_lse = torch.empty((1, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError, match="out must be"):
        fa.attn_fwd(q, q, q, out=bad_out)
    with pytest.raises(ValueError, match="lse must be"):
        fa.attn_fwd(q, q, q, lse=bad_lse)
    with pytest.raises(ValueError, match="out must be"):
        fa.prepare_fwd(q, q, q, bad_out)
    with pytest.raises(ValueError, match="workspace must be"):
        fa.attn_decode_splitkv(q, q, q, 2, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    out, lse = fa.attn_fwd(q, q, q)
    with pytest.raises(ValueError, match="dk must be"):
        fa.attn_bwd(q, q, q, out, lse, q, dk=torch.empty((1, 2, 64, 64), dtype=torch.bfloat16,
                                                         device="cuda"))
    torch.cuda.synchronize()
