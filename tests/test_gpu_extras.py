"""GPU parity of the extras -- per-batch key lengths (seqlens_k) and the additive bias -- on the
prefill (attn_fwd_ex) and split-KV decode (attn_decode_splitkv_ex) paths, and of the routing
entry attn_forward, against the CPU fp64 oracle.  Every call goes through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, compare, say, to_f64, upload  # noqa: E402
from oracle import attention as A  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu

META_M_MAX_ABS = 1e-4   # plus 4 fp32 ulps of |m|: a large bias makes large maxima
META_L_REL = 1e-2
PARTIAL_MAX_ABS = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


def _s32(d):
    return float(np.float32(1.0 / np.sqrt(d)))


def _lens(L):
    return torch.as_tensor(np.asarray(L, np.int32), device="cuda")


def _bias(bits):
    return I.to_device(bits, "bf16")


def _bias64(bits):
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def _prefill(B, Hq, Hkv, Nq, Nk, d, causal, seed, L=None, bias_bits=None):
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    s32 = _s32(d)
    bshape = None if bias_bits is None else bias_bits.shape
    say(f"prefill_ex B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} seed={seed} "
        f"lens={None if L is None else list(L)} bias={bshape}")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=causal, scale=s32,
                              seqlens_k=None if L is None else _lens(L),
                              bias=None if bias_bits is None else _bias(bias_bits))
    torch.cuda.synchronize()
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), s32, causal, seqlens_k=L,
                                      bias=None if bias_bits is None else _bias64(bias_bits))
    return to_f64(out), to_f64(lse), O_ref, lse_ref


# (B, Hq, Hkv, Nq, Nk capacity, d, causal): ragged capacities and lengths (0, 1, a whole number of
# 64-key blocks, the capacity), Nq above and below the lengths, GQA, head dim 64
VARLEN_CASES = [
    (4, 4, 2, 200, 333, 128, True),
    (4, 4, 2, 200, 333, 128, False),
    (5, 2, 2, 130, 130, 64, True),
    (3, 8, 2, 64, 1000, 128, True),
    (6, 2, 1, 300, 256, 128, False),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_prefill_varlen(case):
    B, Hq, Hkv, Nq, Nk, d, causal = case
    L = I.draw_seqlens(500 + Nk, B, Nk)
    if B > 3:
        L[3] = 128  # a whole number of 64-key blocks
    out, lse, O_ref, lse_ref = _prefill(B, Hq, Hkv, Nq, Nk, d, causal, 510 + Nq, L=L)
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=f"varlen {case}")


def test_prefill_varlen_matches_truncated_tensors():
    # a batch element with L keys gives what a K/V of exactly L keys gives, bit for bit
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 150, 400, 128
    x = I.draw_qkv(520, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    L = np.array([400, 257, 64], np.int32)
    say("prefill varlen vs truncated tensors")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=True, seqlens_k=_lens(L))
    for b in range(B):
        ob, lb = fa.attn_fwd(q[b:b + 1].contiguous(), k[b:b + 1, :, :L[b]].contiguous(),
                             v[b:b + 1, :, :L[b]].contiguous(), causal=True)
        torch.cuda.synchronize()
        assert torch.equal(out[b:b + 1].view(torch.int16), ob.view(torch.int16)), b
        assert torch.equal(lse[b:b + 1].view(torch.int32), lb.view(torch.int32)), b


def test_prefill_ex_without_extras_is_attn_fwd():
    x = I.draw_qkv(521, 2, 4, 4, 333, 333, 128)
    q, k, v = upload(x)
    say("attn_fwd_ex without extras vs attn_fwd")
    a, la = fa.attn_fwd_ex(q, k, v, causal=True)
    b, lb = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))


# (B, Hq, Hkv, Nq, Nk, d, causal, bias_b, bias_h, kind, std, masked_frac)
BIAS_CASES = [
    (2, 4, 2, 300, 300, 128, True, 1, 1, "normal", 1.0, 0.0),
    (2, 4, 2, 300, 300, 128, False, 2, 4, "normal", 3.0, 0.0),
    (2, 4, 2, 200, 332, 128, True, 2, 1, "alibi", 0.0, 0.0),
    (2, 4, 4, 257, 260, 64, True, 1, 4, "normal", 1.0, 0.2),
    (1, 2, 2, 130, 64, 128, False, 1, 2, "normal", 2.0, 0.5),
    (3, 8, 2, 128, 128, 64, False, 3, 8, "alibi", 0.0, 0.1),
    # a bias large enough to move the running max by more than the lazy threshold
    (1, 2, 1, 256, 512, 128, True, 1, 1, "normal", 12.0, 0.0),
]


@pytest.mark.parametrize("case", BIAS_CASES, ids=lambda c: "B{}_Hq{}_Nq{}_Nk{}_d{}_{}_b{}x{}_{}_{}_{}".format(
    c[0], c[1], c[3], c[4], c[5], "causal" if c[6] else "full", c[7], c[8], c[9], c[10], c[11]))
def test_prefill_bias(case):
    B, Hq, Hkv, Nq, Nk, d, causal, bb, bh, kind, std, frac = case
    bits = I.draw_bias(600 + Nq + Nk, bb, bh, Nq, Nk, kind, std, frac)
    out, lse, O_ref, lse_ref = _prefill(B, Hq, Hkv, Nq, Nk, d, causal, 610 + Nq, bias_bits=bits)
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what=f"bias {case}")


def test_prefill_bias_and_varlen_together():
    B, Hq, Hkv, Nq, Nk, d = 4, 4, 2, 180, 360, 128
    L = I.draw_seqlens(620, B, Nk)
    bits = I.draw_bias(621, B, 1, Nq, Nk, "normal", 1.5, 0.1)
    for causal in (True, False):
        out, lse, O_ref, lse_ref = _prefill(B, Hq, Hkv, Nq, Nk, d, causal, 622, L=L, bias_bits=bits)
        compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
                what=f"bias+varlen causal={causal}")


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True)])
def test_prefill_paired_grid_with_extras(d, causal):
    # a grid of several rounds of workgroups runs paired query blocks (blocks nqt-1-i and i in
    # one workgroup); here with an odd number of query blocks (9: the middle one runs alone),
    # GQA, per-batch key lengths (the capacity, 0, 1 and a ragged one) and a per-head bias with
    # -inf entries, full tensors against the oracle
    B, Hq, Hkv, Nq, Nk = 4, 32, 8, 1100, 1100
    assert B * Hq * ((Nq + 127) // 128 + 1) // 2 >= 512  # the paired grid is taken
    L = I.draw_seqlens(650 + d, B, Nk)
    bits = I.draw_bias(651 + d, 1, Hq, Nq, Nk, "normal", 2.0, 0.05)
    out, lse, O_ref, lse_ref = _prefill(B, Hq, Hkv, Nq, Nk, d, causal, 652 + d, L=L, bias_bits=bits)
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"paired grid d={d} causal={causal} lens={list(L)}")


@pytest.mark.parametrize("slope", [0.02, 0.5, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_bias_rising_max(slope, causal):
    # a bias rising along the keys lifts every row's max block after block: by 64*slope per
    # 64-key block (natural units), i.e. below the lazy bound, within the in-register shift, and
    # beyond it (the block is then recomputed from K)
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 256, 640, 128
    ramp = (slope * np.arange(Nk, dtype=np.float32))[None, None, None, :]
    rows = np.linspace(0.0, 3.0, Nq, dtype=np.float32)[None, None, :, None]
    bits = I.bf16_bits_from_f32(np.broadcast_to(ramp + rows, (1, 1, Nq, Nk)))
    out, lse, O_ref, lse_ref = _prefill(B, Hq, Hkv, Nq, Nk, d, causal, 660, bias_bits=bits)
    # rows' LSE reach ~1300 at slope 2; the plain 1e-3 bound holds (measured at most 3.4e-4)
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"rising bias slope={slope} causal={causal}")


def test_prefill_bias_masked_rows():
    # rows whose every key is masked by a -inf bias: output 0 and lse -inf, like Nk = 0
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 2, 100, 128, 128
    b32 = I.bf16_bits_to_f32(I.draw_bias(630, 1, Hq, Nq, Nk, "normal"))
    b32[0, 0, 5, :] = -np.inf
    b32[0, 1, 70:90, :] = -np.inf
    b32[0, 1, 95, :64] = -np.inf  # the first block only
    bits = I.bf16_bits_from_f32(b32)
    out, lse, O_ref, lse_ref = _prefill(B, Hq, Hkv, Nq, Nk, d, False, 631, bias_bits=bits)
    assert np.all(out[0, 0, 5] == 0) and np.isneginf(lse[0, 0, 5])
    assert np.all(out[0, 1, 70:90] == 0) and np.all(np.isneginf(lse[0, 1, 70:90]))
    compare(out, lse, O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS, what="masked rows")


def test_prefill_bias_full_size_sampled():
    # the causal prefill workload (B=2, H=16, N=2048, d=128) with a padding-style bias shared by
    # the batch and heads, in the launch configuration of the benchmark; sampled rows
    w = I.WORKLOADS["prefill_causal_b2h16n2048"]
    x = w.draw()
    q, k, v = upload(x)
    bits = I.draw_bias(640, 1, 1, w.Nq, w.Nk, "normal", 1.0, 0.05)
    s32 = _s32(w.d)
    say("prefill bias full size, sampled rows")
    out, lse = fa.attn_fwd_ex(q, k, v, causal=True, scale=s32, bias=_bias(bits))
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, 1000, 1023, 1024, 2046, 2047} |
                           set(np.random.default_rng(641).integers(0, w.Nq, 16).tolist())))
    idx = torch.as_tensor(rows, device="cuda")
    O_ref, lse_ref = A.attention_rows_fp64(*x.as_f64(), s32, True, rows, bias=_bias64(bits))
    compare(to_f64(out[:, :, idx]), to_f64(lse[:, :, idx]), O_ref, lse_ref, BF16_MAX_ABS,
            BF16_MEAN_ABS, what="bias full size")


def _decode(B, Hq, Hkv, Nq, Nk, d, causal, S, seed, L=None, bias_bits=None):
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    s32 = _s32(d)
    bshape = None if bias_bits is None else bias_bits.shape
    say(f"decode_ex B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal} S={S} seed={seed} "
        f"lens={None if L is None else list(L)} bias={bshape}")
    out, lse, ws = fa.attn_decode_splitkv_ex(q, k, v, S, causal=causal, scale=s32,
                                             seqlens_k=None if L is None else _lens(L),
                                             bias=None if bias_bits is None else _bias(bias_bits))
    torch.cuda.synchronize()
    b64 = None if bias_bits is None else _bias64(bias_bits)
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), s32, causal, seqlens_k=L, bias=b64)
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"decode_ex B{B} Nq{Nq} Nk{Nk} S{S}")
    # per-split partials and (m, l) metadata against the oracle's split model
    f = ws.view(torch.float32)
    n = B * Hq * Nq * S
    O_s = to_f64(f[: n * d].view(B, Hq, Nq, S, d))
    ml = f[n * d: n * d + 2 * n].view(B, Hq, Nq, S, 2)
    m_s, l_s = to_f64(ml[..., 0]), to_f64(ml[..., 1])
    rO, rm, rl = A.splitkv_partials_fp64(*x.as_f64(), s32, causal, S, bias=b64, seqlens_k=L)
    empty = rl == 0
    assert np.array_equal(l_s == 0, empty), "empty-split pattern differs"
    assert np.all(np.isneginf(m_s[empty])) and np.all(O_s[empty] == 0)
    full = ~empty
    if full.any():
        tol = META_M_MAX_ABS + 4 * 2.0**-23 * np.abs(rm[full])
        assert np.all(np.abs(m_s[full] - rm[full]) <= tol)
        assert (np.abs(l_s[full] - rl[full]) / rl[full]).max() <= META_L_REL
        assert np.abs(O_s[full] - rO[full]).max() <= PARTIAL_MAX_ABS


# (B, Hq, Hkv, Nq, Nk capacity, d, causal, n_splits)
DECODE_VARLEN = [
    (4, 8, 2, 1, 1000, 128, True, 16),
    (4, 8, 2, 4, 1000, 128, True, 3),
    (5, 4, 4, 1, 300, 64, False, 7),
    (3, 32, 8, 4, 2048, 128, True, 1),
]


@pytest.mark.parametrize("case", DECODE_VARLEN, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_S{}".format(
    *c[:6], "causal" if c[6] else "full", c[7]))
def test_decode_varlen(case):
    B, Hq, Hkv, Nq, Nk, d, causal, S = case
    L = I.draw_seqlens(700 + Nk, B, Nk)
    _decode(B, Hq, Hkv, Nq, Nk, d, causal, S, 710 + Nk, L=L)


# (B, Hq, Hkv, Nq, Nk, d, causal, n_splits, bias_b, bias_h, kind, std, masked_frac)
DECODE_BIAS = [
    (2, 8, 2, 1, 1000, 128, True, 16, 1, 1, "normal", 1.0, 0.0),
    (2, 8, 2, 4, 1000, 128, True, 5, 2, 8, "normal", 4.0, 0.3),
    (3, 4, 1, 4, 512, 64, False, 4, 3, 1, "alibi", 0.0, 0.0),
    (1, 4, 4, 2, 64, 128, True, 64, 1, 4, "normal", 1.0, 0.5),
]


@pytest.mark.parametrize("case", DECODE_BIAS, ids=lambda c: "B{}_Hq{}_Nq{}_Nk{}_d{}_S{}_b{}x{}_{}_{}".format(
    c[0], c[1], c[3], c[4], c[5], c[7], c[8], c[9], c[10], c[12]))
def test_decode_bias(case):
    B, Hq, Hkv, Nq, Nk, d, causal, S, bb, bh, kind, std, frac = case
    bits = I.draw_bias(800 + Nk + S, bb, bh, Nq, Nk, kind, std, frac)
    _decode(B, Hq, Hkv, Nq, Nk, d, causal, S, 810 + Nk, bias_bits=bits)


def test_decode_full_size_varlen_and_bias():
    # the GQA decode workload (B=8, Hq=32, Hkv=8, Nq=4, KV capacity 8192, 16 splits) with a
    # length mix and a per-head bias with some masked keys
    w = I.WORKLOADS["decode_gqa_nq4"]
    L = I.draw_seqlens(900, w.B, w.Nk)
    bits = I.draw_bias(901, 1, w.Hq, w.Nq, w.Nk, "normal", 2.0, 0.02)
    _decode(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, True, w.n_splits, w.seed, L=L, bias_bits=bits)


@pytest.mark.parametrize("Nq", [1, 31, 32, 40])
def test_forward_routes_by_query_rows(Nq):
    # below 32 query rows attn_forward is the split-KV path with the library's split count,
    # from 32 on it is the prefill kernel: bit-identical to calling those directly
    B, Hq, Hkv, Nk, d = 2, 8, 2, 700, 128
    x = I.draw_qkv(950 + Nq, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    L = np.array([700, 333], np.int32)
    bits = I.draw_bias(951, B, 1, Nq, Nk, "normal")
    lens, bias = _lens(L), _bias(bits)
    say(f"attn_forward Nq={Nq}")
    out, lse, ws = fa.attn_forward(q, k, v, causal=True, seqlens_k=lens, bias=bias)
    if Nq < 32:
        S = fa.attn_decode_num_splits(B, Hq, Hkv, Nq, Nk)
        ref, lref, _ = fa.attn_decode_splitkv_ex(q, k, v, S, causal=True, seqlens_k=lens,
                                                 bias=bias)
        assert ws is not None and ws.numel() == fa.attn_forward_workspace_bytes(B, Hq, Hkv, Nq,
                                                                                 Nk, d)
    else:
        ref, lref = fa.attn_fwd_ex(q, k, v, causal=True, seqlens_k=lens, bias=bias)
        assert ws is None
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lref.view(torch.int32))
    O_ref, lse_ref = A.attention_fp64(*x.as_f64(), _s32(d), True, seqlens_k=L, bias=_bias64(bits))
    compare(to_f64(out), to_f64(lse), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what=f"attn_forward Nq={Nq}")


def test_invalid_extras_raise():
    q = torch.zeros((2, 4, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 2, 12, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="seqlens_k"):
        fa.attn_fwd_ex(q, k, k, seqlens_k=torch.zeros(3, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="seqlens_k"):
        fa.attn_fwd_ex(q, k, k, seqlens_k=torch.zeros(2, dtype=torch.int64, device="cuda"))
    bad = torch.zeros((3, 1, 8, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.AttentionError, match="bias"):
        fa.attn_fwd_ex(q, k, k, bias=bad)
    k10 = torch.zeros((2, 2, 10, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.AttentionError, match="multiple of 4"):
        fa.attn_decode_splitkv_ex(q, k10, k10, 2,
                                  bias=torch.zeros((1, 1, 8, 10), dtype=torch.bfloat16,
                                                   device="cuda"))
