"""The longest key sequence the C ABI accepts, on the prefill and the split-KV decode paths.

One K or V head slice may hold at most 2^32 / (2 d) - 129 keys (2^24 - 129 at head dimension
128, 2^25 - 129 at 64): the kernels address a slice, plus one block of overrun, with 32-bit
buffer offsets, and the ABI rejects anything longer.  At that length the last key block is
ragged.  The fp64 oracle cannot hold slices of 4 GiB, so these cases use a closed form that
follows from the definition (the same reasoning as the oracle pin for identical keys):

  every query row is c·e0 and every key is 0 except the last 64, which are β·e0, so a row's
  visible scores are 0 (n - m of them) and S = scale·c·β (m of them, m = the special keys it
  sees); its values are v0 for ordinary keys and v1 for the special ones.  Then
      LSE = ln((n - m) + m e^S),   O = ((n - m) v0 + m e^S v1) / ((n - m) + m e^S).

With S ≈ 13 the last 64 keys, at the far end of the 4 GiB slice, carry about half the weight of
a full row and the millions of ordinary keys the other half, so special keys read from the
wrong place or as zero, or ordinary keys miscounted by a few percent, move O or LSE outside the
tolerance.  The jump of the running max in the last block also exercises the in-register
rescale."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, LSE_MAX_ABS, say, to_f64  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402

pytestmark = pytest.mark.gpu

HEAD_DIMS = (128, 64)


def beta(d):
    # exact in bf16; S = scale·c·β ≈ 12.7 (d = 128) or 13 (d = 64), so ordinary and special keys
    # carry weight of the same order
    return 36.0 if d == 128 else 26.0


def nk_max(d):
    return (1 << 32) // (2 * d) - 129  # (Nk + 128) * d * 2 bytes must stay below 2^32

N_SPECIAL = 64
C_Q = 4.0                  # exact in bf16
V0 = 0.5                   # ordinary values (exact)
V1 = -2.0                  # special values (exact)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


@pytest.fixture(scope="module", params=HEAD_DIMS, ids=lambda d: f"d{d}")
def big_kv(request):
    D = request.param
    NK = nk_max(D)
    say(f"allocating K and V with {NK} keys at d = {D} (2 x {NK * D * 2 / 2**30:.2f} GiB)")
    k = torch.zeros((1, 1, NK, D), dtype=torch.bfloat16, device="cuda")
    k[0, 0, NK - N_SPECIAL:, 0] = beta(D)
    v = torch.full((1, 1, NK, D), V0, dtype=torch.bfloat16, device="cuda")
    v[0, 0, NK - N_SPECIAL:, :] = V1
    torch.cuda.synchronize()
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def _expected(Nq, Hq, causal, scale, NK, D):
    """Closed-form O [1, Hq, Nq, D] and LSE [1, Hq, Nq] in fp64."""
    S = float(np.float32(scale)) * C_Q * beta(D)
    off = NK - Nq
    O = np.empty((1, Hq, Nq, D))
    L = np.empty((1, Hq, Nq))
    for i in range(Nq):
        n = (i + off + 1) if causal else NK
        m = max(0, n - (NK - N_SPECIAL))
        w_sp = m * math.exp(S)
        den = (n - m) + w_sp
        O[0, :, i, :] = ((n - m) * V0 + w_sp * V1) / den
        L[0, :, i] = math.log(den)
    return O, L


def _check(out, lse, O_ref, L_ref, what):
    o, l = to_f64(out), to_f64(lse)
    err = np.abs(o - O_ref)
    lerr = float(np.abs(l - L_ref).max())
    say(f"  {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} lse={lerr:.3e}")
    assert float(err.max()) <= BF16_MAX_ABS and float(err.mean()) <= BF16_MEAN_ABS, what
    assert lerr <= LSE_MAX_ABS, what


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_prefill_at_the_maximum_key_length(big_kv, causal):
    k, v = big_kv
    NK, D = k.shape[2], k.shape[3]
    Hq, Nq = 2, 128  # two query heads share the one K/V head
    q = torch.zeros((1, Hq, Nq, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = C_Q
    scale = 1.0 / math.sqrt(D)
    say(f"prefill Nq={Nq} Nk={NK} d={D} causal={causal}")
    out, lse = fa.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check(out, lse, *_expected(Nq, Hq, causal, scale, NK, D), f"prefill d={D} causal={causal}")


@pytest.mark.parametrize("Nq", [1, 4])
def test_decode_at_the_maximum_key_length(big_kv, Nq):
    k, v = big_kv
    NK, D = k.shape[2], k.shape[3]
    Hq = 4
    q = torch.zeros((1, Hq, Nq, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = C_Q
    scale = 1.0 / math.sqrt(D)
    say(f"decode Nq={Nq} Nk={NK} d={D} n_splits=16")
    out, lse, _ = fa.attn_decode_splitkv(q, k, v, 16, causal=True, scale=scale)
    torch.cuda.synchronize()
    _check(out, lse, *_expected(Nq, Hq, True, scale, NK, D), f"decode d={D} Nq={Nq}")


@pytest.mark.parametrize("D", HEAD_DIMS)
def test_one_more_key_is_rejected(D):
    # the ABI's limit, checked without allocating: one key more is refused
    lib = fa.load()
    q = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16, device="cuda")
    rc = lib.attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), None, 1, 1, 1, 1,
                      nk_max(D) + 1, D, 0.0, 1, None)
    assert rc == -2  # ATTN_ERR_SHAPE, before anything is launched


def test_backward_at_the_maximum_key_length(big_kv):
    """Gradients at the longest accepted key length (GQA: two query heads, one K/V head; Nq = 64
    causal, so row i sees every ordinary key and the first i + 1 special keys).  With dO = g·1
    every head contributes the same, and the chain rule of the closed form gives, per row i
    (P_ord = 1/den_i, P_sp = E/den_i, E = e^S, dP = d g v, D_i = d g O_i):
        dV_j = 2 g Σ_i P_ij,   dK_j = 2 scale c e0 Σ_i P_ij (dP_j - D_i),
        dQ_i = scale β e0 Σ_{special j ≤ i + off} P_ij (dP_j - D_i).
    The millions of ordinary keys must all get bit-identical gradients (checked on the GPU);
    one of them, every special key and every dQ row are compared with the closed form."""
    k, v = big_kv
    NK, D = k.shape[2], k.shape[3]
    Hq, Nq, g = 2, 64, 0.25
    q = torch.zeros((1, Hq, Nq, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = C_Q
    dout = torch.full((1, Hq, Nq, D), g, dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(D)
    s32 = float(np.float32(scale))
    say(f"backward Nq={Nq} Nk={NK} d={D}")
    out, lse = fa.attn_fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.attn_bwd(q, k, v, out, lse, dout, causal=True, scale=scale)
    torch.cuda.synchronize()

    # closed form, fp64
    E = math.exp(s32 * C_Q * beta(D))
    n_ord = NK - N_SPECIAL
    i = np.arange(Nq)
    m = i + 1                                   # special keys row i sees
    den = n_ord + m * E
    O = (n_ord * V0 + m * E * V1) / den
    Drow = D * g * O
    dp_ord, dp_sp = D * g * V0, D * g * V1
    dv_ord = Hq * g * np.sum(1.0 / den)
    dk_ord = Hq * s32 * C_Q * np.sum((dp_ord - Drow) / den)
    sp = np.arange(N_SPECIAL)                   # special key s is seen by rows i >= s
    vis = i[None, :] >= sp[:, None]
    dv_sp = Hq * g * np.sum(np.where(vis, E / den[None, :], 0.0), axis=1)
    dk_sp = Hq * s32 * C_Q * np.sum(np.where(vis, E * (dp_sp - Drow[None, :]) / den[None, :], 0.0),
                                    axis=1)
    dq0 = s32 * beta(D) * m * E * (dp_sp - Drow) / den   # the same for both heads

    # every ordinary key: identical gradients, dK only in dimension 0
    ordv = dv[0, 0, :n_ord]  # bf16 views: min / max compare bits exactly without copies
    ordk = dk[0, 0, :n_ord]
    assert float(ordv.min()) == float(ordv.max()), "ordinary keys' dV differ"
    assert float(ordk[:, 0].min()) == float(ordk[:, 0].max()), "ordinary keys' dK differ"
    assert float(ordk[:, 1:].abs().max()) == 0.0
    got_v, got_k = float(ordv[0, 0]), float(ordk[0, 0])
    say(f"  ordinary dV {got_v:.6e} vs {dv_ord:.6e}, dK {got_k:.6e} vs {dk_ord:.6e}")
    assert abs(got_v - dv_ord) <= 2e-2 * abs(dv_ord)
    assert abs(got_k - dk_ord) <= 2e-2 * abs(dk_ord) + 1e-9

    # the special keys and dQ, row by row (relative to each tensor's largest value)
    gv = to_f64(dv[0, 0, n_ord:])
    gk = to_f64(dk[0, 0, n_ord:])
    gq = to_f64(dq[0])
    for name, got, ref in (("dV special", gv, np.repeat(dv_sp[:, None], D, axis=1)),
                           ("dK special", gk[:, 0], dk_sp),
                           ("dQ", gq[:, :, 0], np.broadcast_to(dq0, (Hq, Nq)))):
        scale_ref = float(np.abs(ref).max())
        err = float(np.abs(got - ref).max()) / scale_ref
        say(f"  {name}: max|ref|={scale_ref:.3e} max_rel={err:.3e}")
        assert err <= 2e-2, name
    assert float(np.abs(gk[:, 1:]).max()) == 0.0 and float(np.abs(gq[:, :, 1:]).max()) == 0.0
