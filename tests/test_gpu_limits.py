"""The longest key sequence the C ABI accepts, on the prefill and the split-KV decode paths.

At head dimension 128 one K or V head slice may hold at most 2^24 - 129 keys: the kernels address
a slice, plus one block of overrun, with 32-bit buffer offsets, and the ABI rejects anything
longer.  At that length the last key block is ragged (63 keys).  The fp64 oracle cannot
hold slices of 4 GiB, so these cases use a closed form that follows from the definition (the same
reasoning as the oracle pin for identical keys):

  every query row is c·e0 and every key is 0 except the last 64, which are β·e0, so a row's
  visible scores are 0 (n - m of them) and S = scale·c·β (m of them, m = the special keys it
  sees); its values are v0 for ordinary keys and v1 for the special ones.  Then
      LSE = ln((n - m) + m e^S),   O = ((n - m) v0 + m e^S v1) / ((n - m) + m e^S).

With S ≈ 12.7 the last 64 keys, at the far end of the 4 GiB slice, carry about half the weight
of a full row and the 16.7 million ordinary keys the other half, so special keys read from the
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

D = 128
NK_MAX = (1 << 24) - 129   # (Nk + 128) * d * 2 bytes must stay below 2^32
N_SPECIAL = 64
C_Q, BETA = 4.0, 36.0      # exact in bf16; S = scale·c·β ≈ 12.7
V0 = 0.5                   # ordinary values (exact)
V1 = -2.0                  # special values (exact)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


@pytest.fixture(scope="module")
def big_kv():
    say(f"allocating K and V with {NK_MAX} keys (2 x {NK_MAX * D * 2 / 2**30:.2f} GiB)")
    k = torch.zeros((1, 1, NK_MAX, D), dtype=torch.bfloat16, device="cuda")
    k[0, 0, NK_MAX - N_SPECIAL:, 0] = BETA
    v = torch.full((1, 1, NK_MAX, D), V0, dtype=torch.bfloat16, device="cuda")
    v[0, 0, NK_MAX - N_SPECIAL:, :] = V1
    torch.cuda.synchronize()
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def _expected(Nq, Hq, causal, scale):
    """Closed-form O [1, Hq, Nq, D] and LSE [1, Hq, Nq] in fp64."""
    S = float(np.float32(scale)) * C_Q * BETA
    off = NK_MAX - Nq
    O = np.empty((1, Hq, Nq, D))
    L = np.empty((1, Hq, Nq))
    for i in range(Nq):
        n = (i + off + 1) if causal else NK_MAX
        m = max(0, n - (NK_MAX - N_SPECIAL))
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
    Hq, Nq = 2, 128  # two query heads share the one K/V head
    q = torch.zeros((1, Hq, Nq, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = C_Q
    scale = 1.0 / math.sqrt(D)
    say(f"prefill Nq={Nq} Nk={NK_MAX} causal={causal}")
    out, lse = fa.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check(out, lse, *_expected(Nq, Hq, causal, scale), f"prefill causal={causal}")


@pytest.mark.parametrize("Nq", [1, 4])
def test_decode_at_the_maximum_key_length(big_kv, Nq):
    k, v = big_kv
    Hq = 4
    q = torch.zeros((1, Hq, Nq, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = C_Q
    scale = 1.0 / math.sqrt(D)
    say(f"decode Nq={Nq} Nk={NK_MAX} n_splits=16")
    out, lse, _ = fa.attn_decode_splitkv(q, k, v, 16, causal=True, scale=scale)
    torch.cuda.synchronize()
    _check(out, lse, *_expected(Nq, Hq, True, scale), f"decode Nq={Nq}")


def test_one_more_key_is_rejected():
    # the ABI's limit, checked without allocating: one key more is refused
    lib = fa.load()
    q = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16, device="cuda")
    rc = lib.attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), None, 1, 1, 1, 1,
                      NK_MAX + 1, D, 0.0, 1, None)
    assert rc == -2  # ATTN_ERR_SHAPE, before anything is launched
