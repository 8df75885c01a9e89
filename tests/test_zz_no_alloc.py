"""The decode entry point that allocates nothing (attn_decode_splitkv_noalloc), on the GPU.

It runs the kernels of attn_decode_splitkv with the split partials in the library's fixed device
scratch instead of a caller workspace, so its outputs must equal attn_decode_splitkv's bit for
bit: checked on two calls in a row, the second on a smaller problem (the scratch keeps the first
call's contents), then once more on the first problem, plus the size limit.  Every call goes
through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import BF16_MAX_ABS, BF16_MEAN_ABS, compare, say, to_f64, upload  # noqa: E402
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


def _s32(d):
    return float(np.float32(1.0 / np.sqrt(d)))


def _both(B, Hq, Hkv, Nq, Nk, d, S, causal, seed):
    x = I.draw_qkv(seed, B, Hq, Hkv, Nq, Nk, d)
    q, k, v = upload(x)
    say(f"noalloc decode B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} S{S} causal={causal} seed={seed}")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), device=q.device)
    fa.attn_decode_splitkv_noalloc(q, k, v, S, causal=causal, scale=_s32(d), out=out, lse=lse)
    ref_out, ref_lse, _ = fa.attn_decode_splitkv(q, k, v, S, causal=causal, scale=_s32(d))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "lse differs"
    return x, out, lse


def test_noalloc_equals_workspace_entry_point_twice_then_smaller():
    # the GQA decode workload at Nq = 4 (8.5 MB of partials), then a smaller problem with other
    # shapes and split count, then the first again
    first = (8, 32, 8, 4, 8192, 128, 16, True, 5)
    second = (2, 8, 2, 3, 1000, 64, 7, True, 77)
    x, out, lse = _both(*first)
    _both(*first)
    x2, out2, lse2 = _both(*second)
    O_ref, lse_ref = A.attention_fp64(*x2.as_f64(), _s32(64), True)
    compare(to_f64(out2), to_f64(lse2), O_ref, lse_ref, BF16_MAX_ABS, BF16_MEAN_ABS,
            what="noalloc second call vs oracle")
    _both(*first)


def test_noalloc_size_limit():
    # partials beyond the 32 MiB scratch are refused before anything is enqueued
    B, Hq, Hkv, Nq, Nk, d, S = 8, 32, 8, 16, 8192, 128, 16  # 34,078,720 bytes
    assert fa.attn_decode_workspace_bytes(B, Hq, Nq, d, S) > 32 << 20
    q = torch.zeros((B, Hq, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    say("noalloc size limit")
    with pytest.raises(fa.AttentionError, match="scratch"):
        fa.attn_decode_splitkv_noalloc(q, k, k, S, out=out)
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all()), "a refused call wrote its output"
    # the largest split count that fits still runs
    S2 = 15  # 31,948,800 bytes
    assert fa.attn_decode_workspace_bytes(B, Hq, Nq, d, S2) <= 32 << 20
    fa.attn_decode_splitkv_noalloc(q, k, k, S2, out=out)
    torch.cuda.synchronize()
    assert bool((out.float() == 0).all())
