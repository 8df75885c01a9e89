"""The library under HIP graph capture: forward, backward and split-KV decode enqueued into one
captured graph (through torch's graph API on the current stream), replayed several times with
eager work and synchronisations in between, every replay bit-identical to the eager results.

The library only enqueues kernels on the caller's stream (it allocates, frees, copies and
synchronises nothing), so its calls can be captured; this checks that the captured kernels
read their inputs and write their outputs afresh on each replay."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import say  # noqa: E402
from scaled_dot_product_fa2_amd import binding as fa  # noqa: E402
from scaled_dot_product_fa2_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    fa.load()
    yield


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replay_matches_eager():
    say("graph capture of forward + backward + decode")
    x = I.draw_qkv(5000, 2, 8, 2, 384, 384, 128)
    q, k, v = (I.to_device(a, "bf16") for a in (x.q, x.k, x.v))
    dout = I.to_device(I.draw_grad(5001, (2, 8, 384, 128)), "bf16")
    xd = I.draw_qkv(5002, 2, 8, 2, 4, 2000, 128)
    qd, kd, vd = (I.to_device(a, "bf16") for a in (xd.q, xd.k, xd.v))

    # outputs and workspaces allocated once, outside the graph
    out, lse = torch.empty_like(q), torch.empty((2, 8, 384), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa.attn_bwd_workspace_bytes(2, 8, 384), dtype=torch.uint8, device="cuda")
    outd = torch.empty_like(qd)
    lsed = torch.empty((2, 8, 4), dtype=torch.float32, device="cuda")
    dws = torch.empty(fa.attn_decode_workspace_bytes(2, 8, 4, 128, 8), dtype=torch.uint8,
                      device="cuda")

    def run():
        fa.attn_fwd(q, k, v, causal=True, out=out, lse=lse)
        fa.attn_bwd(q, k, v, out, lse, dout, causal=True, dq=dq, dk=dk, dv=dv, workspace=bws)
        fa.attn_decode_splitkv(qd, kd, vd, 8, causal=True, out=outd, lse=lsed, workspace=dws)

    # eager reference
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv, outd, lsed)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream, as torch asks
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    for rep in range(4):
        # poison every output between replays, with eager work in between
        for t in (out, lse, dq, dk, dv, outd, lsed):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv", "decode out", "decode lse"),
                              (out, lse, dq, dk, dv, outd, lsed), ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: {name} differs from eager"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays
    # inputs changed in place are picked up by the next replay
    q.copy_(torch.flip(q, dims=[2]))
    g.replay()
    torch.cuda.synchronize()
    o2, l2 = fa.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(o2)) and torch.equal(_bits(lse), _bits(l2))
    assert np.isfinite(ref[0].float().cpu().numpy()).all()
