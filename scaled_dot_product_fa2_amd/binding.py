"""ctypes binding of ``libsdpa_fa2.so`` (C ABI in ``include/sdpa_fa2.h``).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no fallback: if the library is
missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsdpa_fa2.so")

ATTN_OK = 0
_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None

_c_int, _c_float, _vp, _c_size = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_SIGNATURES = {
    "attn_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "attn_fwd_f32": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "attn_decode_workspace_bytes": (_c_size, [_c_int] * 5),
    "attn_decode_splitkv": (_c_int, [_vp] * 6 + [_c_size] + [_c_int] * 6 +
                            [_c_float, _c_int, _c_int, _vp]),
    "attn_fwd_ex": (_c_int, [_vp] * 5 + [_vp, _vp, _c_int, _c_int] + [_c_int] * 6 +
                    [_c_float, _c_int, _vp]),
    "attn_decode_splitkv_ex": (_c_int, [_vp] * 6 + [_c_size] + [_vp, _vp, _c_int, _c_int] +
                               [_c_int] * 6 + [_c_float, _c_int, _c_int, _vp]),
    "attn_decode_splitkv_noalloc": (_c_int, [_vp] * 5 + [_c_int] * 6 +
                                    [_c_float, _c_int, _c_int, _vp]),
    "attn_decode_num_splits": (_c_int, [_c_int] * 5),
    "attn_forward_workspace_bytes": (_c_size, [_c_int] * 6),
    "attn_forward": (_c_int, [_vp] * 6 + [_c_size] + [_vp, _vp, _c_int, _c_int] + [_c_int] * 6 +
                     [_c_float, _c_int, _vp]),
    "attn_bwd_workspace_bytes": (_c_size, [_c_int] * 3),
    "attn_bwd": (_c_int, [_vp] * 10 + [_c_size] + [_c_int] * 6 + [_c_float, _c_int, _vp]),
    "attn_bwd_ex": (_c_int, [_vp] * 10 + [_c_size] + [_vp, _vp, _c_int, _c_int] + [_c_int] * 6 +
                    [_c_float, _c_int, _vp]),
    "attn_status_string": (ctypes.c_char_p, [_c_int]),
}
EXPORTED = tuple(_SIGNATURES)


class AttentionError(RuntimeError):
    pass


def hip_runtimes_mapped():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return sorted(paths)


def load(path: str = LIB_PATH, require_single_runtime: bool = True) -> ctypes.CDLL:
    """Load the library once.  torch is imported first so that the library binds to the HIP
    runtime torch already mapped (both carry the SONAME libamdhip64.so.7)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        import torch  # noqa: F401  (maps torch's HIP runtime before ours is resolved)

        if not os.path.exists(path):
            raise AttentionError(
                f"HIP attention library not found at {path}; build it with "
                "`python -m scaled_dot_product_fa2_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        rts = hip_runtimes_mapped()
        if require_single_runtime and len(rts) > 1:
            raise AttentionError(f"two HIP runtimes are mapped into this process: {rts}")
        _lib = lib
        return lib


def status_string(rc: int) -> str:
    return load().attn_status_string(rc).decode()


def _check_rc(rc: int, what: str):
    if rc != ATTN_OK:
        raise AttentionError(f"{what}: {status_string(rc)} (status {rc})")


def _ptr(t) -> Optional[int]:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _validate(q, k, v, dtype):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, heads, seq, head_dim]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, Hq, Nq, d = q.shape
    return B, Hq, k.shape[1], Nq, k.shape[2], d


def _check_like(name, t, shape, dtype, device):
    """A caller-supplied output or workspace must match exactly what the kernels will write."""
    import torch

    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape) or
            t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on "
                         f"{device}")
    return t


def _out_lse(q, B, Hq, Nq, out, lse, want_lse):
    """The output and logsumexp tensors: allocated when not given, checked when given."""
    import torch

    out = torch.empty_like(q) if out is None else _check_like("out", out, q.shape, q.dtype,
                                                              q.device)
    if lse is None:
        if want_lse:
            lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    else:
        lse = _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    return out, lse


def _check_workspace(workspace, device):
    import torch

    if (not isinstance(workspace, torch.Tensor) or workspace.device != device or
            not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return workspace


def _extras(q, B, Hq, Nq, Nk, seqlens_k, bias):
    """Marshal the optional per-batch key lengths (int32 [B]) and bias (bf16 [1|B, 1|Hq, Nq, Nk])
    into (seqlens_ptr, bias_ptr, bias_b, bias_h); shape rules beyond these are the library's."""
    import torch

    sp = None
    if seqlens_k is not None:
        if (not isinstance(seqlens_k, torch.Tensor) or seqlens_k.dtype != torch.int32 or
                seqlens_k.device != q.device or tuple(seqlens_k.shape) != (B,) or
                not seqlens_k.is_contiguous()):
            raise ValueError(f"seqlens_k must be a contiguous int32 [{B}] tensor on {q.device}")
        sp = seqlens_k.data_ptr()
    if bias is None:
        return sp, None, 1, 1
    if (not isinstance(bias, torch.Tensor) or bias.dtype != torch.bfloat16 or
            bias.device != q.device or bias.dim() != 4 or not bias.is_contiguous() or
            tuple(bias.shape[2:]) != (Nq, Nk)):
        raise ValueError(f"bias must be a contiguous bf16 [1|B, 1|Hq, {Nq}, {Nk}] tensor on "
                         f"{q.device}")
    return sp, _ptr(bias), int(bias.shape[0]), int(bias.shape[1])


def attn_fwd(q, k, v, causal: bool = True, scale: float = 0.0, out=None, lse=None,
             want_lse: bool = True) -> Tuple[object, object]:
    """Fused attention forward on bf16 [B,H,N,d] tensors; returns (out bf16, lse fp32 or None)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    rc = load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                         float(scale), int(bool(causal)), _stream(q.device))
    _check_rc(rc, "attn_fwd")
    return out, lse


def attn_fwd_ex(q, k, v, causal: bool = True, scale: float = 0.0, seqlens_k=None, bias=None,
                out=None, lse=None, want_lse: bool = True):
    """``attn_fwd`` with optional per-batch key lengths (int32 [B] on the device) and an additive
    bf16 bias [1|B, 1|Hq, Nq, Nk]; returns (out, lse)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    sp, bp, bb, bh = _extras(q, B, Hq, Nq, Nk, seqlens_k, bias)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    rc = load().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), sp, bp, bb, bh, B, Hq,
                            Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream(q.device))
    _check_rc(rc, "attn_fwd_ex")
    return out, lse


def attn_fwd_f32(q, k, v, causal: bool = True, scale: float = 0.0, out=None, lse=None,
                 want_lse: bool = True):
    """The same on float32 tensors (fp32 arithmetic throughout)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.float32)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    rc = load().attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq,
                             Nk, d, float(scale), int(bool(causal)), _stream(q.device))
    _check_rc(rc, "attn_fwd_f32")
    return out, lse


def attn_decode_workspace_bytes(B: int, Hq: int, Nq: int, d: int, n_splits: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits))


def attn_decode_splitkv(q, k, v, n_splits: int, causal: bool = True, scale: float = 0.0,
                        out=None, lse=None, workspace=None, want_lse: bool = True):
    """Split-KV decode on bf16 tensors; returns (out, lse, workspace).

    ``workspace`` (a uint8 CUDA tensor of at least ``attn_decode_workspace_bytes`` bytes) may be
    passed in to reuse memory; it then holds the fp32 partials [B,Hq,Nq,S,d] followed by the
    (m, l) metadata [B,Hq,Nq,S,2].
    """
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    need = attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits) if n_splits >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    rc = load().attn_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                    int(n_splits), _stream(q.device))
    _check_rc(rc, "attn_decode_splitkv")
    return out, lse, workspace


def attn_decode_splitkv_ex(q, k, v, n_splits: int, causal: bool = True, scale: float = 0.0,
                           seqlens_k=None, bias=None, out=None, lse=None, workspace=None,
                           want_lse: bool = True):
    """``attn_decode_splitkv`` with optional per-batch key lengths and bias; returns
    (out, lse, workspace)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    sp, bp, bb, bh = _extras(q, B, Hq, Nq, Nk, seqlens_k, bias)
    need = attn_decode_workspace_bytes(B, Hq, Nq, d, n_splits) if n_splits >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    rc = load().attn_decode_splitkv_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                       _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), sp, bp, bb,
                                       bh, B, Hq, Hkv, Nq, Nk, d, float(scale),
                                       int(bool(causal)), int(n_splits), _stream(q.device))
    _check_rc(rc, "attn_decode_splitkv_ex")
    return out, lse, workspace


def attn_decode_splitkv_noalloc(q, k, v, n_splits: int, causal: bool = True, scale: float = 0.0,
                                out=None, lse=None, want_lse: bool = True):
    """Split-KV decode through the entry point that allocates nothing (its partials live in the
    library's fixed device scratch); returns (out, lse).  Pass ``out`` (and ``lse``) to keep the
    whole call free of allocations."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    rc = load().attn_decode_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B,
                                            Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                            int(n_splits), _stream(q.device))
    _check_rc(rc, "attn_decode_splitkv_noalloc")
    return out, lse


def attn_decode_num_splits(B: int, Hq: int, Hkv: int, Nq: int, Nk: int) -> int:
    return int(load().attn_decode_num_splits(B, Hq, Hkv, Nq, Nk))


def attn_forward_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().attn_forward_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))


def attn_forward(q, k, v, causal: bool = True, scale: float = 0.0, seqlens_k=None, bias=None,
                 out=None, lse=None, workspace=None, want_lse: bool = True):
    """One call for any query length: split-KV below 32 query rows, the prefill kernel otherwise
    (the library decides); returns (out, lse, workspace)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    sp, bp, bb, bh = _extras(q, B, Hq, Nq, Nk, seqlens_k, bias)
    need = attn_forward_workspace_bytes(B, Hq, Hkv, Nq, Nk, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_workspace(workspace, q.device)
    out, lse = _out_lse(q, B, Hq, Nq, out, lse, want_lse)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().attn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
                             ws_bytes, sp, bp, bb, bh, B, Hq, Hkv, Nq, Nk, d, float(scale),
                             int(bool(causal)), _stream(q.device))
    _check_rc(rc, "attn_forward")
    return out, lse, workspace


def attn_bwd(q, k, v, out, lse, dout, causal: bool = True, scale: float = 0.0, dq=None, dk=None,
             dv=None, workspace=None, seqlens_k=None, bias=None):
    """Gradients (dq, dk, dv) of the forward on bf16 [B,H,N,d] tensors (d 64 or 128), given the
    forward's output and logsumexp and the gradient ``dout`` of the loss w.r.t. the output.  With
    ``seqlens_k`` and / or ``bias`` (as for ``attn_fwd_ex``) it is the backward of the forward
    with those extras (``attn_bwd_ex``; no gradient is taken for the bias)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    for name, t, dt in (("out", out, torch.bfloat16), ("dout", dout, torch.bfloat16)):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or t.shape != q.shape or \
                not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous {dt} tensor shaped like q")
    if (not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or
            tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be the forward's contiguous float32 [B, Hq, Nq] logsumexp")
    dq = torch.empty_like(q) if dq is None else _check_like("dq", dq, q.shape, q.dtype, q.device)
    dk = torch.empty_like(k) if dk is None else _check_like("dk", dk, k.shape, k.dtype, q.device)
    dv = torch.empty_like(v) if dv is None else _check_like("dv", dv, v.shape, v.dtype, q.device)
    need = attn_bwd_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size())
    tail = (B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream(q.device))
    if seqlens_k is None and bias is None:
        rc = load().attn_bwd(*head, *tail)
    else:
        rc = load().attn_bwd_ex(*head, *_extras(q, B, Hq, Nq, Nk, seqlens_k, bias), *tail)
    _check_rc(rc, "attn_bwd")
    return dq, dk, dv


def attn_bwd_workspace_bytes(B: int, Hq: int, Nq: int) -> int:
    return int(load().attn_bwd_workspace_bytes(B, Hq, Nq))


def prepare_bwd(q, k, v, out, lse, dout, dq, dk, dv, workspace, causal: bool = True,
                scale: float = 0.0, seqlens_k=None, bias=None):
    """A zero-argument callable that enqueues ``attn_bwd`` (``attn_bwd_ex`` with
    ``seqlens_k`` or ``bias``) with these tensors (timing loops)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    for name, t, ref in (("out", out, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k),
                         ("dv", dv, v)):
        _check_like(name, t, ref.shape, ref.dtype, q.device)
    _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    _check_workspace(workspace, q.device)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size())
    tail = (B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream(q.device))
    if seqlens_k is None and bias is None:
        fn, args = load().attn_bwd, head + tail
    else:
        fn = load().attn_bwd_ex
        args = head + tuple(_extras(q, B, Hq, Nq, Nk, seqlens_k, bias)) + tail

    def call():
        rc = fn(*args)
        if rc != ATTN_OK:
            _check_rc(rc, "attn_bwd")
    return call


def prepare_fwd(q, k, v, out, lse=None, causal: bool = True, scale: float = 0.0, seqlens_k=None,
                bias=None):
    """A zero-argument callable that enqueues ``attn_fwd`` (``attn_fwd_ex`` when extras are
    given) with these tensors on the current stream, with every argument marshalled once up
    front (for timing loops)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    _check_like("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    tail = (B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream(q.device))
    if seqlens_k is None and bias is None:
        fn, name = load().attn_fwd, "attn_fwd"
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)) + tail
    else:
        fn, name = load().attn_fwd_ex, "attn_fwd_ex"
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                *_extras(q, B, Hq, Nq, Nk, seqlens_k, bias)) + tail

    def call():
        rc = fn(*args)
        if rc != ATTN_OK:
            _check_rc(rc, name)
    return call


def prepare_decode(q, k, v, n_splits: int, out, lse, workspace, causal: bool = True,
                   scale: float = 0.0, seqlens_k=None, bias=None):
    """The same for ``attn_decode_splitkv`` (``attn_decode_splitkv_ex`` with extras)."""
    import torch

    B, Hq, Hkv, Nq, Nk, d = _validate(q, k, v, torch.bfloat16)
    _check_like("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        _check_like("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    _check_workspace(workspace, q.device)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    tail = (B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), int(n_splits),
            _stream(q.device))
    if seqlens_k is None and bias is None:
        fn, name, args = load().attn_decode_splitkv, "attn_decode_splitkv", head + tail
    else:
        fn, name = load().attn_decode_splitkv_ex, "attn_decode_splitkv_ex"
        args = head + tuple(_extras(q, B, Hq, Nq, Nk, seqlens_k, bias)) + tail

    def call():
        rc = fn(*args)
        if rc != ATTN_OK:
            _check_rc(rc, name)
    return call
