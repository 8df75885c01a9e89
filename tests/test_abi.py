"""The C-ABI library on the CPU: it loads, exports every symbol the header declares, and rejects
invalid arguments with the documented status codes before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from scaled_dot_product_fa2_amd import binding as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa_fa2.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from scaled_dot_product_fa2_amd import build

        build.build()
    return fa.load()


def _header():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    return re.findall(r"SDPA_FA2_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", _header())


def _status_codes():
    return {name: int(val) for name, val in re.findall(r"(ATTN_\w+)\s*=\s*(-?\d+)", _header())}


def test_every_declared_symbol_is_exported(lib):
    declared = _declared_functions()
    assert sorted(declared) == sorted(fa.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_only_the_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {fa.LIB_PATH}").read()
    text = [ln.split()[-1] for ln in out.splitlines() if " T " in ln]
    assert sorted(text) == sorted(fa.EXPORTED)


def test_one_hip_runtime(lib):
    assert len(fa.hip_runtimes_mapped()) == 1


def test_status_strings(lib):
    codes = _status_codes()
    assert codes["ATTN_OK"] == 0 and len(set(codes.values())) == len(codes)
    for name, val in codes.items():
        s = fa.status_string(val)
        assert s and s != "unknown status", name
    assert fa.status_string(12345) == "unknown status"


def test_workspace_bytes(lib):
    assert lib.attn_decode_workspace_bytes(8, 32, 4, 128, 16) == 8 * 32 * 4 * 16 * 130 * 4
    assert lib.attn_decode_workspace_bytes(8, 32, 1, 64, 3) == 8 * 32 * 1 * 3 * 66 * 4
    assert lib.attn_decode_workspace_bytes(-1, 32, 1, 64, 3) == 0
    assert lib.attn_decode_workspace_bytes(2**30, 2**30, 2**30, 128, 2**30) == 0  # overflow


C = _status_codes()
A16 = 0x10000  # a fake, 16-byte-aligned address: never dereferenced, every case below fails first
GOOD = dict(B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=128, scale=0.0, causal=1)


def _fwd(lib, q=A16, k=A16, v=A16, o=A16, lse=None, f32=False, **kw):
    a = {**GOOD, **kw}
    fn = lib.attn_fwd_f32 if f32 else lib.attn_fwd
    return fn(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
              a["scale"], a["causal"], None)


def _dec(lib, q=A16, k=A16, v=A16, o=A16, lse=None, ws=A16, ws_bytes=1 << 40, S=2, **kw):
    a = {**GOOD, **kw}
    return lib.attn_decode_splitkv(q, k, v, o, lse, ws, ws_bytes, a["B"], a["Hq"], a["Hkv"],
                                   a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], S, None)


@pytest.mark.parametrize("f32", [False, True])
def test_forward_validation(lib, f32):
    assert _fwd(lib, f32=f32, B=-1) == C["ATTN_ERR_SHAPE"]
    assert _fwd(lib, f32=f32, Nk=-5) == C["ATTN_ERR_SHAPE"]
    assert _fwd(lib, f32=f32, Nq=1 << 30) == C["ATTN_ERR_SHAPE"]
    assert _fwd(lib, f32=f32, d=96) == C["ATTN_ERR_HEADDIM"]
    assert _fwd(lib, f32=f32, d=256) == C["ATTN_ERR_HEADDIM"]
    assert _fwd(lib, f32=f32, Hq=3) == C["ATTN_ERR_GQA"]
    assert _fwd(lib, f32=f32, Hkv=0) == C["ATTN_ERR_GQA"]
    assert _fwd(lib, f32=f32, scale=float("nan")) == C["ATTN_ERR_SCALE"]
    assert _fwd(lib, f32=f32, scale=float("inf")) == C["ATTN_ERR_SCALE"]
    assert _fwd(lib, f32=f32, scale=-0.5) == C["ATTN_ERR_SCALE"]
    # positive scales below 2^-32 (subnormals among them) are refused: 1/scale must stay finite
    # for the bias, which the kernels carry in units of the unscaled dot product
    assert _fwd(lib, f32=f32, scale=2.0**-33) == C["ATTN_ERR_SCALE"]
    assert _fwd(lib, f32=f32, scale=1e-45) == C["ATTN_ERR_SCALE"]
    assert _fwd(lib, f32=f32, scale=2.0**-32, lse=A16 + 2) == C["ATTN_ERR_ALIGN"]  # accepted
    assert _fwd(lib, f32=f32, q=None) == C["ATTN_ERR_NULL"]
    assert _fwd(lib, f32=f32, o=None) == C["ATTN_ERR_NULL"]
    assert _fwd(lib, f32=f32, k=None) == C["ATTN_ERR_NULL"]
    assert _fwd(lib, f32=f32, q=A16 + 8) == C["ATTN_ERR_ALIGN"]
    assert _fwd(lib, f32=f32, v=A16 + 2) == C["ATTN_ERR_ALIGN"]
    assert _fwd(lib, f32=f32, lse=A16 + 2) == C["ATTN_ERR_ALIGN"]
    # empty problems succeed without touching anything (NULL pointers allowed)
    assert _fwd(lib, f32=f32, q=None, k=None, v=None, o=None, B=0) == C["ATTN_OK"]
    assert _fwd(lib, f32=f32, q=None, k=None, v=None, o=None, Nq=0) == C["ATTN_OK"]
    assert _fwd(lib, f32=f32, q=None, k=None, v=None, o=None, Hq=0, Hkv=0) == C["ATTN_OK"]


def test_decode_validation(lib):
    assert _dec(lib, S=0) == C["ATTN_ERR_SPLITS"]
    assert _dec(lib, S=9) == C["ATTN_ERR_SPLITS"]           # more splits than keys
    assert _dec(lib, S=2, Nk=0, k=None, v=None) == C["ATTN_ERR_SPLITS"]
    assert _dec(lib, ws=None) == C["ATTN_ERR_WORKSPACE"]
    need = lib.attn_decode_workspace_bytes(1, 4, 8, 128, 2)
    assert _dec(lib, ws_bytes=need - 1) == C["ATTN_ERR_WORKSPACE"]
    assert _dec(lib, ws=A16 + 4) == C["ATTN_ERR_ALIGN"]
    assert _dec(lib, d=80) == C["ATTN_ERR_HEADDIM"]
    assert _dec(lib, Hq=6, Hkv=4) == C["ATTN_ERR_GQA"]
    assert _dec(lib, q=None) == C["ATTN_ERR_NULL"]
    assert _dec(lib, scale=float("-inf")) == C["ATTN_ERR_SCALE"]
    assert _dec(lib, scale=3e-39) == C["ATTN_ERR_SCALE"]  # subnormal
    assert _dec(lib, B=0, q=None, k=None, v=None, o=None, ws=None) == C["ATTN_OK"]


def test_binding_requires_the_library(monkeypatch, tmp_path):
    # the product path has no fallback: a missing library is an error, not a CPU computation
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(fa.AttentionError, match="not found"):
        fa.load(str(tmp_path / "missing.so"))


def test_ctypes_signatures_match_header(lib):
    hdr = _header()
    for name, (res, args) in fa._SIGNATURES.items():
        m = re.search(r"SDPA_FA2_API\s+[\w\s\*]+?\b" + name + r"\s*\(([^;]*)\);", hdr, re.S)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip()]
        assert len(params) == len(args), name
        for p, a in zip(params, args):
            p = p.strip()
            if "*" in p:
                assert a is ctypes.c_void_p, (name, p)
            elif p.startswith("size_t"):
                assert a is ctypes.c_size_t, (name, p)
            elif p.startswith("float"):
                assert a is ctypes.c_float, (name, p)
            else:
                assert p.startswith("int") and a is ctypes.c_int, (name, p)


def _fwd_ex(lib, q=A16, k=A16, v=A16, o=A16, lse=None, seqlens=None, bias=None, bb=1, bh=1,
            **kw):
    a = {**GOOD, **kw}
    return lib.attn_fwd_ex(q, k, v, o, lse, seqlens, bias, bb, bh, a["B"], a["Hq"], a["Hkv"],
                           a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], None)


def _dec_ex(lib, q=A16, k=A16, v=A16, o=A16, lse=None, ws=A16, ws_bytes=1 << 40, seqlens=None,
            bias=None, bb=1, bh=1, S=2, **kw):
    a = {**GOOD, **kw}
    return lib.attn_decode_splitkv_ex(q, k, v, o, lse, ws, ws_bytes, seqlens, bias, bb, bh,
                                      a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                      a["scale"], a["causal"], S, None)


@pytest.mark.parametrize("which", ["fwd", "dec"])
def test_extras_validation(lib, which):
    call = _fwd_ex if which == "fwd" else _dec_ex
    base = dict(B=2, Hq=4, Hkv=2, Nq=8, Nk=12)
    # the common checks come first, exactly as in the plain entry points
    assert call(lib, **{**base, "d": 96}) == C["ATTN_ERR_HEADDIM"]
    assert call(lib, q=None, **base) == C["ATTN_ERR_NULL"]
    # bias dims: batch 1 or B, heads 1 or Hq; Nk a multiple of 4
    for bb, bh in ((3, 1), (1, 2), (0, 1), (2, 5), (-1, 4)):
        assert call(lib, bias=A16, bb=bb, bh=bh, **base) == C["ATTN_ERR_BIAS"], (bb, bh)
    assert call(lib, bias=A16, bb=2, bh=4, **{**base, "Nk": 10}) == C["ATTN_ERR_BIAS"]
    assert call(lib, bias=A16 + 8, bb=1, bh=1, **base) == C["ATTN_ERR_ALIGN"]
    assert call(lib, seqlens=A16 + 2, **base) == C["ATTN_ERR_ALIGN"]
    # without a bias its dims are not looked at, nor is Nk % 4
    assert call(lib, bb=7, bh=9, **{**base, "d": 96, "Nk": 10}) == C["ATTN_ERR_HEADDIM"]
    # empty problems succeed with any extras
    assert call(lib, q=None, k=None, v=None, o=None, ws=None, seqlens=A16, bias=A16, bb=1, bh=1,
                **{**base, "B": 0}) == C["ATTN_OK"]


def test_decode_ex_workspace_and_splits(lib):
    assert _dec_ex(lib, S=0) == C["ATTN_ERR_SPLITS"]
    assert _dec_ex(lib, ws=None) == C["ATTN_ERR_WORKSPACE"]
    need = lib.attn_decode_workspace_bytes(1, 4, 8, 128, 2)
    assert _dec_ex(lib, ws_bytes=need - 1) == C["ATTN_ERR_WORKSPACE"]


def test_num_splits(lib):
    # 8 x 8 KV heads, 4 query rows each: 64 workgroups per split -> 16 splits for ~1024
    assert lib.attn_decode_num_splits(8, 32, 8, 1, 8192) == 16
    # few workgroups per split, but no split shorter than 256 keys
    assert lib.attn_decode_num_splits(1, 8, 8, 1, 512) == 2
    assert lib.attn_decode_num_splits(1, 8, 8, 1, 100) == 1
    assert lib.attn_decode_num_splits(1, 1, 1, 1, 1 << 24) == 256  # capped
    assert lib.attn_decode_num_splits(64, 64, 64, 16, 8192) == 1   # the grid is full already
    assert lib.attn_decode_num_splits(0, 8, 8, 1, 512) == 1
    assert lib.attn_decode_num_splits(1, 6, 4, 1, 512) == 1        # invalid GQA


def test_forward_workspace_and_routing(lib):
    # prefill route from 32 query rows on: no workspace
    assert lib.attn_forward_workspace_bytes(2, 16, 16, 32, 4096, 128) == 0
    s = lib.attn_decode_num_splits(8, 32, 8, 31, 8192)
    assert lib.attn_forward_workspace_bytes(8, 32, 8, 31, 8192, 128) == \
        lib.attn_decode_workspace_bytes(8, 32, 31, 128, s)

    def fwd(ws=A16, ws_bytes=1 << 40, **kw):
        a = {**GOOD, **kw}
        return lib.attn_forward(A16, A16, A16, A16, None, ws, ws_bytes, None, None, 1, 1, a["B"],
                                a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                a["causal"], None)

    # below 32 rows the split-KV path runs, so its workspace is required
    assert fwd(ws=None, Nq=8) == C["ATTN_ERR_WORKSPACE"]
    assert fwd(ws_bytes=1, Nq=31, Nk=64) == C["ATTN_ERR_WORKSPACE"]
    assert fwd(ws=None, Nq=8, d=96) == C["ATTN_ERR_HEADDIM"]
    assert fwd(ws=None, B=0) == C["ATTN_OK"]


def _bwd(lib, ws=A16, ws_bytes=1 << 40, lse=A16, dout=A16, dq=A16, dk=A16, dv=A16, q=A16, k=A16,
         v=A16, o=A16, **kw):
    a = {**GOOD, **kw}
    return lib.attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, a["B"], a["Hq"], a["Hkv"],
                        a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], None)


def test_backward_validation(lib):
    assert lib.attn_bwd_workspace_bytes(2, 16, 2048) == 2 * 16 * 2048 * 8
    assert lib.attn_bwd_workspace_bytes(-1, 16, 2048) == 0
    assert _bwd(lib, d=96) == C["ATTN_ERR_HEADDIM"]  # head dim 64 or 128
    assert _bwd(lib, B=-1) == C["ATTN_ERR_SHAPE"]
    assert _bwd(lib, Hq=3) == C["ATTN_ERR_GQA"]
    assert _bwd(lib, scale=float("nan")) == C["ATTN_ERR_SCALE"]
    assert _bwd(lib, scale=2.0**-40) == C["ATTN_ERR_SCALE"]
    for name in ("lse", "dout", "dq", "q", "o", "k", "v", "dk", "dv"):
        assert _bwd(lib, **{name: None}) == C["ATTN_ERR_NULL"], name
    assert _bwd(lib, dq=A16 + 8) == C["ATTN_ERR_ALIGN"]
    assert _bwd(lib, lse=A16 + 2) == C["ATTN_ERR_ALIGN"]
    assert _bwd(lib, ws=None) == C["ATTN_ERR_WORKSPACE"]
    assert _bwd(lib, ws_bytes=lib.attn_bwd_workspace_bytes(1, 4, 8) - 1) == C["ATTN_ERR_WORKSPACE"]
    assert _bwd(lib, ws=A16 + 4) == C["ATTN_ERR_ALIGN"]
    # nothing on either side: nothing to do, NULL everywhere is fine
    assert _bwd(lib, B=0, q=None, k=None, v=None, o=None, lse=None, dout=None, dq=None, dk=None,
                dv=None, ws=None) == C["ATTN_OK"]
    # no query rows: the query-side pointers and the workspace are not needed (dk, dv are)
    assert _bwd(lib, Nq=0, q=None, o=None, lse=None, dout=None, dq=None, ws=None, k=None) == \
        C["ATTN_ERR_NULL"]


def test_backward_with_lengths_validation(lib):
    # attn_bwd_ex checks what attn_bwd checks, plus the alignment of the length array
    def bwd_ex(seqlens, bias=None, bias_b=1, bias_h=1, **kw):
        a = {**GOOD, **kw}
        return lib.attn_bwd_ex(A16, A16, A16, A16, A16, A16, A16, A16, A16, A16, 1 << 40, seqlens,
                               bias, bias_b, bias_h, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"],
                               a["d"], a["scale"], a["causal"], None)

    assert bwd_ex(A16 + 2) == C["ATTN_ERR_ALIGN"]
    assert bwd_ex(None, bias=A16, bias_b=3) == C["ATTN_ERR_BIAS"]   # neither 1 nor B
    assert bwd_ex(None, bias=A16, Nk=GOOD["Nk"] + 1) == C["ATTN_ERR_BIAS"]  # Nk % 4 != 0
    assert bwd_ex(None, bias=A16 + 8) == C["ATTN_ERR_ALIGN"]
    assert bwd_ex(A16, d=96) == C["ATTN_ERR_HEADDIM"]
    assert bwd_ex(A16, Hq=3) == C["ATTN_ERR_GQA"]
    assert bwd_ex(None, B=0) == C["ATTN_OK"]
