"""Register, scratch and LDS budgets of every gfx950 kernel instance (CPU: compiles only).

Each HIP source is compiled for gfx950 with the library's own flags and the compiler's
kernel-resource-usage remarks; the test then checks, for every instantiated kernel, that

  * nothing spills: ScratchSize is 0 bytes per lane and no VGPR spills (a spill would put
    private memory traffic on the hot path);
  * the occupancy each kernel's design assumes still holds: the forward runs two 4-wave
    workgroups per CU (2 waves per SIMD, at most 256 VGPRs and 80 KB of LDS each), the four-wave
    decode splits and both backward kernels 2 waves per SIMD, the one-wave decode splits 1, the
    small kernels (combine, fp32 forward) at least 4.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

import pytest

from scaled_dot_product_fa2_amd import build as B

SOURCES = ["fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip"]

# (kernel name pattern, minimum waves per SIMD, maximum LDS bytes per workgroup or None)
BUDGETS = [
    (r"fwd_bf16_kernel<", 2, 81920),
    (r"fwd_f32_kernel<", 4, None),
    (r"decode_split_kernel<\d+, \w+, \w+, 1>", 1, None),
    (r"decode_split_kernel<\d+, \w+, \w+, 4>", 2, None),
    (r"decode_combine_kernel<", 4, None),
    (r"bwd_dq_kernel<", 2, None),
    (r"bwd_dkdv_kernel<", 2, None),
]


def _remarks(src, outdir):
    cmd = [B.hipcc(), *B.HIP_FLAGS, "--offload-device-only", "-c", os.path.join(B.CSRC, src),
           "-o", os.path.join(outdir, src + ".o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stderr


def _parse(text):
    """{demangled kernel name: {field: value}} from the remarks of one compilation."""
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            kernels[cur][m.group(1).strip()] = m.group(2)
    names = list(kernels)
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    demangled = r.stdout.splitlines() if r.returncode == 0 else names
    return {d: kernels[n] for n, d in zip(names, demangled)}


@pytest.fixture(scope="module")
def resources():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            texts = list(ex.map(lambda s: _remarks(s, tmp), SOURCES))
    out = {}
    for t in texts:
        out.update(_parse(t))
    return out


def test_every_kernel_is_reported(resources):
    # 8 forward (d x causal x bias), 4 fp32 forward, 16 decode splits (d x causal x bias x
    # waves), 2 combines, 8 dq, 8 dk/dv
    assert len(resources) == 46, sorted(resources)
    for pat, _, _ in BUDGETS:
        assert any(re.search(pat, k) for k in resources), pat


def test_no_scratch_and_no_spills(resources):
    for name, r in resources.items():
        assert int(r["ScratchSize"]) == 0, f"{name}: scratch {r['ScratchSize']} bytes/lane"
        assert int(r["VGPRs Spill"]) == 0, f"{name}: {r['VGPRs Spill']} VGPRs spilled"
        assert r.get("Dynamic Stack", "False") == "False", name


def test_occupancy_and_lds_budgets(resources):
    for name, r in resources.items():
        budget = [b for b in BUDGETS if re.search(b[0], name)]
        assert len(budget) == 1, f"{name}: no budget"
        _, waves, lds = budget[0]
        assert int(r["Occupancy"]) >= waves, f"{name}: {r['Occupancy']} waves/SIMD < {waves}"
        assert int(r["VGPRs"]) + int(r["AGPRs"]) <= 512 // waves, name
        if lds is not None:
            assert int(r["LDS Size"]) <= lds, f"{name}: {r['LDS Size']} bytes of LDS > {lds}"
