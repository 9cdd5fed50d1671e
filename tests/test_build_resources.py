"""Every kernel of the library builds without register spills: each HIP source
is compiled for gfx950 (device code only) with the compiler's per-kernel
resource report, and every kernel must report no VGPR spill and no scratch
memory.  The attention kernel must also keep two wavefronts per SIMD, which
its two-role design relies on."""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from bit_kv_cache_kv4_amd import build as kbuild

HIPCC = kbuild.HIPCC


def _report(src):
    out = os.path.join("/tmp", "kv4_res_%d_%s.o" % (os.getpid(), os.path.basename(src)))
    cmd = [HIPCC] + kbuild.FLAGS + ["--cuda-device-only", "-c", src, "-o", out,
                                    "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if os.path.exists(out):
        os.remove(out)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: \s*([A-Za-z ]+?(?:\[[^\]]*\])?):\s*(\S+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = m.group(2)
    return kernels


@pytest.fixture(scope="module")
def resources():
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        reports = list(ex.map(_report, kbuild.sources()))
    merged = {}
    for r in reports:
        merged.update(r)
    return merged


def test_every_kernel_is_spill_free(resources):
    assert len(resources) >= 10
    bad = {k: v for k, v in resources.items()
           if v.get("VGPRs Spill", "0") != "0" or v.get("ScratchSize [bytes/lane]", "0") != "0"}
    assert not bad, "kernels with spills or scratch: %s" % bad


def test_attention_keeps_two_wavefronts_per_simd(resources):
    attn = {k: v for k, v in resources.items() if "sparse_mla_f32q_kernel" in k or "sparse_mla_bf16_kernel" in k}
    assert len(attn) == 4                                   # {bf16, fp32 queries} x {352, 288-byte rows}
    for k, v in attn.items():
        assert int(v["Occupancy [waves/SIMD]"]) >= 2, (k, v)
