"""The built kernels' gfx950 assembly keeps the matrix-core fences and contains
no forbidden instruction (see isa_scan.py).  Compiles each HIP source with the
library's own flags to device assembly; needs hipcc, no GPU."""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", "bit_quantized_moe_q2_amd"))
import build as B  # noqa: E402

from isa_scan import forbidden, mfma_srcc_gaps  # noqa: E402

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


@pytest.fixture(scope="module")
def assembly():
    if not os.path.exists(B._hipcc()):
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="ds4q_isa_")

    def one(src):
        out = os.path.join(tmp, src + ".s")
        cmd = [B._hipcc(), *B.HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, open(out).read()

    try:
        with ThreadPoolExecutor(max_workers=min(8, len(HIP_SOURCES))) as ex:
            yield dict(ex.map(one, HIP_SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_srcc_overwrite_near_mfma(assembly, src):
    hits = mfma_srcc_gaps(assembly[src], limit=8)
    assert not hits, "\n".join(f"{k[:70]} L{a}: {i} | L{b}: {j} after {ws} wait states"
                               for k, a, i, b, j, ws in hits[:10])


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_forbidden_instructions(assembly, src):
    bad = forbidden(assembly[src])
    assert not bad, bad[:10]


def test_scanner_finds_planted_gap():
    # a write of the accumulator input three instructions after the MFMA
    text = "\n".join([
        "_Zk:",
        "\tv_mfma_i32_16x16x64_i8 v[10:13], v[10:13], v[36:39], v[14:17]",
        "\tv_mul_f32_e32 v56, v24, v18",
        "\tv_cvt_f32_ubyte0_e32 v24, v24",
        "\tv_lshrrev_b32_e32 v24, 28, v25",
        "\tv_cndmask_b32_e64 v14, v19, v21, s[0:1]",
    ])
    hits = mfma_srcc_gaps(text, limit=8)
    assert len(hits) == 1 and hits[0][5] == 3
    # the fence's s_nop 7 makes it 8 wait states: no hit
    fenced = text.replace("\tv_mul_f32_e32 v56, v24, v18", "\ts_nop 7\n\tv_mul_f32_e32 v56, v24, v18")
    assert not mfma_srcc_gaps(fenced, limit=8)
    # a write of an unrelated register, or a read of the accumulator, is no hit
    assert not mfma_srcc_gaps(text.replace("v_cndmask_b32_e64 v14,", "v_cndmask_b32_e64 v15x,"), limit=8)
    assert not mfma_srcc_gaps(text.replace("v_cndmask_b32_e64 v14, v19", "v_cndmask_b32_e64 v40, v14"), limit=8)
    # a buffer load writes its first operand, unless it loads to LDS (then
    # that operand is the offset it reads)
    load = text.replace("\tv_cndmask_b32_e64 v14, v19, v21, s[0:1]", "\tbuffer_load_dwordx4 v[14:17], v20, s[4:7], 0 offen")
    assert len(mfma_srcc_gaps(load, limit=8)) == 1
    assert not mfma_srcc_gaps(text.replace("\tv_cndmask_b32_e64 v14, v19, v21, s[0:1]",
                                           "\tbuffer_load_dwordx4 v14, s[4:7], s62 offen lds"), limit=8)


def test_forbidden_scan_finds_planted():
    assert forbidden("\ts_store_dword s0, s[2:3], 0x0\n\tv_add_f32 v0, v1, v2\n")
    assert forbidden("\tv_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]\n")
    assert not forbidden("\tv_pk_add_f16 v0, v1, v2\n\ts_load_dword s0, s[2:3], 0x0\n")
