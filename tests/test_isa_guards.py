"""Guards on the generated gfx950 assembly (CPU only: hipcc cross-compiles).

* The direct HBM->LDS copies are inline assembly that sets M0 itself.  That is
  sound only while the compiler keeps no value of its own in M0 across them, so
  every M0 access in the attention kernels must be one of those copies: an
  s_mov_b32 into M0, an s_nop, then the copy.
* No packed fp32 arithmetic (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32) in any
  kernel: the build disables the feature, and this checks that it stays so.
"""

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from attention_qk_norm_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]
COPY_SOURCES = ["k_prefill.hip", "k_prefill_wide.hip", "k_decode.hip"]


@pytest.fixture(scope="module")
def assembly():
    if not os.path.exists(B.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="qwattn_isa_")

    def compile_one(src):
        out = os.path.join(tmp, src + ".s")
        cmd = ([B.HIPCC] + B.FLAGS + list(B.SOURCE_FLAGS.get(src, ())) +
               ["--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out])
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, open(out).read()

    try:
        with ThreadPoolExecutor(max_workers=min(8, len(HIP_SOURCES))) as ex:
            yield dict(ex.map(compile_one, HIP_SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def instructions(text):
    """Instruction lines (comments, labels and directives dropped)."""
    out = []
    for ln in text.splitlines():
        ln = ln.split(";")[0].strip()
        if not ln or ln.endswith(":") or ln.startswith("."):
            continue
        out.append(ln)
    return out


@pytest.mark.parametrize("src", COPY_SOURCES)
def test_m0_only_in_the_copies(assembly, src):
    ins = instructions(assembly[src])
    copies = 0
    for i, ln in enumerate(ins):
        if not re.search(r"\bm0\b", ln):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"{src}: M0 used outside the copies: {ln}"
        assert ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_dwordx4"), \
            f"{src}: M0 write not followed by its copy: {ins[i:i + 3]}"
        copies += 1
    assert copies > 0, f"{src}: no copies found (the check would be vacuous)"


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_packed_fp32(assembly, src):
    bad = [ln for ln in instructions(assembly[src]) if re.match(r"v_pk_(add|mul|fma)_f32\b", ln)]
    assert not bad, f"{src}: packed fp32 instructions: {bad[:3]}"
