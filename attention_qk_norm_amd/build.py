"""Build libqwattn.so in-tree for gfx950 with hipcc.

    python -m attention_qk_norm_amd.build        # or: __graft_entry__.build()

Every source is compiled on each call (one process per file, in parallel),
then linked into ``attention_qk_norm_amd/lib/libqwattn.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libqwattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["qwattn_api.cpp", "k_normrope.hip", "k_prefill.hip", "k_prefill_wide.hip", "k_attn_f32.hip", "k_decode.hip",
           "k_gemm.hip", "k_probe.hip", "k_scratch.hip"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code (the host pass of
# hipcc warns that it does not know the feature; that is harmless).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-source extra flags.  The attention kernels keep their MFMA accumulators
# in arch VGPRs: the softmax reads every score, and the online softmax rescales
# every output accumulator, with VALU; the AGPR form made the compiler shuttle
# them between register files.  The prefill kernels take their work-item list
# and KV-head count as leading scalar arguments, which the wave finds preloaded
# in SGPRs (kernarg preload), so its first dependent load can issue at once.
SOURCE_FLAGS = {"k_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=3"],
                "k_prefill_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=3"],
                "k_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, objdir, extra=()):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + list(SOURCE_FLAGS.get(src, ())) + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    return obj, r.returncode, "\n".join(msgs)


def build(verbose=False, out=None, extra_flags=None):
    """Compile and link; `out` / `extra_flags` ({source: [flags]}) build variants."""
    objdir = os.path.join(PKG, "_build" if out is None else "_build_variant")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    extra_flags = extra_flags or {}
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        results = list(ex.map(lambda s: _compile(s, objdir, extra_flags.get(s, ())), SOURCES))
    failed = False
    for (obj, rc, msg), src in zip(results, SOURCES):
        if msg.strip() and (verbose or rc):
            print(f"--- {src}\n{msg}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("libqwattn: compilation failed")
    lib = LIB if out is None else out
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("libqwattn: link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
