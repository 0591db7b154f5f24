"""The validation layer (qwattn_api.cpp) built for the host alone under
AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launchers replaced
by stand-ins that write every workspace byte the kernels would write
(tests/host_sanitize/).  The driver calls every entry point with invalid
arguments (each must return its status and launch nothing) and with valid
ones whose host arrays and workspaces have exactly the declared sizes, so a
bounds slip in the validation loops or a workspace layout that overruns its
size is a sanitizer report.  A second build plants one such slip (the decode
chunk bound without its per-sequence term) to show the run would catch it.
CPU only: hipcc compiles the host side (--cuda-host-only)."""

import os
import shutil
import subprocess
import tempfile

import pytest

from attention_qk_norm_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = os.path.join(HERE, "host_sanitize")
API = os.path.join(B.CSRC, "qwattn_api.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src, obj):
    cmd = ([B.HIPCC, "-x", "hip", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer"] +
           SAN_FLAGS + ["-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC, "-I", SAN, "-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return obj


def _link(objs, exe):
    r = subprocess.run([CLANG, "-fsanitize=address,undefined"] + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


@pytest.fixture(scope="module")
def objs():
    if not os.path.exists(B.HIPCC) or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang++ not available")
    tmp = tempfile.mkdtemp(prefix="qwattn_san_")
    from concurrent.futures import ThreadPoolExecutor
    srcs = {"api": API, "stubs": os.path.join(SAN, "stubs.cpp"), "main": os.path.join(SAN, "validation_main.cpp")}
    with ThreadPoolExecutor(3) as ex:
        built = dict(zip(srcs, ex.map(lambda k: _compile(srcs[k], os.path.join(tmp, k + ".o")), srcs)))
    yield tmp, built
    shutil.rmtree(tmp, ignore_errors=True)


def test_validation_layer_clean_under_asan_ubsan(objs):
    tmp, o = objs
    r = _run(_link([o["api"], o["stubs"], o["main"]], os.path.join(tmp, "validation")))
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_sanitizer_catches_a_planted_workspace_overrun(objs):
    tmp, o = objs
    text = open(API).read()
    planted = text.replace("  return most + n_seq;", "  return most;")
    assert planted != text
    src = os.path.join(tmp, "planted_api.cpp")
    open(src, "w").write(planted)
    exe = _link([_compile(src, os.path.join(tmp, "planted.o")), o["stubs"], o["main"]], os.path.join(tmp, "planted"))
    r = _run(exe)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
