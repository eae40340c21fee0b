"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is compiled again with both sanitizers on its host code only
(argument checks, size arithmetic, kernel-name tables, the allocation-free
scratch lookup; the device code is compiled as usual and never runs here),
and every host-side C-ABI check of test_abi.py runs against that build in a
child process with the sanitizer runtime preloaded.  Any out-of-bounds
access, overflowing signed arithmetic or other undefined behaviour on those
paths aborts the child and fails the test.  CPU only: the checks never
launch a kernel.
"""

import os
import shutil
import subprocess
import sys

import pytest

import exact_attention_103_amd as fa
from exact_attention_103_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Host-only sanitizers (each -fsanitize directly after -Xarch_host), a
# shared sanitizer runtime so the child can preload it into Python.
SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-omit-frame-pointer -Xarch_host -shared-libsan").split()


def _asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(B.hipcc())), "..", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    return None


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="host-only validation checks")
def test_c_abi_host_checks_under_sanitizers(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("sanitizer runtime not found")
    lib = str(tmp_path / "libfa_sanitized.so")
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE
    cmd = [hipcc, *flags, "-I", B.INCLUDE, "-I", B.CSRC,
           *[os.path.join(B.CSRC, s) for s in B.SOURCES], "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    child = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})\n"
        "import exact_attention_103_amd as fa\n"
        f"fa._lib = fa.load_library({lib!r})\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',\n"
        f"    {os.path.join(ROOT, 'tests', 'test_abi.py')!r},\n"
        # these inspect the shipped libraries' files, not host behaviour
        "    '-k', 'not exports and not serial and not profiled']))\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
