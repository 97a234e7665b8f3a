"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled again with the sanitizers on its host half only (the
device code is unchanged), linked into a separate library, and the CPU ABI
tests run against it in a child process: argument validation, the
validate-before-touching-weights order of create and load, the status
strings and the thread-local error text, with every out-of-range enum and
NULL the tests pass.  Any report aborts the child (halt_on_error), so the
test fails on the first finding.  CPU only."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from tensor_dit_transformer_amd import build as B  # noqa: E402

OUT = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT, "libtp_shard_sanitized.so")
# each sanitizer flag is passed to the host compilation alone
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _runtime():
    found = sorted(glob.glob(os.path.join(os.path.dirname(B.HIPCC), "..", "llvm", "lib", "clang", "*",
                                          "lib", "linux", "libclang_rt.asan-x86_64.so")))
    found += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return os.path.realpath(found[0]) if found else None


def _build():
    import concurrent.futures as cf
    os.makedirs(OUT, exist_ok=True)
    flags = [f for f in B.CFLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN

    def one(src):
        obj = os.path.join(OUT, os.path.basename(src)[:-4] + ".o")
        cmd = [B.HIPCC, *flags, *B.FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(one, B.sources()))
    cmd = [B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *HOST_SAN, "-shared-libasan",
           "-o", LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]


@pytest.mark.slow
def test_abi_tests_pass_under_host_asan_and_ubsan():
    rt = _runtime()
    assert rt, "clang AddressSanitizer runtime not found"
    _build()
    env = dict(os.environ)
    env["TP_SHARD_LIB"] = LIB
    # the sanitizer runtime must be the first library loaded; anything already
    # preloaded stays, after it
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout
