"""Host sanitizer tier (CPU only): the fp64 oracle rebuilt with AddressSanitizer
+ UndefinedBehaviorSanitizer runs its pins, mutant checks and thread-count
determinism tests; rebuilt with ThreadSanitizer it runs its worker pool
(prefill and gradient, 1 vs 8 threads, bitwise equal); and the C ABI's
argument checks run host-only under ASan + UBSan with the kernel launchers
replaced by counting doubles (tests/sanitize/).

The instrumented oracle is a shared library loaded into a Python child
process, so that process starts with the sanitizer runtime preloaded.  The
tests are skipped when the environment already preloads a library (that
setting is left alone)."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="gcc/g++ missing")
no_preload = pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                                reason="the environment preloads a library already")


def _child_env(preload, lib, **extra):
    env = dict(os.environ, LD_PRELOAD=preload, KDA_ORACLE_LIB=lib, PYTHONPATH=ROOT,
               OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    env.update(extra)
    return env


@needs_gcc
@no_preload
def test_oracle_pins_under_asan_ubsan(tmp_path):
    rt = _runtime("libasan.so")
    if rt is None:
        pytest.skip("no libasan")
    lib = oracle.build(out=str(tmp_path / "oracle_asan.so"), force=True,
                       extra_flags=["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                    "-fno-omit-frame-pointer", "-g"])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py"), os.path.join(HERE, "test_oracle_grad.py"),
                        os.path.join(HERE, "test_oracle_mutants.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=600,
                       env=_child_env(rt, lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                                      UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


TSAN_SCRIPT = r"""
import numpy as np, oracle
lib = oracle.load()
rng = np.random.default_rng(3)
T, H, dk, dv = 300, 3, 32, 32
q = rng.standard_normal((T, H, dk)); k = rng.standard_normal((T, H, dk)); v = rng.standard_normal((T, H, dv))
q /= np.linalg.norm(q, axis=-1, keepdims=True); k /= np.linalg.norm(k, axis=-1, keepdims=True)
la = -np.exp(rng.uniform(-4, 0, (T, H, dk))); beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
cu = [0, 100, 100, 300]
s0 = 0.02 * rng.standard_normal((3, H, dv, dk))
o1, f1 = oracle.prefill(q, k, v, la, beta, cu, s0, nthreads=1)
o8, f8 = oracle.prefill(q, k, v, la, beta, cu, s0, nthreads=8)
assert np.array_equal(o1, o8) and np.array_equal(f1, f8)
d_o = rng.standard_normal((T, H, dv)); d_f = rng.standard_normal((3, H, dv, dk))
g1 = oracle.prefill_grad(q, k, v, la, beta, cu, s0, d_o, d_f, nthreads=1)
g8 = oracle.prefill_grad(q, k, v, la, beta, cu, s0, d_o, d_f, nthreads=8)
assert all(np.array_equal(g1[n], g8[n]) for n in g1)
print("TSAN_OK")
"""


@needs_gcc
@no_preload
def test_oracle_threads_under_tsan(tmp_path):
    rt = _runtime("libtsan.so")
    if rt is None:
        pytest.skip("no libtsan")
    lib = oracle.build(out=str(tmp_path / "oracle_tsan.so"), force=True, extra_flags=["-fsanitize=thread", "-g"])
    r = subprocess.run([sys.executable, "-c", TSAN_SCRIPT], cwd=ROOT, capture_output=True, text=True, timeout=600,
                       env=_child_env(rt, lib, TSAN_OPTIONS="halt_on_error=1:report_signal_unsafe=0"))
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "TSAN_OK" in out, out[-4000:]
    assert "ThreadSanitizer" not in out, out[-4000:]


@needs_gcc
@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"), reason="HIP headers missing")
def test_abi_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "gated_delta_rule_88_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "kda_api.cpp"),
           os.path.join(HERE, "sanitize", "abi_stubs.cpp"), os.path.join(HERE, "sanitize", "abi_driver.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "0 failures" in out
