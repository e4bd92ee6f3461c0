"""CPU robustness: the oracle and the host side of libdgdenoise built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through their
interfaces (tests/sanitize/*.c).  Any out-of-bounds access, use after free,
leak (oracle) or undefined operation -- including reading an out-of-range
enum a C caller stored in an ABI struct -- aborts the driver.  Device code
is built unsanitized (the sanitizer flags go to the host compilation only)
and never runs: every call the ABI driver makes is answered or rejected
before any device work."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "uniform_state_discrete_dg_amd", "csrc")
LLVM = "/opt/rocm/llvm/bin"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, env=None, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def _env(**extra):
    env = dict(os.environ)
    env.update(extra)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=gnu11", *SAN_FLAGS, "-fopenmp", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "dg_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=_env(OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                             UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.stdout.strip() == "ok" and "runtime error" not in r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_host_abi_under_address_and_undefined_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    host_san = []
    for f in SAN_FLAGS:           # host compilation only; the device code is built as usual
        host_san += ["-Xarch_host", f]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", *host_san, "-x", "hip", "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "driver.o")
    _run([os.path.join(LLVM, "clang"), "-std=gnu11", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([os.path.join(LLVM, "clang++"), "-fsanitize=address,undefined", *objs, drv, "-L/opt/rocm/lib",
          "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
                             HIP_VISIBLE_DEVICES=""))
    assert r.stdout.strip() == "ok" and "runtime error" not in r.stderr
