"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

Two builds, each tested in a child process with its sanitizer runtime preloaded:
  * the oracle (oracle.c) built with gcc -fsanitize=address,undefined, running the oracle
    pins (tests/test_oracle_pins.py);
  * libw8a8.so with the host side of its C-ABI layer (abi.hip: argument validation, status
    codes, dispatch) built with clang's AddressSanitizer and UndefinedBehaviorSanitizer
    (device code unchanged, the other objects as built), running the host-side ABI tests
    (tests/test_abi_cpu.py), which make no compute call.
A sanitizer report fails the child (halt_on_error) and so the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _child(env_extra, args, timeout, log_dir):
    """Run pytest on `args` in a child process; sanitizer reports go to files in log_dir (a
    report ends the child with a non-zero status before pytest can print it)."""
    env = dict(os.environ)
    env.update(env_extra)
    log = os.path.join(str(log_dir), "san")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0:log_path={log}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *args], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=timeout)
    reports = "".join(open(f).read() for f in sorted(glob.glob(log + "*")))
    out = r.stdout + r.stderr
    assert not reports, reports[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                           "-shared", "-fPIC", "-std=c11", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    out = _child({"W8A8_ORACLE_LIB": lib, "LD_PRELOAD": libasan, "OMP_NUM_THREADS": "4"},
                 ["tests/test_oracle_pins.py"], timeout=900, log_dir=tmp_path)
    assert " passed" in out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libw8a8_san.so")
    # host-side sanitizers only: each -fsanitize applies to the host compilation (-Xarch_host);
    # every source's host code (argument checks, dispatch, plans, the autotuning table)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    csrc = os.path.join(ROOT, "w8a8_activation_quantized_amd", "csrc")
    objs, procs = [], []
    for f in ("abi", "quantize", "gemm", "mv", "sdpa", "diag"):
        o = str(tmp_path / (f + "_san.o"))
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                                       "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-Xclang",
                                       "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-c",
                                       os.path.join(csrc, f + ".hip"), "-o", o],
                                      stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL))
    assert all(pr.wait() == 0 for pr in procs), "sanitizer build failed"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", lib, *objs])
    out = _child({"W8A8_LIB": lib, "LD_PRELOAD": rt[-1]}, ["tests/test_abi_cpu.py"], timeout=900, log_dir=tmp_path)
    assert " passed" in out
