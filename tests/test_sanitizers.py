"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The oracle (plain C, gcc) is rebuilt with -fsanitize=address,undefined and
its pin tests run against that build; the library's host code (argument
checks, layouts, plans, the binding's calls) is rebuilt by hipcc with the
sanitizers on the host pass only (-Xarch_host: GPU code is never built with
them) and the C-ABI tests run against that build. Each run is a child
process with the sanitizer runtime preloaded, leak detection off (the
interpreter's own allocations are not ours to check) and the first error
fatal, so any report fails the test. Builds go to _build/san/ and are reused
while the sources are unchanged."""
import glob
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "san")
CSRC = os.path.join(ROOT, "dynamic_quantized_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _digest(files):
    h = hashlib.sha256()
    for f in sorted(files):
        with open(f, "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _run(args, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env.pop("PYTEST_ADDOPTS", None)
    r = subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    return r.returncode, (r.stdout + r.stderr)[-6000:]


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan():
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    assert asan and ubsan, "gcc's sanitizer runtimes are missing"
    src = os.path.join(ROOT, "oracle", "oracle.c")
    os.makedirs(SAN, exist_ok=True)
    lib = os.path.join(SAN, f"liboracle_san_{_digest([src])}.so")
    if not os.path.exists(lib):
        subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                        src, "-o", lib, "-lm"], check=True)
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_pins*.py")))
    rc, out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *pins],
                   {"DQ_ORACLE_LIB": lib, "LD_PRELOAD": f"{asan}:{ubsan}",
                    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}, timeout=1200)
    assert rc == 0, out
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out


def test_library_host_code_under_asan_and_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rts, "clang's AddressSanitizer runtime is missing"
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    hdrs = sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(ROOT, "include", "dqip.h")]
    tag = _digest(srcs + hdrs)
    out_dir = os.path.join(SAN, f"dqip_{tag}")
    lib = os.path.join(out_dir, "libdqip_san.so")
    if not os.path.exists(lib):
        os.makedirs(out_dir, exist_ok=True)
        host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
        flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *host_san]
        procs, objs = [], []
        for s in srcs:
            o = os.path.join(out_dir, os.path.basename(s) + ".o")
            objs.append(o)
            procs.append(subprocess.Popen([HIPCC, *flags, "-c", s, "-o", o], stdout=subprocess.DEVNULL,
                                          stderr=subprocess.PIPE))
        for p in procs:
            _, err = p.communicate()
            assert p.returncode == 0, err.decode()[-3000:]
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san, *objs, "-o", lib],
                       check=True)
    rc, out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                    os.path.join(ROOT, "tests", "test_abi.py")],
                   {"DQIP_LIB_PATH": lib, "LD_PRELOAD": rts[0],
                    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}, timeout=900)
    assert rc == 0, out
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
