"""Address and undefined-behaviour sanitizers on the CPU code (no GPU needed).

* The oracle is rebuilt with -fsanitize=address,undefined (g++) and the fast
  pins run against it in a child process with the sanitizer runtimes
  preloaded; any heap overflow, use after free, signed overflow, bad shift or
  misaligned access ends that process with a report.
* A copy of the oracle with an out-of-bounds write planted in it must be
  stopped by the same harness, which shows the harness is live.
* The host side of libep (the C-ABI argument checks that run before any
  launch) is rebuilt with the sanitizers on the host pass only, linked with
  the library's unchanged kernel objects, and the boundary tests run against
  it.  Every call there fails its host checks, so nothing touches a GPU.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle.build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "ep_oracle.cpp")
CSRC = os.path.join(ROOT, "combine_ep_layout_09_amd", "csrc")
OBJS = os.path.join(ROOT, "combine_ep_layout_09_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

PINS_SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._LIB_PATH = {lib!r}
from tests import test_oracle_mutants as mut
for pin in mut._fast_pins():
    pin()
print("PINS_OK", flush=True)
"""


def _gcc_runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="ep_sanitizers_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _build_oracle(src_text, out):
    src = out + ".cpp"
    with open(src, "w") as f:
        f.write(src_text)
    flags = [f for f in obuild.CXXFLAGS if f != "-O2"]
    subprocess.run(["g++", *flags, "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-w",
                    src, "-o", out], check=True)


def _run_pins(lib):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("g++ sanitizer runtimes not installed")
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=f"{asan}:{ubsan}")
    code = PINS_SCRIPT.format(root=ROOT, lib=lib)
    return subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                          timeout=600)


def test_oracle_pins_clean_under_asan_ubsan(workdir):
    lib = os.path.join(workdir, "liboracle_san.so")
    _build_oracle(open(ORACLE_SRC).read(), lib)
    r = _run_pins(lib)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "PINS_OK" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


def test_sanitizer_harness_stops_a_planted_overflow(workdir):
    src = open(ORACLE_SRC).read()
    anchor = "for (int64_t r = 0; r < R; ++r) src_of_slot[r] = -1;"
    assert src.count(anchor) == 1
    lib = os.path.join(workdir, "liboracle_overflow.so")
    _build_oracle(src.replace(anchor, "for (int64_t r = 0; r <= R + 64; ++r) src_of_slot[r] = -1;"),
                  lib)
    r = _run_pins(lib)
    assert r.returncode != 0 and "PINS_OK" not in r.stdout
    assert "AddressSanitizer" in r.stderr, (r.stdout + r.stderr)[-4000:]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_libep_host_checks_clean_under_asan_ubsan(workdir):
    rt = _clang_asan_runtime()
    kernel_objs = sorted(glob.glob(os.path.join(OBJS, "*.hip.o")))
    if rt is None or not os.path.exists(HIPCC) or not kernel_objs:
        pytest.skip("hipcc, its ASan runtime or the built kernel objects are missing")
    api_obj = os.path.join(workdir, "ep_api_san.o")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    *host_san, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c",
                    os.path.join(CSRC, "ep_api.hip"), "-o", api_obj],
                   check=True, capture_output=True)
    others = [o for o in kernel_objs if os.path.basename(o) != "ep_api.hip.o"]
    lib = os.path.join(workdir, "libep_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *host_san[:4],
                    "-shared-libsan", api_obj, *others, "-o", lib], check=True,
                   capture_output=True)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import combine_ep_layout_09_amd as ep\n"
            "ep._LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, lib, os.path.join(ROOT, "tests", "test_boundary.py")))
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=rt)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
