"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every HIP source is compiled again with the sanitizers on its host half only
(each -fsanitize= after -Xarch_host: the device code is built as usual and
never runs here), linked into a separate library in a temporary folder, and
driven by tests/abi_host_driver.cpp, built with the same sanitizers: plans
of thousands of random descriptors and their tables, the host mirror of the
consumer order, size queries, and the argument checks of every run call
(which refuse before any device work).  A sanitizer report aborts the driver
(-fno-sanitize-recover=all); a wrong answer fails it."""

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "communication_overlap_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.slow


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), os.path.join(ROCM, "bin", "hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_host_code_is_clean_under_address_and_undefined_behavior_sanitizers(tmp_path):
    hipcc = _hipcc()
    objs = []
    cmds = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src)[:-4] + ".o"))
        objs.append(obj)
        cmds.append([hipcc, "--offload-arch=gfx950", "-O3", "-g", "-std=c++17", "-fPIC", *SAN,
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{INCLUDE}", f"-I{CSRC}",
                     "-c", src, "-o", obj])
    with ThreadPoolExecutor(min(8, len(cmds))) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds):
            assert r.returncode == 0, r.stderr[-3000:]
    # The objects carry their device code already; the host linker joins them.
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    lib = str(tmp_path / "libovl_san.so")
    r = subprocess.run([clang, "-shared", "-fPIC", "-fsanitize=address,undefined", "-o", lib, *objs,
                        f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_host_driver")
    r = subprocess.run([clang, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}", f"-I{os.path.join(ROCM, 'include')}",
                        os.path.join(ROOT, "tests", "abi_host_driver.cpp"), lib, f"-Wl,-rpath,{tmp_path}",
                        f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "host driver ok" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_the_sanitizers_are_live(tmp_path):
    """The same driver flags catch a planted heap overflow (so a clean run
    above means something)."""
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    src = tmp_path / "overflow.cpp"
    src.write_text("#include <vector>\nint main(int c, char**){std::vector<int> v(4); return v.data()[c + 4];}\n")
    exe = str(tmp_path / "overflow")
    subprocess.run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", str(src),
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
