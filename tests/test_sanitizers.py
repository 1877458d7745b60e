"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/naju_oracle.c), built with gcc and the sanitizers
  together with tests/sanitize/oracle_driver.c, runs every oracle function on
  small seeded inputs (ragged lengths, a single token, an empty sequence, both
  state sizes, with and without every optional argument); leak checking on.
* The host side of libnaju.so: every HIP source is built with the sanitizers on
  its host code only (the device code is unchanged), and
  tests/sanitize/api_driver.cpp drives the argument checks, the workspace and
  checkpoint sizing over a range of shapes up to the largest accepted, and the
  empty-problem paths -- every call returns before any device work, so no GPU
  is needed.  Leak checking is off there: the HIP runtime, loaded with the
  library, keeps allocations until exit.

A sanitizer report makes the driver exit nonzero (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_naju_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SOURCES = ["naju_api.hip", "naju_fwd.hip", "naju_fwd_mfma.hip", "naju_fwd_mfma64.hip",
           "naju_bwd.hip", "naju_bwd_mfma.hip", "naju_step.hip", "naju_mixer.hip"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_sanitizer_build_reports_an_overflow(tmp_path):
    """The gcc sanitizer flags used below do catch a heap overflow here."""
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    src = tmp_path / "canary.c"
    src.write_text("#include <stdlib.h>\nint main(void) { volatile int *p = malloc(4 * sizeof(int));"
                   " int v = p[4]; free((void *)p); return v & 0; }\n")
    exe = str(tmp_path / "canary")
    rc, out = _run(["gcc", "-O0", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    str(src), "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe])
    assert rc != 0 and "heap-buffer-overflow" in out, out[-2000:]


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "naju_oracle.c"),
           "-o", exe, "-lm"]
    rc, out = _run(cmd)
    assert rc == 0, "build failed:\n" + out[-3000:]
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = _run([exe], env=env)
    assert rc == 0 and "oracle driver: ok" in out, out[-5000:]


def test_library_host_side_under_asan_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("hipcc / clang++ not found")
    # sanitizers on the host compilation only (each -fsanitize= behind -Xarch_host)
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
             "-Wno-unused-command-line-argument", "-Wno-inline-asm",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        return _run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]) + (obj,)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for rc, out, _ in results:
        assert rc == 0, "hipcc failed:\n" + out[-3000:]
    lib = str(tmp_path / "libnaju_san.so")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] +
                   [o for _, _, o in results] +
                   ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, "link failed:\n" + out[-3000:]
    exe = str(tmp_path / "api_driver")
    driver_cmd = [CLANGXX, "-O1", "-g", "-std=c++17"]
    driver_cmd += ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    driver_cmd += ["-fno-omit-frame-pointer", "-I" + os.path.join(ROOT, "include"),
                   os.path.join(HERE, "api_driver.cpp"), "-o", exe, "-L" + str(tmp_path),
                   "-lnaju_san", "-Wl,-rpath," + str(tmp_path), "-L/opt/rocm/lib", "-lamdhip64",
                   "-Wl,-rpath,/opt/rocm/lib"]
    rc, out = _run(driver_cmd)
    assert rc == 0, "driver build failed:\n" + out[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    rc, out = _run([exe], env=env)
    assert rc == 0 and "api driver: ok" in out, out[-5000:]
