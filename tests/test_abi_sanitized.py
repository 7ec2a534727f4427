"""Host validation of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled with both sanitizers on its host pass
(the device code is built as usual but never runs), linked with
tests/sanitize/abi_driver.cpp, and run on the CPU:
the driver feeds extreme and invalid arguments to every entry point, each of
which must return its documented status before any launch.  A sanitizer
finding aborts the run."""

import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_video_cube_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    from block_sparse_video_cube_amd import build

    # The sanitizers apply to the host pass only (-Xarch_host); the device
    # code is built as usual (gfx950) so the objects link, but never runs.
    common = ["-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmds, objs = [], []
    for src in build.SOURCES:
        obj = os.path.join(tmp_path, src + ".o")
        cmds.append([HIPCC, f"--offload-arch={build.ARCH}", "-Xclang", "-target-feature", "-Xclang",
                     "-packed-fp32-ops", *common, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    drv = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
    objs.append(os.path.join(tmp_path, "abi_driver.o"))
    cmds.append([HIPCC, "--offload-host-only", *common, "-c", drv, "-o", objs[-1]])
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
    for r in results:
        assert r.returncode == 0, r.stderr[-3000:]
    exe = os.path.join(tmp_path, "abi_driver")
    r = subprocess.run([HIPCC, f"--offload-arch={build.ARCH}", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr[-3000:])
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "abi_driver: 0 failures" in r.stdout
