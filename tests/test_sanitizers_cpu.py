"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two instrumented builds, each exercised by the CPU tests that already cover
it, in a child process with the sanitizer runtime preloaded and every report
fatal:
  * the fp64 oracle (gcc, -fsanitize=address,undefined) under the oracle's
    pins (test_oracle_pins.py);
  * the library's host code, the argument checks of every entry point
    (fa_api.hip, fa_noalloc.hip built by hipcc with the sanitizers on the
    host side only, linked with the uninstrumented kernel objects) under the
    C ABI tests (test_abi_cpu.py), which call every entry point with valid
    and invalid arguments.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from tiled_attention_fa_amd import build as hipbuild  # noqa: E402

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run_tests(test_file, env_extra, preload):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", lib, os.path.join(ROOT, "oracle", "fa_oracle.c"), "-lm"], check=True)
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                        check=True).stdout.strip()
    out = _run_tests("test_oracle_pins.py", {"FA_TEST_LIBORACLE": lib}, rt)
    print(out.strip().splitlines()[-1])


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return hits[-1]


def test_abi_host_code_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    host_srcs = ("fa_api.hip", "fa_noalloc.hip")
    objs = []
    for name in host_srcs:
        objs.append(hipbuild._compile(os.path.join(hipbuild.CSRC, name), HOST_SAN + ["-g"], str(tmp_path)))
    # the kernels, uninstrumented (device code cannot be), from the regular
    # build folder, compiled here if that build has not run
    kernel_srcs = [s for s in sorted(glob.glob(os.path.join(hipbuild.CSRC, "*.hip")))
                   if os.path.basename(s) not in host_srcs]
    kdir = tmp_path / "kernels"
    kdir.mkdir()
    for s in kernel_srcs:
        built = os.path.join(hipbuild.BUILD_DIR, os.path.basename(s) + ".o")
        if os.path.exists(built) and os.path.getmtime(built) >= os.path.getmtime(s):
            objs.append(built)
        else:
            objs.append(hipbuild._compile(s, [], str(kdir)))
    lib = str(tmp_path / "libfa_san.so")
    subprocess.run([hipbuild.hipcc(), f"--offload-arch={hipbuild.ARCH}", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    *objs, "-o", lib], check=True, capture_output=True)
    out = _run_tests("test_abi_cpu.py", {"FA_TEST_LIBFA": lib}, rt)
    print(out.strip().splitlines()[-1])
