"""CPU sanitizer runs (no GPU):
* the oracle under AddressSanitizer + UndefinedBehaviorSanitizer, driven over
  every function and its edge cases (tests/oracle_sanitize_driver.c);
* the oracle under ThreadSanitizer, the same calls from eight threads at once
  (as the test suite's thread pool makes them);
* the C ABI's host code (argument validation, workspace planning, the
  no-device paths: tests/test_abi_cpu.py) in a library whose host half is
  built with AddressSanitizer + UndefinedBehaviorSanitizer.
Kernels are not instrumented: device-side sanitizers are not used here."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")
ORACLE = os.path.join(ROOT, "oracle", "triattn_oracle.c")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _gcc_supports(flag, tmp_path):
    src = tmp_path / "probe.c"
    src.write_text("int main(void){return 0;}\n")
    r = subprocess.run(["gcc", flag, str(src), "-o", str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def _run_driver(tmp_path, flags, name):
    exe = tmp_path / name
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", *flags, DRIVER, ORACLE, "-lm", "-lpthread",
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", f"{name}: rc {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    if not _gcc_supports("-fsanitize=address,undefined", tmp_path):
        pytest.skip("gcc has no address/undefined sanitizer runtime here")
    _run_driver(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"], "drv_asan")


def test_oracle_threads_under_thread_sanitizer(tmp_path):
    if not _gcc_supports("-fsanitize=thread", tmp_path):
        pytest.skip("gcc has no thread sanitizer runtime here")
    _run_driver(tmp_path, ["-fsanitize=thread", "-DTHREADS"], "drv_tsan")


def _clang_asan_runtime():
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_host_code_under_address_sanitizer(tmp_path):
    """tests/test_abi_cpu.py against a library whose api.hip host code is built
    with ASan + UBSan (the kernels' objects are the regular build's)."""
    objs = [os.path.join(ROOT, "long_reasoning_decode_amd", "_build", f"{n}.o")
            for n in ("score", "select", "decode", "calib")]
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run __graft_entry__.build() first)")
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime not found")
    api_o = tmp_path / "api_asan.o"
    lib = tmp_path / "libtriattn_asan.so"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
                    "-Xarch_host", "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-c", os.path.join(ROOT, "long_reasoning_decode_amd", "csrc", "api.hip"),
                    "-o", str(api_o)], check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-Xarch_host", "-shared-libsan",
                    "-o", str(lib), str(api_o), *objs], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, TRIATTN_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, f"ABI tests under ASan failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert "passed" in r.stdout
