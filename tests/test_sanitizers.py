"""The oracle and the library's host-side checks under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

Both are rebuilt with the sanitizers into a temporary folder: the oracle's C
files with gcc, the library with hipcc, the sanitizers on its host code only
(the device code is built without optimisation and never launched here). The
CPU tests that drive each of them then run again in a child process with the
matching sanitizer runtime preloaded (the Python interpreter itself is not
instrumented): the oracle's pins (every oracle function on its worked
examples, closed forms and edge cases) and the C ABI's argument, workspace,
plan and status checks. Any report ends the child with an error (halt on
error, no recovery from undefined behaviour), which fails the test.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1:detect_odr_violation=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _run_child(preload: str, setup: str, tests: list, tmp) -> None:
    """pytest over `tests` (their CPU cases) in a child process whose first
    statements are `setup` (pointing a loader at the sanitized build)."""
    driver = tmp / "driver.py"
    driver.write_text(
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        f"{setup}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-x', '-q', '-s', '-m', 'not gpu', '-p', 'no:cacheprovider'] + {tests!r}))\n")
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, str(driver)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    lines = r.stderr.splitlines()
    first = next((k for k, l in enumerate(lines) if "runtime error" in l or "ERROR: AddressSanitizer" in l), None)
    report = "\n".join(lines[first:first + 12]) if first is not None else r.stderr[-4000:]
    out = r.stdout[-3000:] + "\n" + report
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, out


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    srcs = [os.path.join(ROOT, "oracle", f) for f in ("ssd_oracle.c", "ssd_oracle_bwd.c")]
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11", "-o",
                    str(lib)] + srcs + ["-lm", "-lpthread"], check=True)
    tests = sorted(os.path.relpath(p, ROOT) for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle*.py")))
    _run_child(asan, f"import oracle\noracle._LIB_PATH = {str(lib)!r}", tests, tmp_path)


def _clang_asan_runtime(hipcc: str):
    r = subprocess.run([hipcc, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if os.path.isabs(path) and os.path.exists(path):
        return path
    hits = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def test_library_host_checks_under_asan_ubsan(tmp_path):
    from selective_state_space_46_amd import build
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not installed")
    rt = _clang_asan_runtime(hipcc)
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in build.compile_flags() if f != "-O3"] + ["-O1", "-g", "-Xarch_device", "-O0"] + san

    def compile_one(src):
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run([hipcc] + flags + ["-c", src, "-o", str(obj)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return str(obj)

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, build.sources()))
    lib = tmp_path / "libssd_san.so"
    r = subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={build.ARCH}", "-shared-libsan"] + san +
                       ["-o", str(lib)] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    _run_child(rt, f"import selective_state_space_46_amd as ssd\nssd._LIB_PATH = {str(lib)!r}",
               ["tests/test_abi.py", "tests/test_host_logic.py"], tmp_path)
