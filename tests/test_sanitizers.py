"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU reference (oracle/oracle.cpp) is rebuilt with g++
  -fsanitize=address,undefined and the reference's own pin tests run
  against that build in a child process (the sanitizer runtimes preloaded
  into Python, leak checks off for the interpreter).
* The host side of the C ABI (qstate_api.cpp: argument checks, layout,
  launch parameters) is built with the same flags into a harness
  (tests/san/abi_host_harness.cpp) whose stand-in dispatcher checks every
  launch's parameters; no GPU is involved.
* A planted heap overflow in a throwaway library shows the sanitizer is live
  in the child process."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not found")
    d = tmp_path_factory.mktemp("san")
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return d, env


def test_sanitizer_is_live(san_env):
    d, env = san_env
    src = d / "planted.cpp"
    src.write_text('extern "C" int poke(int n) { int* a = new int[4]; a[n] = 1; int r = a[0];'
                   ' delete[] a; return r; }\n'
                   'extern "C" int twice(int x) { return x + x; }\n')
    for flags, call, finding in (
            (["-fsanitize=address"], "poke(4)", "heap-buffer-overflow"),
            (["-fsanitize=undefined", "-fno-sanitize-recover=all"], "twice(2**30)",
             "signed integer overflow")):
        lib = d / f"libplanted_{len(flags)}.so"
        subprocess.run(["g++", "-shared", "-fPIC", "-g", "-O0", *flags, "-o", str(lib), str(src)],
                       check=True)
        code = f"import ctypes; ctypes.CDLL({str(lib)!r}).{call}"
        p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                           text=True, timeout=120)
        assert p.returncode != 0 and finding in p.stderr, p.stderr[-2000:]


def test_oracle_pins_under_sanitizers(san_env):
    d, env = san_env
    lib = d / "liboracle_san.so"
    subprocess.run(["g++", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", *SAN, "-o", str(lib), os.path.join(ROOT, "oracle", "oracle.cpp")],
                   check=True)
    env = dict(env, QSTATE_ORACLE_LIB=str(lib))
    tests = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in tests]],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    tail = (p.stdout + p.stderr)[-3000:]
    assert p.returncode == 0, tail
    assert "passed" in p.stdout and "ERROR: AddressSanitizer" not in p.stderr, tail


def test_abi_host_side_under_sanitizers(san_env):
    d, _ = san_env
    exe = d / "abi_host_harness"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "bit_recurrent_state_amd", "csrc"),
                    os.path.join(ROOT, "bit_recurrent_state_amd", "csrc", "qstate_api.cpp"),
                    os.path.join(ROOT, "tests", "san", "abi_host_harness.cpp"), "-o", str(exe)],
                   check=True)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert p.returncode == 0, (p.stdout + p.stderr)[-3000:]
    assert p.stdout.startswith("ok:"), p.stdout
