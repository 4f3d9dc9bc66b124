"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): the library and the oracle.

Every source is compiled with the sanitizers on the host side only (device code is built as
usual) into a private copy of libgdn.so; then
  * tests/c/abi_check.c, built with the same clang and sanitizers, runs against it, and
  * the ctypes ABI suite (tests/test_abi_cpu.py) runs against it in a child process that
    preloads the ASan runtime.
Both exercise the argument validation, which runs before any HIP call.  The float64 C oracle
(test infrastructure) is built with gcc's sanitizers and runs its pin and form tests.  A
sanitizer report stops the child with a non-zero status (leak checking is off: the HIP and
OpenMP runtimes keep their allocations until exit).
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_deltanet_recurrence_rule_amd")
ROCM_CLANG = "/opt/rocm/llvm/bin/clang"

# sanitizers on the host pass only; each -fsanitize= follows its -Xarch_host
HOST_SAN = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-omit-frame-pointer".split()
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _asan_runtime():
    r = subprocess.run([ROCM_CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    from gated_deltanet_recurrence_rule_amd import build as gdn_build

    if shutil.which(gdn_build.HIPCC) is None and not os.path.exists(gdn_build.HIPCC):
        pytest.skip("hipcc not available")
    if not os.path.exists(ROCM_CLANG) or _asan_runtime() is None:
        pytest.skip("the ROCm clang sanitizer runtime is not available")
    out = tmp_path_factory.mktemp("san")
    lib = gdn_build.build(extra_flags=["-O1", "-g", *HOST_SAN], out=str(out / "libgdn.so"),
                          build_dir=str(out / "obj"))
    return lib


def test_plain_c_program_under_sanitizers(san_lib, tmp_path):
    rt_dir = os.path.dirname(_asan_runtime())
    lib_dir = os.path.dirname(san_lib)
    exe = str(tmp_path / "abi_check")
    cmd = [ROCM_CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-shared-libsan", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe, "-L", lib_dir, "-lgdn",
           "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + rt_dir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env={**os.environ, **SAN_ENV})
    assert r.returncode == 0 and "all ok" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_abi_suite_under_sanitizers(san_lib, tmp_path):
    runner = tmp_path / "run_abi.py"
    runner.write_text(textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        from gated_deltanet_recurrence_rule_amd import binding
        binding.LIB_PATH = {san_lib!r}
        import pytest
        sys.exit(pytest.main(["-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
                              {os.path.join(ROOT, "tests", "test_abi_cpu.py")!r}]))
    """))
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": _asan_runtime()}
    r = subprocess.run([sys.executable, str(runner)], capture_output=True, text=True, timeout=600, env=env,
                       cwd=str(tmp_path))
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stdout + r.stderr and "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert " passed" in r.stdout, tail


def test_oracle_under_sanitizers(tmp_path):
    """The float64 C oracle, built with gcc's ASan and UBSan, runs its pin and form tests."""
    import oracle

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's ASan runtime is not available")
    lib = str(tmp_path / "libgdn_oracle.so")
    r = subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fopenmp",
                        "-shared", "-fPIC", "-Wall", oracle.SRC_PATH, "-o", lib, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    runner = tmp_path / "run_oracle.py"
    runner.write_text(textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import oracle
        oracle.LIB_PATH = {lib!r}
        import pytest
        sys.exit(pytest.main(["-q", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
                              {os.path.join(ROOT, "tests", "test_oracle_forms.py")!r},
                              {os.path.join(ROOT, "tests", "test_oracle_pins.py")!r}]))
    """))
    env = {**os.environ, "LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    r = subprocess.run([sys.executable, str(runner)], capture_output=True, text=True, timeout=900, env=env,
                       cwd=str(tmp_path))
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stdout + r.stderr and "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert " passed" in r.stdout, tail
