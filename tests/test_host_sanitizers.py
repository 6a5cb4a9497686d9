"""Host code under AddressSanitizer, UndefinedBehaviorSanitizer and ThreadSanitizer
(CPU only).

Drives in ``tests/sanitize/`` are compiled with the planner, the engine and the C ABI
(device code replaced by stubs that no call reaches) and run: the planner over many plan
shapes, flags, budgets, fallbacks and dry runs, and the C ABI over its size queries,
argument checks and error paths, with ``-fsanitize=address,undefined`` (UBSan
non-recoverable); and the C ABI from eight threads at once with ``-fsanitize=thread``.
A sanitizer report makes the drive exit nonzero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_bounded_streaming_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CXX = os.path.join(ROCM, "llvm", "bin", "clang++")
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-w"]


TSAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include", "-w"]


def _build_and_run(tmp_path, sources, libs=(), flags=FLAGS):
    if not os.path.exists(CXX):
        pytest.skip("clang++ of the ROCm toolchain is not available")
    exe = str(tmp_path / "drive")
    build = subprocess.run([CXX, *flags, *sources, "-o", exe, *libs], stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
    assert build.returncode == 0, build.stdout[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=600)
    assert run.returncode == 0 and "runtime error" not in run.stdout and "ERROR:" not in run.stdout \
        and "WARNING: ThreadSanitizer" not in run.stdout, run.stdout[-4000:]
    return run.stdout


def test_planner_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, [os.path.join(SAN, "planner_drive.cpp"), os.path.join(CSRC, "plan.cpp")])
    assert "plans built" in out


def test_c_abi_under_sanitizers(tmp_path):
    if shutil.which("nm") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("the HIP runtime library is not available to link")
    out = _build_and_run(tmp_path, [os.path.join(SAN, "abi_drive.cpp"), os.path.join(SAN, "stubs.cpp"),
                                    os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
                                    os.path.join(CSRC, "engine.cpp")],
                         libs=[f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    assert "plans created" in out


def test_c_abi_from_many_threads_under_thread_sanitizer(tmp_path):
    if not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("the HIP runtime library is not available to link")
    out = _build_and_run(tmp_path, [os.path.join(SAN, "threads_drive.cpp"), os.path.join(SAN, "stubs.cpp"),
                                    os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
                                    os.path.join(CSRC, "engine.cpp")],
                         libs=[f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], flags=TSAN_FLAGS)
    assert "plans created" in out
