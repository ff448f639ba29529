"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code (no GPU):

- the C ABI (csrc/kda_api.cpp and the host scheduling policy csrc/kda_plan.cpp) with the
  device launchers stubbed out, driven through every validation path of every entry point
  and through calls that pass validation (tests/sanitize/abi_driver.cpp);
- the fp64 oracle (oracle/kda_oracle.c) on a small packed batch with empty and one-token
  sequences, several threads and a pair subset (tests/sanitize/oracle_driver.c).

Both are built with g++/gcc -fsanitize=address,undefined -fno-sanitize-recover=all and
must exit cleanly."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_sequence_chunked_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(
    os.path.join(ROCM, "lib", "libamdhip64.so")), reason="needs g++ and the HIP runtime")
def test_c_abi_host_paths_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
         f"-I{ROOT}/include", f"-I{CSRC}"] + SAN +
        [os.path.join(CSRC, "kda_api.cpp"), os.path.join(CSRC, "kda_plan.cpp"),
         os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"),
         f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = run([exe], env=env)
    assert "0 unexpected results" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11"] + SAN + [os.path.join(ROOT, "oracle", "kda_oracle.c"),
                                     os.path.join(HERE, "oracle_driver.c"), "-lpthread",
                                     "-lm", "-o", exe])
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="abort_on_error=1",
                            UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"))
    assert "0 problems" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
