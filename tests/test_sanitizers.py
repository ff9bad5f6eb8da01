"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

  * the CPU oracle (oracle/oracle.c) with a driver that runs every exported
    function on small ragged inputs (tests/sanitize/oracle_driver.c), built
    with gcc;
  * the C ABI's host code (every csrc/*.hip, sanitizers on the host side only:
    each -fsanitize= sits behind -Xarch_host, the GPU code is built as usual
    and never runs) with a driver that makes every call the library must
    answer on the host (tests/sanitize/abi_host_driver.cpp).

Any out-of-bounds access, leak or undefined behaviour aborts the driver."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(exe):
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{exe} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fopenmp", "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(SAN, "oracle_driver.c"), "-lm"], check=True)
    assert "oracle driver ok" in run(exe)


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "sparse_attention_token_lightning_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g"] + HOST_SAN +
                   ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
                    "-I", os.path.join(ROOT, "include"), "-o", exe] + srcs + [os.path.join(SAN, "abi_host_driver.cpp")],
                   check=True, capture_output=True)
    assert "abi host driver ok" in run(exe)
