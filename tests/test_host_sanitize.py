"""The library's host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

tests/host_san/ holds two randomized drivers:
  * fuzz_abi: the C boundary (sweeps of 1..40 jobs of every format and path,
    launches of more than 4 GiB of weights, which take the stream kernel's
    big step shape, allocation-free sweeps in a row on the shared scratch,
    the verify head, round replay, attention verify, pack)
    built from the
    library's own host sources, with the HIP runtime and the kernel launchers
    replaced by host stand-ins that touch every region each kernel would
    touch.  Valid calls get buffers and workspaces of exactly the documented
    sizes; invalid ones must be rejected before any launch.
  * fuzz_oracle: quantize -> pack -> unpack -> dequant -> sweep round trips
    through the oracle's C functions.
Each is built with gcc/g++ (host code only) and run on a few seeds; any
sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
CSRC = os.path.join(ROOT, "self_speculative_verify_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_san")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build(cmd):
    r = subprocess.run(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]


@pytest.fixture(scope="module")
def bins(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("no host compiler")
    if not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("no HIP headers")
    d = tmp_path_factory.mktemp("san")
    abi, orc = str(d / "fuzz_abi"), str(d / "fuzz_oracle")
    _build(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-o", abi,
            os.path.join(HERE, "fuzz_abi.cpp"), os.path.join(HERE, "hip_stub.cpp"),
            os.path.join(CSRC, "qgemm_host.cpp"), os.path.join(CSRC, "attn_host.cpp")])
    _build(["gcc", "-std=c11", *SAN, "-pthread", "-o", orc,
            os.path.join(HERE, "fuzz_oracle.c"), os.path.join(ROOT, "oracle", "qg_oracle.c"), "-lm"])
    return abi, orc


def _run(binary, seed, iters):
    r = subprocess.run([binary, str(seed), str(iters)], stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                       text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok "), (r.returncode, r.stdout, r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    return int(r.stdout.split()[1])


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_abi_under_sanitizers(bins, seed):
    assert _run(bins[0], seed, 300) >= 300


@pytest.mark.parametrize("seed", [21, 22])
def test_oracle_under_sanitizers(bins, seed):
    assert _run(bins[1], seed, 300) == 300
