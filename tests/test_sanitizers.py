"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only):
the plan/accumulator bookkeeping of the HIP library (fuzzed with random and
invalid layouts), the matrix-core kernels' workgroup-to-tile map, and the C
oracle (driven through its pins)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_rmsnorm_backward_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def test_plan_bookkeeping_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    subprocess.run(["g++", "-std=c++17", *SAN, f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "native", "plan_fuzz.cpp"),
                    os.path.join(CSRC, "plan.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan fuzz: ok" in r.stdout


def test_gemm_tile_map_takes_every_tile_once(tmp_path):
    """The constexpr tile map that linear.hip launches with, run on the host."""
    exe = str(tmp_path / "tile_map_check")
    subprocess.run(["g++", "-std=c++17", *SAN, f"-I{CSRC}",
                    os.path.join(ROOT, "tests", "native", "tile_map_check.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "tile map: ok" in r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    """Rebuild the oracle with the sanitizers and run every pin against it."""
    import oracle
    from tests import test_oracle_pins as pins
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", *oracle.GCC_FLAGS, *SAN, *oracle.SRCS, "-o", so, "-lm"], check=True)
    # the sanitizer runtime must be loaded first: run the pins in a child process
    code = (
        "import sys, inspect; sys.path.insert(0, %r)\n"
        "import oracle\n"
        "from tests import test_oracle_pins as pins\n"
        "orc = oracle.load_library(%r)\n"
        "for pin in list(pins.PINS) + list(pins.LINEAR_PINS) + list(pins.EMBEDDING_PINS):\n"
        "    args = [orc] + ([1e-6] if 'eps' in inspect.signature(pin).parameters else [])\n"
        "    pin(*args)\n"
        "print('oracle pins under sanitizers: ok')\n" % (ROOT, so))
    asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    ubsan_rt = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                              text=True).stdout.strip()
    env = {**os.environ, "LD_PRELOAD": f"{asan_rt} {ubsan_rt}", "ASAN_OPTIONS": "detect_leaks=0"}
    r = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ok" in r.stdout
