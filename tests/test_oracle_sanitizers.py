"""The oracle's C source under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): every pin runs against a sanitized build, and a planted
out-of-bounds access in a copy of the source is reported, which shows the
sanitized build is live."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _build(src, out):
    subprocess.run(["gcc", *FLAGS, src, "-o", out, "-lm"], check=True, capture_output=True, text=True)
    return out


def _pins(lib, log, tests="tests/test_oracle_pins.py"):
    """Run the pins against `lib`; returns (exit status, sanitizer reports)."""
    env = dict(os.environ, SDNQ_ORACLE_LIB=lib, LD_PRELOAD=_runtime(), OMP_NUM_THREADS="4",
               ASAN_OPTIONS=f"detect_leaks=0:log_path={log}", UBSAN_OPTIONS=f"print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    d = os.path.dirname(log)
    reports = "".join(open(os.path.join(d, f)).read() for f in os.listdir(d) if f.startswith(os.path.basename(log)))
    return r.returncode, reports + r.stderr


@pytest.mark.slow
def test_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if _runtime() is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = _build(oracle._SRC, str(tmp_path / "liboracle_san.so"))
    rc, reports = _pins(lib, str(tmp_path / "san"))
    assert rc == 0, reports[-3000:]
    assert "AddressSanitizer" not in reports and "runtime error" not in reports


@pytest.mark.slow
def test_a_planted_out_of_bounds_read_is_reported(tmp_path):
    if _runtime() is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(oracle._SRC).read()
    old = "    for (int64_t i = 0; i < n; i++)\n        out[i] = bf16_decode(h[i]);"
    assert src.count(old) == 1
    bad = tmp_path / "oob.c"
    bad.write_text(src.replace(old, "    for (int64_t i = 0; i <= n; i++)\n        out[i] = bf16_decode(h[i]);"))
    lib = _build(str(bad), str(tmp_path / "liboracle_oob.so"))
    rc, reports = _pins(lib, str(tmp_path / "san"))
    assert rc != 0 and "AddressSanitizer" in reports and "oracle_f32_from_bf16" in reports
