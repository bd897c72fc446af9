"""The CPU code built with AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/gdn_oracle.c), compiled with its own flags plus
  -fsanitize=address,undefined, runs every pin, and every planted mistake of
  test_oracle_mutants.py is still caught (by a pin, or by a sanitizer report).
* The C ABI's host code (gated_deltanet_recurrent_amd/csrc/gdn_api.cpp: the
  argument validation that runs before anything is enqueued) is compiled for
  the host alone with g++ and the same sanitizers, against test-only
  launchers that count their calls (tests/sanitize/launch_stub.cpp) and a
  stand-in HIP header (tests/sanitize/hip/), and runs test_abi_host.py; refused
  calls must not reach a launcher.

Each sanitized library is loaded into a Python subprocess that has the ASan
runtime preloaded; any sanitizer report aborts that process, which fails the
test.  No GPU is used.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g"]


def _runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    if p.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _env():
    env = dict(os.environ)
    pre = _runtime()
    env["LD_PRELOAD"] = pre + ((" " + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = ROOT
    return env


def _python(code, env, cwd=ROOT):
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          cwd=cwd, timeout=600)


def _build_oracle(src, out):
    import oracle
    cmd = ["gcc", *oracle.CFLAGS, *SAN, "-I", os.path.dirname(oracle.SRC), "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


PINS_SCRIPT = """
import sys
import oracle
from tests import test_oracle_pins as pins
orc = oracle.Oracle({so!r})
failed = []
for pin in pins.PINS:
    try:
        pin(orc)
    except (AssertionError, ValueError, FloatingPointError):
        failed.append(pin.__name__)
print("FAILED_PINS", len(failed), ",".join(failed))
"""


def test_oracle_pins_under_sanitizers(tmp_path):
    env = _env()
    so = _build_oracle(os.path.join(ROOT, "oracle", "gdn_oracle.c"), str(tmp_path / "san.so"))
    r = _python(PINS_SCRIPT.format(so=so), env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "FAILED_PINS 0 " in r.stdout, r.stdout[-2000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_planted_mistakes_under_sanitizers(tmp_path):
    from tests.test_oracle_mutants import MUTANTS
    import oracle
    env = _env()
    src = open(oracle.SRC).read()
    shutil.copy(os.path.join(os.path.dirname(oracle.SRC), "gdn_oracle.h"), tmp_path)

    def run(m):
        name, old, new = m
        assert old in src, f"mutation site not found: {old!r}"
        tag = "".join(c if c.isalnum() else "_" for c in name)
        c_path = tmp_path / f"m_{tag}.c"
        c_path.write_text(src.replace(old, new))
        so = _build_oracle(str(c_path), str(tmp_path / f"m_{tag}.so"))
        r = _python(PINS_SCRIPT.format(so=so), env)
        by_pin = r.returncode == 0 and "FAILED_PINS 0 " not in r.stdout
        by_sanitizer = r.returncode != 0 and ("runtime error" in r.stderr or
                                              "AddressSanitizer" in r.stderr)
        return name, by_pin, by_sanitizer, r.returncode, r.stderr[-1500:]

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        results = list(ex.map(run, MUTANTS))
    for name, by_pin, by_sanitizer, rc, err in results:
        assert by_pin or by_sanitizer, (name, rc, err)


API_SCRIPT = """
import ctypes as C, sys
import pytest
import gated_deltanet_recurrent_amd as gdn
gdn.LIB_PATH = {so!r}
gdn._lib = None
L = gdn.lib()
L.gdn_stub_launches.restype = C.c_int64
rc = pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi_host.py"])
print("PYTEST_RC", int(rc))
print("LAUNCHES_AFTER_HOST_TESTS", L.gdn_stub_launches())
# calls that pass validation reach exactly the launchers they should
S, q, k, v, g, b, o = (C.c_void_p(0x7f0000000000 + (i << 32)) for i in range(7))
before = L.gdn_stub_launches()
assert L.gdn_step(S, q, k, v, g, b, o, 3, 48, 16, 128, 128, None) == 0
assert L.gdn_stub_launches() == before + 1
assert L.gdn_step(S, q, k, v, g, b, S, 3, 48, 16, 128, 128, None) == gdn.GDN_EINVAL
assert L.gdn_stub_launches() == before + 1
print("STUB_CHECKS_OK")
"""


def test_api_validation_under_sanitizers(tmp_path):
    env = _env()
    so = str(tmp_path / "libgdn_hostcheck.so")
    csrc = os.path.join(ROOT, "gated_deltanet_recurrent_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-fPIC", "-shared", "-Wall", *SAN,
           "-I", os.path.join(ROOT, "tests", "sanitize"), "-I", os.path.join(ROOT, "include"),
           "-I", csrc, "-o", so, os.path.join(csrc, "gdn_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp")]
    subprocess.run(cmd, check=True, capture_output=True)
    r = _python(API_SCRIPT.format(so=so), env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-4000:])
    assert "PYTEST_RC 0" in r.stdout, r.stdout[-3000:]
    # every call in the host tests is refused or a no-op: nothing was launched
    assert "LAUNCHES_AFTER_HOST_TESTS 0" in r.stdout, r.stdout[-3000:]
    assert "STUB_CHECKS_OK" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    """The harness above would notice a memory error: an oracle copy whose
    mark reads one float past the end of S aborts with an ASan report."""
    import oracle
    env = _env()
    src = open(oracle.SRC).read()
    old = "memcpy(slab->S_snap, S, ns * sizeof(float));"
    assert old in src
    shutil.copy(os.path.join(os.path.dirname(oracle.SRC), "gdn_oracle.h"), tmp_path)
    c_path = tmp_path / "overflow.c"
    c_path.write_text(src.replace(old, "memcpy(slab->S_snap, S, (ns + 1) * sizeof(float));"))
    so = _build_oracle(str(c_path), str(tmp_path / "overflow.so"))
    r = _python(PINS_SCRIPT.format(so=so), env)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])
