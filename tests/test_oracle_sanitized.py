"""The C oracle under the host sanitizers: tests/sanitize/oracle_drive.c runs
every oracle entry point on small seeded inputs and edge cases (zero length,
empty batch, one state, optional pointers left NULL, more threads than
channels, argument errors) and checks two identities (scan = decode steps,
SSD on heads = S6 with the head's A).  Built with gcc, once with
AddressSanitizer + UndefinedBehaviorSanitizer (leak detection on) and once
with ThreadSanitizer (the oracle splits channels over threads); any finding
aborts the driver.  Host code only; no GPU involved."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(ROOT, "oracle", "mssm_oracle.c"), os.path.join(HERE, "sanitize", "oracle_drive.c")]
GCC = shutil.which("gcc")


def _build_and_run(tmp_path, name, flags, env=None):
    exe = str(tmp_path / name)
    cmd = [GCC, "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer", "-pthread", *flags, *SRC, "-lm",
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0:
        pytest.skip(f"{name}: the sanitizer runtime is not available here ({b.stderr.strip()[:200]})")
    return subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)


@pytest.mark.skipif(GCC is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = _build_and_run(tmp_path, "drive_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"], env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "oracle drive: ok" in out, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]


@pytest.mark.skipif(GCC is None, reason="gcc not found")
def test_oracle_under_tsan(tmp_path):
    r = _build_and_run(tmp_path, "drive_tsan", ["-fsanitize=thread"])
    out = r.stdout + r.stderr
    if r.returncode != 0 and "FATAL: ThreadSanitizer" in out and "data race" not in out:
        pytest.skip("ThreadSanitizer cannot run in this environment: " + out.strip()[:200])
    assert r.returncode == 0 and "oracle drive: ok" in out, out[-3000:]
    assert "ThreadSanitizer" not in out, out[-3000:]
