"""The oracle's pins again, with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, gcc), in a child process that
preloads the sanitizer runtime.  Catches out-of-bounds accesses and
undefined arithmetic in the reference itself."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def test_pins_under_sanitizers(tmp_path):
    src = os.path.join(ROOT, "oracle", "lags_oracle.c")
    lib = str(tmp_path / "liblags_oracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", src, "-o", lib]
    subprocess.run(cmd, check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("the AddressSanitizer runtime is not installed")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle as O, pins\n"
            "orc = O.Oracle(%r)\n"
            "for p in pins.ALL_FAST_PINS:\n"
            "    p(orc)\n"
            "print('pins ok')\n") % (ROOT, HERE, lib)
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         timeout=600)
    assert res.returncode == 0 and "pins ok" in res.stdout, res.stdout[-2000:] + res.stderr[-4000:]
