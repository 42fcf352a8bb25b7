"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: tests/oracle_sanitize.c drives
every oracle function (every payload format, the expert-parallel chain, conversions of special
values, rejected arguments) in a build with -fsanitize=address,undefined; any out-of-bounds access,
leak or undefined arithmetic aborts it. CPU only."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "moe_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize.c"), "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
