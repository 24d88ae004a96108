"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (every entry point, driven by host_checks/oracle_driver.c on small,
ragged and degenerate inputs with exactly sized buffers) and the two exhaustive
arithmetic checks are built with gcc -fsanitize=address,undefined and
-fno-sanitize-recover=all, so any out-of-bounds access, use after free, leak,
signed overflow, invalid shift or similar undefined behaviour aborts the run."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
FLAGS = ["-std=c99", "-O1", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(tmp_path, name, sources, extra=(), args=()):
    exe = str(tmp_path / name)
    subprocess.run(["gcc", *FLAGS, *SAN, *extra, *sources, "-o", exe, "-lm"], check=True)
    res = subprocess.run([exe, *args], capture_output=True, text=True, timeout=600, env=ENV)
    print(res.stdout)
    print(res.stderr)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
    return res


def test_oracle_under_asan_ubsan(tmp_path):
    res = _build_and_run(tmp_path, "oracle_driver",
                         [os.path.join(HERE, "host_checks", "oracle_driver.c"),
                          os.path.join(ROOT, "oracle", "fp4q_oracle.c")],
                         ["-I", os.path.join(ROOT, "oracle")])
    assert "ran clean" in res.stdout


@pytest.mark.parametrize("check,args", [("division_check", ()), ("dequant_division_check", ("16",))])
def test_host_arithmetic_checks_under_asan_ubsan(tmp_path, check, args):
    # the dequantization check covers every divisor in its plain build; here every 16th
    _build_and_run(tmp_path, check, [os.path.join(HERE, "host_checks", check + ".c")], args=args)
