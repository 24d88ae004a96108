"""Host checks of the exact-arithmetic building blocks the kernels rely on.

The kernels divide by block scales with a precomputed reciprocal pair (one
multiplication and one fused multiply-add per element) instead of IEEE division,
and form the pair from the hardware reciprocal estimate plus one Newton step.
host_checks/division_check.c verifies both exhaustively over every dividend
significand and every E4M3 divisor (CPU only, libm fmaf).  Dequantization divides
by the FP32 tensor scale with a corrected reciprocal; host_checks/
dequant_division_check.c verifies it for every dividend the decoders of all block
formats (NVFP4, IF4, the variants) can form against every divisor significand."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_corrected_reciprocal_division_is_exact(tmp_path):
    exe = str(tmp_path / "division_check")
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "host_checks", "division_check.c"), "-o", exe, "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout


def test_dequant_division_is_exact(tmp_path):
    exe = str(tmp_path / "dequant_division_check")
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "host_checks", "dequant_division_check.c"), "-o", exe, "-lm"],
                   check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
