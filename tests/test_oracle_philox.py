"""Pin the oracle's Philox4x32-10 against rocRAND's independent implementation.

rocRAND ships Philox4x32-10 as host-callable source (rocrand_philox4x32_10.h); a
small helper program (rocrand_philox_ref.cpp) seeds its engine so that it evaluates
the bijection at a chosen (counter, key), and the oracle must agree word for word.
The helper maps counter words 0-1 through rocRAND's `offset` argument (times 4), so
the test keeps word 1 below 2^30.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers / hipcc not available")
    exe = str(tmp_path_factory.mktemp("rr") / "rr")
    subprocess.run([hipcc, "-O1", "-x", "c++", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(rows):
        text = "".join("%08x %08x %08x %08x %08x %08x\n" % tuple(int(v) for v in r) for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w, 16) for w in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint32)

    return run


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(123)
    rows = rng.integers(0, 2**32, size=(300, 6), dtype=np.uint64).astype(np.uint32)
    rows[:, 1] &= np.uint32(0x3FFFFFFF)
    special = np.array([[0, 0, 0, 0, 0, 0], [1, 0, 0, 0, 0, 0], [0, 0, 1, 0, 0, 0],
                        [0, 0, 0, 1, 4, 0], [0, 0, 0, 1, 0xFFFFFFFF, 0xFFFFFFFF],
                        [7, 0, 1, 0, 40, 0], [0x3FFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 1, 2]],
                       dtype=np.uint32)
    rows = np.concatenate([special, rows])
    ref = rocrand_ref(rows)
    got = np.stack([oracle.philox4x32_10(r[:4], r[4:]) for r in rows])
    assert np.array_equal(got, ref)


def test_sr_draws_and_rht_signs_use_the_stated_counters(rocrand_ref):
    seed = 0x0000000500000029
    key = [seed & 0xFFFFFFFF, seed >> 32]
    idx = np.array([0, 1, 2, 7, 8, 9, 15, 16, 12345, 2**33 + 5], dtype=np.uint64)
    rows = []
    for stream in (0, 1):
        for i in idx.tolist():
            g = i >> 3
            rows.append([g & 0xFFFFFFFF, g >> 32, stream, 0] + key)
    ref = rocrand_ref(np.array(rows, dtype=np.uint32))
    k = 0
    for stream in (0, 1):
        got = oracle.sr_bits16(seed, stream, idx)
        for n, i in enumerate(idx.tolist()):
            word = int(ref[k + n][(i >> 1) & 3])
            expect = (word & 0xFFFF) if (i & 1) else (word >> 16)
            assert got[n] == expect
        k += len(idx)
    sref = rocrand_ref(np.array([[0, 0, 0, 1] + key], dtype=np.uint32))[0]
    assert np.array_equal(oracle.rht_signs(seed), sref)


def test_sr_draws_are_uniform_16_bit():
    # 2^20 draws: every 16-bit value class is hit about equally (chi-square, 256 bins)
    d = oracle.sr_bits16(99, 0, np.arange(1 << 20, dtype=np.uint64))
    assert d.max() < 65536
    h = np.bincount(d >> 8, minlength=256)
    e = d.size / 256
    chi2 = float(((h - e) ** 2 / e).sum())
    assert chi2 < 400           # 255 dof: mean 255, sd ~22.6
    # the two streams are different draws
    d1 = oracle.sr_bits16(99, 1, np.arange(1 << 12, dtype=np.uint64))
    assert np.count_nonzero(d1 != d[: 1 << 12]) > 4000
