"""Pins for the oracle's random Hadamard transform (CPU only).

Checked against: the Sylvester recursion built independently, H H^T = 128 I in
integers, an independent fast Walsh-Hadamard transform in binary64, orthogonality
(norm preservation), inverse-after-forward, and the Wgrad identity the page
states: the transformed operands give the same product (dY H)(H^T x) = dY x.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si


def _sylvester(n):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _oracle_h():
    return np.array([[oracle.hadamard_entry(i, t) for t in range(128)] for i in range(128)], dtype=np.int64)


def _signs(mask):
    return np.array([-1.0 if (int(mask[t >> 5]) >> (t & 31)) & 1 else 1.0 for t in range(128)])


def test_hadamard_is_sylvester_and_orthogonal():
    h = _oracle_h()
    assert np.array_equal(h, _sylvester(128))
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def _fwht_rows(a):
    """Unnormalised fast Walsh-Hadamard transform along axis 0 (length 128), binary64."""
    a = a.astype(np.float64).copy()
    h = 1
    while h < a.shape[0]:
        a = a.reshape(-1, 2, h, a.shape[-1])
        x, y = a[:, 0].copy(), a[:, 1].copy()
        a[:, 0], a[:, 1] = x + y, x - y
        a = a.reshape(-1, a.shape[-1])
        h *= 2
    return a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rht_matches_independent_fast_transform(dtype):
    rows, cols = 256, 24
    x = si.wgrad_activation(rows, cols, seed=3) if dtype == "bf16" else si.weight(rows, cols, seed=3, std=1.0)
    xf = si.bf16_bits_to_f32(x) if dtype == "bf16" else x
    mask = oracle.rht_signs(4)
    s = _signs(mask)
    y = oracle.rht(x, mask)
    ref = np.empty_like(y)
    for c in range(0, rows, 128):
        blk = xf[c:c + 128].astype(np.float64) * s[:, None]
        ref[c:c + 128] = (_fwht_rows(blk) / np.sqrt(128.0)).astype(np.float32)
    if dtype == "bf16":
        # bf16 inputs: both binary64 sums are exact, so the roundings agree bit for bit
        assert np.array_equal(y, ref)
    else:
        assert np.max(np.abs(y - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2 ** -23


def test_rht_preserves_norms_and_inverts():
    x = si.wgrad_gradient(384, 16, seed=6)
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    mask = oracle.rht_signs(11)
    y = oracle.rht(x, mask)
    for c in range(0, 384, 128):
        n0 = np.linalg.norm(xf[c:c + 128], axis=0)
        n1 = np.linalg.norm(y[c:c + 128].astype(np.float64), axis=0)
        assert np.allclose(n0, n1, rtol=1e-6, atol=0)
    back = oracle.rht(y, mask, inverse=True)
    assert np.allclose(back, xf, rtol=0, atol=4e-7 * np.max(np.abs(xf)))


def test_rht_unit_vectors_give_signed_hadamard_columns():
    mask = oracle.rht_signs(5)
    s = _signs(mask)
    h = _sylvester(128)
    e = np.zeros((128, 128), np.float32)
    e[np.arange(128), np.arange(128)] = 1.0            # column j is the unit vector e_j
    y = oracle.rht(e, mask)
    expect = (h * s[None, :] / np.sqrt(128.0)).astype(np.float32)   # column t: s_t H[:, t] / sqrt(128)
    assert np.array_equal(y, expect)


def test_wgrad_product_is_preserved():
    """Per the page, W'grad = q(dY H) q(H^T x) relies on (dY H)(H^T x) = dY x; in the
    token-major layout that is B_G^T B_X = G^T X for the same transform on both."""
    g = si.bf16_bits_to_f32(si.wgrad_gradient(256, 12, seed=1)).astype(np.float64)
    xa = si.bf16_bits_to_f32(si.wgrad_activation(256, 10, seed=1)).astype(np.float64)
    mask = oracle.rht_signs(9)
    bg = oracle.rht(si.f32_to_bf16_bits(g.astype(np.float32)), mask).astype(np.float64)
    bx = oracle.rht(si.f32_to_bf16_bits(xa.astype(np.float32)), mask).astype(np.float64)
    lhs, rhs = bg.T @ bx, g.T @ xa
    assert np.allclose(lhs, rhs, rtol=1e-5, atol=1e-6 * np.max(np.abs(rhs)))


def test_rht_column_equals_full_transform_column():
    x = si.wgrad_gradient(256, 20, seed=2)
    mask = oracle.rht_signs(1)
    y = oracle.rht(x, mask)
    for j in (0, 7, 19):
        assert np.array_equal(oracle.rht_column(x, j, mask), y[:, j])
