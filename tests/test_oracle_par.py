"""The row-range split used for full-size parity gives the oracle's whole-tensor bytes."""
import numpy as np

import oracle
import oracle.par as op
import synth_inputs as si


def test_split_oracle_equals_whole_tensor_oracle():
    a = si.activation(272, 400, seed=3)
    gs = oracle.tensor_scale(oracle.amax(a))
    assert op.amax(a) == oracle.amax(a)
    for colwise in (False, True):
        for rnd in (oracle.RTN, oracle.SR):
            c, s = op.quantize_nvfp4(a, colwise, gs, rnd=rnd, seed=5)
            cw, sw, _ = oracle.quantize_nvfp4(a, colwise=colwise, gs=gs, rnd=rnd, seed=5)
            assert np.array_equal(c, cw) and np.array_equal(s, sw)
    w = si.weight(96, 160, seed=1)
    gw = oracle.tensor_scale(oracle.amax(w))
    c, s = op.quantize_nvfp4_2d(w, gw)
    cw, sw, _ = oracle.quantize_nvfp4_2d(w, gs=gw)
    assert np.array_equal(c, cw) and np.array_equal(s, sw)
    y = op.dequantize(oracle.FMT_NVFP4_2D, c, s, gw, 96, 160)
    assert np.array_equal(y.view(np.uint32), oracle.dequantize(oracle.FMT_NVFP4_2D, c, s, gw, 96, 160).view(np.uint32))
    c, s = op.quantize_mxfp4_rtn(w)
    cw, sw = oracle.quantize_mxfp4(w)
    assert np.array_equal(c, cw) and np.array_equal(s, sw)
    m = si.if4_mix(200, 64, seed=2)
    gm = oracle.tensor_scale(oracle.amax(m))
    c, s = op.quantize_if4(m, gm)
    cw, sw, _ = oracle.quantize_if4(m, gs=gm)
    assert np.array_equal(c, cw) and np.array_equal(s, sw)
    y = op.dequantize(oracle.FMT_IF4, c, s, gm, 200, 64)
    assert np.array_equal(y.view(np.uint32), oracle.dequantize(oracle.FMT_IF4, c, s, gm, 200, 64).view(np.uint32))
    g = si.wgrad_gradient(512, 72, seed=1)
    sg = oracle.rht_signs(4)
    assert np.array_equal(op.rht(g, sg).view(np.uint32), oracle.rht(g, sg).view(np.uint32))
