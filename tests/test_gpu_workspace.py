"""The caller-owned workspace and graph capture (GPU).

A workspace carries the tensor-amax hand-over between the kernels of a call.  These
tests check that (1) nothing of one call leaks into the next, with the tensor amax
falling from call to call so that a stale maximum would win; (2) a call captured into a
HIP graph on a fresh stream -- the first call the stream ever sees -- replays correctly
when the input changes between replays; (3) calls without a workspace give the same
bytes as calls with one; (4) a workspace can be destroyed and re-created.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from block_scaled_fp4_05_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_two_pass_state_does_not_leak_between_calls():
    """Falling tensor amax over many calls of every two-pass kind on one workspace."""
    ws = B.Workspace()
    rng = np.random.default_rng(3)
    base = rng.standard_normal((256, 384)).astype(np.float32)
    signs = oracle.rht_signs(9)
    for k in range(12):
        x = base * np.float32(2.0 ** -k)
        bits = si.f32_to_bf16_bits(x)
        xd = dev_bf16(bits)
        kind = k % 4
        if kind == 0:      # IF4: amax pass, then the IF4 quantizer
            out = B.quantize_if4(xd, ws=ws)
            c, s, gs = oracle.quantize_if4(bits)
            assert np.array_equal(host(out["codes"]), c) and np.array_equal(host(out["scales"]), s)
        elif kind == 1:    # 16x16
            out = B.quantize_nvfp4_2d(xd, ws=ws)
            c, s, gs = oracle.quantize_nvfp4_2d(bits)
            assert np.array_equal(host(out["codes"]), c) and np.array_equal(host(out["scales"]), s)
        elif kind == 2:    # RHT: transform amax pass, then the fused column-wise quantizer
            out = B.quantize_nvfp4(xd, B.COLWISE, rht_signs=signs.tolist(), ws=ws)
            y = host(B.rht(xd, signs.tolist()))
            gs = oracle.tensor_scale(float(np.max(np.abs(y))))
            c, s, _ = oracle.quantize_nvfp4(y, colwise=True, gs=gs)
            assert np.array_equal(host(out["col_codes"]), c) and np.array_equal(host(out["col_scales"]), s)
        else:              # MXFP4 reporting the amax
            out = B.quantize_mxfp4(xd, with_amax=True, ws=ws)
            gs = None
            assert host(out["amax"])[0] == np.float32(oracle.amax(bits))
        if gs is not None:
            assert host(out["tensor_scale"])[0] == np.float32(gs)
            if kind != 2:
                assert host(out["amax"])[0] == np.float32(oracle.amax(bits))
    torch.cuda.synchronize()
    ws.close()


def test_graph_capture_first_call_on_a_fresh_stream_replays_correctly():
    rows, cols = 512, 768
    ws = B.Workspace()                       # created before capture: capture allocates nothing
    x = torch.empty(rows, cols, dtype=torch.bfloat16, device=DEV)
    inputs = [si.activation(rows, cols, seed=s) for s in (51, 52, 53)]
    # the largest magnitude falls from replay to replay, so a stale amax would show
    inputs = [si.f32_to_bf16_bits(si.bf16_bits_to_f32(b) * np.float32(4.0 ** -i)) for i, b in enumerate(inputs)]
    x.copy_(dev_bf16(inputs[0]))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv = B.quantize_nvfp4(x, B.ROWWISE | B.COLWISE, ws=ws)
        i4 = B.quantize_if4(x, ws=ws)
        mx = B.quantize_mxfp4(x, with_amax=True, ws=ws)
        nv_none = B.quantize_nvfp4(x, B.ROWWISE, ws=None)
    for i, bits in enumerate(inputs):
        x.copy_(dev_bf16(bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rc, rs, gs = oracle.quantize_nvfp4(bits)
        cc, cs, _ = oracle.quantize_nvfp4(bits, colwise=True)
        assert host(nv["amax"])[0] == np.float32(oracle.amax(bits)), i
        assert host(nv["tensor_scale"])[0] == gs, i
        assert np.array_equal(host(nv["row_codes"]), rc) and np.array_equal(host(nv["row_scales"]), rs), i
        assert np.array_equal(host(nv["col_codes"]), cc) and np.array_equal(host(nv["col_scales"]), cs), i
        assert np.array_equal(host(nv_none["row_codes"]), rc) and host(nv_none["tensor_scale"])[0] == gs, i
        c4, s4, g4 = oracle.quantize_if4(bits)
        assert np.array_equal(host(i4["codes"]), c4) and np.array_equal(host(i4["scales"]), s4), i
        assert host(mx["amax"])[0] == np.float32(oracle.amax(bits)), i
        cm, sm = oracle.quantize_mxfp4(bits)
        assert np.array_equal(host(mx["codes"]), cm) and np.array_equal(host(mx["scales"]), sm), i
        # eager work on the same workspace between replays (the one-pass kernel here)
        eager = B.quantize_nvfp4(x, B.ROWWISE | B.COLWISE, ws=ws)
        assert torch.equal(eager["row_codes"], nv["row_codes"]) and torch.equal(eager["col_codes"], nv["col_codes"])
        assert torch.equal(eager["amax"], nv["amax"])
    del g
    torch.cuda.synchronize()
    ws.close()


def test_graph_capture_of_rht_2d_variant_dequant_and_gemm_calls_replays_correctly():
    """The other two-pass calls and the GEMM epilogue amax under capture: the RHT
    column-wise quantizer with SR, NVFP4 16x16, the IF6 variant with its dequantization,
    and an MXFP4 GEMM reporting max |C|.  Each replay, on a new input, stores what the same
    calls made eagerly on that input store (each eager path is checked against the oracle
    elsewhere)."""
    rows, cols = 512, 768
    ws = B.Workspace()
    signs = B.fp4q_rht_signs_from_seed(11)
    x = torch.empty(rows, cols, dtype=torch.bfloat16, device=DEV)
    inputs = [si.activation(rows, cols, seed=s) for s in (61, 62, 63)]
    inputs = [si.f32_to_bf16_bits(si.bf16_bits_to_f32(b) * np.float32(3.0 ** -i)) for i, b in enumerate(inputs)]
    x.copy_(dev_bf16(inputs[0]))
    torch.cuda.synchronize()

    def calls():
        r = B.quantize_nvfp4(x, B.COLWISE, rnd=B.SR, sr_seed=7, rht_signs=signs, ws=ws)
        t = B.quantize_nvfp4_2d(x, ws=ws)
        v = B.quantize_variant(x, B.VAR_IF6, ws=ws)
        y = B.dequantize_variant(B.VAR_IF6, v["codes"], v["scales"], v["tensor_scale"], rows, cols, torch.bfloat16)
        m = B.quantize_mxfp4(x, ws=ws)
        amax = torch.empty(1, dtype=torch.float32, device=DEV)
        c = B.gemm_mxfp4(m, m, torch.bfloat16, amax=amax)
        return {"rc": r["col_codes"], "rs": r["col_scales"], "rts": r["tensor_scale"], "tc": t["codes"],
                "tsc": t["scales"], "vc": v["codes"], "vs": v["scales"], "y": y, "c": c, "camax": amax}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = calls()
    for i, bits in enumerate(inputs):
        x.copy_(dev_bf16(bits))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = calls()
        torch.cuda.synchronize()
        for k in cap:
            assert torch.equal(cap[k], eager[k]), (i, k)
        assert cap["camax"].item() == cap["c"].float().abs().max().item(), i
    del g
    torch.cuda.synchronize()
    ws.close()


@pytest.mark.parametrize("shape", [(256, 512), (4000, 2608)])
def test_no_workspace_equals_workspace(shape):
    rows, cols = shape
    bits = si.activation(rows, cols, seed=61)
    xd = dev_bf16(bits)
    a = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE, ws=None)
    b = B.quantize_nvfp4(xd, B.ROWWISE | B.COLWISE)
    for k in ("row_codes", "row_scales", "col_codes", "col_scales", "amax", "tensor_scale"):
        assert torch.equal(a[k], b[k]), k
    a = B.quantize_if4(xd, ws=None)
    b = B.quantize_if4(xd)
    for k in ("codes", "scales", "amax", "tensor_scale"):
        assert torch.equal(a[k], b[k]), k


def test_workspace_destroy_and_recreate():
    bits = si.activation(128, 256, seed=71)
    xd = dev_bf16(bits)
    rc, rs, gs = oracle.quantize_nvfp4(bits)
    for _ in range(3):
        ws = B.Workspace()
        out = B.quantize_nvfp4(xd, B.ROWWISE, ws=ws)
        assert np.array_equal(host(out["row_codes"]), rc) and host(out["tensor_scale"])[0] == gs
        ws.close()
    with pytest.raises(B.Fp4qError):
        B.quantize_mxfp4(xd, with_amax=True, ws=None)
