"""Benchmark: FP4-quantized elements/s and achieved HBM GB/s on one MI355X.

Headline workload (the default; one step = the whole hot path for one batch): IF4 of a
bf16 [32768 x 8192] tensor (rows 50 % N(0,1), 25 % U(-1,1), 25 % Laplace(0,1), then
0.1 % of all elements x50) -- tensor amax, per-16 block FP4-or-INT4 choice flagged in
the E4M3 scale's sign bit -- then the dequantization round trip back to bf16.  It is the
largest workload that fits one GPU.  The same run also times the other full-size
workloads and reports them in the same JSON line (`config.other_workloads`):
NVFP4 1x16 row-wise + column-wise of a bf16 [8192 x 4096] activation, NVFP4 16x16 and
MXFP4 of an fp32 [8192 x 8192] weight, and the Wgrad pair (two bf16 [16384 x 4096]
operands, 128-token random Hadamard transform, column-wise NVFP4, SR on the gradient).

Inputs are synthetic, seeded, and resident in HBM before timing starts.  Consecutive
steps rotate over input/output sets whose total exceeds the 256 MB Infinity Cache, so
no step reads an earlier step's data from cache; the single-step distribution is taken
with a 1 GiB buffer written between steps.  Before anything is timed, the CPU-baseline
leg runs the oracle on a sample of the headline input and checks the GPU's output for
that sample byte for byte (the run fails otherwise), once on one thread and once on all
host cores.

`roofline` reports the dominant kernel: algorithmic bytes per launch (compulsory input
read + code/scale writes) over that kernel's mean duration, timed with HIP events on the
stream it runs on.  `traffic` is read from a committed counter summary under profiles/
while its recorded source digest matches the kernel's sources, else null.

`--config NAME` runs one workload alone as the line (also `mxfp6`, `gemm`, `gemm_nvfp4`
and the `copy` calibration); `--gpus N` with N > 1 exits: this library runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_MFMA_FP4_TFLOPS = 10100.0
METRIC = "FP4-quantized elements/s and achieved HBM GB/s (% of MI355X peak)"

# The sources each profiled kernel is built from; a change to any other file leaves its
# recorded counters valid.
QUANT_SOURCES = ["fp4q_quant.hip", "fp4q_dev.hpp", "fp4q_internal.hpp"]
KERNEL_SOURCES = {
    "k_if4": QUANT_SOURCES, "k_nvfp4_fused": QUANT_SOURCES, "k_nvfp4_2d": QUANT_SOURCES,
    "k_amax_wide": QUANT_SOURCES, "k_dequant": QUANT_SOURCES,
    "k_rht_nvfp4_col": ["fp4q_rht.hip", "fp4q_dev.hpp", "fp4q_internal.hpp"],
    "k_rht_amax": ["fp4q_rht.hip", "fp4q_dev.hpp", "fp4q_internal.hpp"],
    "k_variant": ["fp4q_variant.hip", "fp4q_dev.hpp", "fp4q_internal.hpp"],
    "k_dequant_variant": ["fp4q_variant.hip", "fp4q_dev.hpp", "fp4q_internal.hpp"],
    "k_mxfp4": QUANT_SOURCES, "k_mxfp6": QUANT_SOURCES,
    "k_gemm_mxfp4": ["fp4q_gemm.hip", "fp4q_internal.hpp"],
    "k_gemm_nvfp4": ["fp4q_gemm.hip", "fp4q_internal.hpp"],
}


def source_digest(kernel: str | None = None) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_05_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel) or sorted(os.listdir(csrc))
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str):
    """HBM bytes per launch from profiles/traffic.json if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or ent.get("source_digest") != source_digest(kernel):
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _u8(*shape):
    import torch
    return torch.empty(*shape, dtype=torch.uint8, device="cuda")


def _f1():
    import torch
    return torch.zeros(1, dtype=torch.float32, device="cuda")


def _timed_oracle(fn, threads: int):
    """Runs fn() with the split oracle on `threads` host threads; returns (result, seconds)."""
    import oracle.par as op
    op.set_threads(threads)
    try:
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0
    finally:
        op.set_threads(None)


def _cpu_line(elements: int, t1: float, tn: float, n: int, sample: str) -> dict:
    return {"value": elements / tn, "unit": "elements/s", "cores": n, "kind": "oracle", "sample": sample,
            "single_core_value": elements / t1, "cpu_model": cpu_model(), "parity_checked": True}


# --------------------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------------------

class Workload:
    name = ""
    dtype = "bf16"
    elements = 0
    algo_bytes = 0           # compulsory bytes of the whole step
    kernel = ""              # dominant kernel (symbol substring)
    kernel_bytes = 0         # algorithmic bytes per launch of the dominant kernel
    sets = 2                 # input/output sets the steps rotate over

    def setup(self): ...
    def step(self, i: int): ...
    def kernel_launch(self, i: int): ...          # the dominant kernel alone
    def given_launch(self, i: int): ...           # the call with the tensor amax given
    def cpu_baseline(self, budget_s: float) -> dict | None: ...
    def extra(self, stream) -> dict: return {}


class IF4RoundTrip(Workload):
    """IF4 quantize (amax computed) + dequantize back to bf16, bf16 [32768 x 8192]."""
    name = "if4_roundtrip_bf16_32768x8192"
    rows, cols = 32768, 8192

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        self.quant_bytes = 2 * n + n // 2 + n // 16             # read x, write codes + scales
        self.deq_bytes = n // 2 + n // 16 + 2 * n                # read codes + scales, write bf16
        self.algo_bytes = self.quant_bytes + self.deq_bytes
        self.kernel = "k_if4"
        self.kernel_bytes = self.quant_bytes

    def setup(self):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.ws = B.Workspace()
        self.host = si.if4_mix(self.rows, self.cols, seed=5)
        x0 = _dev_bf16(self.host)
        r, c = self.rows, self.cols
        self.x = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        self.out = [dict(amax=_f1(), ts=_f1(), c=_u8(r, c // 2), s=_u8(r, c // 16),
                         y=torch.empty(r, c, dtype=torch.bfloat16, device="cuda")) for _ in range(self.sets)]

    def _quant(self, i, mode):
        B, k = self.B, i % self.sets
        o = self.out[k]
        B.fp4q_quantize_if4(self.x[k], B.BF16, self.rows, self.cols, mode, o["amax"], o["ts"], o["c"], o["s"],
                            self.ws)

    def _deq(self, i):
        B, o = self.B, self.out[i % self.sets]
        B.fp4q_dequantize(B.FMT_IF4, o["c"], o["s"], o["ts"], self.rows, self.cols, B.BF16, o["y"])

    def step(self, i):
        self._quant(i, self.B.AMAX_COMPUTE)
        self._deq(i)

    def kernel_launch(self, i):
        self._quant(i, self.B.AMAX_GIVEN)

    def given_launch(self, i):
        self._quant(i, self.B.AMAX_GIVEN)

    def extra(self, stream):
        import torch
        B = self.B
        d = {}
        d["amax_pass_ms"] = _event_mean(stream, lambda i: B.fp4q_amax(self.x[i % self.sets], B.BF16, self.rows,
                                                                       self.cols, self.out[i % self.sets]["amax"]))
        d["amax_pass_GBps"] = 2 * self.elements / (d["amax_pass_ms"] * 1e-3) / 1e9
        d["quantize_call_ms"] = _event_mean(stream, lambda i: self._quant(i, B.AMAX_COMPUTE))
        d["quantize_call_GBps"] = self.quant_bytes / (d["quantize_call_ms"] * 1e-3) / 1e9
        d["dequant_bf16_ms"] = _event_mean(stream, self._deq)
        d["dequant_bf16_GBps"] = self.deq_bytes / (d["dequant_bf16_ms"] * 1e-3) / 1e9
        flags = self.out[0]["s"] >= 0x80
        torch.cuda.synchronize()
        r = self.rows
        d["int4_share"] = {"normal": float(flags[:r // 2].float().mean()),
                           "uniform": float(flags[r // 2:3 * r // 4].float().mean()),
                           "laplace": float(flags[3 * r // 4:].float().mean())}
        return d

    def cpu_baseline(self, budget_s):
        """The oracle on the first rows (IF4 quantize with the whole tensor's scale, then
        dequantize), checked byte for byte against the GPU's output for those rows."""
        import numpy as np
        import oracle
        import oracle.par as op
        import torch
        self.step(0)
        torch.cuda.synchronize()
        o = self.out[0]
        gs = oracle.tensor_scale(op.amax(self.host))
        if np.float32(gs) != o["ts"].cpu().numpy()[0]:
            raise AssertionError("bench parity: the tensor scale differs from the oracle's")
        t0 = time.perf_counter()
        c, s, _ = oracle.quantize_if4(np.ascontiguousarray(self.host[:64]), gs=gs)
        oracle.dequantize(oracle.FMT_IF4, c, s, gs, 64, self.cols)
        per_row = (time.perf_counter() - t0) / 64
        nrows = int(min(self.rows, max(64, (budget_s / per_row) // 64 * 64)))
        sample = np.ascontiguousarray(self.host[:nrows])

        def run():
            cc, ss = op.quantize_if4(sample, gs)
            yy = op.dequantize(oracle.FMT_IF4, cc, ss, gs, nrows, self.cols)
            return cc, ss, yy
        (c1, s1, y1), t1 = _timed_oracle(run, 1)
        n = host_cores()
        (cn, sn, yn), tn = _timed_oracle(run, n)
        yb = o["y"][:nrows].view(torch.int16).cpu().numpy().view(np.uint16)
        import synth_inputs as si
        ok = (np.array_equal(o["c"][:nrows].cpu().numpy(), c1) and np.array_equal(o["s"][:nrows].cpu().numpy(), s1)
              and np.array_equal(yb, si.f32_to_bf16_bits(y1)) and np.array_equal(cn, c1)
              and np.array_equal(yn.view(np.uint32), y1.view(np.uint32)))
        if not ok:
            raise AssertionError("bench parity: the GPU's IF4 codes, scales or round trip differ from the oracle's")
        return _cpu_line(nrows * self.cols, t1, tn, n,
                         f"IF4 quantize + dequantize of rows 0..{nrows - 1} ({nrows}x{self.cols} bf16) with the "
                         f"whole tensor's scale; 1 thread {t1:.1f} s, {n} threads {tn:.1f} s")


class ActivationNVFP4(Workload):
    """NVFP4 1x16 row-wise + column-wise, RTN, amax computed (one pass), bf16 [8192 x 4096]."""
    name = "nvfp4_1x16_rowcol_rtn_bf16_8192x4096"
    rows, cols = 8192, 4096
    sets = 4

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        self.algo_bytes = 2 * n + 2 * (n // 2 + n // 16)
        self.kernel = "k_nvfp4_fused"         # the whole step is this one launch
        self.kernel_bytes = self.algo_bytes

    def setup(self):
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.ws = B.Workspace()
        self.host = si.activation(self.rows, self.cols, seed=2)
        x0 = _dev_bf16(self.host)
        self.x = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        r, c = self.rows, self.cols
        self.out = [dict(amax=_f1(), ts=_f1(), rc=_u8(r, c // 2), rs=_u8(r, c // 16), cc=_u8(c, r // 2),
                         cs=_u8(c, r // 16)) for _ in range(self.sets)]

    def _call(self, i, mode):
        B, k = self.B, i % self.sets
        o = self.out[k]
        B.fp4q_quantize_nvfp4(self.x[k], B.BF16, self.rows, self.cols, B.ROWWISE | B.COLWISE, B.RTN, 0, None, mode,
                              o["amax"], o["ts"], o["rc"], o["rs"], o["cc"], o["cs"], self.ws)

    def step(self, i):
        self._call(i, self.B.AMAX_COMPUTE)

    def kernel_launch(self, i):
        self._call(i, self.B.AMAX_COMPUTE)

    def given_launch(self, i):
        # the streaming tile kernel alone; the amax buffers hold what a compute call wrote
        self._call(i, self.B.AMAX_GIVEN)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        import oracle.par as op
        import torch
        self.step(0)
        torch.cuda.synchronize()
        o = self.out[0]
        gs = oracle.tensor_scale(op.amax(self.host))
        t0 = time.perf_counter()
        oracle.quantize_nvfp4_rows(self.host, 0, 64, False, gs)
        oracle.quantize_nvfp4_rows(self.host, 0, 32, True, gs)
        per = (time.perf_counter() - t0) / (64 * self.cols + 32 * self.rows)
        nr = int(min(self.rows, max(64, budget_s / 2 / per / self.cols // 64 * 64)))
        sample = np.ascontiguousarray(self.host[:nr])
        run = lambda: op.quantize_nvfp4(sample, False, gs)
        (c1, s1), t1 = _timed_oracle(run, 1)
        n = host_cores()
        (cn, sn), tn = _timed_oracle(run, n)
        if not (np.array_equal(o["rc"][:nr].cpu().numpy(), c1) and np.array_equal(o["rs"][:nr].cpu().numpy(), s1)
                and np.array_equal(cn, c1)):
            raise AssertionError("bench parity: NVFP4 row-wise codes differ from the oracle's")
        return _cpu_line(nr * self.cols, t1, tn, n, f"row-wise NVFP4 of rows 0..{nr - 1}; 1 thread {t1:.1f} s, "
                                                    f"{n} threads {tn:.1f} s")


class WeightNVFP4MX(Workload):
    """fp32 [8192 x 8192]: MXFP4 (reporting the tensor amax) then NVFP4 16x16 with it."""
    name = "weight_fp32_8192x8192_nvfp4_16x16_and_mxfp4"
    rows = cols = 8192
    dtype = "f32"

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        b2d = 4 * n + n // 2 + n // 256
        bmx = 4 * n + n // 2 + n // 32
        self.algo_bytes = b2d + bmx
        self.kernel = "k_nvfp4_2d"
        self.kernel_bytes = b2d

    def setup(self):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.ws = B.Workspace()
        self.host = si.weight(self.rows, self.cols, seed=3)
        x0 = torch.from_numpy(self.host).to("cuda")
        self.x = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        r, c = self.rows, self.cols
        self.out = [dict(amax=_f1(), ts=_f1(), c=_u8(r, c // 2), s=_u8(r // 16, c // 16), mc=_u8(r, c // 2),
                         ms=_u8(r, c // 32)) for _ in range(self.sets)]

    def step(self, i):
        # MXFP4 first: its pass also reports the tensor amax, which the 16x16 call takes
        # as given, so W is read twice rather than three times (amax, 16x16, MXFP4)
        B, k = self.B, i % self.sets
        o, x = self.out[k], self.x[k]
        B.fp4q_quantize_mxfp4(x, B.F32, self.rows, self.cols, B.RTN, 0, o["mc"], o["ms"], o["amax"], self.ws)
        B.fp4q_quantize_nvfp4_2d(x, B.F32, self.rows, self.cols, B.AMAX_GIVEN, o["amax"], o["ts"], o["c"], o["s"],
                                 None, self.ws)

    def kernel_launch(self, i):
        B, k = self.B, i % self.sets
        o, x = self.out[k], self.x[k]
        B.fp4q_quantize_nvfp4_2d(x, B.F32, self.rows, self.cols, B.AMAX_GIVEN, o["amax"], o["ts"], o["c"], o["s"],
                                 None, self.ws)

    given_launch = kernel_launch

    def extra(self, stream):
        B = self.B
        ms = _event_mean(stream, lambda i: B.fp4q_quantize_mxfp4(
            self.x[i % self.sets], B.F32, self.rows, self.cols, B.RTN, 0, self.out[i % self.sets]["mc"],
            self.out[i % self.sets]["ms"], self.out[i % self.sets]["amax"], self.ws))
        n = self.elements
        return {"mxfp4_with_amax_ms": ms, "mxfp4_with_amax_GBps": (4 * n + n // 2 + n // 32) / (ms * 1e-3) / 1e9}


class WgradRHT(Workload):
    """Two bf16 [16384 x 4096] operands: 128-token RHT, column-wise NVFP4 (gradient SR,
    activation RTN), amax of the transformed tensor computed."""
    name = "wgrad_rht128_nvfp4_col_bf16_2x16384x4096"
    rows, cols = 16384, 4096

    def __init__(self):
        n = self.rows * self.cols
        self.elements = 2 * n
        per = 2 * n + n // 2 + n // 16
        self.algo_bytes = 2 * per
        self.kernel = "k_rht_nvfp4_col"
        self.kernel_bytes = per

    def setup(self):
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.ws = B.Workspace()
        g0 = _dev_bf16(si.wgrad_gradient(self.rows, self.cols, seed=4))
        x0 = _dev_bf16(si.wgrad_activation(self.rows, self.cols, seed=4))
        self.signs = B.fp4q_rht_signs_from_seed(4)
        self.g = [g0] + [g0.clone() for _ in range(self.sets - 1)]
        self.xa = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        r, c = self.rows, self.cols
        self.out = [[dict(amax=_f1(), ts=_f1(), c=_u8(c, r // 2), s=_u8(c, r // 16)) for _ in range(2)]
                    for _ in range(self.sets)]

    def _q(self, x, o, rnd, seed, mode):
        B = self.B
        B.fp4q_quantize_nvfp4(x, B.BF16, self.rows, self.cols, B.COLWISE, rnd, seed, self.signs, mode, o["amax"],
                              o["ts"], None, None, o["c"], o["s"], self.ws)

    def step(self, i):
        k = i % self.sets
        self._q(self.g[k], self.out[k][0], self.B.SR, 40, self.B.AMAX_COMPUTE)
        self._q(self.xa[k], self.out[k][1], self.B.RTN, 41, self.B.AMAX_COMPUTE)

    def kernel_launch(self, i):
        k = i % self.sets
        self._q(self.g[k], self.out[k][0], self.B.SR, 40, self.B.AMAX_GIVEN)

    given_launch = kernel_launch

    def extra(self, stream):
        B = self.B
        rtn = _event_mean(stream, lambda i: self._q(self.xa[i % self.sets], self.out[i % self.sets][1], B.RTN, 41,
                                                    B.AMAX_GIVEN))
        sr = _event_mean(stream, self.kernel_launch, n=50, warm=20)
        flops = 2 * 128 * self.rows * self.cols
        # the transform as a dense contraction on the bf16 MFMA, against its dense peak; the
        # algorithmic minimum, a fast Walsh-Hadamard transform, is 7 adds per element
        util = lambda ms: flops / (ms * 1e-3) / 1e12
        return {"rtn_quantizer_ms": rtn, "mfma_dense_flop_per_operand": flops,
                "mfma_TFLOPs_sr": util(sr), "mfma_frac_of_bf16_peak_sr": util(sr) / PEAK_MFMA_BF16_TFLOPS,
                "mfma_TFLOPs_rtn": util(rtn), "mfma_frac_of_bf16_peak_rtn": util(rtn) / PEAK_MFMA_BF16_TFLOPS,
                "fwht_adds_per_element": 7}


class WeightMXFP6(Workload):
    """MX FP6 (E2M3) of the weight workload's fp32 [8192 x 8192] matrix."""
    name = "weight_fp32_8192x8192_mxfp6_e2m3"
    rows = cols = 8192
    dtype = "f32"

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        self.algo_bytes = 4 * n + n // 4 * 3 + n // 32
        self.kernel = "k_mxfp6"
        self.kernel_bytes = self.algo_bytes

    def setup(self):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        x0 = torch.from_numpy(si.weight(self.rows, self.cols, seed=3)).to("cuda")
        self.x = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        self.out = [(_u8(self.rows, self.cols // 4 * 3), _u8(self.rows, self.cols // 32)) for _ in range(self.sets)]

    def step(self, i):
        B = self.B
        c, s = self.out[i % self.sets]
        B.fp4q_quantize_mxfp6(self.x[i % self.sets], B.F32, self.rows, self.cols, B.FP6_E2M3, c, s)

    kernel_launch = step
    given_launch = step


class GemmMXFP4(Workload):
    """Y = X W^T on MXFP4 operands: X an activation [8192 x 8192] (N(0,1), 1 % of the
    columns x30, bf16), W the weight workload's matrix; Y in bf16."""
    name = "fprop_gemm_mxfp4_8192x8192x8192_bf16_out"
    m = n = k = 8192
    bound, peak, unit = "mfma", PEAK_MFMA_FP4_TFLOPS, "TFLOP/s"
    dtype = "fp4"   # E2M1 x E2M1 products, fp32 accumulation
    metric = "MXFP4 GEMM FLOP/s and % of MI355X dense FP4 matrix-core peak"

    def __init__(self):
        self.flops = 2 * self.m * self.n * self.k
        self.elements = self.flops
        self.algo_bytes = (self.m + self.n) * (self.k // 2 + self.k // 32) + 2 * self.m * self.n
        self.kernel = "k_gemm_mxfp4"
        self.kernel_bytes = self.algo_bytes

    def setup(self):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        qa = B.quantize_mxfp4(_dev_bf16(si.activation(self.m, self.k, seed=2)))
        qb = B.quantize_mxfp4(torch.from_numpy(si.weight(self.n, self.k, seed=3)).to("cuda"))
        self.ops = [(qa, qb)] + [({k: v.clone() for k, v in qa.items()}, {k: v.clone() for k, v in qb.items()})
                                 for _ in range(self.sets - 1)]
        self.y = [torch.empty(self.m, self.n, dtype=torch.bfloat16, device="cuda") for _ in range(self.sets)]

    def step(self, i):
        B = self.B
        qa, qb = self.ops[i % self.sets]
        B.fp4q_gemm_mxfp4(qa["codes"], qa["scales"], qb["codes"], qb["scales"], self.m, self.n, self.k, B.BF16,
                          self.y[i % self.sets])

    kernel_launch = step
    given_launch = step


class GemmNVFP4Wgrad(GemmMXFP4):
    """dY^T X from the Wgrad workload's RHT-quantized operands: [4096 x 4096] over 16384
    tokens, bf16 out, on the f16 MFMA after an exact decode (dense peak 2.5 PFLOP/s, as bf16)."""
    name = "wgrad_gemm_nvfp4_rht_4096x4096x16384_bf16_out"
    m = n = 4096
    k = 16384
    bound, peak, unit = "mfma", PEAK_MFMA_BF16_TFLOPS, "TFLOP/s"
    dtype = "f16"   # exact f16 decodes of r * s, fp32 accumulation
    metric = "NVFP4 GEMM FLOP/s and % of MI355X dense f16/bf16 matrix-core peak"

    def __init__(self):
        self.flops = 2 * self.m * self.n * self.k
        self.elements = self.flops
        self.algo_bytes = (self.m + self.n) * (self.k // 2 + self.k // 16) + 2 * self.m * self.n
        self.kernel = "k_gemm_nvfp4"
        self.kernel_bytes = self.algo_bytes

    def setup(self):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        signs = B.fp4q_rht_signs_from_seed(4)
        qg = B.quantize_nvfp4(_dev_bf16(si.wgrad_gradient(self.k, self.m, seed=4)), B.COLWISE, rnd=B.SR, sr_seed=40,
                              rht_signs=signs)
        qx = B.quantize_nvfp4(_dev_bf16(si.wgrad_activation(self.k, self.n, seed=4)), B.COLWISE, rht_signs=signs)
        pick = lambda q: (q["col_codes"], q["col_scales"], q["tensor_scale"])
        ops = (pick(qg), pick(qx))
        self.ops = [ops] + [(tuple(t.clone() for t in ops[0]), tuple(t.clone() for t in ops[1]))
                            for _ in range(self.sets - 1)]
        self.y = [torch.empty(self.m, self.n, dtype=torch.bfloat16, device="cuda") for _ in range(self.sets)]

    def step(self, i):
        B = self.B
        (ac, as_, ga), (bc, bs, gb) = self.ops[i % self.sets]
        B.fp4q_gemm_nvfp4(ac, as_, ga, bc, bs, gb, self.m, self.n, self.k, 0, B.BF16, self.y[i % self.sets])

    kernel_launch = step
    given_launch = step

    def extra(self, stream):
        """The same product with IF4 operands (fp4q_quantize_if4 of dY^T and X^T, no RHT):
        one IF4 operand (A) and both, against the NVFP4 product above."""
        import torch
        import synth_inputs as si
        B = self.B
        t = lambda b: _dev_bf16(b).t().contiguous()
        qa = B.quantize_if4(t(si.wgrad_gradient(self.k, self.m, seed=4)))
        qb = B.quantize_if4(t(si.wgrad_activation(self.k, self.n, seed=4)))
        (nc, ns, ng), _ = self.ops[0]
        y = self.y[0]
        one = lambda i: B.fp4q_gemm_nvfp4(qa["codes"], qa["scales"], qa["tensor_scale"], nc, ns, ng, self.m, self.n,
                                          self.k, B.IF4_A, B.BF16, y)
        both = lambda i: B.fp4q_gemm_nvfp4(qa["codes"], qa["scales"], qa["tensor_scale"], qb["codes"], qb["scales"],
                                           qb["tensor_scale"], self.m, self.n, self.k, B.IF4_A | B.IF4_B, B.BF16, y)
        share = float(((qa["scales"] & 0x80) != 0).float().mean().item())
        return {"if4_a_ms": _event_mean(stream, one, n=20, warm=10),
                "if4_both_ms": _event_mean(stream, both, n=20, warm=10), "if4_int4_block_share_a": share}


class BlockVariants(Workload):
    """The block formats compared with IF4 on the IF4 workload's bf16 [32768 x 8192]
    tensor: Four Over Six, NVINT4, IF3 and IF6 (NVFP4 two-level scaling, 16-element
    blocks), each quantized with the tensor amax given and dequantized back to bf16."""
    name = "block_variants_46_nvint4_if3_if6_bf16_32768x8192"
    rows, cols = 32768, 8192

    def __init__(self):
        from block_scaled_fp4_05_amd import binding as B
        n = self.rows * self.cols
        self.vars = [(B.VAR_46, "four_over_six"), (B.VAR_NVINT4, "nvint4"), (B.VAR_IF3, "if3"), (B.VAR_IF6, "if6")]
        self.bits = {v: B.VARIANT_BITS[v] for v, _ in self.vars}
        self.qbytes = {v: 2 * n + n * self.bits[v] // 8 + n // 16 for v, _ in self.vars}
        self.dbytes = {v: n * self.bits[v] // 8 + n // 16 + 2 * n for v, _ in self.vars}
        self.elements = n * len(self.vars)
        self.algo_bytes = sum(self.qbytes.values()) + sum(self.dbytes.values())
        self.kernel = "k_variant"             # the IF6 quantizer, the heaviest of the four
        self.kernel_bytes = self.qbytes[B.VAR_IF6]

    def setup(self):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.ws = B.Workspace()
        x0 = _dev_bf16(si.if4_mix(self.rows, self.cols, seed=5))
        r, c = self.rows, self.cols
        self.x = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        self.amax = [_f1() for _ in range(self.sets)]
        for k in range(self.sets):
            B.fp4q_amax(self.x[k], B.BF16, r, c, self.amax[k])
        self.out = [{v: dict(ts=_f1(), c=_u8(r, c * self.bits[v] // 8), s=_u8(r, c // 16),
                             y=torch.empty(r, c, dtype=torch.bfloat16, device="cuda")) for v, _ in self.vars}
                    for _ in range(self.sets)]

    def _quant(self, i, v):
        B, k = self.B, i % self.sets
        o = self.out[k][v]
        B.fp4q_quantize_variant(self.x[k], B.BF16, self.rows, self.cols, v, B.AMAX_GIVEN, self.amax[k], o["ts"],
                                o["c"], o["s"], self.ws)

    def _deq(self, i, v):
        B, o = self.B, self.out[i % self.sets][v]
        B.fp4q_dequantize_variant(v, o["c"], o["s"], o["ts"], self.rows, self.cols, B.BF16, o["y"])

    def step(self, i):
        for v, _ in self.vars:
            self._quant(i, v)
            self._deq(i, v)

    def kernel_launch(self, i):
        self._quant(i, self.B.VAR_IF6)

    given_launch = kernel_launch

    def extra(self, stream):
        d = {}
        for v, nm in self.vars:
            q = _event_mean(stream, lambda i, v=v: self._quant(i, v))
            dq = _event_mean(stream, lambda i, v=v: self._deq(i, v))
            d[nm] = {"bits": self.bits[v], "quantize_ms": q, "quantize_GBps": self.qbytes[v] / (q * 1e-3) / 1e9,
                     "dequant_bf16_ms": dq, "dequant_GBps": self.dbytes[v] / (dq * 1e-3) / 1e9}
        return d


class DeviceCopy(Workload):
    """Calibration, not a hot-path row: a plain device-to-device copy of 64 MiB."""
    name = "device_copy_64MiB"
    nbytes = 64 << 20
    sets = 4

    def __init__(self):
        self.elements = self.nbytes // 2
        self.algo_bytes = 2 * self.nbytes
        self.kernel = "copy"
        self.kernel_bytes = self.algo_bytes

    def setup(self):
        import torch
        n = self.nbytes // 2
        self.src = [torch.randn(n, device="cuda").to(torch.bfloat16) for _ in range(self.sets)]
        self.dst = [torch.empty_like(t) for t in self.src]

    def step(self, i):
        k = i % self.sets
        self.dst[k].copy_(self.src[k])

    kernel_launch = step
    given_launch = step


HEADLINE = IF4RoundTrip
OTHERS = [ActivationNVFP4, WeightNVFP4MX, WgradRHT, BlockVariants]
WORKLOADS = {"if4": IF4RoundTrip, "activation": ActivationNVFP4, "weight": WeightNVFP4MX, "wgrad": WgradRHT,
             "variants": BlockVariants,
             "mxfp6": WeightMXFP6, "gemm": GemmMXFP4, "gemm_nvfp4": GemmNVFP4Wgrad, "copy": DeviceCopy}


# --------------------------------------------------------------------------------------

def _event_mean(stream, fn, n: int = 100, warm: int = 50) -> float:
    """Mean ms of n back-to-back fn(i) between two HIP events on `stream`, after `warm`
    untimed launches that bring the clocks to the level a stream of such launches runs at."""
    import torch
    for i in range(warm):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def copy_reference(stream) -> float:
    """GB/s (bytes read + written) of a plain device copy of 512 MiB, beyond the 256 MB
    Infinity Cache: the bandwidth a streaming kernel can reach on this machine, beside the
    8 TB/s of the specification."""
    import torch
    n = 1 << 29
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    ms = _event_mean(stream, lambda i: dst.copy_(src), n=20, warm=5)
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def run(wl: Workload, steps: int, warmup: int, cpu_budget: float, flush, copy_gbps: float | None = None) -> dict:
    import torch
    wl.setup()
    cb = wl.cpu_baseline(cpu_budget) if cpu_budget > 0 else None    # includes the parity check
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    # whole-step throughput: K consecutive steps between two synchronizations
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(warmup + i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    # the dominant kernel alone, back to back, HIP events on the stream it runs on
    nk = max(steps, 100)
    k_mean = _event_mean(stream, wl.kernel_launch, nk)
    mfma = getattr(wl, "bound", "hbm") == "mfma"
    if mfma:
        achieved, peak, unit = wl.flops / (k_mean * 1e-3) / 1e12, wl.peak, wl.unit
    else:
        achieved, peak, unit = wl.kernel_bytes / (k_mean * 1e-3) / 1e9, PEAK_HBM_GBPS, "GB/s"
    step_gbps = wl.algo_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": getattr(wl, "metric", METRIC),
        "value": wl.elements / (ms_per_step * 1e-3),
        "unit": "FLOP/s" if mfma else "elements/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "elements_per_step": wl.elements, "algorithmic_bytes_per_step": wl.algo_bytes,
                   "whole_step_GBps": step_gbps, "whole_step_frac_of_hbm_peak": step_gbps / PEAK_HBM_GBPS},
        "roofline": {"bound": "mfma" if mfma else "hbm", "kernel": wl.kernel, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak, "traffic": counter_traffic(wl.kernel),
                     "kernel_ms_mean": k_mean, "kernel_launches_timed": nk,
                     "algorithmic_bytes_per_launch": wl.kernel_bytes},
    }
    # single steps from cold caches: a 1 GiB write between steps, each step between its own events
    st = []
    for i in range(steps):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        wl.step(i)
        b.record(stream)
        torch.cuda.synchronize()
        st.append(a.elapsed_time(b))
    st.sort()
    pick = lambda q: st[min(len(st) - 1, int(q * (len(st) - 1) + 0.5))]
    line["config"]["cold_step_ms_p10"], line["config"]["cold_step_ms_p50"], line["config"]["cold_step_ms_p90"] = (
        pick(0.1), pick(0.5), pick(0.9))
    if not mfma:
        g_ms = _event_mean(stream, wl.given_launch, nk)
        line["config"]["amax_given_ms"] = g_ms
        line["config"]["amax_given_GBps"] = wl.kernel_bytes / (g_ms * 1e-3) / 1e9
    else:
        line["config"]["whole_step_TFLOPs"] = wl.flops / (ms_per_step * 1e-3) / 1e12
    line["config"].update(wl.extra(stream))
    if copy_gbps and not mfma:
        line["config"]["copy_reference_GBps"] = copy_gbps
        line["config"]["whole_step_frac_of_copy"] = step_gbps / copy_gbps
        line["roofline"]["frac_of_copy"] = achieved / copy_gbps
    if cb is not None:
        line["cpu_baseline"] = cb
    return line


def _summary(line: dict) -> dict:
    """The other workloads' figures, carried inside the headline line."""
    c, r = line["config"], line["roofline"]
    keep = {k: v for k, v in c.items() if k not in ("workload",)}
    return {"workload": c["workload"], "value": line["value"], "unit": line["unit"], "dtype": line["dtype"],
            "ms_per_step": line["ms_per_step"], **keep,
            "roofline": {k: r[k] for k in ("bound", "kernel", "achieved", "peak", "unit", "frac", "frac_of_copy",
                                           "traffic", "kernel_ms_mean") if k in r}}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 50 warm-up steps: after the host-side set-up the GPU's clocks need a few
    # milliseconds of load to settle, and the VALU-bound kernels run up to 8 % slower
    # until they have (IF4 round trip: 328 us per step over 20 steps after 5, 303 us over
    # 100 after 50, 305 us over 200 after 200); the cold single steps are reported apart
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="headline", choices=["headline"] + list(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of single-thread oracle work for cpu_baseline (0: skip it and its parity check)")
    ap.add_argument("--no-others", action="store_true", help="headline only (e.g. under a profiler)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU: every step is one GPU's share of the work "
                                   "(the multi-GPU sharding is described, not built), so --gpus must be 1"}))
        return 2
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    from block_scaled_fp4_05_amd import binding as B
    B.lib()
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush = lambda: scratch.fill_(1)
    copy_gbps = copy_reference(torch.cuda.current_stream())
    if a.config == "headline":
        line = run(HEADLINE(), a.steps, a.warmup, a.cpu_budget, flush, copy_gbps)
        if not a.no_others:
            others = []
            for cls in OTHERS:
                torch.cuda.empty_cache()
                others.append(_summary(run(cls(), a.steps, a.warmup, 0.0, flush, copy_gbps)))
                print(f"# timed {others[-1]['workload']}", file=sys.stderr, flush=True)
            line["config"]["other_workloads"] = others
    else:
        line = run(WORKLOADS[a.config](), a.steps, a.warmup, a.cpu_budget if a.config != "copy" else 0.0, flush,
                   copy_gbps)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
