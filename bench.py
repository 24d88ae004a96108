"""Benchmark: FP4-quantized elements/s and achieved HBM GB/s on one MI355X.

Default workload (one step = the whole hot path for one batch): NVFP4 1x16
quantization of a bf16 activation [8192 x 4096] (N(0,1), 1% of the columns x30),
round-to-nearest, row-wise AND transposed column-wise codes + E4M3 scales + the
FP32 tensor scale -- tensor amax pass included.  Inputs are synthetic and already
resident in HBM; consecutive steps rotate over several input/output buffer sets
whose total exceeds the 256 MB Infinity Cache, so no step reads another step's
data from cache.

Other workloads (`--config`): weight [8192 x 8192] fp32 NVFP4 16x16 + MXFP4
("weight"), MX FP6 E2M3 of the same weight ("mxfp6"), the Wgrad pair with the 128x128
RHT ("wgrad"), IF4 + dequantize on [32768 x 8192] ("if4"), and the GEMM that consumes MXFP4 operands, Y = X W^T with
8192 x 8192 x 8192 and bf16 output ("gemm"; measured in FLOP/s against the dense
FP4 matrix-core peak), and the NVFP4 weight-gradient GEMM dY^T X on the Wgrad
workload's RHT-quantized operands ("gemm_nvfp4"; against the dense bf16 peak, the
MFMA it runs on).  Each prints one JSON line; `--config all` prints one per
workload.

The roofline object reports the dominant kernel: algorithmic bytes per launch
(compulsory input read + code/scale writes) over that kernel's mean duration,
timed with HIP events on the stream it runs on.  `traffic` is read from a committed
counter summary under profiles/ when its recorded source digest matches the
current kernel sources, else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_MFMA_FP4_TFLOPS = 10100.0


# The sources each profiled kernel is built from; a change to any other file leaves its
# recorded counters valid.
KERNEL_SOURCES = {
    "k_nvfp4_fused": ["fp4q_quant.hip", "fp4q_dev.hpp", "fp4q_internal.hpp"],
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


# --------------------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------------------

class Workload:
    name = ""
    elements = 0
    algo_bytes = 0           # compulsory bytes of the whole step
    kernel = ""              # dominant kernel (symbol substring)
    kernel_bytes = 0         # algorithmic bytes per launch of the dominant kernel

    def setup(self, nbuf: int): ...
    def step(self, i: int): ...
    def kernel_launch(self, i: int): ...
    def cpu_baseline(self, budget_s: float) -> dict: ...


def _dev_bf16(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


class ActivationNVFP4(Workload):
    name = "nvfp4_1x16_rowcol_rtn_bf16_8192x4096"
    rows, cols = 8192, 4096

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        self.algo_bytes = 2 * n + 2 * (n // 2 + n // 16)
        self.kernel = "k_nvfp4_fused"         # the whole step is this one launch
        self.kernel_bytes = self.algo_bytes

    def setup(self, nbuf):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.host = si.activation(self.rows, self.cols, seed=2)
        x0 = _dev_bf16(self.host)
        self.x = [x0] + [x0.clone() for _ in range(nbuf - 1)]
        r, c = self.rows, self.cols
        u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")
        self.out = [dict(amax=torch.zeros(1, device="cuda"), ts=torch.zeros(1, device="cuda"),
                         rc=u8(r, c // 2), rs=u8(r, c // 16), cc=u8(c, r // 2), cs=u8(c, r // 16))
                    for _ in range(nbuf)]

    def _call(self, i, mode):
        B, o, x = self.B, self.out[i % len(self.out)], self.x[i % len(self.x)]
        B.fp4q_quantize_nvfp4(x, B.BF16, self.rows, self.cols, B.ROWWISE | B.COLWISE, B.RTN, 0, None, mode,
                              o["amax"], o["ts"], o["rc"], o["rs"], o["cc"], o["cs"])

    def step(self, i):
        self._call(i, self.B.AMAX_COMPUTE)

    def kernel_launch(self, i):
        self._call(i, self.B.AMAX_COMPUTE)

    def given_launch(self, i):
        # the same call with the tensor amax supplied (AMAX_GIVEN): the streaming tile
        # kernel alone; the amax buffers hold the values a compute-mode call wrote
        self._call(i, self.B.AMAX_GIVEN)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        bits = self.host
        t0 = time.perf_counter()
        amax = oracle.amax(bits)
        gs = oracle.tensor_scale(amax)
        t_amax = time.perf_counter() - t0
        # calibrate on 64 rows, then size the sample to the budget
        t0 = time.perf_counter()
        oracle.quantize_nvfp4(np.ascontiguousarray(bits[:64]), gs=gs)
        oracle.quantize_nvfp4(np.ascontiguousarray(bits[:64]), colwise=True, gs=gs)
        per_row = (time.perf_counter() - t0) / 64
        nrows = int(min(self.rows, max(64, (budget_s / per_row) // 16 * 16)))
        sample = np.ascontiguousarray(bits[:nrows])
        t0 = time.perf_counter()
        oracle.quantize_nvfp4(sample, gs=gs)
        oracle.quantize_nvfp4(sample, colwise=True, gs=gs)
        dt = time.perf_counter() - t0
        per_elem = dt / (nrows * self.cols) + t_amax / (self.rows * self.cols)
        return {"value": 1.0 / per_elem, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"tensor amax over all {self.rows}x{self.cols} values, then row-wise and column-wise "
                          f"NVFP4 of rows 0..{nrows - 1} ({nrows}x{self.cols} bf16), single thread, "
                          f"{dt + t_amax:.1f} s"}


class WeightNVFP4MX(Workload):
    name = "weight_fp32_8192x8192_nvfp4_16x16_and_mxfp4"
    rows = cols = 8192

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        b2d = 4 * n + n // 2 + n // 256
        bmx = 4 * n + n // 2 + n // 32
        self.algo_bytes = b2d + bmx
        self.kernel = "k_nvfp4_2d"
        self.kernel_bytes = b2d

    def setup(self, nbuf):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.host = si.weight(self.rows, self.cols, seed=3)
        x0 = torch.from_numpy(self.host).to("cuda")
        nbuf = min(nbuf, 2)                      # 268 MB each: two copies already exceed the cache
        self.x = [x0] + [x0.clone() for _ in range(nbuf - 1)]
        r, c = self.rows, self.cols
        u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")
        self.out = [dict(amax=torch.zeros(1, device="cuda"), ts=torch.zeros(1, device="cuda"), c=u8(r, c // 2),
                         s=u8(r // 16, c // 16), mc=u8(r, c // 2), ms=u8(r, c // 32)) for _ in range(nbuf)]

    def step(self, i):
        # MXFP4 first: its pass also reports the tensor amax, which the 16x16 call takes
        # as given, so W is read twice rather than three times (amax, 16x16, MXFP4)
        B, o, x = self.B, self.out[i % len(self.out)], self.x[i % len(self.x)]
        B.fp4q_quantize_mxfp4(x, B.F32, self.rows, self.cols, B.RTN, 0, o["mc"], o["ms"], o["amax"])
        B.fp4q_quantize_nvfp4_2d(x, B.F32, self.rows, self.cols, B.AMAX_GIVEN, o["amax"], o["ts"], o["c"], o["s"],
                                 None)

    def kernel_launch(self, i):
        B, o, x = self.B, self.out[i % len(self.out)], self.x[i % len(self.x)]
        B.fp4q_quantize_nvfp4_2d(x, B.F32, self.rows, self.cols, B.AMAX_GIVEN, o["amax"], o["ts"], o["c"], o["s"],
                                 None)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        w = self.host
        gs = oracle.tensor_scale(oracle.amax(w))
        t0 = time.perf_counter()
        oracle.quantize_nvfp4_2d(np.ascontiguousarray(w[:16]), gs=gs)
        oracle.quantize_mxfp4(np.ascontiguousarray(w[:16]))
        per_row = (time.perf_counter() - t0) / 16
        nrows = int(min(self.rows, max(16, (budget_s / per_row) // 16 * 16)))
        s = np.ascontiguousarray(w[:nrows])
        t0 = time.perf_counter()
        oracle.quantize_nvfp4_2d(s, gs=gs)
        oracle.quantize_mxfp4(s)
        dt = time.perf_counter() - t0
        return {"value": nrows * self.cols / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"NVFP4 16x16 + MXFP4 of rows 0..{nrows - 1}, single thread, {dt:.1f} s"}


class WeightMXFP6(Workload):
    """MX FP6 (E2M3) of the weight workload's fp32 [8192 x 8192] matrix: one read of W,
    codes packed four per three bytes plus E8M0 scales."""
    name = "weight_fp32_8192x8192_mxfp6_e2m3"
    rows = cols = 8192

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        self.algo_bytes = 4 * n + n // 4 * 3 + n // 32
        self.kernel = "k_mxfp6"
        self.kernel_bytes = self.algo_bytes

    def setup(self, nbuf):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.host = si.weight(self.rows, self.cols, seed=3)
        x0 = torch.from_numpy(self.host).to("cuda")
        nbuf = min(nbuf, 2)
        self.x = [x0] + [x0.clone() for _ in range(nbuf - 1)]
        u8 = lambda *sh: torch.empty(*sh, dtype=torch.uint8, device="cuda")
        self.out = [(u8(self.rows, self.cols // 4 * 3), u8(self.rows, self.cols // 32)) for _ in range(nbuf)]

    def step(self, i):
        B = self.B
        c, s = self.out[i % len(self.out)]
        B.fp4q_quantize_mxfp6(self.x[i % len(self.x)], B.F32, self.rows, self.cols, B.FP6_E2M3, c, s)

    def kernel_launch(self, i):
        self.step(i)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        w = self.host
        oracle.lib()
        t0 = time.perf_counter()
        oracle.quantize_mxfp6(np.ascontiguousarray(w[:4]), oracle.E2M3)
        per_row = (time.perf_counter() - t0) / 4
        nrows = int(min(self.rows, max(4, budget_s / per_row)))
        t0 = time.perf_counter()
        oracle.quantize_mxfp6(np.ascontiguousarray(w[:nrows]), oracle.E2M3)
        dt = time.perf_counter() - t0
        return {"value": nrows * self.cols / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"MX FP6 E2M3 of rows 0..{nrows - 1}, single thread, {dt:.1f} s"}


class WgradRHT(Workload):
    name = "wgrad_rht128_nvfp4_col_bf16_2x16384x4096"
    rows, cols = 16384, 4096

    def __init__(self):
        n = self.rows * self.cols
        self.elements = 2 * n
        per = 2 * n + n // 2 + n // 16
        self.algo_bytes = 2 * per
        self.kernel = "k_rht_nvfp4_col"
        self.kernel_bytes = per

    def setup(self, nbuf):
        import torch
        import oracle
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.g_host = si.wgrad_gradient(self.rows, self.cols, seed=4)
        self.x_host = si.wgrad_activation(self.rows, self.cols, seed=4)
        self.signs = B.fp4q_rht_signs_from_seed(4)
        self.g = [_dev_bf16(self.g_host)]
        self.xa = [_dev_bf16(self.x_host)]
        r, c = self.rows, self.cols
        u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")
        self.out = [dict(amax=torch.zeros(1, device="cuda"), ts=torch.zeros(1, device="cuda"), c=u8(c, r // 2),
                         s=u8(c, r // 16)) for _ in range(2)]

    def _q(self, x, o, rnd, seed, mode):
        B = self.B
        B.fp4q_quantize_nvfp4(x, B.BF16, self.rows, self.cols, B.COLWISE, rnd, seed, self.signs, mode, o["amax"],
                              o["ts"], None, None, o["c"], o["s"])

    def step(self, i):
        self._q(self.g[0], self.out[0], self.B.SR, 40, self.B.AMAX_COMPUTE)
        self._q(self.xa[0], self.out[1], self.B.RTN, 41, self.B.AMAX_COMPUTE)

    def kernel_launch(self, i):
        self._q(self.g[0], self.out[0], self.B.SR, 40, self.B.AMAX_GIVEN)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        signs = np.array(self.signs, dtype=np.uint32)
        t0 = time.perf_counter()
        y = oracle.rht(np.ascontiguousarray(self.g_host[:128]), signs)
        oracle.quantize_nvfp4(y, colwise=True, rnd=oracle.SR, seed=40)
        per_chunk = time.perf_counter() - t0
        nch = int(min(self.rows // 128, max(1, budget_s / per_chunk)))
        t0 = time.perf_counter()
        y = oracle.rht(np.ascontiguousarray(self.g_host[:128 * nch]), signs)
        oracle.quantize_nvfp4(y, colwise=True, rnd=oracle.SR, seed=40)
        dt = time.perf_counter() - t0
        return {"value": 128 * nch * self.cols / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"RHT (binary64) + column-wise NVFP4 SR of the gradient's first {128 * nch} tokens, "
                          f"single thread, {dt:.1f} s"}


class IF4RoundTrip(Workload):
    name = "if4_bf16_32768x8192"
    rows, cols = 32768, 8192

    def __init__(self):
        n = self.rows * self.cols
        self.elements = n
        self.algo_bytes = 2 * n + n // 2 + n // 16
        self.kernel = "k_if4"
        self.kernel_bytes = self.algo_bytes

    def setup(self, nbuf):
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        self.host = si.if4_mix(self.rows, self.cols, seed=5)
        self.x = [_dev_bf16(self.host)]
        r, c = self.rows, self.cols
        u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")
        self.out = [dict(amax=torch.zeros(1, device="cuda"), ts=torch.zeros(1, device="cuda"), c=u8(r, c // 2),
                         s=u8(r, c // 16))]
        self.y = torch.empty(r, c, dtype=torch.float32, device="cuda")

    def step(self, i):
        B, o = self.B, self.out[0]
        B.fp4q_quantize_if4(self.x[0], B.BF16, self.rows, self.cols, B.AMAX_COMPUTE, o["amax"], o["ts"], o["c"], o["s"])

    def kernel_launch(self, i):
        B, o = self.B, self.out[0]
        B.fp4q_quantize_if4(self.x[0], B.BF16, self.rows, self.cols, B.AMAX_GIVEN, o["amax"], o["ts"], o["c"], o["s"])

    def dequant(self):
        B, o = self.B, self.out[0]
        B.fp4q_dequantize(B.FMT_IF4, o["c"], o["s"], o["ts"], self.rows, self.cols, B.F32, self.y)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        gs = oracle.tensor_scale(oracle.amax(self.host))
        t0 = time.perf_counter()
        oracle.quantize_if4(np.ascontiguousarray(self.host[:16]), gs=gs)
        per_row = (time.perf_counter() - t0) / 16
        nrows = int(min(self.rows, max(16, budget_s / per_row)))
        t0 = time.perf_counter()
        oracle.quantize_if4(np.ascontiguousarray(self.host[:nrows]), gs=gs)
        dt = time.perf_counter() - t0
        return {"value": nrows * self.cols / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
                "sample": f"IF4 of rows 0..{nrows - 1} ({nrows}x{self.cols}), single thread, {dt:.1f} s"}


class GemmMXFP4(Workload):
    """Y = X W^T on MXFP4 operands (the forward GEMM after quantization): X an activation
    [8192 tokens x 8192] drawn as the activation workload's (N(0,1), 1% of the columns
    x30, bf16), W the weight workload's [8192 x 8192] N(0, 0.02^2) fp32; both quantized
    by fp4q_quantize_mxfp4 during setup, Y in bf16."""
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

    def setup(self, nbuf):
        import numpy as np
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        xb = si.activation(self.m, self.k, seed=2)
        w = si.weight(self.n, self.k, seed=3)
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to("cuda")
        qa = B.quantize_mxfp4(x)
        qb = B.quantize_mxfp4(torch.from_numpy(w).to("cuda"))
        torch.cuda.synchronize()
        self.host = {key: t.cpu().numpy() for key, t in (("ac", qa["codes"]), ("as", qa["scales"]),
                                                        ("bc", qb["codes"]), ("bs", qb["scales"]))}
        del x
        nbuf = min(nbuf, 2)   # 67 MB of operands + 134 MB of output per set: two sets exceed the cache
        self.ops = [(qa, qb)] + [({k: v.clone() for k, v in qa.items()}, {k: v.clone() for k, v in qb.items()})
                                 for _ in range(nbuf - 1)]
        self.y = [torch.empty(self.m, self.n, dtype=torch.bfloat16, device="cuda") for _ in range(nbuf)]

    def step(self, i):
        B = self.B
        qa, qb = self.ops[i % len(self.ops)]
        B.fp4q_gemm_mxfp4(qa["codes"], qa["scales"], qb["codes"], qb["scales"], self.m, self.n, self.k, B.BF16,
                          self.y[i % len(self.y)])

    def kernel_launch(self, i):
        self.step(i)

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        h = self.host
        oracle.lib()                                  # load (and if needed build) before timing
        t0 = time.perf_counter()
        oracle.gemm_mxfp4(h["ac"][:1], h["as"][:1], h["bc"][:32], h["bs"][:32])
        per_out = (time.perf_counter() - t0) / 32
        nout = int(max(64, min(self.m * 64, budget_s / per_out)))
        rows, cols = max(1, nout // 64), 64
        t0 = time.perf_counter()
        oracle.gemm_mxfp4(np.ascontiguousarray(h["ac"][:rows]), np.ascontiguousarray(h["as"][:rows]),
                          np.ascontiguousarray(h["bc"][:cols]), np.ascontiguousarray(h["bs"][:cols]))
        dt = time.perf_counter() - t0
        return {"value": 2.0 * rows * cols * self.k / dt, "unit": "FLOP/s", "cores": 1, "kind": "oracle",
                "sample": f"outputs [0..{rows - 1}] x [0..{cols - 1}] of Y (k = {self.k}), exact binary64 sums, "
                          f"single thread, {dt:.1f} s"}


class GemmNVFP4Wgrad(GemmMXFP4):
    """The weight gradient dY^T X from the Wgrad workload's operands (bf16 [16384 tokens x
    4096] each; 128-token RHT with seed 4; the gradient with SR, seed 40, the activation
    with RTN), quantized column-wise to NVFP4 during setup: C [4096 x 4096] over k = 16384
    tokens, bf16 out, on the bf16 MFMA after an exact decode."""
    name = "wgrad_gemm_nvfp4_rht_4096x4096x16384_bf16_out"
    m = n = 4096
    k = 16384
    bound, peak, unit = "mfma", PEAK_MFMA_BF16_TFLOPS, "TFLOP/s"
    dtype = "bf16"   # exact bf16 decode of E2M1 x E4M3, bf16 products, fp32 accumulation
    metric = "NVFP4 GEMM FLOP/s and % of MI355X dense bf16 matrix-core peak"

    def __init__(self):
        self.flops = 2 * self.m * self.n * self.k
        self.elements = self.flops
        self.algo_bytes = (self.m + self.n) * (self.k // 2 + self.k // 16) + 2 * self.m * self.n
        self.kernel = "k_gemm_nvfp4"
        self.kernel_bytes = self.algo_bytes

    def setup(self, nbuf):
        import numpy as np
        import torch
        import synth_inputs as si
        from block_scaled_fp4_05_amd import binding as B
        self.B = B
        to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to("cuda")
        g = to_dev(si.wgrad_gradient(self.k, self.m, seed=4))
        x = to_dev(si.wgrad_activation(self.k, self.n, seed=4))
        signs = B.fp4q_rht_signs_from_seed(4)
        qg = B.quantize_nvfp4(g, B.COLWISE, rnd=B.SR, sr_seed=40, rht_signs=signs)
        qx = B.quantize_nvfp4(x, B.COLWISE, rnd=B.RTN, rht_signs=signs)
        torch.cuda.synchronize()
        del g, x
        pick = lambda q: (q["col_codes"], q["col_scales"], q["tensor_scale"])
        self.host = {key: t.cpu().numpy() for key, t in zip(("ac", "as", "ga", "bc", "bs", "gb"), pick(qg) + pick(qx))}
        nbuf = min(nbuf, 2)
        ops = (pick(qg), pick(qx))
        self.ops = [ops] + [(tuple(t.clone() for t in ops[0]), tuple(t.clone() for t in ops[1])) for _ in range(nbuf - 1)]
        self.y = [torch.empty(self.m, self.n, dtype=torch.bfloat16, device="cuda") for _ in range(nbuf)]

    def step(self, i):
        B = self.B
        (ac, as_, ga), (bc, bs, gb) = self.ops[i % len(self.ops)]
        B.fp4q_gemm_nvfp4(ac, as_, ga, bc, bs, gb, self.m, self.n, self.k, B.BF16, self.y[i % len(self.y)])

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        h = self.host
        ga, gb = float(h["ga"][0]), float(h["gb"][0])
        oracle.lib()
        t0 = time.perf_counter()
        oracle.gemm_nvfp4(h["ac"][:1], h["as"][:1], ga, h["bc"][:16], h["bs"][:16], gb)
        per_out = (time.perf_counter() - t0) / 16
        nout = int(max(64, min(self.m * 64, budget_s / per_out)))
        rows, cols = max(1, nout // 64), 64
        t0 = time.perf_counter()
        oracle.gemm_nvfp4(np.ascontiguousarray(h["ac"][:rows]), np.ascontiguousarray(h["as"][:rows]), ga,
                          np.ascontiguousarray(h["bc"][:cols]), np.ascontiguousarray(h["bs"][:cols]), gb)
        dt = time.perf_counter() - t0
        return {"value": 2.0 * rows * cols * self.k / dt, "unit": "FLOP/s", "cores": 1, "kind": "oracle",
                "sample": f"outputs [0..{rows - 1}] x [0..{cols - 1}] of dY^T X (k = {self.k}), exact binary64 "
                          f"sums, single thread, {dt:.1f} s"}


class DeviceCopy(Workload):
    """Calibration, not a hot-path row: a plain device-to-device copy of 64 MiB.  It gives
    the copy rate this machine reaches and the factor between rocprofv3's FETCH_SIZE /
    WRITE_SIZE and bytes actually moved (each is known to be 64 MiB per launch)."""
    name = "device_copy_64MiB"
    nbytes = 64 << 20

    def __init__(self):
        self.elements = self.nbytes // 2
        self.algo_bytes = 2 * self.nbytes
        self.kernel = "copyBuffer"
        self.kernel_bytes = self.algo_bytes

    def setup(self, nbuf):
        import torch
        n = self.nbytes // 2
        self.src = [torch.randn(n, device="cuda").to(torch.bfloat16) for _ in range(nbuf)]
        self.dst = [torch.empty_like(t) for t in self.src]

    def step(self, i):
        k = i % len(self.src)
        self.dst[k].copy_(self.src[k])

    def kernel_launch(self, i):
        self.step(i)

    def cpu_baseline(self, budget_s):
        return None


WORKLOADS = {"activation": ActivationNVFP4, "weight": WeightNVFP4MX, "wgrad": WgradRHT, "if4": IF4RoundTrip,
             "mxfp6": WeightMXFP6, "gemm": GemmMXFP4, "gemm_nvfp4": GemmNVFP4Wgrad}
CALIBRATION = {"copy": DeviceCopy}


# --------------------------------------------------------------------------------------

def run(wl: Workload, steps: int, warmup: int, cpu_budget: float) -> dict:
    import torch
    wl.setup(nbuf=4)
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    # whole-step timing
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    # dominant kernel alone: back-to-back launches between two HIP events recorded on
    # the stream the kernel runs on (torch's current stream, which the binding uses)
    stream = torch.cuda.current_stream()
    nk = max(steps, 20)
    for i in range(4):
        wl.kernel_launch(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(nk):
        wl.kernel_launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    k_mean = e0.elapsed_time(e1) / nk
    mfma = getattr(wl, "bound", "hbm") == "mfma"
    if mfma:
        achieved = wl.flops / (k_mean * 1e-3) / 1e12
        peak, unit = wl.peak, wl.unit
    else:
        achieved = wl.kernel_bytes / (k_mean * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBPS, "GB/s"
    value = wl.elements / (ms_per_step * 1e-3)
    line = {
        "metric": getattr(wl, "metric", "FP4-quantized elements/s and achieved HBM GB/s (% of MI355X peak)"),
        "value": value,
        "unit": "FLOP/s" if mfma else "elements/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": getattr(wl, "dtype", "f32"),
        "data": "synthetic",
        "config": {"workload": wl.name, "elements_per_step": wl.elements, "algorithmic_bytes_per_step": wl.algo_bytes,
                   "whole_step_GBps": wl.algo_bytes / (ms_per_step * 1e-3) / 1e9,
                   "whole_step_frac_of_hbm_peak": wl.algo_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "roofline": {"bound": "mfma" if mfma else "hbm", "kernel": wl.kernel, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak, "traffic": counter_traffic(wl.kernel),
                     "kernel_ms_mean": k_mean, "kernel_launches_timed": nk,
                     "algorithmic_bytes_per_launch": wl.kernel_bytes},
    }
    # distribution of single steps: a separate pass, each step between its own events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        wl.step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    st = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda q: st[min(len(st) - 1, int(q * (len(st) - 1) + 0.5))]
    line["config"]["step_ms_p10"], line["config"]["step_ms_p50"], line["config"]["step_ms_p90"] = (
        pick(0.1), pick(0.5), pick(0.9))
    if mfma:
        flops_s = wl.flops / (ms_per_step * 1e-3)
        line["config"]["whole_step_TFLOPs"] = flops_s / 1e12
        line["config"]["whole_step_frac_of_peak"] = flops_s / 1e12 / wl.peak
        if cpu_budget > 0:
            cb = wl.cpu_baseline(cpu_budget)
            if cb is not None:
                line["cpu_baseline"] = cb
        return line
    # the call with the tensor amax given by the caller (no amax pass)
    given = getattr(wl, "given_launch", wl.kernel_launch)
    for i in range(4):
        wl.step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(nk):
        given(i)
    e1.record(stream)
    torch.cuda.synchronize()
    g_ms = e0.elapsed_time(e1) / nk
    line["config"]["amax_given_ms"] = g_ms
    line["config"]["amax_given_GBps"] = wl.kernel_bytes / (g_ms * 1e-3) / 1e9
    if isinstance(wl, WgradRHT):
        flops = 2 * 128 * (wl.rows * wl.cols)            # dense 128x128 contraction over one operand
        line["roofline"]["mfma_tflops_in_kernel"] = flops / (k_mean * 1e-3) / 1e12
        line["roofline"]["mfma_frac_of_bf16_peak"] = line["roofline"]["mfma_tflops_in_kernel"] / PEAK_MFMA_BF16_TFLOPS
    if isinstance(wl, IF4RoundTrip):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wl.dequant()
        e0.record(stream)
        for _ in range(5):
            wl.dequant()
        e1.record(stream)
        torch.cuda.synchronize()
        dq = e0.elapsed_time(e1) / 5
        n = wl.rows * wl.cols
        line["config"]["dequant_ms"] = dq
        line["config"]["dequant_GBps"] = (n // 2 + n // 16 + 4 * n) / (dq * 1e-3) / 1e9
    if cpu_budget > 0:
        cb = wl.cpu_baseline(cpu_budget)
        if cb is not None:
            line["cpu_baseline"] = cb
    return line


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="activation", choices=list(WORKLOADS) + list(CALIBRATION) + ["all"])
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline (0: skip)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; every step is one GPU's share "
                                   "(see the sharding notes), so --gpus must be 1"}))
        return 2
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    from block_scaled_fp4_05_amd import binding as B
    B.lib()
    names = list(WORKLOADS) if a.config == "all" else [a.config]
    for n in names:
        wl = WORKLOADS[n]() if n in WORKLOADS else CALIBRATION[n]()
        line = run(wl, a.steps, a.warmup, a.cpu_budget)
        print(json.dumps(line), flush=True)
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
