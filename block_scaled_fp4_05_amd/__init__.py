"""block_scaled_fp4_05_amd -- block-scaled FP4 quantization for MI355X (gfx950).

The work happens in libfp4q.so (hand-written HIP kernels behind the C ABI in
include/fp4q.h); :mod:`.binding` marshals torch tensors and streams into it.
"""
from .binding import (  # noqa: F401
    AMAX_COMPUTE, AMAX_GIVEN, BF16, COLWISE, F32, FMT_IF4, FMT_MXFP4, FMT_NVFP4, FMT_NVFP4_2D, ROWWISE, RTN, SR,
    Fp4qError, Workspace, amax, dequantize, fp4q_abi_version, fp4q_amax, fp4q_dequantize, fp4q_quantize_if4,
    fp4q_quantize_mxfp4, fp4q_quantize_nvfp4, fp4q_quantize_nvfp4_2d, fp4q_rht, fp4q_rht_signs_from_seed,
    fp4q_status_string, lib, quantize_if4, quantize_mxfp4, quantize_nvfp4, quantize_nvfp4_2d, rht, stream_workspace,
)
