"""fp8_precision_numerics_amd — per-tensor-scaled FP8 GEMM with delayed scaling on
AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libfp8mi.so (include/fp8mi.h) built from
the HIP sources under csrc/; this package is its Python binding (argument
marshalling), a holder for one tensor's delayed-scaling buffers, and the
sequencing of one FP8 linear layer's forward and backward GEMMs (Fp8Linear).
"""

from ._binding import (ACCUM_EXACT, ACCUM_MFMA_FP8, BF16, E4M3, E5M2, EXPORTED_SYMBOLS, F32, QUANTIZE_WORKSPACE_BYTES, Fp8Error, fp8_amax_update, fp8_gemm,  # noqa: F401
                       fp8_dequant_sum, fp8_gemm_mx, fp8_gemm_requant, fp8_grouped_gemm, fp8_quantize, fp8_quantize_blockwise, fp8_quantize_mx, fp8_quantize_update, fp8_quantize_update_noalloc, fp8_shared_scale, library_path, load_library, mx_scale_ld, mx_scale_pos,
                       status_string, version)
from .linear import Fp8Linear  # noqa: F401
from .state import DelayedScalingState, Recipe  # noqa: F401
