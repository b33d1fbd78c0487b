"""CPU oracle for FP8 quantization and the scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU statement of what the GPU path computes.  Only the test suite, the smoke
check of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``quantize_scaled_gemm_amd``) never imports,
calls or links anything here, and nothing here imports the product path: the
two share no kernels, headers, helpers, tables or constants.

Sources, cited per function:
  * "Low-Precision Training Guide" (Megatron Core developer guide): the recipe
    names (delayed, tensorwise, mxfp8, blockwise), the block shapes, the
    margin knob, the amax history length and compute algorithm.
  * "Benefits of Using FP8 Precision with MegaDLMs and Required Hardware": the
    E4M3 format flag and the hybrid mode; the FP8 store of the MLP
    activation's input (activation_func_fp8_input_store).
  * "How to reduce cuda memory usage of fp8?" (TransformerEngine issue 1764):
    why a transposed FP8 copy of each operand exists (the backward pass reads
    it).
  * Outside the pages, named where used: the OCP 8-bit floating point
    specification (bit layouts of E4M3 and E5M2, maxima 448 and 57344) and the
    OCP Microscaling v1.0 specification (the E8M0 scale byte).

Every reading taken where the pages are silent is listed in the module that
takes it.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (closed forms, exhaustive enumeration, exact
rational brute force, an independent library cast).  No function here is
"parity unpinned".
"""

from .fp8 import (  # noqa: F401
    FORMATS,
    decode_exact,
    decode_table,
    encode_exact,
    encode,
    dequantize,
)
from .recipes import (  # noqa: F401
    amax,
    tensorwise_scale,
    cast_transpose,
    quantize_tensorwise,
    DelayedState,
    amax_update,
    mx_exponent,
    mx_quantize,
    block_scale,
    block_quantize_1x128,
    block_quantize_128x128,
)
from .gemm import (  # noqa: F401
    gemm_per_tensor,
    gemm_mx,
    gemm_block,
    gemm_exact_fraction,
    accumulate,
    wgrad_bf16,
    tolerance_check,
    mx_operand,
    mfma_accumulation_bound,
)
from . import nvfp4  # noqa: F401  (NVFP4: E2M1 elements, E4M3 1x16 block scales, fp32 tensor scale)
from .activation import (  # noqa: F401
    gelu,
    gelu_grad,
    act_fp8_store_fwd,
    act_fp8_store_bwd,
    elementwise_check,
)
