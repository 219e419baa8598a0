"""fp64 CPU oracle of one MiniMax H3 Omni-Transformer block forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark do.  It shares no code with the HIP path; the only
common module is the seeded input generator, which holds none of the
block's arithmetic.

Every function is a plain numpy float64 statement of what the pages define;
see `oracle.block` for the citations and for the readings taken where the
pages are silent.  Parity status: every step is pinned by the CPU tests in
tests/test_oracle_*.py (closed forms, invariants, library special cases and
brute force); the block's numeric values as a whole are pinned only through
those steps and block-level invariants, since the pages print no worked
numeric example of the block.
"""
from .block import (  # noqa: F401
    token_table, rms_normalize, adaln_modulate, linear, qk_rmsnorm,
    rope_inv_freq, rope3d, attention, silu, swiglu, gate_residual,
    block_forward, BRANCH_ATTN, BRANCH_FFN,
)
from .stack import shifted_sigma, euler_coefficients, euler_update, stack_forward  # noqa: F401
from .io import patchify, unpatchify, project_inputs, project_outputs  # noqa: F401
from .fp8 import (e4m3_decode, e4m3_encode, quantize_rows, gemm_fp8, E4M3_MAX,  # noqa: F401
                  quantize_qkv, dequantize_qkv)
