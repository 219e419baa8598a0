"""C-ABI behaviour on the GPU that the CPU tests cannot reach.

A HIP error left behind in the calling thread by some earlier, unrelated
call (here a failed hipSetDevice) must not be reported as the library
call's own failure: the call runs and its result is right.
"""
import ctypes

import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs

from gpu_util import TOL, assert_close, widen

pytestmark = pytest.mark.gpu


def test_stale_hip_error_is_not_reported_as_the_calls_own():
    import torch
    blk.load()
    # the HIP runtime libh3blk is linked against (already loaded under this name)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipPeekAtLastError.restype = ctypes.c_int
    n, F = 37, 96
    gu_h = inputs.draw_rows(None, (n, 2 * F), 77, dtype="bf16")
    gu = torch.from_numpy(gu_h.view(np.int16)).view(torch.bfloat16).cuda()
    h = torch.full((n, F), float("nan"), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    assert hip.hipSetDevice(1 << 20) != 0          # no such device: the error stays behind
    assert hip.hipPeekAtLastError() != 0
    blk.h3_swiglu(gu, h, n, F, blk.H3_BF16)         # raises on any status but H3_OK
    torch.cuda.synchronize()
    ref = oracle.swiglu(inputs.widen(gu_h, "bf16"), F)
    assert_close("swiglu_after_stale_error", widen(h, "bf16"), ref, TOL["bf16"])
