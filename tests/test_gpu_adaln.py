"""GPU parity of h3_adaln_modulate against the fp64 oracle on every row.

Wide rows (more than 4 x 64 sixteen-byte vectors: 2560 and 5376 bf16
values, 1536 fp32 values) take the run-of-rows kernel, narrow ones the
row-per-wavefront kernel.  Cases cover ragged row counts (n not a multiple
of the four-row batch, fewer rows than one batch), intervals that change the
modality set inside a batch and across workgroups, both branches, and rows
whose vectors do not divide evenly among the 256 threads."""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import device_inputs

from gpu_util import TOL, assert_close, widen

pytestmark = pytest.mark.gpu


def _segments(n, n_sets, cuts):
    pts = sorted({0, n} | {c for c in cuts if 0 < c < n})
    return [inputs.Segment(start=a, length=b - a, mod_set=(i * 2 + 1) % n_sets, T=b - a, kind="audio")
            for i, (a, b) in enumerate(zip(pts[:-1], pts[1:]))]


@pytest.mark.parametrize("dtype,dim", [("bf16", 5376), ("bf16", 2560), ("bf16", 256), ("f32", 1536), ("f32", 192)])
@pytest.mark.parametrize("n,cuts,br", [(1, (), 0), (3, (1, 2), 1), (37, (5, 6, 17, 33), 0),
                                       (1001, (3, 250, 251, 600, 997), 1),
                                       # more rows than the wide-row grid: each workgroup
                                       # takes rows w, w + G, ... across interval changes
                                       (3001, (2, 700, 701, 1023, 1025, 2047, 2999), 0)])
def test_adaln_all_rows(dtype, dim, n, cuts, br):
    import torch
    n_sets = 3
    x_h = inputs.draw_rows(None, (n, dim), 71 + n + dim, dtype=dtype)
    mod = np.random.Generator(np.random.PCG64(72 + dim)).standard_normal((n_sets, 6, dim)).astype(np.float32)
    segs = _segments(n, n_sets, cuts)
    d = device_inputs(None, {"x": x_h, "mod": mod})
    y = torch.full_like(d["x"], float("nan"))
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    blk.h3_adaln_modulate(d["x"], y, n, dim, d["mod"], n_sets, br, blk.segments(segs), len(segs), 1e-6, dt)
    torch.cuda.synchronize()
    ref = oracle.adaln_modulate(inputs.widen(x_h, dtype), mod.astype(np.float64), br, segs, 1e-6)
    assert_close(f"adaln_{dtype}_{dim}_{n}", widen(y, dtype), ref, TOL[dtype])
