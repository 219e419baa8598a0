"""GPU parity of the input/output adapters against the fp64 oracle.

* h3_patchify / h3_unpatchify move bits: they must equal the oracle's
  rearrangement of the same bits exactly, padding columns must be zero, and
  unpatchify(patchify(x)) must give x back bit for bit.
* Packing (patchify + input projections into the interval rows of the
  packed sequence) and unpacking (output projections + unpatchify) at the
  tiny fp32 workload end to end (1e-5), and at the 15 s 768p workload
  (92840 tokens, bf16) on sampled rows (2e-2), with the unpatchify of the
  projected video tokens checked bit for bit.
"""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import adapters, blk, inputs
from video_audio_diffusion_amd.block import device_inputs, host_array

from gpu_util import TOL, assert_close

pytestmark = pytest.mark.gpu


def _dev(a):
    return device_inputs(None, {"a": a})["a"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape,patch,ld", [((91, 48, 84, 24), (1, 2, 2), 128), ((3, 4, 6, 24), (1, 2, 2), 96),
                                            ((4, 6, 2, 8), (2, 3, 1), 56), ((600, 1, 1, 32), (1, 1, 1), 64),
                                            ((5, 2, 2, 16), (5, 2, 2), 328)])
def test_patchify_bit_exact(dtype, shape, patch, ld):
    import torch
    lat = inputs.draw_rows(None, shape, 700 + shape[0], dtype=dtype)
    T, H, W, C = shape
    pt, ph, pw = patch
    n = (T // pt) * (H // ph) * (W // pw)
    P = pt * ph * pw * C
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d_lat = _dev(lat)
    tok = torch.full((n, ld), float("nan"), dtype=tdt, device="cuda")
    blk.h3_patchify(d_lat, T, H, W, C, pt, ph, pw, tok, ld, dt)
    back = torch.full_like(d_lat, float("nan"))
    blk.h3_unpatchify(tok, ld, T, H, W, C, pt, ph, pw, back, dt)
    torch.cuda.synchronize()
    got = host_array(tok, dtype)
    want = oracle.patchify(lat, patch)            # bits rearranged, never converted
    assert np.array_equal(got[:, :P], want), "patchify moved the wrong values"
    assert np.all(inputs.widen(got[:, P:], dtype) == 0), "padding columns not zero"
    assert np.array_equal(host_array(back, dtype), lat), "unpatchify(patchify(x)) != x"


def _tiny():
    c = inputs.CONFIGS[1]
    return adapters.AdapterConfig(block=c, text_width=64)


def _weights(acfg, host):
    w_in = {m: adapters.pad_columns(_dev(host["w_in/" + m]), acfg.k_pad(m)) for m in ("text", "video", "audio")}
    w_out = {m: _dev(host["w_out/" + m]) for m in ("video", "audio")}
    return adapters.AdapterWeights(w_in, w_out)


def _oracle_features(acfg, host):
    c = acfg.block
    feats = {}
    for s in c.segments:
        a = inputs.widen(host["feat/" + s.kind], c.dtype)
        m = inputs.modality(s.kind)
        feats[s.kind] = a if m == "text" else oracle.patchify(a, acfg.patch(m))
    return feats


def test_tiny_pack_and_unpack_end_to_end():
    import torch
    acfg = _tiny()
    c = acfg.block
    host = inputs.make_adapter_inputs(c, acfg.text_width)
    ad = adapters.H3Adapters(acfg, _weights(acfg, host))
    feats = {s.kind: _dev(host["feat/" + s.kind]) for s in c.segments}
    x = torch.full((c.n_tok, c.dim), float("nan"), dtype=torch.float32, device="cuda")
    ad.pack(feats, x)
    lat_out = {k: torch.empty(inputs.adapter_shapes(c, acfg.text_width)["feat/" + k], dtype=torch.float32,
                              device="cuda") for k in adapters.TARGET_KINDS}
    ad.unpack(x, lat_out)
    torch.cuda.synchronize()
    f64 = {k: v.astype(np.float64) for k, v in host.items()}
    w_in = {s.kind: f64["w_in/" + inputs.modality(s.kind)] for s in c.segments}
    x_ref = oracle.project_inputs(_oracle_features(acfg, host), w_in, c.segments, c.dim)
    assert_close("adapters_pack", host_array(x, "f32"), x_ref, TOL["f32"])
    outs = oracle.project_outputs(host_array(x, "f32"), {k: f64["w_out/" + k] for k in adapters.TARGET_KINDS},
                                  c.segments)
    video = [s for s in c.segments if s.kind == "video"][0]
    v_ref = oracle.unpatchify(outs["video"], (video.T, video.H, video.W), acfg.patch("video"), acfg.video_channels)
    assert_close("adapters_unpack_video", host_array(lat_out["video"], "f32"), v_ref, TOL["f32"])
    assert_close("adapters_unpack_audio", host_array(lat_out["audio"], "f32").reshape(outs["audio"].shape),
                 outs["audio"], TOL["f32"])


def test_768p15s_pack_and_unpack_sampled():
    import torch
    c = inputs.CONFIGS[3]
    acfg = adapters.AdapterConfig(block=c)
    host = inputs.make_adapter_inputs(c, acfg.text_width)
    ad = adapters.H3Adapters(acfg, _weights(acfg, host))
    feats = {s.kind: _dev(host["feat/" + s.kind]) for s in c.segments}
    x = torch.full((c.n_tok, c.dim), float("nan"), dtype=torch.bfloat16, device="cuda")
    ad.pack(feats, x)
    lat_out = {k: torch.empty(inputs.adapter_shapes(c, acfg.text_width)["feat/" + k], dtype=torch.bfloat16,
                              device="cuda") for k in adapters.TARGET_KINDS}
    ad.unpack(x, lat_out)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(c, n_random=256)
    idx = torch.from_numpy(rows).cuda()
    x_rows = inputs.widen(host_array(x.index_select(0, idx), "bf16"), "bf16")
    feats64 = _oracle_features(acfg, host)
    for s in c.segments:
        m = inputs.modality(s.kind)
        sel = rows[(rows >= s.start) & (rows < s.start + s.length)]
        ref = oracle.linear(feats64[s.kind][sel - s.start], inputs.widen(host["w_in/" + m], "bf16"))
        assert_close(f"pack_{s.kind}", x_rows[np.isin(rows, sel)], ref, TOL["bf16"])
    for s in c.segments:
        if s.kind not in adapters.TARGET_KINDS:
            continue
        m = inputs.modality(s.kind)
        sel = rows[(rows >= s.start) & (rows < s.start + s.length)]
        proj = ad.proj[s.kind] if m == "video" else lat_out[s.kind].reshape(s.length, -1)
        got = inputs.widen(host_array(proj.index_select(0, torch.from_numpy(sel - s.start).cuda()), "bf16"), "bf16")
        ref = oracle.linear(x_rows[np.isin(rows, sel)], inputs.widen(host["w_out/" + m], "bf16"))
        assert_close(f"unpack_{s.kind}", got, ref, TOL["bf16"])
    video = [s for s in c.segments if s.kind == "video"][0]
    want = oracle.unpatchify(host_array(ad.proj["video"], "bf16"), (video.T, video.H, video.W),
                             acfg.patch("video"), acfg.video_channels)
    assert np.array_equal(host_array(lat_out["video"], "bf16"), want), "unpatchify of the projected tokens"
