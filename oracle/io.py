"""fp64 oracle of the input and output adapters around the backbone.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "MiniMax-H3: native audio-video joint generation" notes, section 2.2
  (every input is mapped by its own projection to the common hidden width
  before the packed sequence is formed), section 2.3 (the backbone predicts
  update directions for the video and the audio latents), section 3 (the
  modality-specific parameters sit in the input/output projections and the
  AdaLN branch), the section 3.2 table (text features are 5120 wide), 4.1
  (f16t4d24 visual latent with 24 channels, then a 1x2x2 patchify; one
  visual patch is 96 values wide before its projection) and 4.3 (audio
  latents: 40 tokens per second per channel, 32 channels per token);
* "MiniMax-H3 paper reading", 7.3 (patchify with patch (1, 2, 2) over
  (t, h, w), then flatten(0, 2): t slowest, w fastest).

Readings (the pages give no formula for these steps):
* a latent is channels-last, [T, H, W, C];
* the values of one patch are ordered (dt, dh, dw, c), channels fastest;
* an audio token is one latent vector of 32 channels (a 1x1x1 patch);
* every projection is a bias-free linear map, like those inside the block:
  the rows of an interval in the packed sequence are features . W_in^T, and
  the adapter output of an interval is x_out[rows] . W_out^T, unpatchified
  back to the latent grid for video.
"""
import numpy as np

from .block import linear


def patchify(latent, patch):
    """[T, H, W, C] -> [(T/pt)(H/ph)(W/pw), pt*ph*pw*C], tokens in (t, h, w)
    order with w fastest, patch values in (dt, dh, dw, c) order."""
    T, H, W, C = latent.shape
    pt, ph, pw = patch
    if T % pt or H % ph or W % pw:
        raise ValueError("latent grid not divisible by the patch")
    x = np.asarray(latent).reshape(T // pt, pt, H // ph, ph, W // pw, pw, C)
    x = x.transpose(0, 2, 4, 1, 3, 5, 6)
    return x.reshape((T // pt) * (H // ph) * (W // pw), pt * ph * pw * C)


def unpatchify(tokens, grid, patch, channels):
    """Inverse of `patchify`: tokens [n, pt*ph*pw*C] of a (T', H', W') token
    grid -> latent [T' pt, H' ph, W' pw, C]."""
    Tp, Hp, Wp = grid
    pt, ph, pw = patch
    x = np.asarray(tokens)[:, :pt * ph * pw * channels].reshape(Tp, Hp, Wp, pt, ph, pw, channels)
    x = x.transpose(0, 3, 1, 4, 2, 5, 6)
    return x.reshape(Tp * pt, Hp * ph, Wp * pw, channels)


def project_inputs(features, weights, segments, dim):
    """The packed sequence's hidden states: rows of interval s are
    features[s] . weights[s]^T ([notes] 2.2).  `features` and `weights` map
    an interval's kind to its [len, K] features and [dim, K] projection."""
    n = segments[-1].start + segments[-1].length
    x = np.zeros((n, dim))
    for s in segments:
        f = np.asarray(features[s.kind], dtype=np.float64)
        if f.shape[0] != s.length:
            raise ValueError(f"{s.kind}: {f.shape[0]} feature rows for {s.length} tokens")
        x[s.start:s.start + s.length] = linear(f, weights[s.kind])
    return x


def project_outputs(x_out, weights, segments):
    """Per-interval output projections x_out[rows] . W_out^T for the kinds in
    `weights` ([notes] 2.3 and 3)."""
    return {s.kind: linear(np.asarray(x_out, dtype=np.float64)[s.start:s.start + s.length], weights[s.kind])
            for s in segments if s.kind in weights}
