"""Input and output adapters around the backbone, as libh3blk calls.

"MiniMax-H3: native audio-video joint generation" notes: every input is
mapped by its own projection to the common hidden width before packing
(section 2.2); the backbone predicts the update of the video and audio
latents (2.3); the modality-specific parameters are the input/output
projections and the AdaLN branch (3); the visual latent has 24 channels and
is cut into 1x2x2 patches of 96 values (4.1); an audio token carries 32
latent channels (4.3); text features are 5120 wide (3.2 table).

Input side, per interval of the packed sequence:
    video / audio : h3_patchify(latent) -> token rows zero-padded to K_pad,
                    then h3_gemm_bf16(tokens, W_in) straight into the
                    interval's rows of x
    text          : h3_gemm_bf16(features, W_in) into its rows
Output side, per generation target (kinds "video" and "audio"):
    h3_gemm_bf16(x_out rows, W_out) -> [len, P]; video then h3_unpatchify
    back to its latent grid (an audio token row already is its latent).

Weights are stored [out][K_pad] with zero columns past the feature width,
so the zero-padded token rows give exactly the unpadded product.  This
module only allocates buffers and issues the calls.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

from . import blk
from .inputs import modality

VIDEO_PATCH = (1, 2, 2)
VIDEO_CHANNELS = 24
AUDIO_CHANNELS = 32
TARGET_KINDS = ("video", "audio")


@dataclass(frozen=True)
class AdapterConfig:
    block: object                       # BlockConfig: segments, hidden width, dtype
    text_width: int = 5120
    video_channels: int = VIDEO_CHANNELS
    audio_channels: int = AUDIO_CHANNELS
    video_patch: Tuple[int, int, int] = VIDEO_PATCH
    name: str = field(default="", compare=False)

    @property
    def k_step(self) -> int:
        return 64 if self.block.dtype == "bf16" else 32

    def patch(self, mod: str) -> Tuple[int, int, int]:
        return self.video_patch if mod == "video" else (1, 1, 1)

    def channels(self, mod: str) -> int:
        return self.video_channels if mod == "video" else self.audio_channels

    def feature_width(self, mod: str) -> int:
        """Values per token before the input projection."""
        if mod == "text":
            return self.text_width
        pt, ph, pw = self.patch(mod)
        return pt * ph * pw * self.channels(mod)

    def k_pad(self, mod: str) -> int:
        """Contraction width of the input GEMM: the feature width rounded up
        to the GEMM's k-step."""
        k = self.feature_width(mod)
        return -(-k // self.k_step) * self.k_step

    def latent_shape(self, seg) -> Tuple[int, ...]:
        """[T, H, W, C] latent of a video/audio interval; [len, width] text."""
        mod = modality(seg.kind)
        if mod == "text":
            return (seg.length, self.text_width)
        pt, ph, pw = self.patch(mod)
        return (seg.T * pt, seg.H * ph, seg.W * pw, self.channels(mod))


@dataclass
class AdapterWeights:
    w_in: Dict[str, object]     # modality -> [D, K_pad], zero columns past the feature width
    w_out: Dict[str, object]    # "video" / "audio" -> [P, D]


def pad_columns(w, k_pad: int):
    """[rows, K] weight -> [rows, k_pad] with zero columns past K (a one-time
    weight layout step, on the device)."""
    import torch
    if w.shape[1] == k_pad:
        return w.contiguous()
    out = torch.zeros(w.shape[0], k_pad, dtype=w.dtype, device=w.device)
    out[:, :w.shape[1]] = w
    return out


class H3Adapters:
    """Input packing and output unpacking of one packed sequence."""

    def __init__(self, acfg: AdapterConfig, weights: AdapterWeights, device="cuda"):
        import torch
        self.cfg = acfg
        self.w = weights
        c = acfg.block
        self.dt = blk.H3_BF16 if c.dtype == "bf16" else blk.H3_F32
        self.tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.tok: Dict[str, object] = {}
        self.proj: Dict[str, object] = {}
        for s in c.segments:
            mod = modality(s.kind)
            if mod != "text":
                self.tok[s.kind] = torch.empty(s.length, acfg.k_pad(mod), dtype=self.tdt, device=device)
            if s.kind in TARGET_KINDS:
                self.proj[s.kind] = torch.empty(s.length, acfg.feature_width(mod), dtype=self.tdt, device=device)

    def pack(self, feats: Dict[str, object], x, stream: Optional[int] = None, mark=None):
        """x [N, D] <- per-interval input projections of `feats` (kind ->
        latent [T, H, W, C] for video/audio, features [len, width] for text).
        `mark(name)`, if given, is called before each library call."""
        a, c = self.cfg, self.cfg.block
        D = c.dim
        st = blk.current_stream() if stream is None else stream
        mark = mark or (lambda name: None)
        for s in c.segments:
            mod = modality(s.kind)
            if mod == "text":
                A, K = feats[s.kind], a.text_width
            else:
                T, H, W, C = a.latent_shape(s)
                A, K = self.tok[s.kind], a.k_pad(mod)
                mark("patchify_" + s.kind)
                blk.h3_patchify(feats[s.kind], T, H, W, C, *a.patch(mod), A, K, self.dt, st)
            mark("gemm_in_" + s.kind)
            blk.h3_gemm_bf16(A, K, self.w.w_in[mod], K, x[s.start:s.start + s.length], D, s.length, D, K,
                             self.dt, st)
        return x

    def unpack(self, x_out, latents: Dict[str, object], stream: Optional[int] = None, mark=None):
        """latents[kind] <- output projection of the target intervals' rows
        of x_out (video unpatchified to [T, H, W, C], audio [len, 32])."""
        a, c = self.cfg, self.cfg.block
        D = c.dim
        st = blk.current_stream() if stream is None else stream
        mark = mark or (lambda name: None)
        for s in c.segments:
            if s.kind not in TARGET_KINDS:
                continue
            mod = modality(s.kind)
            P = a.feature_width(mod)
            out = self.proj[s.kind] if mod == "video" else latents[s.kind]
            mark("gemm_out_" + s.kind)
            blk.h3_gemm_bf16(x_out[s.start:s.start + s.length], D, self.w.w_out[mod], D, out, P, s.length, P, D,
                             self.dt, st)
            if mod == "video":
                T, H, W, C = a.latent_shape(s)
                mark("unpatchify_" + s.kind)
                blk.h3_unpatchify(out, P, T, H, W, C, *a.patch(mod), latents[s.kind], self.dt, st)
        return latents
