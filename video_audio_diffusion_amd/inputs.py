"""Seeded synthetic inputs for one H3-Omni-Transformer block.

This module describes workloads and draws their input tensors.  It holds none
of the block's arithmetic: the fp64 oracle and the HIP path both take the
exact arrays produced here, so the only thing they share is the input bits.

Shapes and the packed-sequence layout follow the MiniMax H3 pages:

* backbone widths (hidden 5376, 56 heads x 128, FFN 14336): the
  "MiniMax-H3: native audio-video joint generation" notes, section 3.2 table;
* packed sequence of intervals (text, visual condition, audio, target video)
  with their index ranges kept: same notes, section 2.2;
* video token grid: 1x2x2 patchify of an f16t4d24 latent, so a 768p 16:9
  frame becomes a 24 x 42 token grid and tokens are flattened with t slowest
  and w fastest ("minimax-h3" reading notes, section 7.3);
* audio at 40 latent tokens per second per channel (notes section 4.3).

The tensors are:
    x      [N, D]           activations, N(0, 1)
    mod    [3, 6, D] fp32   cached AdaLN outputs per modality set, N(0, 1);
                            chunk order (shift1, scale1, gate1, shift2,
                            scale2, gate2), sets (text, visual, audio)
    w_qkv  [3I, D]          rows [q heads | k heads | v heads], N(0, 0.02^2)
    w_o    [D, I]
    w_gu   [2F, D]          rows [gate | up]
    w_d    [D, F]
    gamma_q, gamma_k [d]    per-head RMSNorm gains (1, or 4 for the
                            peaked-softmax variant)

Floating-point tensors of a bf16 workload are drawn in fp32 and rounded to
bf16 with round-to-nearest-even; they are held as uint16 bit patterns.
"""
from __future__ import annotations

import os
from dataclasses import dataclass, field, replace
from typing import Dict, List, Sequence, Tuple

import numpy as np

MOD_TEXT, MOD_VISUAL, MOD_AUDIO = 0, 1, 2
N_MOD_SETS = 3
N_MOD_CHUNKS = 6          # shift, scale, gate for the attention and FFN branch

TENSOR_IDS = {"x": 1, "mod": 2, "w_qkv": 3, "w_o": 4, "w_gu": 5, "w_d": 6}


@dataclass(frozen=True)
class Segment:
    """One interval [start, start+length) of the packed sequence."""
    start: int
    length: int
    mod_set: int
    T: int
    H: int = 1
    W: int = 1
    t0: int = 0
    h0: int = 0
    w0: int = 0
    kind: str = ""

    def __post_init__(self):
        if self.T * self.H * self.W != self.length:
            raise ValueError(f"segment {self.kind}: T*H*W != length")


@dataclass(frozen=True)
class BlockConfig:
    name: str
    index: int
    dim: int
    heads: int
    head_dim: int
    ffn: int
    rope_split: Tuple[int, int, int]
    rope_base: float
    dtype: str                     # "f32" or "bf16"
    segments: Tuple[Segment, ...]
    eps: float = 1e-6
    w_std: float = 0.02
    gamma: float = 1.0
    description: str = field(default="", compare=False)

    @property
    def inner(self) -> int:
        return self.heads * self.head_dim

    @property
    def n_tok(self) -> int:
        return sum(s.length for s in self.segments)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def pack(parts: Sequence[Tuple[str, int, int, int, int]]) -> Tuple[Segment, ...]:
    """Lay out (kind, mod_set, T, H, W) parts back to back from token 0."""
    segs: List[Segment] = []
    start = 0
    for kind, mod_set, T, H, W in parts:
        n = T * H * W
        segs.append(Segment(start, n, mod_set, T, H, W, kind=kind))
        start += n
    return tuple(segs)


def latent_frames(seconds: float, fps: int = 24) -> int:
    """Latent frames of a temporally causal t4 VAE: the first frame alone,
    then one latent frame per 4 video frames."""
    return 1 + int(round(seconds * fps)) // 4


def token_grid(height: int, width: int, stride: int = 32) -> Tuple[int, int]:
    """Token grid of a frame after 16x VAE downsampling and 2x2 patchify."""
    return height // stride, width // stride


FULL = dict(dim=5376, heads=56, head_dim=128, ffn=14336,
            rope_split=(64, 32, 32), rope_base=10000.0, dtype="bf16")

CONFIGS: Dict[int, BlockConfig] = {
    1: BlockConfig(
        name="tiny-f32", index=1, dim=192, heads=4, head_dim=64, ffn=512,
        rope_split=(16, 24, 24), rope_base=10000.0, dtype="f32",
        segments=pack([("text", MOD_TEXT, 16, 1, 1),
                       ("audio", MOD_AUDIO, 8, 1, 1),
                       ("video", MOD_VISUAL, 2, 4, 6)]),
        description="tiny fp32 block, 72 tokens"),
    2: BlockConfig(
        name="768p-16x9-4s", index=2, **FULL,
        segments=pack([("text", MOD_TEXT, 256, 1, 1),
                       ("audio", MOD_AUDIO, 160, 1, 1),
                       ("video", MOD_VISUAL, 25, 24, 42)]),
        description="full-width bf16 block, 4 s 16:9 768p, 25616 tokens"),
    3: BlockConfig(
        name="768p-16x9-15s", index=3, **FULL,
        segments=pack([("text", MOD_TEXT, 512, 1, 1),
                       ("audio", MOD_AUDIO, 600, 1, 1),
                       ("video", MOD_VISUAL, 91, 24, 42)]),
        description="full-width bf16 block, 15 s 16:9 768p, 92840 tokens"),
    4: BlockConfig(
        name="ref2va-9x16-15s", index=4, **FULL,
        segments=pack([("text", MOD_TEXT, 512, 1, 1)]
                      + [(f"ref_image{i}", MOD_VISUAL, 1, 42, 24) for i in range(9)]
                      + [("ref_video", MOD_VISUAL, 90, 42, 24)]
                      + [(f"ref_audio{i}", MOD_AUDIO, 600, 1, 1) for i in range(3)]
                      + [("audio", MOD_AUDIO, 600, 1, 1)]
                      + [("video", MOD_VISUAL, 91, 42, 24)]),
        description="Ref2VA-style long sequence, 9:16 15 s target, 194432 tokens"),
}


# ---------------------------------------------------------------- the stack

# Update mask ([notes] section 5): the sampler moves the generation targets
# (intervals of kind "video" and "audio") and leaves text and reference
# intervals as they are.  Their schedules' shifts ([notes] section 6: video
# 12, audio 3).
TARGET_SHIFTS: Dict[str, float] = {"video": 12.0, "audio": 3.0}


@dataclass(frozen=True)
class StackConfig:
    """The 50-block backbone ([notes] section 3.2 table) and one Euler step
    (step `step` of `n_steps`) over the packed sequence of `block`."""
    name: str
    block: BlockConfig
    n_blocks: int = 50
    n_steps: int = 50
    step: int = 0
    shifts: Tuple[Tuple[str, float], ...] = tuple(TARGET_SHIFTS.items())
    description: str = ""

    @property
    def n_tok(self) -> int:
        return self.block.n_tok


STACKS: Dict[int, StackConfig] = {
    5: StackConfig(name="stack50-768p-16x9-15s", block=CONFIGS[3],
                   description="50 blocks and one Euler step at 92840 tokens"),
}
STACK_TINY = StackConfig(name="stack50-tiny-f32", block=CONFIGS[1],
                         description="50 tiny fp32 blocks and one Euler step (parity)")


def stack_seed(cfg_index: int, block: int, tensor: str) -> int:
    """Seed of one block's tensor in a stack (inside the workload's range of
    1000 seeds, above the single-block ids)."""
    return 1000 * cfg_index + 100 + 8 * block + TENSOR_IDS[tensor]


def make_stack_block(cfg: BlockConfig, block: int) -> Dict[str, np.ndarray]:
    """Weights, modulation table and gains of block `block` of a stack."""
    D, I, F = cfg.dim, cfg.inner, cfg.ffn
    shapes = {"mod": ((N_MOD_SETS, N_MOD_CHUNKS, D), 1.0), "w_qkv": ((3 * I, D), cfg.w_std),
              "w_o": ((D, I), cfg.w_std), "w_gu": ((2 * F, D), cfg.w_std), "w_d": ((D, F), cfg.w_std)}
    out: Dict[str, np.ndarray] = {}
    for name, (shape, std) in shapes.items():
        dt = "f32" if name == "mod" else cfg.dtype
        a = np.empty(shape, dtype=np.uint16 if dt == "bf16" else np.float32)
        _fill_normal(a, stack_seed(cfg.index, block, name), std, dt)
        out[name] = a
    out["gamma_q"] = np.full(cfg.head_dim, cfg.gamma, dtype=np.float32)
    out["gamma_k"] = np.full(cfg.head_dim, cfg.gamma, dtype=np.float32)
    return out


def permuted(cfg: BlockConfig, order: Sequence[int]) -> Tuple[BlockConfig, np.ndarray]:
    """The same workload with its segments re-packed in `order`.

    Returns the new config and the row map `rows` such that token i of the
    new sequence is token rows[i] of the original one.  Grids, position
    offsets and modality sets travel with their segments."""
    segs = [cfg.segments[i] for i in order]
    new, rows, start = [], [], 0
    for s in segs:
        new.append(replace(s, start=start))
        rows.append(np.arange(s.start, s.start + s.length))
        start += s.length
    return replace(cfg, segments=tuple(new)), np.concatenate(rows)


# ---------------------------------------------------------------- bf16 bits

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    chunk = 1 << 24
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for i in range(0, flat_u.size, chunk):
        v = flat_u[i:i + chunk]
        bias = ((v >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_o[i:i + chunk] = ((v + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 copy of a stored tensor (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws -> the stored representation of the workload's dtype."""
    a = np.asarray(a, dtype=np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


# ---------------------------------------------------------------- draws

_CHUNK = 1 << 22          # elements per independently seeded chunk


def _fill_normal(out: np.ndarray, seed: int, std: float, dtype: str) -> None:
    """Fill `out` (flat view) with N(0, std^2) draws: chunk c of 2^22 elements
    comes from PCG64(SeedSequence([seed, c])), so chunks can be drawn by
    several threads and the result does not depend on the thread count."""
    import concurrent.futures as cf

    flat = out.reshape(-1)

    def one(c):
        lo = c * _CHUNK
        hi = min(flat.size, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, c])))
        a = g.standard_normal(size=hi - lo, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        flat[lo:hi] = f32_to_bf16_bits(a) if dtype == "bf16" else a

    n_chunks = (flat.size + _CHUNK - 1) // _CHUNK
    workers = min(16, os.cpu_count() or 1, max(1, n_chunks))
    if workers == 1:
        for c in range(n_chunks):
            one(c)
    else:
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(n_chunks)))


def draw(cfg_index: int, tensor: str, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """Seeded N(0, std^2) tensor in the stored representation of `dtype`
    (seed 1000 * workload index + tensor id)."""
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    _fill_normal(out, 1000 * cfg_index + TENSOR_IDS[tensor], std, dtype)
    return out


def make_inputs(cfg: BlockConfig, tensors: Sequence[str] = tuple(TENSOR_IDS)) -> Dict[str, np.ndarray]:
    """Draw the seeded input tensors of `cfg` (only those named in `tensors`)."""
    D, I, F = cfg.dim, cfg.inner, cfg.ffn
    shapes = {"x": ((cfg.n_tok, D), 1.0), "mod": ((N_MOD_SETS, N_MOD_CHUNKS, D), 1.0),
              "w_qkv": ((3 * I, D), cfg.w_std), "w_o": ((D, I), cfg.w_std),
              "w_gu": ((2 * F, D), cfg.w_std), "w_d": ((D, F), cfg.w_std)}
    out: Dict[str, np.ndarray] = {}
    for name in tensors:
        shape, std = shapes[name]
        out[name] = draw(cfg.index, name, shape, std, "f32" if name == "mod" else cfg.dtype)
    out["gamma_q"] = np.full(cfg.head_dim, cfg.gamma, dtype=np.float32)
    out["gamma_k"] = np.full(cfg.head_dim, cfg.gamma, dtype=np.float32)
    return out


# ---------------------------------------------------------------- adapters

ADAPTER_TENSOR_IDS = {"feat": 1, "w_in": 2, "w_out": 3}
MODALITY_IDS = {"text": 0, "video": 1, "audio": 2}


def modality(kind: str) -> str:
    """Interval kind -> "text", "video" (video, reference video and images)
    or "audio" (audio and reference audio)."""
    if kind == "text":
        return "text"
    if "audio" in kind:
        return "audio"
    if "video" in kind or "image" in kind:
        return "video"
    raise ValueError(f"no modality for interval kind {kind!r}")


def adapter_shapes(cfg: BlockConfig, text_width: int, video_channels: int = 24, audio_channels: int = 32,
                   video_patch=(1, 2, 2)) -> Dict[str, tuple]:
    """Shapes of the adapter inputs: "feat/<kind>" -> channels-last latent
    [T, H, W, C] of a video/audio interval ([len, text_width] for text);
    "w_in/<modality>" -> [dim, values per token]; "w_out/<modality>" ->
    [values per token, dim] for video and audio."""
    pt, ph, pw = video_patch
    width = {"text": text_width, "video": pt * ph * pw * video_channels, "audio": audio_channels}
    out = {}
    for s in cfg.segments:
        m = modality(s.kind)
        out["feat/" + s.kind] = ((s.length, text_width) if m == "text" else
                                 (s.T * pt, s.H * ph, s.W * pw, video_channels) if m == "video" else
                                 (s.T, s.H, s.W, audio_channels))
        out["w_in/" + m] = (cfg.dim, width[m])
        if m != "text":
            out["w_out/" + m] = (width[m], cfg.dim)
    return out


def make_adapter_inputs(cfg: BlockConfig, text_width: int, **geom) -> Dict[str, np.ndarray]:
    """Seeded adapter inputs: features and latents N(0,1), projections
    N(0, w_std^2), in the stored representation of cfg.dtype.  Seed:
    1000 * workload index + 600 + 10 * (interval or modality id) + tensor id."""
    out = {}
    for name, shape in adapter_shapes(cfg, text_width, **geom).items():
        kind, key = name.split("/")
        if kind == "feat":
            sub = [s.kind for s in cfg.segments].index(key)
            std = 1.0
        else:
            sub = MODALITY_IDS[key]
            std = cfg.w_std
        a = np.empty(shape, dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
        _fill_normal(a, 1000 * cfg.index + 600 + 10 * sub + ADAPTER_TENSOR_IDS[kind], std, cfg.dtype)
        out[name] = a
    return out


def draw_rows(cfg: BlockConfig, shape, seed: int, dtype: str = None) -> np.ndarray:
    """Extra seeded N(0,1) tensors (per-call parity inputs, peaked variants)."""
    out = np.empty(shape, dtype=np.uint16 if (dtype or cfg.dtype) == "bf16" else np.float32)
    _fill_normal(out, seed, 1.0, dtype or cfg.dtype)
    return out


def sample_rows(cfg: BlockConfig, n_random: int = 2048, seed: int = 7) -> np.ndarray:
    """Rows checked at full size: every segment boundary +-1, the first and
    last rows, and seeded random rows."""
    n = cfg.n_tok
    rows = {0, n - 1}
    for s in cfg.segments:
        for r in (s.start - 1, s.start, s.start + 1, s.start + s.length - 2,
                  s.start + s.length - 1, s.start + s.length):
            if 0 <= r < n:
                rows.add(r)
    g = np.random.Generator(np.random.PCG64(seed))
    rows.update(int(r) for r in g.integers(0, n, size=min(n_random, n)))
    return np.array(sorted(rows), dtype=np.int64)
