"""Workload shapes pinned to the numbers the pages print (tests/golden/h3_shapes.json)."""
import json
import os

import numpy as np

from video_audio_diffusion_amd import inputs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "h3_shapes.json")))


def test_video_token_grid_worked_example():
    g = GOLD["video_worked_example"]
    T, H, W, _ = g["video_THWC"]
    lat = g["latent_THWC"]
    assert [T // g["vae_temporal"], H // g["vae_spatial"], W // g["vae_spatial"]] == lat[:3]
    assert lat[3] == g["latent_channels"]
    # 1x2x2 patchify on the latent; the token grid helper works in pixels
    assert [lat[0], lat[1] // 2, lat[2] // 2] == g["tokens_THW"]
    assert inputs.token_grid(H, W) == tuple(g["tokens_THW"][1:])


def test_video_worked_example_2():
    g = GOLD["video_worked_example_2"]
    T, H, W = g["video_THW"]
    assert [T // 4, H // 16, W // 16, 24] == g["latent_THWC"]


def test_patch_width():
    g = GOLD["video_worked_example"]
    assert g["latent_channels"] * int(np.prod(g["patch"])) == GOLD["patch_width"]["value"]


def test_full_width_configs_match_backbone_table():
    b = GOLD["backbone"]
    for idx in (2, 3, 4):
        c = inputs.CONFIGS[idx]
        assert (c.dim, c.heads, c.head_dim, c.ffn) == (b["hidden"], b["heads"], b["head_dim"], b["ffn"])
        assert c.inner == b["inner"]


def test_adaln_table_size():
    b = GOLD["backbone"]
    assert inputs.N_MOD_SETS * inputs.N_MOD_CHUNKS * b["hidden"] == GOLD["adaln_out_features"]["value"]


def test_block_params_times_blocks_is_loaded_weight_size():
    b = GOLD["backbone"]
    D, I, F = b["hidden"], b["inner"], b["ffn"]
    per_block = 3 * I * D + D * I + 2 * F * D + D * F
    assert per_block == 385_351_680
    w = GOLD["weights_loaded_for_inference"]
    total = per_block * b["blocks"]
    assert abs(total - w["params"]) / w["params"] < w["tolerance_rel"]
    assert abs(2 * total - w["bytes_bf16"]) / w["bytes_bf16"] < w["tolerance_rel"]


def test_audio_token_rate():
    a = GOLD["audio_tokens"]
    assert a["seconds"] * a["latent_hz"] == a["tokens_per_channel"]
    # the 4 s / 15 s workloads take 40 tokens per second
    assert inputs.CONFIGS[2].segments[1].length == 4 * a["latent_hz"]
    assert inputs.CONFIGS[3].segments[1].length == 15 * a["latent_hz"]


def test_workload_token_counts():
    assert inputs.CONFIGS[1].n_tok == 72
    assert inputs.CONFIGS[2].n_tok == 25616
    assert inputs.CONFIGS[3].n_tok == 92840
    assert inputs.CONFIGS[4].n_tok == 194432
    assert inputs.latent_frames(4) == 25 and inputs.latent_frames(15) == 91
    v = inputs.CONFIGS[3].segments[-1]
    assert (v.T, v.H, v.W) == (91,) + inputs.token_grid(768, 1360)


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1.0 + 2 ** -8 + 2 ** -20],
                    dtype=np.float32)
    got = inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(vals))
    # 1+2^-8 is a tie between 1 and 1+2^-7: the even mantissa (1.0) wins;
    # 1+3*2^-8 ties between 1+2^-7 and 1+2^-6: the even one (1+2^-6) wins;
    # just above a tie rounds up
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 1.0 + 2 ** -7]


def test_inputs_are_seeded():
    c = inputs.CONFIGS[1]
    a = inputs.make_inputs(c)
    b = inputs.make_inputs(c)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (72, 192) and a["w_qkv"].shape == (768, 192)
    assert abs(a["w_qkv"].std() - 0.02) < 0.002
