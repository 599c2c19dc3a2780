"""Seeded input generator: determinism, rounding, and the workload shapes the pages print."""
import json
import math
import os

import numpy as np

from joint_video_audio_trigflow_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_high_res_shape_matches_printed_latent():
    g = json.load(open(os.path.join(GOLDEN, "pages_workload_shapes.json")))
    _, frames, ch, hh, ww = g["high_res_latent_shape"]
    assert frames * hh * ww == g["high_res_video_tokens"]
    hr = inputs.CONFIGS["high-res"]
    assert hr.Nv == g["high_res_video_tokens"] and hr.Cv == ch == g["latent_channels"]
    # the same 32x spatial packing at the standard resolution
    py, px = g["standard_pixels"]
    sy = g["high_res_pixels"][0] // hh
    assert inputs.CONFIGS["standard"].Nv == frames * (py // sy) * (px // sy)


def test_bf16_rounding_is_round_to_nearest_even():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 spacing at 1
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 1e-6, -one - ulp / 2, 3.0e38])
    r = inputs.round_bf16(x)
    assert r[0] == one                    # tie -> even
    assert r[1] == one + 2 * ulp          # tie -> even
    assert r[2] == one + ulp              # above tie -> up
    assert r[3] == -one
    assert np.isfinite(r[4])
    y = np.random.default_rng(0).standard_normal(1000)
    ry = inputs.round_bf16(y)
    assert np.all(np.abs(ry - y) <= np.abs(y) * 2.0 ** -8)
    assert np.array_equal(inputs.round_bf16(ry), ry)


def test_generator_is_deterministic_and_shaped():
    for name in ("tiny", "small", "stress"):
        cfg = inputs.CONFIGS[name]
        a = inputs.make_data(cfg)
        b = inputs.make_data(cfg)
        for k in a:
            assert np.array_equal(a[k], b[k])
        assert a["z0_v"].shape == (cfg.B, cfg.Nv, cfg.Cv)
        assert a["z0_a"].shape == (cfg.B, cfg.Na, cfg.Ca)
        assert a["text"].shape == (cfg.B, cfg.Nt, cfg.d)
        assert a["text_mask"].sum(1).tolist() == [cfg.Ntv] * cfg.B
        w = inputs.make_weights(cfg, "teacher")
        assert w["w_qkv"].shape == (3 * cfg.d, cfg.d)
        assert not np.array_equal(w["w_t"], inputs.make_weights(cfg, "student")["w_t"])


def test_timestep_ranges():
    t = inputs.make_data(inputs.CONFIGS["stress"])["t"]
    assert np.all((t[:4] > 0.01) & (t[:4] < 0.1))
    assert np.all((t[4:] > math.pi / 2 - 0.1) & (t[4:] < math.pi / 2 - 0.01))
    t = inputs.make_data(inputs.CONFIGS["small"])["t"]
    assert np.all((t > 0.05) & (t < math.pi / 2 - 0.05))


def test_padding_matches_sixty_percent():
    assert inputs.CONFIGS["standard"].Ntv == 256 - round(0.6 * 256)
