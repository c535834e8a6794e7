"""The seeded generators: slices equal the same rows of the whole tensor; bf16 rounding is RNE."""
import numpy as np
import torch

from prefix_shared_branch_amd import inputs


def test_slice_consistency():
    cfg = inputs.replace(inputs.CONFIGS["tiny"], P=33000)
    whole = inputs.prompt_k(cfg)
    part = inputs.prompt_k(cfg, 1234, 4321)
    np.testing.assert_array_equal(whole[1234:4321], part)
    # rows straddling a chunk boundary
    rpc = inputs.CHUNK_ELEMS // (cfg.Hkv * cfg.Dqk)
    b = inputs.prompt_v(cfg, rpc - 3, rpc + 5)
    np.testing.assert_array_equal(inputs.prompt_v(cfg)[rpc - 3:rpc + 5], b)


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = (g.standard_normal(100000) * 3).astype(np.float32)
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_config_recipes():
    tiny = inputs.CONFIGS["tiny"]
    R = inputs.response_lengths(tiny)
    assert R.shape == (4,) and R.min() >= 64 and R.max() <= 128
    r = inputs.rewards(tiny)
    assert set(np.unique(r)).issubset({0.0, 1.0})
    mla = inputs.CONFIGS["mla"]
    assert mla.ldk == 576 and mla.ldv == 576
    v = inputs.prompt_v(inputs.replace(mla, P=3), 0, 3)
    k = inputs.prompt_k(inputs.replace(mla, P=3), 0, 3)
    np.testing.assert_array_equal(v, k[:, :, :512])
    s = inputs.bf16_bits_to_f64(inputs.prompt_k(inputs.replace(mla, P=2000)))
    assert abs(s.std() - 1 / 24) < 1e-3
