"""Pins of the seeded input generators (CPU only)."""

import numpy as np
import torch

from synth import CONFIGS
from synth import inputs as S


def test_splitmix64_published_sequence():
    # splitmix64 seeded with state 0: the generator adds the golden gamma before mixing,
    # so its outputs are mix(k * gamma) for k = 1, 2, 3 (Steele, Lea & Flood 2014)
    gamma = 0x9E3779B97F4A7C15
    outs = [S.splitmix64_scalar((k * gamma) & ((1 << 64) - 1)) for k in range(0, 3)]
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    v = S.splitmix64(np.array([0, gamma, 2 * gamma % (1 << 64)], dtype=np.uint64))
    assert [int(a) for a in v] == outs


def test_value_generator_statistics_and_bounds():
    t = S.value_rows(0, np.arange(2000), 256, "f32").astype(np.float64)
    assert abs(t.mean()) < 2e-4
    assert abs(t.std() - 0.02) < 2e-4
    assert np.abs(t).max() <= 0.02 * 3.4642
    # rows are addressable: a row drawn alone equals the same row drawn in a block
    np.testing.assert_array_equal(S.value_rows(0, [1234], 256, "f32")[0], t[1234].astype(np.float32))


def test_value_rows_bf16_is_rounded_f32():
    f = S.value_rows(3, np.arange(64), 128, "f32")
    b = S.value_rows(3, np.arange(64), 128, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_make_inputs_shapes_and_prefix():
    cfg = CONFIGS["pkm_1m_bf16"].with_(T=64, n_sub=32)
    a = S.make_inputs(cfg, seed=0)
    assert a["x"].shape == (64, 1024) and a["x"].dtype == np.uint16
    assert a["W_q"].shape == (1024, 2048)
    assert a["subkeys"].shape == (4, 2, 32, 256)
    b = S.make_inputs(cfg, seed=0, T=10)
    np.testing.assert_array_equal(a["x"][:10], b["x"])
    x = S.bf16_bits_to_f32(a["x"]).astype(np.float64)
    assert abs(x.std() - 1.0) < 0.01
