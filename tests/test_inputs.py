"""The seeded input module: determinism and bf16 rounding (CPU)."""
import numpy as np
import torch

from dual_window_attention_amd import inputs as I


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 0.0]   # ties to even
    bits = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = I.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_seeded_per_tensor():
    cfg = I.CONFIGS[1].scaled(seq=64)
    a = I.attention_inputs(cfg)
    b = I.attention_inputs(cfg)
    np.testing.assert_array_equal(a["q"].data, b["q"].data)
    assert not np.array_equal(a["q"].data[..., :8], a["k"].data[..., :8].repeat(2, axis=2))
    w1 = I.layer_weights(cfg)
    assert w1["w_down0"].shape == (cfg.d_model, cfg.d_ff)
    beta = I.beta_for(cfg)
    assert beta.shape == (1, 1) and 0 <= beta[0, 0] < 1
    cm = I.beta_for(cfg, chunk_mean=True)
    assert cm[0, 0] == np.float32(beta[0, 0] / 64)
    ragged = I.beta_for(cfg, seq=100, chunk_mean=True) * np.array([64, 36], np.float32)
    np.testing.assert_allclose(ragged, I.beta_for(cfg, seq=100), rtol=1e-6)


def test_outlier_keys_fraction():
    cfg = I.CONFIGS[4].scaled(batch=1, seq=4096)
    k = I.attention_inputs(cfg)["k"].f32()
    rms = np.sqrt((k.astype(np.float64) ** 2).mean(-1))
    frac = (rms > 4.0).mean()
    assert 0.04 < frac < 0.06


def test_stored_64k_layer_rows_match_the_generators():
    """The stored oracle rows of the 64K layer were written from exactly the
    inputs the generators produce now (else rerun make_layer_golden.py)."""
    from tests.golden import make_layer_golden as G
    ref = np.load(G.OUT)
    cfg = I.CONFIGS[3]
    q, k, v, x, w = G.inputs64(cfg)
    fp = G.fingerprint({"q": q, "k": k, "v": v, "x": x, **w})
    assert sorted(fp) == sorted(n for n in ref.files if n.startswith("fp_"))
    for n, a in fp.items():
        np.testing.assert_allclose(a, ref[n], rtol=1e-12, err_msg=n)
