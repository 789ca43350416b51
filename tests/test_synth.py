"""Seeded synthetic inputs: reproducibility, bf16 rounding, and the structure
each workload asks for (bias channel, correlated tokens, Zipf popularity)."""
import numpy as np

from intra_expert_activation_amd import synth


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5, 0.0,
                  np.float32(3.4e38), np.inf], np.float32)
    b = synth.f32_to_bf16_bits(f)
    # 1+2^-8 is halfway between 1 and 1+2^-7: ties go to the even mantissa (1.0);
    # 1+3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties go to 1+2^-6.
    np.testing.assert_array_equal(
        synth.bf16_bits_to_f32(b),
        np.array([1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5, 0.0, np.inf, np.inf], np.float32))
    assert synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] & 0x7F80 == 0x7F80


def test_reproducible_and_prefix():
    c = synth.config(4, I=128, E=16)
    a1 = synth.make_layer(c)
    a2 = synth.make_layer(c)
    for k in ("w_gate", "w_up", "w_down", "ws_gate"):
        np.testing.assert_array_equal(a1[k], a2[k])
    x64, l64 = synth.make_tokens(c, 2)
    x8, l8 = synth.make_tokens(c, 2, 8)
    np.testing.assert_array_equal(x8, x64[:8])
    np.testing.assert_array_equal(l8, l64[:8])
    xc, _ = synth.make_tokens(c, 1)
    assert xc.shape[0] == synth.CALIB_TOKENS and not np.array_equal(xc[:8], x8)


def test_weight_scale_and_bias_channel():
    c = synth.config(2, E=4, I=256)
    L = synth.make_layer(c)
    wg = synth.bf16_bits_to_f32(L["w_gate"])
    body = wg[:, :, :-1]
    assert abs(body.std() - 0.02) < 1e-3 and abs(body.mean()) < 1e-3
    bias = wg[:, :, -1]
    assert abs(bias.mean() + 1.5) < 0.1 and abs(bias.std() - 0.5) < 0.1
    x, _ = synth.make_tokens(c, 2)
    xf = synth.bf16_bits_to_f32(x)
    assert (xf[:, -1] == 1.0).all()
    # correlated tokens: pairwise correlation close to rho = 0.9
    z = xf[:, :-1]
    z = (z - z.mean(1, keepdims=True)) / z.std(1, keepdims=True)
    corr = (z @ z.T) / z.shape[1]
    off = corr[~np.eye(len(corr), dtype=bool)]
    assert abs(off.mean() - 0.9) < 0.02


def test_zipf_popularity_skew():
    c = synth.config(4)
    _, logits = synth.make_tokens(c, 2)
    K = c["K"]
    top = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    counts = np.bincount(top.ravel(), minlength=c["E"])
    # Gumbel-top-k over ln p: the most popular experts are picked far more often
    assert counts.max() >= 40 and (counts == 0).sum() >= 5
