"""The seeded input generator: slices agree with whole draws, bf16 rounding
is round-to-nearest-even, tokens are in range."""
import numpy as np

import datagen


def test_slices_match_whole_draws_across_chunks():
    C = datagen.CHUNK
    whole = datagen.draw_flat(0, 3, 0, 2 * C + 17, "bf16")
    for st, sp in [(0, 10), (5, C + 3), (C - 4, C + 4), (2 * C, 2 * C + 17)]:
        assert np.array_equal(whole[st:sp], datagen.draw_flat(0, 3, st, sp, "bf16"))


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 3.0e-39], np.float32)
    got = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, np.nan], np.float32)
    assert np.array_equal(got[:4], want[:4])
    # subnormal input stays within one bf16 ulp
    assert abs(got[4] - x[4]) <= 2.0 ** -133


def test_init_statistics_and_tokens():
    shape = datagen.PRESETS["tiny"]
    w = datagen.init_tensor(shape, "wq", 0)
    assert w.shape == (128, 128) and abs(w.std() - 0.02) < 1e-3 and abs(w.mean()) < 1e-3
    assert np.all(datagen.init_tensor(shape, "attn_norm") == 1)
    tok = datagen.tokens(shape)
    assert tok.shape == (2, 64) and tok.min() >= 0 and tok.max() < shape.vocab
    s = datagen.PRESETS["1.3b"]
    a = datagen.init_tensor(s, "wd", 3, rows=slice(100, 102))
    assert np.array_equal(a, datagen.draw_flat(0, datagen.tensor_id(s, "wd", 3), 100 * s.d_ff, 102 * s.d_ff,
                                               "bf16").reshape(2, -1))
    b16 = datagen.f32_to_bf16_bits(a)
    assert np.array_equal(datagen.bf16_bits_to_f32(b16), a)  # already bf16-representable
