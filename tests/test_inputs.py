"""The seeded input generators (CPU only)."""

import numpy as np

from linear_attention_ssm_chunk_amd import inputs as I


def test_bf16_round_trip_and_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 0.0], np.float32)
    b = I.f32_to_bf16_bits(x)
    y = I.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins -> 1.0
    assert list(y) == [1.0, 1.0, 1.0 + 2 ** -7, -2.5, 0.0]


def test_workload_shapes_and_distributions():
    p = I.make_workload(1)
    assert p.lengths == [256] and p.q.shape == (256, 1, 128) and p.v.shape == (256, 1, 128)
    qn = np.linalg.norm(I.bf16_to_f64(p.q), axis=-1)
    assert np.all(np.abs(qn - 1) < 1e-2)
    assert np.all(p.g < 0) and np.all((p.beta > 0) & (p.beta < 1))
    assert np.all(p.h0 == 0)
    # same seed, same draw
    p2 = I.make_workload(1)
    assert np.array_equal(p.k, p2.k) and np.array_equal(p.g, p2.g)


def test_ragged_lengths_rule():
    L, s = I.ragged_lengths(4)
    assert len(L) == 8 and all(1 <= x <= 16384 and x % 64 for x in L)
    assert abs(sum(L) - 32768) <= 3277 and s >= 4


def test_conv_packing_places_heads():
    p = I.make_problem([70], 2, 6, seed=0)
    c = I.pack_conv(p)
    assert c["qk_row"] == 2 * 2 * 128 + 6 * 128 and c["gb_row"] == 12
    assert np.array_equal(c["conv"][5, c["k_off"] + 128: c["k_off"] + 256], p.k[5, 1])
    assert np.array_equal(c["conv"][5, c["v_off"] + 3 * 128: c["v_off"] + 4 * 128], p.v[5, 3])
    assert c["gb"][9, c["beta_off"] + 4] == p.beta[9, 4]
