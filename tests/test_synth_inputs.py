"""Host-side checks of the seeded input generator (no GPU needed)."""
import numpy as np

import synth


def test_streams_are_deterministic_and_distinct():
    a = synth.normal_bf16((9, 1), (700, 64), 0.02, chunk_rows=128)
    b = synth.normal_bf16((9, 1), (700, 64), 0.02, chunk_rows=128)
    c = synth.normal_bf16((9, 2), (700, 64), 0.02, chunk_rows=128)
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1.5, 3.140625, 1 + 2 ** -9], np.float32)
    bits = synth.f32_to_bf16_bits(x)
    assert bits.tolist() == [0x3F80, 0x3F82, 0xBFC0, 0x4049, 0x3F80]
    assert np.array_equal(synth.bf16_bits_to_f32(bits), np.array([1, 1 + 2 ** -6, -1.5, 3.140625, 1], np.float32))


def test_weight_statistics_and_shapes():
    w = synth.layer_weights(1, 0, synth.TINY)
    assert w["wq"].shape == (256, 256) and w["w_down"].shape == (256, 688) and w["w_gate"].shape == (688, 256)
    v = synth.bf16_bits_to_f32(w["w_gate"]).astype(np.float64)
    assert abs(v.std() - 0.02) < 0.001 and abs(v.mean()) < 0.001
    assert np.all(w["attn_norm"] == 0x3F80)


def test_free_order_is_a_permutation():
    p = synth.free_order(3, 4200)
    assert sorted(p.tolist()) == list(range(4200)) and not np.array_equal(p, np.arange(4200))


def test_scatter_places_positions_by_block_table():
    H, D = 2, 4
    pk = np.zeros((5, H, 16, D), np.uint16)
    pv = np.zeros((5, H, D, 16), np.uint16)
    row = np.array([3, 0, 4], np.int32)
    n = 37
    k = np.arange(n * H * D, dtype=np.uint16).reshape(n, H, D)
    synth.scatter_kv_into_pool(pk, pv, row, k, k + 1)
    for p in range(n):
        assert np.array_equal(pk[row[p // 16], :, p % 16, :], k[p])
        assert np.array_equal(pv[row[p // 16], :, :, p % 16], k[p] + 1)
