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


def test_pool_layout_write_and_read_by_block_table():
    """The tests' own encoding of the documented pool layout: positions land in the slot their block-table
    row names, K as [page][h][o][d], V as [page][h][o/4][d][o%4], and read back unchanged."""
    from tests import pool_layout as pl
    H, D, P = 2, 8, 5
    kb = np.zeros(pl.block_elems(P, H, D), np.uint16)
    vb = np.zeros_like(kb)
    row = np.array([3, 0, 4], np.int32)
    n = 37
    k = np.arange(n * H * D, dtype=np.uint16).reshape(n, H, D)
    pl.write_history(kb, vb, row, k, k + 1, H, D)
    kv = kb.reshape(P, H, 16, D)
    vv = vb.reshape(P, H, 4, D, 4)
    for p in range(n):
        pg, o = row[p // 16], p % 16
        assert np.array_equal(kv[pg, :, o, :], k[p]) and np.array_equal(vv[pg, :, o // 4, :, o % 4], k[p] + 1)
        rk, rv = pl.read_slot(kb, vb, pg, o, H, D)
        assert np.array_equal(rk, k[p]) and np.array_equal(rv, k[p] + 1)
    written = np.zeros((P, 16), bool)
    for p in range(n):
        written[row[p // 16], p % 16] = True
    assert pl.unwritten_equal(kb, np.zeros_like(kb), written, H, D, "k")
    assert not pl.unwritten_equal(kb, np.zeros_like(kb), np.zeros((P, 16), bool), H, D, "k")


def test_literal_gamma_model_weights():
    mw = synth.model_weights(1, synth.TINY, norm_gamma="literal")
    g = np.concatenate([synth.bf16_bits_to_f32(mw.layers[0]["attn_norm"]), synth.bf16_bits_to_f32(mw.final_norm)])
    assert abs(g.std() - 0.02) < 0.004 and not np.array_equal(mw.final_norm, mw.layers[0]["attn_norm"])
