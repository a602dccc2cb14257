"""Layer-step parity: llmdec_layer_decode / llmdec_layer_prefill against the oracle's layer_step.

Full-size cases are the 7B-layer workloads: decode at batch 1 with 2048
cached tokens, decode over 32 sequences with contexts in [128, 4096], and a
4 x 512 prefill.  Small cases cover the batched (skinny) and tiled matrix
paths with ragged sizes and chunked prefill (new tokens after a cached prefix).
"""
import numpy as np
import pytest

import synth
from oracle import decoder as od
from oracle import pages as op
from tests.gpu_util import assert_close, assert_stored_bf16, banner, f32_from_bf16
from tests import pool_layout as pl
from tests.layer_harness import LayerCase

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    from kv_cached_transformer_amd import llmdec
    llmdec.lib()
    return llmdec


@pytest.fixture(scope="module")
def R():
    from kv_cached_transformer_amd import runtime
    return runtime


TINY1 = synth.ModelShape(n_layers=1, hidden=256, n_heads=4, n_kv_heads=4, head_dim=64, intermediate=688, vocab=1024)
# grouped-query shapes: 4 query heads over 2 K/V heads; a 7B-sized layer with 32 query heads over 8
TINY1_GQA = synth.ModelShape(n_layers=1, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=688,
                             vocab=1024)
GQA7B_LAYER = synth.ModelShape(n_layers=1, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, intermediate=11008,
                               vocab=32000)


def check_new_slots(case, new_tokens, tag):
    """New K/V written by the step: the slot set exactly (sentinel), the values as the oracle's bf16 roundings."""
    H, D = case.shape.n_kv_heads, case.shape.head_dim
    kblk, vblk = case.pool_blocks()
    written = np.zeros((case.num_pages, 16), bool)
    got, ref = [], []
    for s, p in new_tokens:
        pg, off = op.slot_of(case.bt[s], p)
        written[pg, off] = True
        gk, gv = pl.read_slot(kblk, vblk, pg, off, H, D)
        got += [f32_from_bf16(gk), f32_from_bf16(gv)]
        ref += [case.kv.k[(0, s)][p], case.kv.v[(0, s)][p]]
    assert_stored_bf16(f"{tag} new K/V", np.stack(got), np.stack(ref))
    # everything else is either the seeded history (unchanged) or the 0xFFFF sentinel
    assert pl.unwritten_equal(case.kblk0, kblk, written, H, D, "k"), f"{tag}: a K slot outside the new tokens changed"
    assert pl.unwritten_equal(case.vblk0, vblk, written, H, D, "v"), f"{tag}: a V slot outside the new tokens changed"


def run_decode(L, R, shape, workload, ctxs, x_in, tag):
    banner(f"{tag}: layer_decode n={len(ctxs)}")
    case = LayerCase(L, R, shape, workload, ctxs, [1] * len(ctxs))
    n = len(ctxs)
    ws = case.workspace(n)
    xd = R.dev_f32(x_in)
    ctx_d = R.dev_i32(ctxs)  # device buffers stay referenced until the stream has run
    L.llmdec_layer_decode(case.cfg, case.packed.struct, 0, xd.data_ptr(), n, ctx_d.data_ptr(),
                          case.bt_dev.data_ptr(), case.max_pages, case.pool.handle, ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert ws.error_bits() == 0
    got = xd.cpu().numpy()
    ref = od.layer_step(shape, case.lw.tensors, 0, x_in, list(range(n)), ctxs, case.kv)
    assert_close(f"{tag} layer output", got, ref)
    check_new_slots(case, [(s, c) for s, c in enumerate(ctxs)], tag)


def run_prefill(L, R, shape, workload, starts, lens, x_in, tag):
    banner(f"{tag}: layer_prefill starts={starts[:4]} lens={lens[:4]}")
    case = LayerCase(L, R, shape, workload, starts, lens)
    n = len(lens)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ws = case.workspace(T)
    xd = R.dev_f32(x_in)
    cu_d, st_d = R.dev_i32(cu), R.dev_i32(starts)
    L.llmdec_layer_prefill(case.cfg, case.packed.struct, 0, xd.data_ptr(), n, T, max(lens), cu_d.data_ptr(),
                           st_d.data_ptr(), case.bt_dev.data_ptr(), case.max_pages, case.pool.handle,
                           ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert ws.error_bits() == 0
    got = xd.cpu().numpy()
    seqs = np.repeat(np.arange(n), lens)
    pos = np.concatenate([np.arange(s0, s0 + ln) for s0, ln in zip(starts, lens)])
    ref = od.layer_step(shape, case.lw.tensors, 0, x_in, seqs, pos, case.kv)
    assert_close(f"{tag} layer output", got, ref)
    check_new_slots(case, list(zip(seqs.tolist(), pos.tolist())), tag)


# ----------------------------------------------------------------------------- small shapes
def test_decode_tiny_batch1(L, R):
    run_decode(L, R, TINY1, 91, [37], synth.hidden_input(91, 1, 256), "tiny decode b1")


def test_decode_tiny_batched_ragged(L, R):
    ctxs = [0, 15, 16, 17, 100, 3]
    run_decode(L, R, TINY1, 92, ctxs, synth.hidden_input(92, len(ctxs), 256), "tiny decode b6")


def test_prefill_tiny_chunked(L, R):
    starts, lens = [0, 16, 5, 0], [1, 17, 40, 64]
    run_prefill(L, R, TINY1, 93, starts, lens, synth.hidden_input(93, sum(lens), 256), "tiny prefill chunked")


@pytest.mark.parametrize("starts,lens", [([0], [64]), ([0, 7], [33, 32]), ([3, 0, 16], [1, 63, 15])])
def test_prefill_tiny_at_the_row_boundary(L, R, starts, lens):
    """64 rows take the streaming products with the fp16 pair and the RoPE/append kernel; 65 and 79 rows
    the tiled products with RoPE and the append in their epilogues (one row past a 16-row block)."""
    n = sum(lens)
    run_prefill(L, R, TINY1, 99 + n, starts, lens, synth.hidden_input(99 + n, n, 256), f"tiny prefill {n} rows")


def test_prefill_tiny_single_token(L, R):
    run_prefill(L, R, TINY1, 94, [20], [1], synth.hidden_input(94, 1, 256), "tiny prefill 1 token")


# ----------------------------------------------------------------------------- 7B layer workloads
def test_7b_layer_decode_batch1_ctx2048(L, R):
    run_decode(L, R, synth.LLAMA7B_LAYER, 2, [2048], synth.hidden_input(2, 1, 4096), "7B decode b1 ctx2048")


def test_7b_layer_decode_batch32(L, R):
    ctxs = synth.context_lengths(3, 32, 128, 4096)
    run_decode(L, R, synth.LLAMA7B_LAYER, 3, ctxs.tolist(), synth.hidden_input(3, 32, 4096), "7B decode b32")


def test_7b_layer_prefill_4x512(L, R):
    lens = [512] * 4
    run_prefill(L, R, synth.LLAMA7B_LAYER, 4, [0] * 4, lens, synth.hidden_input(4, 2048, 4096), "7B prefill 4x512")


# ----------------------------------------------------------------------------- grouped-query attention
def test_decode_tiny_gqa_batched_ragged(L, R):
    ctxs = [0, 15, 16, 17, 100, 3]
    run_decode(L, R, TINY1_GQA, 95, ctxs, synth.hidden_input(95, len(ctxs), 256), "tiny GQA decode b6")


def test_prefill_tiny_gqa_chunked(L, R):
    starts, lens = [0, 16, 5, 0], [1, 17, 40, 64]
    run_prefill(L, R, TINY1_GQA, 96, starts, lens, synth.hidden_input(96, sum(lens), 256), "tiny GQA prefill")


def test_gqa_7b_sized_layer_decode_batch8(L, R):
    ctxs = synth.context_lengths(97, 8, 128, 2048)
    run_decode(L, R, GQA7B_LAYER, 97, ctxs.tolist(), synth.hidden_input(97, 8, 4096), "GQA 32/8 decode b8")


def test_gqa_7b_sized_layer_prefill(L, R):
    lens = [256, 100]
    run_prefill(L, R, GQA7B_LAYER, 98, [0, 37], lens, synth.hidden_input(98, sum(lens), 4096), "GQA 32/8 prefill")


# ----------------------------------------------------------------------------- device-side argument errors
@pytest.mark.parametrize("n", [1, 2])
def test_decode_bad_page_and_position_set_error_bits(L, R, n):
    """A block-table entry naming a page that does not exist, and a position past the block-table row, are
    caught on the device: the sticky error bits say which, and no K/V slot is written.  n = 1 runs the
    one-row q|k|v product with RoPE and the append in its epilogue, n = 2 the RoPE/append kernel."""
    banner(f"decode with a bad page / position, {n} sequence(s)")
    ctxs = [37] * n
    case = LayerCase(L, R, TINY1, 99, ctxs, [1] * n, build_oracle=False)
    x_in = synth.hidden_input(99, n, 256)
    bad = case.bt.copy()
    bad[:, 37 // 16] = case.num_pages + 3          # the new token's page (block 2) does not exist
    for bt, ctx, bit in [(bad, ctxs, L.ERR_PAGE), (case.bt, [case.max_pages * 16] * n, L.ERR_POS)]:
        ws = case.workspace(n)
        xd, bt_d, ctx_d = R.dev_f32(x_in), R.dev_i32(bt), R.dev_i32(ctx)
        L.llmdec_layer_decode(case.cfg, case.packed.struct, 0, xd.data_ptr(), n, ctx_d.data_ptr(), bt_d.data_ptr(),
                              case.max_pages, case.pool.handle, ws.ptr, ws.nbytes, R.stream())
        torch.cuda.synchronize()
        assert ws.error_bits() & bit, f"error bit {bit} not set (bits {ws.error_bits()})"
        kblk, vblk = case.pool_blocks()
        assert np.array_equal(kblk, case.kblk0) and np.array_equal(vblk, case.vblk0), "a K/V slot was written"


@pytest.mark.parametrize("n_tok", [40, 80])
def test_prefill_bad_page_and_position_set_error_bits(L, R, n_tok):
    """The same checks in a prefill: new tokens whose block-table entries name pages that do not exist, and
    new tokens past the block-table row, set the sticky error bits and write no K/V slot.  40 tokens run
    the RoPE/append kernel after a batched product; 80 run the tiled q|k|v products, which apply RoPE and
    the append in their epilogue."""
    banner(f"prefill of {n_tok} tokens with a bad page / position")
    ctx = 37
    case = LayerCase(L, R, TINY1, 99, [ctx], [n_tok], build_oracle=False)
    x_in = synth.hidden_input(99, n_tok, 256)
    bad = case.bt.copy()
    bad[0, ctx // 16:(ctx + n_tok - 1) // 16 + 1] = case.num_pages + 3  # every new token's page
    cu_d = R.dev_i32(np.array([0, n_tok], np.int32))
    for bt, start, bit in [(bad, ctx, L.ERR_PAGE), (case.bt, case.max_pages * 16, L.ERR_POS)]:
        ws = case.workspace(n_tok)
        xd, bt_d, st_d = R.dev_f32(x_in), R.dev_i32(bt), R.dev_i32(np.array([start], np.int32))
        L.llmdec_layer_prefill(case.cfg, case.packed.struct, 0, xd.data_ptr(), 1, n_tok, n_tok, cu_d.data_ptr(),
                               st_d.data_ptr(), bt_d.data_ptr(), case.max_pages, case.pool.handle, ws.ptr,
                               ws.nbytes, R.stream())
        torch.cuda.synchronize()
        assert ws.error_bits() & bit, f"error bit {bit} not set (bits {ws.error_bits()})"
        kblk, vblk = case.pool_blocks()
        assert np.array_equal(kblk, case.kblk0) and np.array_equal(vblk, case.vblk0), "a K/V slot was written"
