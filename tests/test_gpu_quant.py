"""Group-quantized weights on the device against the oracle's dequantization.

The quantized matrix-vector product (llmdec_op_linear_q8) and the quantized decode layer
(llmdec_layer_decode_q8) are compared with oracle.quant / oracle.decoder fed the dequantized
matrices in float64.  The product runs in fp32 from the unrounded activation, so it is held to
fp32-level agreement besides the hidden-state bound; the layer is held to the hidden-state bound
and its new K/V slots to the stored-bf16 rule of the other layer tests.
"""
import numpy as np
import pytest

import synth
from oracle import decoder as od
from oracle import quant as oq
from tests.gpu_util import assert_close, banner
from tests.layer_harness import LayerCase
from tests.test_gpu_layers import TINY1, TINY1_GQA, check_new_slots

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


def dequantized(m, bits=8, cols=None):
    codes, scales, zeros = m
    if bits == 4:
        codes = oq.unpack_nibbles(codes, cols)
    return oq.dequantize(codes, od.widen_bf16(scales), zeros)


def op_linear(L, bits):
    return L.llmdec_op_linear_q8 if bits == 8 else L.llmdec_op_linear_q4


# (rows, cols): several lanes' chunks and steps, a short last group (688 = 5 x 128 + 48), a ragged
# last step (1040 = 1024 + 16), 14 steps (the largest k), and the 7B shapes
SHAPES = [(16, 256), (64, 688), (12, 1040), (8, 14336), (4, 16), (4, 144), (4096, 4096), (4096, 11008), (12288, 4096)]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_linear_q8(L, R, rows, cols, bits):
    banner(f"op_linear_q{bits} {rows}x{cols}")
    m = synth.q_matrix(bits, 60, 0, cols % 7, rows, cols)
    w = R.Q8Matrix(m, bits, cols)
    x = synth.rng(61, rows, cols).standard_normal(cols).astype(np.float32)
    base = synth.rng(62, rows, cols).standard_normal(rows).astype(np.float32)
    xd = R.dev_f32(x)
    out = R.dev_f32(np.full(rows, np.nan, np.float32))
    acc = R.dev_f32(base)
    op_linear(L, bits)(xd.data_ptr(), cols, w.ptr, rows, out.data_ptr(), 0, R.stream())
    op_linear(L, bits)(xd.data_ptr(), cols, w.ptr, rows, acc.data_ptr(), 1, R.stream())
    torch.cuda.synchronize()
    codes = m[0] if bits == 8 else oq.unpack_nibbles(m[0], cols)
    ref = oq.linear_q8(x[None, :], codes, od.widen_bf16(m[1]), m[2])[0]
    got = out.cpu().numpy()
    assert_close(f"q{bits} {rows}x{cols} store", got, ref)
    assert_close(f"q{bits} {rows}x{cols} store (fp32 level)", got, ref, max_abs=1e-4, rel_l2=1e-5)
    assert_close(f"q{bits} {rows}x{cols} accumulate", acc.cpu().numpy(), base.astype(np.float64) + ref,
                 max_abs=1e-4, rel_l2=1e-5)


@pytest.mark.parametrize("bits", [8, 4])
def test_linear_q8_group_isolation(L, R, bits):
    """A one-hot activation picks out one column: out[r] = (code - zero) * scale of that column's group,
    for a column in every group position of a row with a short last group."""
    rows, cols = 8, 688
    m = synth.q_matrix(bits, 63, 0, 0, rows, cols)
    w = R.Q8Matrix(m, bits, cols)
    W = dequantized(m, bits, cols)
    out = R.dev_f32(np.zeros(rows, np.float32))
    for c in (0, 15, 16, 127, 128, 511, 640, 687):
        x = np.zeros(cols, np.float32)
        x[c] = 1.0
        xd = R.dev_f32(x)
        op_linear(L, bits)(xd.data_ptr(), cols, w.ptr, rows, out.data_ptr(), 0, R.stream())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, W[:, c].astype(np.float32).astype(np.float64)), f"column {c}"


def run_decode_q8(L, R, shape, workload, ctx, tag, bits=8):
    banner(f"{tag}: layer_decode_q{bits} ctx={ctx}")
    case = LayerCase(L, R, shape, workload, [ctx], [1], pack=False)
    qw = synth.q_layer_weights(bits, workload, 0, shape)
    layer = R.Q8Layer(case.cfg, qw, bits)
    x_in = synth.hidden_input(workload, 1, shape.hidden)
    ws = case.workspace(1)
    xd = R.dev_f32(x_in)
    ctx_d = R.dev_i32([ctx])
    decode = L.llmdec_layer_decode_q8 if bits == 8 else L.llmdec_layer_decode_q4
    decode(case.cfg, layer.struct, 0, xd.data_ptr(), 1, ctx_d.data_ptr(), case.bt_dev.data_ptr(),
           case.max_pages, case.pool.handle, ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert ws.error_bits() == 0
    shapes = shape.matrix_shapes()
    dense = {k: dequantized(v, bits, shapes[k][1]) for k, v in qw.items() if k not in ("attn_norm", "mlp_norm")}
    dense.update(attn_norm=qw["attn_norm"], mlp_norm=qw["mlp_norm"])
    ref = od.layer_step(shape, dense, 0, x_in, [0], [ctx], case.kv)
    assert_close(f"{tag} layer output", xd.cpu().numpy(), ref)
    check_new_slots(case, [(0, ctx)], tag)


def test_decode_q8_tiny(L, R):
    run_decode_q8(L, R, TINY1, 64, 37, "tiny q8 decode")


def test_decode_q8_tiny_gqa_page_start(L, R):
    run_decode_q8(L, R, TINY1_GQA, 65, 32, "tiny GQA q8 decode")


def test_decode_q8_7b_layer_ctx2048(L, R):
    run_decode_q8(L, R, synth.LLAMA7B_LAYER, 66, 2048, "7B q8 decode b1 ctx2048")


def test_decode_q4_tiny(L, R):
    run_decode_q8(L, R, TINY1, 68, 37, "tiny q4 decode", bits=4)


def test_decode_q4_tiny_gqa_page_start(L, R):
    run_decode_q8(L, R, TINY1_GQA, 69, 32, "tiny GQA q4 decode", bits=4)


def test_decode_q4_7b_layer_ctx2048(L, R):
    run_decode_q8(L, R, synth.LLAMA7B_LAYER, 70, 2048, "7B q4 decode b1 ctx2048", bits=4)


def test_decode_q8_rejects_batches(L, R):
    case = LayerCase(L, R, TINY1, 67, [5, 9], [1, 1], pack=False, build_oracle=False)
    layer = R.Q8Layer(case.cfg, synth.q8_layer_weights(67, 0, TINY1))
    ws = case.workspace(2)
    xd = R.dev_f32(np.zeros((2, 256), np.float32))
    ctx_d = R.dev_i32([5, 9])
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_layer_decode_q8(case.cfg, layer.struct, 0, xd.data_ptr(), 2, ctx_d.data_ptr(),
                                 case.bt_dev.data_ptr(), case.max_pages, case.pool.handle, ws.ptr, ws.nbytes,
                                 R.stream())
    assert e.value.status == L.LLMDEC_E_UNSUPPORTED
