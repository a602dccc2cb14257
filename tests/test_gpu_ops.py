"""Per-kernel parity: each libllmdec operation against the CPU oracle on seeded inputs.

Sizes span several tiles plus a ragged tail; edge cases include one-token
contexts, page boundaries (15, 16, 17 tokens) and planted argmax ties.
"""
import numpy as np
import pytest

import synth
from oracle import decoder as od
from oracle import pages as op
from tests import pool_layout as pl
from tests.gpu_util import (assert_close, assert_rounded, assert_stored_bf16, assert_within_rounding_bound, banner,
                            f16_ulp, f32_from_bf16, f64_from_f16, report, unpack_tiled)

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


class Shape:
    def __init__(self, H, D, I=688, V=1024, layers=1, Hk=None):
        self.n_layers, self.hidden, self.n_heads, self.n_kv_heads, self.head_dim = layers, H * D, H, Hk or H, D
        self.intermediate, self.vocab, self.page_size, self.rms_eps, self.rope_theta = I, V, 16, 1e-6, 10000.0


def bf16_normal(rng, shape, std=1.0):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ----------------------------------------------------------------------------- RMSNorm
# above 64 rows: 64-column groups of kpad = n + 32 at each block shape of the many-row kernel (5, 17, 64, 65
# and 128 groups, the last at the widest packed stride, 8192)
@pytest.mark.parametrize("rows,n", [(1, 4096), (3, 256), (80, 256), (70, 4096), (133, 1024), (200, 4064), (72, 8160)])
def test_rmsnorm(L, R, rows, n):
    """fp32 output against the oracle; the packed fp16 output is the nearest-even fp16 of the device's own
    fp32 value, bit for bit (both roundings taken in the same precision), and the fp16 pair's lo part is
    the rounding of what hi leaves."""
    banner(f"rmsnorm rows={rows} n={n}")
    rng = np.random.default_rng(100 + rows)
    x = (rng.standard_normal((rows, n)) * 3).astype(np.float32)
    g = synth.f32_to_bf16_bits(1 + 0.1 * rng.standard_normal(n).astype(np.float32))
    xd, gd = R.dev_f32(x), R.dev_u16(g)
    out = torch.empty(rows, n, dtype=torch.float32, device="cuda")
    kpad = n + 32   # one extra k-tile: must come back zeroed
    hi = torch.full((((rows + 15) // 16) * 16 * kpad,), -1, dtype=torch.int16, device="cuda")
    lo = torch.full_like(hi, -1)
    L.llmdec_op_rmsnorm(xd.data_ptr(), gd.data_ptr(), rows, n, 1e-6, out.data_ptr(), hi.data_ptr(), lo.data_ptr(),
                        kpad, R.stream())
    torch.cuda.synchronize()
    ref = od.rms_norm(x, od.widen_bf16(g), 1e-6)
    y = out.cpu().numpy().astype(np.float64)
    assert_close("rmsnorm f32", y, ref, max_abs=1e-5, rel_l2=1e-6)
    h_full, l_full = unpack_tiled(R.host_u16(hi), rows, kpad, kpad), unpack_tiled(R.host_u16(lo), rows, kpad, kpad)
    assert np.all(h_full[:, n:] == 0) and np.all(l_full[:, n:] == 0)
    h, l_ = f64_from_f16(h_full[:, :n]), f64_from_f16(l_full[:, :n])
    assert np.array_equal(h, od.round_to_f16(y))
    assert np.array_equal(l_, od.round_to_f16(y - h))
    assert_close("rmsnorm hi+lo", h + l_, ref, max_abs=1e-5, rel_l2=1e-6)
    # packed output only, as the layers ask for it (above 64 rows a kernel that normalises 8 rows per block
    # takes it; its sums of squares add in another order, so its last bits may differ from the above)
    hi2, lo2 = torch.full_like(hi, -1), torch.full_like(hi, -1)
    L.llmdec_op_rmsnorm(xd.data_ptr(), gd.data_ptr(), rows, n, 1e-6, None, hi2.data_ptr(), lo2.data_ptr(), kpad,
                        R.stream())
    torch.cuda.synchronize()
    h2_full, l2_full = unpack_tiled(R.host_u16(hi2), rows, kpad, kpad), unpack_tiled(R.host_u16(lo2), rows, kpad, kpad)
    assert np.all(h2_full[:, n:] == 0) and np.all(l2_full[:, n:] == 0)
    h2, l2 = f64_from_f16(h2_full[:, :n]), f64_from_f16(l2_full[:, :n])
    assert_close("rmsnorm packed-only hi+lo", h2 + l2, ref, max_abs=1e-5, rel_l2=1e-6)
    if rows <= 64:
        assert torch.equal(hi2, hi) and torch.equal(lo2, lo)
    # the single-plane output (as the MLP norm writes it) is the same hi plane
    one = torch.full_like(hi, -1)
    L.llmdec_op_rmsnorm(xd.data_ptr(), gd.data_ptr(), rows, n, 1e-6, None, one.data_ptr(), None, kpad, R.stream())
    torch.cuda.synchronize()
    assert torch.equal(one, hi2)


def test_rmsnorm_eps_inside_root(L, R):
    x = np.full((1, 256), 1e-3, np.float32)
    g = np.full(256, 0x3F80, np.uint16)
    xd, gd = R.dev_f32(x), R.dev_u16(g)
    out = torch.empty(1, 256, dtype=torch.float32, device="cuda")
    L.llmdec_op_rmsnorm(xd.data_ptr(), gd.data_ptr(), 1, 256, 1e-6, out.data_ptr(), None, None, 0, R.stream())
    torch.cuda.synchronize()
    assert np.allclose(out.cpu().numpy(), 1 / np.sqrt(2), rtol=1e-5)


def test_rmsnorm_clips_beyond_f16_range(L, R):
    """Values past fp16's largest finite value are clipped to 65504, not turned into infinities (the
    weights article's remedy for fp16 overflow): gamma = 16384 scales a normalised row past it."""
    x = np.zeros((1, 256), np.float32)
    x[0, :4] = [8.0, -8.0, 0.5, 1.0]
    g = np.full(256, 0x4680, np.uint16)  # bf16 16384: the 8.0 entry normalises to about 1.8e5
    xd, gd = R.dev_f32(x), R.dev_u16(g)
    out = torch.empty(1, 256, dtype=torch.float32, device="cuda")
    act = torch.full((16 * 256,), -1, dtype=torch.int16, device="cuda")
    L.llmdec_op_rmsnorm(xd.data_ptr(), gd.data_ptr(), 1, 256, 1e-6, out.data_ptr(), act.data_ptr(), None, 256,
                        R.stream())
    torch.cuda.synchronize()
    y = out.cpu().numpy().astype(np.float64)[0]
    h = f64_from_f16(unpack_tiled(R.host_u16(act), 1, 256, 256))[0]
    assert abs(y[0]) > 65504 and h[0] == 65504.0 and h[1] == -65504.0
    assert np.array_equal(h, od.round_to_f16(y))


# ----------------------------------------------------------------------------- linear
@pytest.mark.parametrize("parts", [1, 2])
@pytest.mark.parametrize("rows,n,k,acc", [(1, 4096, 4096, 0), (1, 768, 688, 1), (1, 1024, 11008, 0),
                                          (5, 1376, 256, 0), (33, 256, 688, 1), (64, 4096, 4096, 0),
                                          (64, 4096, 11008, 1), (64, 32000, 4096, 0), (17, 12288, 4096, 1),
                                          (100, 512, 256, 0), (300, 784, 1000, 1), (2048, 1024, 4096, 0),
                                          (520, 4096, 11008, 1), (65, 22016, 4096, 0),
                                          # decode-product layouts (row blocks x column waves) not reached above
                                          (17, 512, 256, 0), (17, 512, 1024, 1), (33, 512, 11008, 1),
                                          (33, 4096, 11008, 0), (32, 4096, 4096, 1), (48, 12288, 4096, 0),
                                          # 257 row blocks: the last column group is ragged under a balanced split
                                          (1, 4112, 4096, 0), (40, 4112, 4096, 1),
                                          # one row: the widest input the one-row kernel stages (14336), the
                                          # narrowest (16), and one k-tile past it (the streaming kernel)
                                          (1, 64, 14336, 1), (1, 48, 16, 0), (1, 32, 14352, 0)])
def test_linear(L, R, rows, n, k, acc, parts):
    """rows > 1 (and one row past the one-row kernel's width) take the activation in fp16 (parts = 1) or as
    the fp16 pair (parts = 2): against the oracle fed the same rounded activation the product agrees to
    fp32 accumulation, and against the exact product it stays inside the a-priori bound that the
    activation rounding sets.  One row: fp32 activation, against the exact product."""
    if rows == 1 and k <= 14336 and parts == 2:
        pytest.skip("the one-row kernel takes the fp32 activation whatever act_parts")
    banner(f"linear rows={rows} n={n} k={k} acc={acc} parts={parts}")
    rng = np.random.default_rng(rows * 7 + n + k)
    a = rng.standard_normal((rows, k)).astype(np.float32)
    w = bf16_normal(rng, (n, k), 0.02)
    pm = R.PackedMatrix(n, k, w)
    base = rng.standard_normal((rows, n)).astype(np.float32)
    out = R.dev_f32(base) if acc else torch.empty(rows, n, dtype=torch.float32, device="cuda")
    ws = R.Workspace(L.llmdec_op_linear_ws_bytes(rows, k, n))
    ad = R.dev_f32(a)
    L.llmdec_op_linear(ad.data_ptr(), rows, k, pm.ptr, n, out.data_ptr(), acc, ws.ptr, ws.nbytes, R.stream(),
                       act_parts=parts)
    torch.cuda.synchronize()
    W = od.widen_bf16(w)
    add = base.astype(np.float64) if acc else 0
    a64 = a.astype(np.float64)
    exact = a64 @ W.T + add
    got = out.cpu().numpy()
    if rows == 1 and k <= 14336:
        assert_close(f"linear {rows}x{n}x{k}", got, exact, max_abs=2e-4, rel_l2=1e-5)
    else:
        a_used = od.round_to_f16(a64) if parts == 1 else od.f16_pair(a64)
        assert_close(f"linear {rows}x{n}x{k} (fp16 x{parts})", got, a_used @ W.T + add, max_abs=1e-4, rel_l2=2e-6)
        u = 2.0 ** -11 if parts == 1 else 2.0 ** -21
        assert_within_rounding_bound(f"linear {rows}x{n}x{k} exact", got, exact, np.abs(a64), np.abs(W), u, 1e-4)
    # a second call on the same workspace gives the same bits (split-k partials are added in a fixed order)
    out2 = R.dev_f32(base) if acc else torch.empty(rows, n, dtype=torch.float32, device="cuda")
    L.llmdec_op_linear(ad.data_ptr(), rows, k, pm.ptr, n, out2.data_ptr(), acc, ws.ptr, ws.nbytes, R.stream(),
                       act_parts=parts)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "the same product twice gave different bits"


def test_linear_rejects_bad_act_parts(L, R):
    pm = R.PackedMatrix(16, 32, np.zeros((16, 32), np.uint16))
    ws = R.Workspace(L.llmdec_op_linear_ws_bytes(4, 32, 16))
    a, out = torch.zeros(4, 32, device="cuda"), torch.zeros(4, 16, device="cuda")
    with pytest.raises(L.LlmdecError):
        L.llmdec_op_linear(a.data_ptr(), 4, 32, pm.ptr, 16, out.data_ptr(), 0, ws.ptr, ws.nbytes, R.stream(),
                           act_parts=3)


def test_packed_weights_exact_in_fp16(L, R):
    """The packing carries every bf16 weight within 2^31 of the matrix's largest exactly: a one-hot
    activation row picks one column of W, and its product is that weight (here weights spread over 2^-30
    .. 2^1, so the largest sets the shift and the smallest are far below fp16's own normal range)."""
    rng = np.random.default_rng(77)
    n, k = 64, 96
    mag = np.exp2(rng.uniform(-30, 1, (n, k))) * rng.choice([-1.0, 1.0], (n, k))
    w = synth.f32_to_bf16_bits(mag.astype(np.float32))
    pm = R.PackedMatrix(n, k, w)
    a = np.eye(k, dtype=np.float32)[:80]          # 80 one-hot rows: the tiled kernel
    out = torch.empty(80, n, dtype=torch.float32, device="cuda")
    ws = R.Workspace(L.llmdec_op_linear_ws_bytes(80, k, n))
    ad = R.dev_f32(a)
    L.llmdec_op_linear(ad.data_ptr(), 80, k, pm.ptr, n, out.data_ptr(), 0, ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), od.widen_bf16(w).T[:80])


@pytest.mark.parametrize("parts", [1, 2])
@pytest.mark.parametrize("rows,inter,k", [(1, 688, 256), (7, 11008, 4096), (64, 11008, 4096), (200, 688, 256),
                                          (2048, 11008, 4096)])
def test_swiglu_linear(L, R, rows, inter, k, parts):
    """u = silu(g) * up, g and up the products of the fp16 activation (parts = 1) or of the fp16 pair (parts =
    2), stored in fp16 (parts = 2: as the pair hi + lo).  Against the oracle's value from the same rounded
    activation, each stored fp16 value is its nearest fp16 or, near a rounding boundary, the neighbour
    (fp32 products and silu on the device); the pair carries u to the fp32-level bound."""
    banner(f"swiglu_linear rows={rows} inter={inter} k={k} parts={parts}")
    rng = np.random.default_rng(rows + inter + k)
    a = rng.standard_normal((rows, k)).astype(np.float32)
    wg, wu = bf16_normal(rng, (inter, k), 0.02), bf16_normal(rng, (inter, k), 0.02)
    # fused layout: 16-row blocks alternate gate and up
    gu = np.empty((2 * inter, k), np.uint16)
    gu.reshape(inter // 16, 2, 16, k)[:, 0] = wg.reshape(inter // 16, 16, k)
    gu.reshape(inter // 16, 2, 16, k)[:, 1] = wu.reshape(inter // 16, 16, k)
    pm = R.PackedMatrix(2 * inter, k, gu)
    ld = (inter + 31) // 32 * 32
    act = torch.full((((rows + 15) // 16) * 16 * ld,), -1, dtype=torch.int16, device="cuda")
    lo = torch.full_like(act, -1)
    ws = R.Workspace(L.llmdec_op_linear_ws_bytes(rows, k, 2 * inter))
    ad = R.dev_f32(a)
    L.llmdec_op_swiglu_linear(ad.data_ptr(), rows, k, pm.ptr, inter, act.data_ptr(), ld, ws.ptr, ws.nbytes,
                              R.stream(), act_parts=parts, out_lo=lo.data_ptr() if parts == 2 else None)
    torch.cuda.synchronize()
    a64 = a.astype(np.float64)
    a_used = od.round_to_f16(a64) if parts == 1 else od.f16_pair(a64)
    ref = od.silu(a_used @ od.widen_bf16(wg).T) * (a_used @ od.widen_bf16(wu).T)
    full = unpack_tiled(R.host_u16(act), rows, ld, ld)
    assert np.all(full[:, inter:] == 0)
    hi = f64_from_f16(full[:, :inter])
    # abs_slack: the fp32 products g and up differ from the exact ones by about sqrt(k / 32) * 2^-24 of
    # their size (~1e-6 here), which near u = 0 exceeds fp16's spacing there
    assert_rounded(f"swiglu {rows}x{inter}x{k} x{parts}", hi, ref, od.round_to_f16, f16_ulp, 0.005, abs_slack=1e-5)
    if parts == 2:
        lfull = unpack_tiled(R.host_u16(lo), rows, ld, ld)
        assert np.all(lfull[:, inter:] == 0)
        # the pair carries u to fp32 level: the fp32 sums g and up differ from the exact ones by up to a few
        # sqrt(k / 32) * 2^-24 * |g| (1e-5 at the largest of 2e7 values), times |up| up to about 6
        assert_close(f"swiglu pair {rows}x{inter}x{k}", hi + f64_from_f16(lfull[:, :inter]), ref, max_abs=2e-4,
                     rel_l2=2e-6)


# ----------------------------------------------------------------------------- RoPE + append
@pytest.mark.parametrize("H,D,Hk", [(4, 64, 4), (32, 128, 32), (32, 128, 8), (4, 64, 1)])
def test_rope_append_slots_and_values(L, R, H, D, Hk):
    """Rotation of q (all query heads) and k, and the bf16 K/V stores of the n_kv_heads K/V heads at each
    token's slot, against the oracle; every other slot keeps its sentinel."""
    banner(f"rope_append H={H} D={D} Hk={Hk}")
    shape = Shape(H, D, Hk=Hk)
    cfg = L.make_config(shape)
    rng = np.random.default_rng(7 + H)
    lengths = [1, 16, 17, 40, 300, 4100]   # tokens stored per sequence after this call
    max_pages = 260
    num_pages = sum(op.pages_needed(n) for n in lengths) + 3
    order = rng.permutation(num_pages).astype(np.int32)
    pool = R.Pool(cfg, num_pages, order, fill_bits=0xFFFF)
    ref_pool = op.PagePool(num_pages, order)
    bt = np.full((len(lengths), max_pages), -1, np.int32)
    for s, n in enumerate(lengths):
        row = [-1] * max_pages
        assert pool.alloc(n, bt[s], 0, max_pages) == ref_pool.alloc(n, row, 0, max_pages)[1]
        assert bt[s].tolist() == row
    # new tokens: the last 1..3 positions of each sequence
    toks = [(s, p) for s, n in enumerate(lengths) for p in range(max(0, n - 3), n)]
    T = len(toks)
    h, kv = H * D, Hk * D
    qkv = rng.standard_normal((T, h + 2 * kv)).astype(np.float32)
    qd = R.dev_f32(qkv)
    ws = R.Workspace(8192)
    seq_d, pos_d, bt_d = R.dev_i32([t[0] for t in toks]), R.dev_i32([t[1] for t in toks]), R.dev_i32(bt)
    L.llmdec_op_rope_append(cfg, qd.data_ptr(), T, len(lengths), seq_d.data_ptr(), pos_d.data_ptr(), bt_d.data_ptr(),
                            max_pages,
                            pool.handle, 0, ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert ws.error_bits() == 0
    pos = np.array([t[1] for t in toks])
    q_ref = od.apply_rope(qkv[:, :h].reshape(T, H, D), pos, 1e4).reshape(T, h)
    assert_close("rope q", qd.cpu().numpy()[:, :h], q_ref, max_abs=1e-5, rel_l2=1e-6)
    k_ref = od.round_to_bf16(od.apply_rope(qkv[:, h:h + kv].reshape(T, Hk, D), pos, 1e4))
    v_ref = od.round_to_bf16(qkv[:, h + kv:].astype(np.float64).reshape(T, Hk, D))
    kblk, vblk = pl.host_layer(pool, 0, Hk, D)
    touched_k = np.zeros((num_pages, 16), bool)   # [page][slot]
    ulp_flips = 0
    for i, (s, p) in enumerate(toks):
        pg, off = op.slot_of(bt[s], p)
        gk, gv = pl.read_slot(kblk, vblk, pg, off, Hk, D)
        got_k = f32_from_bf16(gk).astype(np.float64)
        got_v = f32_from_bf16(gv).astype(np.float64)
        assert np.array_equal(got_v, v_ref[i])          # plain rounding: exact
        diff = got_k != k_ref[i]
        ulp_flips += int(diff.sum())
        assert np.all(np.abs(got_k - k_ref[i]) <= np.abs(k_ref[i]) * 2 ** -7 + 1e-30)
        touched_k[pg, off] = True
    assert ulp_flips <= max(2, 0.002 * T * kv), ulp_flips
    # sentinel: every slot not written still holds 0xFFFF in both K and V
    sentinel = np.full_like(kblk, 0xFFFF)
    assert pl.unwritten_equal(kblk, sentinel, touched_k, Hk, D, "k")
    assert pl.unwritten_equal(vblk, sentinel, touched_k, Hk, D, "v")
    # the gather entry point walks the same slots
    s = 4
    n = lengths[s]
    ko = torch.empty(n, Hk, D, dtype=torch.int16, device="cuda")
    vo = torch.empty_like(ko)
    row_d = R.dev_i32(bt[s])
    L.llmdec_debug_gather_kv(pool.handle, 0, row_d.data_ptr(), n, ko.data_ptr(), vo.data_ptr(), R.stream())
    torch.cuda.synchronize()
    kg, vg = R.host_u16(ko), R.host_u16(vo)
    for p in range(n):
        pg, off = op.slot_of(bt[s], p)
        sk, sv = pl.read_slot(kblk, vblk, pg, off, Hk, D)
        assert np.array_equal(kg[p], sk) and np.array_equal(vg[p], sv)


# ----------------------------------------------------------------------------- attention
def _random_pool(L, R, shape, num_pages, rng):
    """A pool whose every slot holds N(0, 1) bf16 values; returns the host K/V blocks (documented layout)."""
    cfg = L.make_config(shape)
    pool = R.Pool(cfg, num_pages, rng.permutation(num_pages).astype(np.int32))
    n = pl.block_elems(num_pages, shape.n_kv_heads, shape.head_dim)
    kblk, vblk = bf16_normal(rng, n), bf16_normal(rng, n)
    pl.upload_layer(pool, 0, kblk, vblk, shape.n_kv_heads, shape.head_dim)
    return cfg, pool, kblk, vblk


def _gather(kblk, vblk, row, n, Hk, D):
    """K[n][Hk][D], V[n][Hk][D] for positions 0..n-1, walking the block-table row."""
    p = np.arange(n)
    pages = np.asarray(row)[p // 16][:, None, None]
    o = (p % 16)[:, None, None]
    h = np.arange(Hk)[None, :, None]
    d = np.arange(D)[None, None, :]
    K = f32_from_bf16(kblk[pl.k_index(pages, h, o, d, Hk, D)]).astype(np.float64)
    V = f32_from_bf16(vblk[pl.v_index(pages, h, o, d, Hk, D)]).astype(np.float64)
    return K, V


@pytest.mark.parametrize("H,D,Hk,ctxs", [(4, 64, 4, [0, 1, 15, 16, 17, 100]),
                                         (32, 128, 32, [0, 15, 16, 2048]),
                                         (8, 128, 8, [4096, 33, 511, 512, 1000, 7]),
                                         (32, 128, 8, [0, 15, 16, 2048, 300]),
                                         (4, 64, 1, [0, 1, 17, 100, 513]),
                                         (4, 64, 4, [2000, 2100, 3]),
                                         (32, 128, 32, [2048, 0, 15, 16, 17, 100, 1, 31, 32, 33, 200, 5, 64,
                                                        65, 127, 128]),
                                         (32, 128, 32, [4000, 2048, 0, 15, 16, 17, 100, 1, 31, 32, 33, 200, 5,
                                                        64, 65, 127])])
def test_decode_attention(L, R, H, D, Hk, ctxs):
    """Query head h attends over K/V head h // (H / Hk) (grouped-query when Hk < H).  The [2000, 2100,
    3] case leaves 16 and 17 block results per head to the combine (one-page partitions, 8 per block):
    the largest count it reads in one pass and one past it.  The last two ask for partitions longer
    than a wave takes: at 2049 tokens one block of eight 17-page partitions (no combine), at 4001 tokens
    two blocks of 16-page ones."""
    banner(f"decode_attention H={H} D={D} Hk={Hk} ctxs={ctxs}")
    shape = Shape(H, D, Hk=Hk)
    g = H // Hk
    rng = np.random.default_rng(11 + H + len(ctxs))
    max_pages = max(op.pages_needed(c + 1) for c in ctxs) + 1
    n = len(ctxs)
    num_pages = sum(op.pages_needed(c + 1) for c in ctxs) + 2
    cfg, pool, k_img, v_img = _random_pool(L, R, shape, num_pages, rng)
    bt = np.full((n, max_pages), -1, np.int32)
    for s, c in enumerate(ctxs):
        pool.alloc(c + 1, bt[s], 0, max_pages)
    q = (rng.standard_normal((n, H * D)) * 1.5).astype(np.float32)
    out = torch.empty(n, H * D, dtype=torch.float32, device="cuda")
    ws = R.Workspace(L.llmdec_workspace_bytes(cfg, n, n, max_pages))
    q_d, ctx_d, bt_d = R.dev_f32(q), R.dev_i32(ctxs), R.dev_i32(bt)
    L.llmdec_op_decode_attention(cfg, q_d.data_ptr(), n, ctx_d.data_ptr(), bt_d.data_ptr(), max_pages, pool.handle, 0, out.data_ptr(), ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert ws.error_bits() == 0
    got = out.cpu().numpy()
    ref = np.empty((n, H * D))
    for s, c in enumerate(ctxs):
        KK, VV = _gather(k_img, v_img, bt[s], c + 1, Hk, D)
        for h in range(H):
            ref[s, h * D:(h + 1) * D] = od.attend(q[s, h * D:(h + 1) * D], KK[:, h // g], VV[:, h // g])
    assert_close("decode attention", got, ref, max_abs=1e-4, rel_l2=1e-5)


@pytest.mark.parametrize("H,D,Hk,seqs", [(4, 64, 4, [(0, 1), (0, 17), (5, 40), (16, 16), (0, 64)]),
                                         (32, 128, 32, [(0, 33), (100, 20), (0, 16)]),
                                         (8, 128, 8, [(0, 512), (37, 300)]),
                                         (32, 128, 8, [(0, 33), (100, 20), (0, 64)]),
                                         (4, 64, 2, [(0, 1), (5, 40), (0, 64)])])
def test_prefill_attention(L, R, H, D, Hk, seqs):
    """Causal attention of new tokens after a cached prefix; query head h reads K/V head h // (H / Hk)."""
    banner(f"prefill_attention H={H} D={D} Hk={Hk} seqs={seqs}")
    shape = Shape(H, D, Hk=Hk)
    g = H // Hk
    rng = np.random.default_rng(21 + H)
    n = len(seqs)
    totals = [s0 + ln for s0, ln in seqs]
    max_pages = max(op.pages_needed(t) for t in totals) + 1
    num_pages = sum(op.pages_needed(t) for t in totals) + 2
    cfg, pool, k_img, v_img = _random_pool(L, R, shape, num_pages, rng)
    bt = np.full((n, max_pages), -1, np.int32)
    for s, t in enumerate(totals):
        pool.alloc(t, bt[s], 0, max_pages)
    cu = np.concatenate([[0], np.cumsum([ln for _, ln in seqs])]).astype(np.int32)
    T = int(cu[-1])
    q = (rng.standard_normal((T, H * D)) * 1.5).astype(np.float32)
    out = torch.full((T, H * D), float("nan"), dtype=torch.float32, device="cuda")
    ws = R.Workspace(8192)
    q_d, cu_d, st_d, bt_d = R.dev_f32(q), R.dev_i32(cu), R.dev_i32([s0 for s0, _ in seqs]), R.dev_i32(bt)
    L.llmdec_op_prefill_attention(cfg, q_d.data_ptr(), n, T, max(ln for _, ln in seqs), cu_d.data_ptr(),
                                  st_d.data_ptr(), bt_d.data_ptr(), max_pages, pool.handle, 0, out.data_ptr(), ws.ptr,
                                  ws.nbytes, R.stream())
    torch.cuda.synchronize()
    assert ws.error_bits() == 0
    got = out.cpu().numpy()
    ref = np.empty((T, H * D))
    for s, (s0, ln) in enumerate(seqs):
        KK, VV = _gather(k_img, v_img, bt[s], s0 + ln, Hk, D)
        for h in range(H):
            K, V = KK[:, h // g], VV[:, h // g]
            for i in range(ln):
                p = s0 + i
                ref[cu[s] + i, h * D:(h + 1) * D] = od.attend(q[cu[s] + i, h * D:(h + 1) * D], K[:p + 1], V[:p + 1])
    assert_close("prefill attention", got, ref, max_abs=1e-5, rel_l2=2e-6)


# ----------------------------------------------------------------------------- SwiGLU gate, greedy head
def test_silu_mul(L, R):
    rng = np.random.default_rng(31)
    g = (rng.standard_normal((3, 688)) * 4).astype(np.float32)
    u = rng.standard_normal((3, 688)).astype(np.float32)
    out = torch.empty(3, 688, dtype=torch.float32, device="cuda")
    g_d, u_d = R.dev_f32(g), R.dev_f32(u)
    L.llmdec_op_silu_mul(g_d.data_ptr(), u_d.data_ptr(), 3, 688, out.data_ptr(), R.stream())
    torch.cuda.synchronize()
    assert_close("silu_mul", out.cpu().numpy(), od.silu(g) * u, max_abs=1e-5, rel_l2=1e-6)


@pytest.mark.parametrize("rows,vocab", [(1, 1024), (3, 1024), (64, 32000), (1, 32000)])
def test_lm_head_argmax(L, R, rows, vocab):
    banner(f"lm_head_argmax rows={rows} vocab={vocab}")
    rng = np.random.default_rng(41 + rows)
    hidden = 4096 if vocab == 32000 else 256
    w = bf16_normal(rng, (vocab, hidden), 0.02)
    # planted ties: rows 10 and 900 of lm_head equal, and row 900 made dominant for input 0
    w[900] = w[10]
    x = rng.standard_normal((rows, hidden)).astype(np.float32)
    x[0] = od.widen_bf16(w[10]).astype(np.float32) * 50
    pm = R.PackedMatrix(vocab, hidden, w)
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    logits = torch.empty(rows, vocab, dtype=torch.float32, device="cuda")
    ws = R.Workspace(L.llmdec_op_linear_ws_bytes(rows, hidden, vocab))
    x_d = R.dev_f32(x)
    L.llmdec_op_lm_head_argmax(x_d.data_ptr(), rows, hidden, pm.ptr, vocab, nxt.data_ptr(), logits.data_ptr(),
                               ws.ptr, ws.nbytes, R.stream())
    torch.cuda.synchronize()
    W = od.widen_bf16(w)
    x64 = x.astype(np.float64)
    ref = x64 @ W.T
    lg = logits.cpu().numpy()
    assert_close("lm_head logits (fp16 input)", lg, od.round_to_f16(x64) @ W.T, max_abs=1e-4, rel_l2=2e-6)
    assert_within_rounding_bound("lm_head logits exact", lg, ref, np.abs(x64), np.abs(W), 2.0 ** -11, 1e-4)
    ids = nxt.cpu().numpy()
    assert ids[0] == 10                          # tie between 10 and 900 -> lowest index
    for r in range(rows):
        assert ids[r] == od.greedy_token(lg[r])  # exact argmax of the device logits
        if od.top2_gap(ref[r]) > 1e-2:
            assert ids[r] == od.greedy_token(ref[r])
