"""Host-only checks of libllmdec: exports, argument validation, and the page allocator.

No device work is launched: these calls either validate and fail before any
launch, or are pure host bookkeeping (the KV pool's free list).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import pages as op

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llmdec.h")


@pytest.fixture(scope="module")
def L():
    from kv_cached_transformer_amd import llmdec
    if not os.path.exists(llmdec.library_path()):
        from kv_cached_transformer_amd import build
        build.build()
    llmdec.lib()
    return llmdec


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llmdec_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported_and_bound(L):
    names = header_functions()
    assert len(names) >= 25
    so = ctypes.CDLL(L.library_path())
    for n in names:
        assert hasattr(so, n), f"{n} declared in llmdec.h but not exported"
        assert n in L.EXPORTED and hasattr(L, n), f"{n} has no binding"


def tiny_cfg(L, **kw):
    import synth
    c = L.make_config(synth.TINY)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_validation_before_launch(L):
    assert L.llmdec_workspace_bytes(tiny_cfg(L), 32, 1, 4) > 0
    assert L.llmdec_workspace_bytes(tiny_cfg(L, page_size=32), 32, 1, 4) == 0
    assert L.llmdec_workspace_bytes(tiny_cfg(L, head_dim=96), 32, 1, 4) == 0
    # grouped K/V heads: n_kv_heads must divide n_heads (4); the q|k|v buffer shrinks with it
    assert 0 < L.llmdec_workspace_bytes(tiny_cfg(L, n_kv_heads=2), 32, 1, 4) < L.llmdec_workspace_bytes(tiny_cfg(L), 32, 1, 4)
    assert L.llmdec_workspace_bytes(tiny_cfg(L, n_kv_heads=3), 32, 1, 4) == 0
    assert L.llmdec_workspace_bytes(tiny_cfg(L, n_kv_heads=0), 32, 1, 4) == 0
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_kv_pool_create(tiny_cfg(L, hidden=300), 1 << 20, 1 << 30, 4)
    assert e.value.status in (L.LLMDEC_E_INVALID, L.LLMDEC_E_UNSUPPORTED)
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_pack_matrix(15, 32, 1 << 20, 1 << 21, 1 << 20)
    assert e.value.status == L.LLMDEC_E_INVALID and "multiple of 16" in str(e.value)
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_pack_matrix(16, 32, 1 << 20, 1 << 21, 100)
    assert e.value.status == L.LLMDEC_E_INVALID


def test_pool_sizing_matches_kv_formula(L):
    import synth
    cfg = L.make_config(synth.LLAMA7B)
    # 128 pages of 16 tokens = one 2048-token request: 1 GiB ([E] §3.4)
    assert L.llmdec_kv_pool_bytes(cfg, 128) == op.pool_bytes(32, 32, 128, 128) == 2 ** 30


def test_pool_rejects_bad_free_order(L):
    cfg = tiny_cfg(L)
    nb = L.llmdec_kv_pool_bytes(cfg, 4)
    with pytest.raises(L.LlmdecError):
        L.llmdec_kv_pool_create(cfg, 1 << 20, nb, 4, np.array([0, 1, 1, 3], np.int32))
    with pytest.raises(L.LlmdecError):
        L.llmdec_kv_pool_create(cfg, 1 << 20, nb - 1, 4)


def test_page_allocator_matches_oracle_bit_for_bit(L):
    """Random grow/free traffic over several sequences: block tables, failures and free counts agree."""
    cfg = tiny_cfg(L)
    num_pages, max_pages, n_seq = 64, 12, 6
    order = np.random.default_rng(5).permutation(num_pages).astype(np.int32)
    # any non-null base: the allocator never dereferences device memory
    h = L.llmdec_kv_pool_create(cfg, 1 << 20, L.llmdec_kv_pool_bytes(cfg, num_pages), num_pages, order)
    ref = op.PagePool(num_pages, order)
    r = np.random.default_rng(6)
    rows = np.full((n_seq, max_pages), -1, np.int32)
    ref_rows = [[-1] * max_pages for _ in range(n_seq)]
    npg = [0] * n_seq
    toks = [0] * n_seq
    for step in range(400):
        s = int(r.integers(n_seq))
        if r.random() < 0.15 and npg[s]:
            pages = rows[s, :npg[s]].copy()
            L.llmdec_kv_pool_free(h, pages)
            assert ref.free(ref_rows[s][:npg[s]]) == op.OK
            rows[s] = -1
            ref_rows[s] = [-1] * max_pages
            npg[s] = 0
            toks[s] = 0
            continue
        want = toks[s] + int(r.integers(1, 40))
        st_ref, n_ref = ref.alloc(want, ref_rows[s], npg[s], max_pages)
        try:
            n_new = L.llmdec_kv_pool_alloc(h, want, rows[s], npg[s], max_pages)
            st = op.OK
        except L.LlmdecError as e:
            st, n_new = e.status, npg[s]
        assert st == st_ref, (step, st, st_ref)
        assert n_new == n_ref
        assert rows[s].tolist() == ref_rows[s]
        npg[s] = n_new
        if st == op.OK:
            toks[s] = want
        assert L.llmdec_kv_pool_free_count(h) == ref.n_free
    # error paths leave everything unchanged
    with pytest.raises(L.LlmdecError):
        L.llmdec_kv_pool_free(h, np.array([num_pages], np.int32))
    free_pages = [p for p in range(num_pages) if p in ref._free]
    if free_pages:
        before = L.llmdec_kv_pool_free_count(h)
        with pytest.raises(L.LlmdecError):
            L.llmdec_kv_pool_free(h, np.array([free_pages[0]], np.int32))
        assert L.llmdec_kv_pool_free_count(h) == before
    L.llmdec_kv_pool_destroy(h)


def test_pool_exhaustion_is_atomic(L):
    cfg = tiny_cfg(L)
    h = L.llmdec_kv_pool_create(cfg, 1 << 20, L.llmdec_kv_pool_bytes(cfg, 3), 3)
    row = np.full(8, -1, np.int32)
    assert L.llmdec_kv_pool_alloc(h, 40, row, 0, 8) == 3
    row2 = np.full(8, -7, np.int32)
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_kv_pool_alloc(h, 1, row2, 0, 8)
    assert e.value.status == L.LLMDEC_E_NO_PAGES and (row2 == -7).all()
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_kv_pool_alloc(h, 200, row, 3, 8)  # 13 pages > row width
    assert e.value.status == L.LLMDEC_E_INVALID
    L.llmdec_kv_pool_destroy(h)


def test_q8_sizes_and_validation_before_launch(L):
    """Group-quantized matrices: packed size = codes + 128 bytes of metadata words per four 1024-column
    steps of a row; unsupported shapes give 0 / E_INVALID; a quantized decode step of more than one
    sequence is E_UNSUPPORTED before anything is launched."""
    assert L.llmdec_q8_matrix_bytes(4096, 4096) == 4096 * 4096 + 4096 * 128
    assert L.llmdec_q8_matrix_bytes(4096, 11008) == 4096 * 11008 + 4096 * 3 * 128
    assert L.llmdec_q8_matrix_bytes(64, 688) == 64 * 688 + 64 * 128
    assert L.llmdec_q8_matrix_bytes(6, 256) == 0            # rows not a multiple of 4
    assert L.llmdec_q8_matrix_bytes(8, 264) == 0            # cols not a multiple of 16
    assert L.llmdec_q8_matrix_bytes(8, 14336) > 0 and L.llmdec_q8_matrix_bytes(8, 14352) == 0
    cfg = tiny_cfg(L)
    assert L.llmdec_q8_packed_layer_bytes(cfg) > 0
    src = L.llmdec_q8_matrix(1 << 20, 1 << 21, 1 << 22)
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_q8_pack_matrix(8, 264, src, 1 << 23, 1 << 20)
    assert e.value.status == L.LLMDEC_E_INVALID
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_q8_pack_matrix(8, 256, src, 1 << 23, 100)
    assert e.value.status == L.LLMDEC_E_INVALID and "needed" in str(e.value)
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_op_linear_q8(1 << 20, 264, 1 << 21, 8, 1 << 22, 0)
    assert e.value.status == L.LLMDEC_E_INVALID
    num_pages = 4
    h = L.llmdec_kv_pool_create(cfg, 1 << 20, L.llmdec_kv_pool_bytes(cfg, num_pages), num_pages)
    try:
        w = L.llmdec_q8_packed_layer(*([1 << 24] * 6))
        ws_bytes = L.llmdec_workspace_bytes(cfg, 2, 2, 4)
        with pytest.raises(L.LlmdecError) as e:
            L.llmdec_layer_decode_q8(cfg, w, 0, 1 << 20, 2, 1 << 21, 1 << 22, 4, h, 1 << 23, ws_bytes)
        assert e.value.status == L.LLMDEC_E_UNSUPPORTED and "n_seqs=2" in str(e.value)
        with pytest.raises(L.LlmdecError) as e:
            L.llmdec_layer_decode_q8(cfg, w, 0, 1 << 20, 1, 1 << 21, 1 << 22, 4, h, 1 << 23, 16)
        assert e.value.status == L.LLMDEC_E_WORKSPACE
    finally:
        L.llmdec_kv_pool_destroy(h)


def test_q4_sizes_and_validation(L):
    """4-bit codes: each row's cols/2 code bytes padded to a multiple of 16, then 256 bytes of metadata words
    per four 2048-column steps; the same shape limits as the 8-bit matrices."""
    assert L.llmdec_q4_matrix_bytes(4096, 4096) == 4096 * 2048 + 4096 * 256
    assert L.llmdec_q4_matrix_bytes(4096, 11008) == 4096 * 5504 + 4096 * 2 * 256
    assert L.llmdec_q4_matrix_bytes(64, 688) == 64 * 352 + 64 * 256
    assert L.llmdec_q4_matrix_bytes(6, 256) == 0 and L.llmdec_q4_matrix_bytes(8, 264) == 0
    assert L.llmdec_q4_matrix_bytes(8, 14336) > 0 and L.llmdec_q4_matrix_bytes(8, 14352) == 0
    assert 0 < L.llmdec_q4_packed_layer_bytes(tiny_cfg(L)) < L.llmdec_q8_packed_layer_bytes(tiny_cfg(L))
    src = L.llmdec_q4_matrix(1 << 20, 1 << 21, 1 << 22)
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_q4_pack_matrix(8, 256, src, 1 << 23, 100)
    assert e.value.status == L.LLMDEC_E_INVALID and "q4_pack_matrix" in str(e.value)


def test_rmsnorm_op_shape_validation_before_launch(L):
    """llmdec_op_rmsnorm refuses shapes its kernels would not cover before anything is launched: n past
    8192 or not a multiple of 32, and a packed stride (ld_packed) below n, not a multiple of 32 or past
    8192 columns (the padding columns n..ld_packed-1 are zeroed only up to there)."""
    p = 1 << 20
    for n, ld in ((8192, 8224), (256, 240), (256, 272), (8224, 8224), (250, 256)):
        with pytest.raises(L.LlmdecError) as e:
            L.llmdec_op_rmsnorm(p, p, 4, n, 1e-6, None, p, None, ld)
        assert e.value.status == L.LLMDEC_E_INVALID, (n, ld)
