"""ctypes binding of libllmdec (include/llmdec.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Device pointers
are plain integers (e.g. ``tensor.data_ptr()``), streams are hipStream_t
handles as integers (``torch.cuda.current_stream().cuda_stream``).  Each call
raises ``LlmdecError`` carrying the library's message when the status is not
LLMDEC_OK.  The library must be built (kv_cached_transformer_amd.build): there
is no other implementation behind these names.
"""
from __future__ import annotations

import ctypes as C
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllmdec.so")

LLMDEC_OK, LLMDEC_E_INVALID, LLMDEC_E_UNSUPPORTED = 0, -1, -2
LLMDEC_E_NO_PAGES, LLMDEC_E_WORKSPACE, LLMDEC_E_HIP = -3, -4, -5
STATUS_NAMES = {0: "OK", -1: "E_INVALID", -2: "E_UNSUPPORTED", -3: "E_NO_PAGES", -4: "E_WORKSPACE", -5: "E_HIP"}

ERR_PAGE, ERR_POS, ERR_TOKEN, ERR_SEQ = 1, 2, 4, 8


class LlmdecError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class llmdec_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "intermediate",
                                         "vocab", "page_size")] + [("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class llmdec_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class llmdec_packed_layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "mlp_norm", "w_qkv", "w_o", "w_gu", "w_down")]


class llmdec_model_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("layers", C.POINTER(llmdec_packed_layer)), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p)]


class llmdec_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int32), ("top_p", C.c_float), ("seed", C.c_uint64),
                ("step", C.c_uint64)]


class llmdec_q8_matrix(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("codes", "scales", "zeros")]


class llmdec_q8_layer_weights(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p)] + [(n, llmdec_q8_matrix) for n in ("wq", "wk", "wv", "wo")] + \
               [("mlp_norm", C.c_void_p)] + [(n, llmdec_q8_matrix) for n in ("w_gate", "w_up", "w_down")]


class llmdec_q8_packed_layer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "mlp_norm", "w_qkv", "w_o", "w_gu", "w_down")]


_lib = None

_P, _I, _Z, _F = C.c_void_p, C.c_int32, C.c_size_t, C.c_float
_CFG = C.POINTER(llmdec_config)
_SIGS = {
    "llmdec_last_error": (C.c_char_p, []),
    "llmdec_packed_matrix_bytes": (_Z, [_I, _I]),
    "llmdec_pack_matrix": (_I, [_I, _I, _P, _P, _Z, _P]),
    "llmdec_packed_layer_bytes": (_Z, [_CFG]),
    "llmdec_pack_layer": (_I, [_CFG, C.POINTER(llmdec_layer_weights), _P, _Z, C.POINTER(llmdec_packed_layer), _P]),
    "llmdec_kv_pool_bytes": (_Z, [_CFG, _I]),
    "llmdec_kv_pool_create": (_I, [_CFG, _P, _Z, _I, C.POINTER(C.c_int32), C.POINTER(_P)]),
    "llmdec_kv_pool_alloc": (_I, [_P, _I, C.POINTER(C.c_int32), C.POINTER(C.c_int32), _I]),
    "llmdec_kv_pool_free": (_I, [_P, C.POINTER(C.c_int32), _I]),
    "llmdec_kv_pool_free_count": (_I, [_P]),
    "llmdec_kv_pool_device_base": (_P, [_P]),
    "llmdec_kv_pool_destroy": (None, [_P]),
    "llmdec_debug_gather_kv": (_I, [_P, _I, _P, _I, _P, _P, _P]),
    "llmdec_workspace_bytes": (_Z, [_CFG, _I, _I, _I]),
    "llmdec_workspace_reset": (_I, [_P, _Z, _P]),
    "llmdec_workspace_error": (_I, [_P, _P, C.POINTER(C.c_uint32)]),
    "llmdec_layer_prefill": (_I, [_CFG, C.POINTER(llmdec_packed_layer), _I, _P, _I, _I, _I, _P, _P, _P, _I, _P, _P,
                                  _Z, _P]),
    "llmdec_layer_decode": (_I, [_CFG, C.POINTER(llmdec_packed_layer), _I, _P, _I, _P, _P, _I, _P, _P, _Z, _P]),
    "llmdec_model_step_greedy": (_I, [_CFG, C.POINTER(llmdec_model_weights), _I, _I, _I, _P, _P, _P, _P, _I, _P, _P,
                                      _P, _P, _Z, _P]),
    "llmdec_model_step_greedy_noalloc": (_I, [_CFG, C.POINTER(llmdec_model_weights), _I, _I, _I, _P, _P, _P, _P, _I,
                                              _P, _P, _P, _P, _P]),
    "llmdec_op_rmsnorm": (_I, [_P, _P, _I, _I, _F, _P, _P, _P, _I, _P]),
    "llmdec_op_linear_ws_bytes": (_Z, [_I, _I, _I]),
    "llmdec_op_linear": (_I, [_P, _I, _I, _P, _I, _P, _I, _I, _P, _Z, _P]),
    "llmdec_op_swiglu_linear": (_I, [_P, _I, _I, _P, _I, _P, _P, _I, _I, _P, _Z, _P]),
    "llmdec_op_rope_append": (_I, [_CFG, _P, _I, _I, _P, _P, _P, _I, _P, _I, _P, _Z, _P]),
    "llmdec_op_decode_attention": (_I, [_CFG, _P, _I, _P, _P, _I, _P, _I, _P, _P, _Z, _P]),
    "llmdec_op_prefill_attention": (_I, [_CFG, _P, _I, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, _Z, _P]),
    "llmdec_op_silu_mul": (_I, [_P, _P, _I, _I, _P, _P]),
    "llmdec_op_lm_head_argmax": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _Z, _P]),
    "llmdec_op_sample": (_I, [_P, _I, _I, C.POINTER(llmdec_sampling), _P, _P]),
    "llmdec_model_step_sample": (_I, [_CFG, C.POINTER(llmdec_model_weights), _I, _I, _I, _P, _P, _P, _P, _I, _P,
                                      C.POINTER(llmdec_sampling), _P, _P, _P, _Z, _P]),
    "llmdec_q4_matrix_bytes": (_Z, [_I, _I]),
    "llmdec_q4_pack_matrix": (_I, [_I, _I, C.POINTER(llmdec_q8_matrix), _P, _Z, _P]),
    "llmdec_q4_packed_layer_bytes": (_Z, [_CFG]),
    "llmdec_q4_pack_layer": (_I, [_CFG, C.POINTER(llmdec_q8_layer_weights), _P, _Z, C.POINTER(llmdec_q8_packed_layer),
                                  _P]),
    "llmdec_op_linear_q4": (_I, [_P, _I, _P, _I, _P, _I, _P]),
    "llmdec_layer_decode_q4": (_I, [_CFG, C.POINTER(llmdec_q8_packed_layer), _I, _P, _I, _P, _P, _I, _P, _P, _Z,
                                    _P]),
    "llmdec_q8_matrix_bytes": (_Z, [_I, _I]),
    "llmdec_q8_pack_matrix": (_I, [_I, _I, C.POINTER(llmdec_q8_matrix), _P, _Z, _P]),
    "llmdec_q8_packed_layer_bytes": (_Z, [_CFG]),
    "llmdec_q8_pack_layer": (_I, [_CFG, C.POINTER(llmdec_q8_layer_weights), _P, _Z, C.POINTER(llmdec_q8_packed_layer),
                                  _P]),
    "llmdec_op_linear_q8": (_I, [_P, _I, _P, _I, _P, _I, _P]),
    "llmdec_layer_decode_q8": (_I, [_CFG, C.POINTER(llmdec_q8_packed_layer), _I, _P, _I, _P, _P, _I, _P, _P, _Z,
                                    _P]),
}
EXPORTED = tuple(_SIGS)


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libllmdec.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m kv_cached_transformer_amd.build`")
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(st):
    if st != LLMDEC_OK:
        raise LlmdecError(st, lib().llmdec_last_error().decode())
    return st


def make_config(shape) -> llmdec_config:
    """llmdec_config from any object with the model-shape attributes."""
    return llmdec_config(shape.n_layers, shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                         shape.intermediate, shape.vocab, getattr(shape, "page_size", 16),
                         float(shape.rms_eps), float(shape.rope_theta))


def _i32p(arr):
    """Host int32 numpy array -> ctypes pointer (None passes NULL)."""
    if arr is None:
        return None
    return arr.ctypes.data_as(C.POINTER(C.c_int32))


# ------------------------------------------------------------------ wrappers (same names as the C ABI)
def llmdec_last_error() -> str:
    return lib().llmdec_last_error().decode()


def llmdec_packed_matrix_bytes(rows, cols):
    return lib().llmdec_packed_matrix_bytes(rows, cols)


def llmdec_pack_matrix(rows, cols, src, dst, dst_bytes, stream=0):
    _check(lib().llmdec_pack_matrix(rows, cols, src, dst, dst_bytes, stream))


def llmdec_packed_layer_bytes(cfg):
    return lib().llmdec_packed_layer_bytes(C.byref(cfg))


def llmdec_pack_layer(cfg, weights: llmdec_layer_weights, dst, dst_bytes, stream=0) -> llmdec_packed_layer:
    out = llmdec_packed_layer()
    _check(lib().llmdec_pack_layer(C.byref(cfg), C.byref(weights), dst, dst_bytes, C.byref(out), stream))
    return out


def llmdec_kv_pool_bytes(cfg, num_pages):
    return lib().llmdec_kv_pool_bytes(C.byref(cfg), num_pages)


def llmdec_kv_pool_create(cfg, dev_base, nbytes, num_pages, free_order=None):
    h = C.c_void_p()
    _check(lib().llmdec_kv_pool_create(C.byref(cfg), dev_base, nbytes, num_pages, _i32p(free_order), C.byref(h)))
    return h


def llmdec_kv_pool_alloc(pool, tokens_needed, row, n_pages, max_pages):
    """Grow a host block-table row (int32 numpy array, modified in place); returns the new page count."""
    n = C.c_int32(n_pages)
    _check(lib().llmdec_kv_pool_alloc(pool, tokens_needed, _i32p(row), C.byref(n), max_pages))
    return n.value


def llmdec_kv_pool_free(pool, pages):
    _check(lib().llmdec_kv_pool_free(pool, _i32p(pages), len(pages)))


def llmdec_kv_pool_free_count(pool):
    return lib().llmdec_kv_pool_free_count(pool)


def llmdec_kv_pool_device_base(pool):
    return lib().llmdec_kv_pool_device_base(pool)


def llmdec_kv_pool_destroy(pool):
    lib().llmdec_kv_pool_destroy(pool)


def llmdec_debug_gather_kv(pool, layer, row_dev, n_tokens, k_out, v_out, stream=0):
    _check(lib().llmdec_debug_gather_kv(pool, layer, row_dev, n_tokens, k_out, v_out, stream))


def llmdec_workspace_bytes(cfg, max_tokens, max_seqs, max_pages):
    return lib().llmdec_workspace_bytes(C.byref(cfg), max_tokens, max_seqs, max_pages)


def llmdec_workspace_reset(ws, ws_bytes, stream=0):
    _check(lib().llmdec_workspace_reset(ws, ws_bytes, stream))


def llmdec_workspace_error(ws, stream=0) -> int:
    bits = C.c_uint32(0)
    _check(lib().llmdec_workspace_error(ws, stream, C.byref(bits)))
    return bits.value


def llmdec_layer_prefill(cfg, w, layer, hidden, n_seqs, n_tokens, max_q_len, cu_seqlens, start_pos, block_tables,
                         max_pages, pool, ws, ws_bytes, stream=0):
    _check(lib().llmdec_layer_prefill(C.byref(cfg), C.byref(w), layer, hidden, n_seqs, n_tokens, max_q_len,
                                      cu_seqlens, start_pos, block_tables, max_pages, pool, ws, ws_bytes, stream))


def llmdec_layer_decode(cfg, w, layer, hidden, n_seqs, ctx_lens, block_tables, max_pages, pool, ws, ws_bytes,
                        stream=0):
    _check(lib().llmdec_layer_decode(C.byref(cfg), C.byref(w), layer, hidden, n_seqs, ctx_lens, block_tables,
                                     max_pages, pool, ws, ws_bytes, stream))


def make_model_weights(embed, packed_layers, final_norm, lm_head_packed):
    """Build the llmdec_model_weights struct; keep the returned tuple alive while it is used."""
    arr = (llmdec_packed_layer * len(packed_layers))(*packed_layers)
    mw = llmdec_model_weights(embed, C.cast(arr, C.POINTER(llmdec_packed_layer)), final_norm, lm_head_packed)
    return mw, arr


def llmdec_model_step_greedy(cfg, mw, n_seqs, n_tokens, max_q_len, tokens, cu_seqlens, start_pos, block_tables,
                             max_pages, pool, next_tokens, logits, ws, ws_bytes, stream=0):
    _check(lib().llmdec_model_step_greedy(C.byref(cfg), C.byref(mw), n_seqs, n_tokens, max_q_len, tokens, cu_seqlens,
                                          start_pos, block_tables, max_pages, pool, next_tokens, logits, ws, ws_bytes,
                                          stream))


def llmdec_model_step_greedy_noalloc(cfg, mw, n_seqs, n_tokens, max_q_len, tokens, cu_seqlens, start_pos,
                                     block_tables, max_pages, pool, next_tokens, logits, error_bits, stream=0):
    _check(lib().llmdec_model_step_greedy_noalloc(C.byref(cfg), C.byref(mw), n_seqs, n_tokens, max_q_len, tokens,
                                                  cu_seqlens, start_pos, block_tables, max_pages, pool, next_tokens,
                                                  logits, error_bits, stream))


def llmdec_op_rmsnorm(x, gamma, rows, n, eps, out_f32, out_act=None, out_lo=None, ld_packed=0, stream=0):
    _check(lib().llmdec_op_rmsnorm(x, gamma, rows, n, eps, out_f32, out_act, out_lo, ld_packed, stream))


def llmdec_op_linear_ws_bytes(rows, k_dim, n_dim):
    return lib().llmdec_op_linear_ws_bytes(rows, k_dim, n_dim)


def llmdec_op_linear(a, rows, k_dim, w_packed, n_dim, out, accumulate, ws, ws_bytes, stream=0, act_parts=1):
    _check(lib().llmdec_op_linear(a, rows, k_dim, w_packed, n_dim, out, int(accumulate), int(act_parts), ws, ws_bytes,
                                  stream))


def llmdec_op_swiglu_linear(a, rows, k_dim, w_gu_packed, inter, out_act, ld_packed, ws, ws_bytes, stream=0,
                            act_parts=1, out_lo=None):
    _check(lib().llmdec_op_swiglu_linear(a, rows, k_dim, w_gu_packed, inter, out_act, out_lo, ld_packed,
                                         int(act_parts), ws, ws_bytes, stream))


def llmdec_op_rope_append(cfg, qkv, n_tokens, n_seqs, seq_of_token, pos_of_token, block_tables, max_pages, pool,
                          layer, ws, ws_bytes, stream=0):
    _check(lib().llmdec_op_rope_append(C.byref(cfg), qkv, n_tokens, n_seqs, seq_of_token, pos_of_token,
                                       block_tables, max_pages, pool, layer, ws, ws_bytes, stream))


def llmdec_op_decode_attention(cfg, q, n_seqs, ctx_lens, block_tables, max_pages, pool, layer, out, ws, ws_bytes,
                               stream=0):
    _check(lib().llmdec_op_decode_attention(C.byref(cfg), q, n_seqs, ctx_lens, block_tables, max_pages, pool, layer,
                                            out, ws, ws_bytes, stream))


def llmdec_op_prefill_attention(cfg, q, n_seqs, n_tokens, max_q_len, cu_seqlens, start_pos, block_tables, max_pages,
                                pool, layer, out, ws, ws_bytes, stream=0):
    _check(lib().llmdec_op_prefill_attention(C.byref(cfg), q, n_seqs, n_tokens, max_q_len, cu_seqlens, start_pos,
                                             block_tables, max_pages, pool, layer, out, ws, ws_bytes, stream))


def llmdec_op_silu_mul(gate, up, rows, n, out, stream=0):
    _check(lib().llmdec_op_silu_mul(gate, up, rows, n, out, stream))


def llmdec_op_lm_head_argmax(x, rows, hidden, lm_head_packed, vocab, next_tokens, logits_out, ws, ws_bytes, stream=0):
    _check(lib().llmdec_op_lm_head_argmax(x, rows, hidden, lm_head_packed, vocab, next_tokens, logits_out, ws,
                                          ws_bytes, stream))


def llmdec_q8_matrix_bytes(rows, cols):
    return lib().llmdec_q8_matrix_bytes(rows, cols)


def llmdec_q8_pack_matrix(rows, cols, src: llmdec_q8_matrix, dst, dst_bytes, stream=0):
    _check(lib().llmdec_q8_pack_matrix(rows, cols, C.byref(src), dst, dst_bytes, stream))


def llmdec_q8_packed_layer_bytes(cfg):
    return lib().llmdec_q8_packed_layer_bytes(C.byref(cfg))


def llmdec_q8_pack_layer(cfg, weights: llmdec_q8_layer_weights, dst, dst_bytes, stream=0) -> llmdec_q8_packed_layer:
    out = llmdec_q8_packed_layer()
    _check(lib().llmdec_q8_pack_layer(C.byref(cfg), C.byref(weights), dst, dst_bytes, C.byref(out), stream))
    return out


def llmdec_op_linear_q8(a, k_dim, w_q8_packed, n_dim, out, accumulate, stream=0):
    _check(lib().llmdec_op_linear_q8(a, k_dim, w_q8_packed, n_dim, out, int(accumulate), stream))


def llmdec_layer_decode_q8(cfg, w, layer, hidden, n_seqs, ctx_lens, block_tables, max_pages, pool, ws, ws_bytes,
                           stream=0):
    _check(lib().llmdec_layer_decode_q8(C.byref(cfg), C.byref(w), layer, hidden, n_seqs, ctx_lens, block_tables,
                                        max_pages, pool, ws, ws_bytes, stream))


def llmdec_op_sample(logits, rows, vocab, params: llmdec_sampling, next_tokens, stream=0):
    _check(lib().llmdec_op_sample(logits, rows, vocab, C.byref(params), next_tokens, stream))


def llmdec_model_step_sample(cfg, mw, n_seqs, n_tokens, max_q_len, tokens, cu_seqlens, start_pos, block_tables,
                             max_pages, pool, params: llmdec_sampling, next_tokens, logits, ws, ws_bytes, stream=0):
    _check(lib().llmdec_model_step_sample(C.byref(cfg), C.byref(mw), n_seqs, n_tokens, max_q_len, tokens, cu_seqlens,
                                          start_pos, block_tables, max_pages, pool, C.byref(params), next_tokens,
                                          logits, ws, ws_bytes, stream))


# 4-bit codes: the same structs (codes two to a byte)
llmdec_q4_matrix, llmdec_q4_layer_weights, llmdec_q4_packed_layer = (llmdec_q8_matrix, llmdec_q8_layer_weights,
                                                                      llmdec_q8_packed_layer)


def llmdec_q4_matrix_bytes(rows, cols):
    return lib().llmdec_q4_matrix_bytes(rows, cols)


def llmdec_q4_pack_matrix(rows, cols, src: llmdec_q8_matrix, dst, dst_bytes, stream=0):
    _check(lib().llmdec_q4_pack_matrix(rows, cols, C.byref(src), dst, dst_bytes, stream))


def llmdec_q4_packed_layer_bytes(cfg):
    return lib().llmdec_q4_packed_layer_bytes(C.byref(cfg))


def llmdec_q4_pack_layer(cfg, weights: llmdec_q8_layer_weights, dst, dst_bytes, stream=0) -> llmdec_q8_packed_layer:
    out = llmdec_q8_packed_layer()
    _check(lib().llmdec_q4_pack_layer(C.byref(cfg), C.byref(weights), dst, dst_bytes, C.byref(out), stream))
    return out


def llmdec_op_linear_q4(a, k_dim, w_q4_packed, n_dim, out, accumulate, stream=0):
    _check(lib().llmdec_op_linear_q4(a, k_dim, w_q4_packed, n_dim, out, int(accumulate), stream))


def llmdec_layer_decode_q4(cfg, w, layer, hidden, n_seqs, ctx_lens, block_tables, max_pages, pool, ws, ws_bytes,
                           stream=0):
    _check(lib().llmdec_layer_decode_q4(C.byref(cfg), C.byref(w), layer, hidden, n_seqs, ctx_lens, block_tables,
                                        max_pages, pool, ws, ws_bytes, stream))
