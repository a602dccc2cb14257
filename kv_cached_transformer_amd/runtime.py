"""Device-memory plumbing around libllmdec for PyTorch callers.

PyTorch only allocates device memory and supplies the stream; every step of
the decoder runs in the library's kernels.  Weights and cache contents are
passed as bf16 bit patterns (numpy uint16), held on the device as int16
tensors.
"""
from __future__ import annotations

import numpy as np
import torch

from . import llmdec as L


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def dev_u16(a: np.ndarray) -> torch.Tensor:
    """Upload a uint16 bit-pattern array as an int16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to("cuda")


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to("cuda")


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


class PackedLayer:
    """One layer packed for the kernels; owns its device buffer."""

    def __init__(self, cfg, tensors: dict, keep_plain: bool = False):
        nbytes = L.llmdec_packed_layer_bytes(cfg)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        plain = {k: dev_u16(v) for k, v in tensors.items()}
        w = L.llmdec_layer_weights(*(plain[k].data_ptr() for k in
                                     ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")))
        self.struct = L.llmdec_pack_layer(cfg, w, self.buf.data_ptr(), nbytes, stream())
        torch.cuda.current_stream().synchronize()
        self.plain = plain if keep_plain else None


class PackedMatrix:
    def __init__(self, rows: int, cols: int, bits: np.ndarray):
        nbytes = L.llmdec_packed_matrix_bytes(rows, cols)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        src = dev_u16(bits)
        L.llmdec_pack_matrix(rows, cols, src.data_ptr(), self.buf.data_ptr(), nbytes, stream())
        torch.cuda.current_stream().synchronize()
        self.ptr = self.buf.data_ptr()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def _q8_upload(m):
    """(codes, scales bits, zeros) host arrays -> device tensors and the llmdec_q8_matrix over them."""
    codes, scales, zeros = m
    t = (dev_u8(codes), dev_u16(scales), dev_u8(zeros))
    return t, L.llmdec_q8_matrix(*(x.data_ptr() for x in t))


class Q8Matrix:
    """One group-quantized matrix packed for the kernels; owns its device buffer.  bits = 8, or 4 (codes
    two to a byte: m[0] is [rows][cols/2] and cols must be given)."""

    def __init__(self, m, bits: int = 8, cols: int = None):
        rows = m[0].shape[0]
        cols = m[0].shape[1] if bits == 8 else cols
        size, pack = ((L.llmdec_q8_matrix_bytes, L.llmdec_q8_pack_matrix) if bits == 8 else
                      (L.llmdec_q4_matrix_bytes, L.llmdec_q4_pack_matrix))
        nbytes = size(rows, cols)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        src, struct = _q8_upload(m)
        pack(rows, cols, struct, self.buf.data_ptr(), nbytes, stream())
        torch.cuda.current_stream().synchronize()
        del src
        self.ptr = self.buf.data_ptr()


class Q8Layer:
    """One layer with group-quantized matrices (bits = 8 or 4), packed; owns its device buffer."""

    def __init__(self, cfg, tensors: dict, bits: int = 8):
        size, pack = ((L.llmdec_q8_packed_layer_bytes, L.llmdec_q8_pack_layer) if bits == 8 else
                      (L.llmdec_q4_packed_layer_bytes, L.llmdec_q4_pack_layer))
        nbytes = size(cfg)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        norms = {k: dev_u16(tensors[k]) for k in ("attn_norm", "mlp_norm")}
        up = {k: _q8_upload(tensors[k]) for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")}
        w = L.llmdec_q8_layer_weights(norms["attn_norm"].data_ptr(), *(up[k][1] for k in ("wq", "wk", "wv", "wo")),
                                      norms["mlp_norm"].data_ptr(), *(up[k][1] for k in ("w_gate", "w_up", "w_down")))
        self.struct = pack(cfg, w, self.buf.data_ptr(), nbytes, stream())
        torch.cuda.current_stream().synchronize()
        del up, norms


class Pool:
    """A device KV pool plus its host handle."""

    def __init__(self, cfg, num_pages: int, free_order=None, fill_bits: int | None = None):
        self.cfg = cfg
        self.num_pages = num_pages
        self.nbytes = L.llmdec_kv_pool_bytes(cfg, num_pages)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        if fill_bits is not None:
            self.buf.view(torch.int16).fill_(np.int16(np.uint16(fill_bits).view(np.int16)))
        fo = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        self.handle = L.llmdec_kv_pool_create(cfg, self.buf.data_ptr(), self.nbytes, num_pages, fo)

    def alloc(self, tokens_needed, row: np.ndarray, n_pages: int, max_pages: int) -> int:
        return L.llmdec_kv_pool_alloc(self.handle, tokens_needed, row, n_pages, max_pages)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            L.llmdec_kv_pool_destroy(h)
            self.handle = None


class Workspace:
    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        self.ptr = self.buf.data_ptr()
        L.llmdec_workspace_reset(self.ptr, self.nbytes, stream())

    def error_bits(self) -> int:
        return L.llmdec_workspace_error(self.ptr, stream())
