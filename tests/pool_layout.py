"""The KV pool's device layout as include/llmdec.h documents it, written out for the tests.

Per layer the pool holds a K block then a V block, layer after layer; with P pages, H K/V heads and
head_dim D, each block has P * H * 16 * D bf16 elements, and the slot of in-page offset o (position
p of a sequence sits in page row[p / 16] at o = p % 16) is found at
    K: ((page * H + h) * 16 + o) * D + d
    V: (((page * H + h) * 4 + o / 4) * D + d) * 4 + o % 4
This module computes those offsets itself, so the tests check the kernels against the documented
formula rather than against product code that shares the kernels' view of the layout.
"""
import numpy as np


def block_elems(num_pages, H, D):
    return num_pages * H * 16 * D


def k_index(page, h, o, d, H, D):
    return ((page * H + h) * 16 + o) * D + d


def v_index(page, h, o, d, H, D):
    return (((page * H + h) * 4 + o // 4) * D + d) * 4 + o % 4


def layer_blocks(flat_u16, layer, num_pages, H, D):
    """(K block, V block) of one layer, as views into a flat array of the whole pool."""
    n = block_elems(num_pages, H, D)
    base = layer * 2 * n
    return flat_u16[base:base + n], flat_u16[base + n:base + 2 * n]


def _hd(H, D):
    return np.arange(H)[:, None], np.arange(D)[None, :]


def read_slot(kblk, vblk, page, o, H, D):
    """K[H][D], V[H][D] (bf16 bits) of one slot."""
    h, d = _hd(H, D)
    return kblk[k_index(page, h, o, d, H, D)], vblk[v_index(page, h, o, d, H, D)]


def write_slot(kblk, vblk, page, o, k, v, H, D):
    h, d = _hd(H, D)
    kblk[k_index(page, h, o, d, H, D)] = k
    vblk[v_index(page, h, o, d, H, D)] = v


def write_history(kblk, vblk, row, k, v, H, D):
    """Positions 0..n-1 of one sequence (k, v: [n][H][D] bf16 bits) into the slots its block-table row names."""
    for p in range(k.shape[0]):
        write_slot(kblk, vblk, int(row[p // 16]), p % 16, k[p], v[p], H, D)


def unwritten_equal(blk_a, blk_b, written, H, D, kind):
    """True when every element of the slots not marked in written[page][o] is equal in both blocks."""
    idx = k_index if kind == "k" else v_index
    pages, offs = np.nonzero(~written)
    h = np.arange(H)[None, :, None]
    d = np.arange(D)[None, None, :]
    at = idx(pages[:, None, None], h, offs[:, None, None], d, H, D)
    return np.array_equal(blk_a[at], blk_b[at])


def host_pool(pool):
    """The whole device pool as host uint16 bits (pool.buf is the caller-owned device buffer)."""
    return pool.buf.cpu().numpy().view(np.uint16)


def upload_layer(pool, layer, kblk, vblk, H, D):
    """Copy host K and V blocks of one layer into the device pool."""
    import torch
    n = block_elems(pool.num_pages, H, D)
    flat = pool.buf.view(torch.int16)
    base = layer * 2 * n
    flat[base:base + n].copy_(torch.from_numpy(np.ascontiguousarray(kblk).view(np.int16)))
    flat[base + n:base + 2 * n].copy_(torch.from_numpy(np.ascontiguousarray(vblk).view(np.int16)))


def host_layer(pool, layer, H, D):
    """(K block, V block) of one layer copied to the host as uint16 bits."""
    n = block_elems(pool.num_pages, H, D)
    flat = pool.buf.view(__import__("torch").int16)
    base = layer * 2 * n
    return (flat[base:base + n].cpu().numpy().view(np.uint16), flat[base + n:base + 2 * n].cpu().numpy().view(np.uint16))


def gather_slots(kblk_t, vblk_t, slots, H, D):
    """K and V (bf16 bits, [n][H][D]) of the given (page, offset) slots, read from device block tensors."""
    import torch
    pg = np.array([p for p, _ in slots])[:, None, None]
    o = np.array([q for _, q in slots])[:, None, None]
    h = np.arange(H)[None, :, None]
    d = np.arange(D)[None, None, :]
    ki = torch.from_numpy(k_index(pg, h, o, d, H, D).astype(np.int64)).to(kblk_t.device)
    vi = torch.from_numpy(v_index(pg, h, o, d, H, D).astype(np.int64)).to(vblk_t.device)
    return kblk_t[ki].cpu().numpy().view(np.uint16), vblk_t[vi].cpu().numpy().view(np.uint16)


def write_sequence_pages(kblk_t, vblk_t, num_pages, pages, k, v, H, D):
    """Write positions 0..n-1 of a sequence into its pages of a device layer (block tensors): the pages
    are fetched, filled on the host with the documented formula (page-major, so the fetched pages form
    a small pool of their own), and written back."""
    import torch
    per = H * 16 * D
    kp, vp = kblk_t.view(num_pages, per), vblk_t.view(num_pages, per)
    idx = torch.from_numpy(np.asarray(pages, np.int64)).to(kblk_t.device)
    kc = kp[idx].cpu().numpy().view(np.uint16).reshape(-1).copy()
    vc = vp[idx].cpu().numpy().view(np.uint16).reshape(-1).copy()
    write_history(kc, vc, np.arange(len(pages)), k, v, H, D)
    kp[idx] = torch.from_numpy(kc.view(np.int16).reshape(len(pages), per)).to(kblk_t.device)
    vp[idx] = torch.from_numpy(vc.view(np.int16).reshape(len(pages), per)).to(vblk_t.device)
