"""Paged KV cache bookkeeping, written out plainly (test infrastructure only).

[E] §3.4: the cache is cut into fixed-size pages of N tokens (16 or 32 is the
recommended size; 16 here); a request takes pages from a list of free pages
when it needs them and returns them when it ends, so requests interleave in
memory; attention finds a token's cache block through a page index.

Readings (the pages are silent on these):
* the free list is a stack whose initial order is given by the caller: the
  first entry of that order is handed out first; pages returned by ``free``
  are pushed in the order given, so the last one returned is reused first;
* growing a sequence to n tokens needs ceil(n / 16) pages; the new pages are
  appended to the sequence's block-table row; if the pool cannot cover the
  growth, nothing changes and the call fails ("no pages");
* position p of a sequence lives in page row[p // 16] at in-page offset p % 16;
* inside a page, K is laid out [kv_head][16][head_dim] and V is laid out
  [kv_head][4][head_dim][4] (quarter of the page, dim, token within the
  quarter); float results do not depend on this, only the pool-image
  comparisons do.

Parity pins: the slot formula against a brute-force page walk, pool sizing
against [E] §3.4's 1 GiB example, paged attention equal to contiguous
attention bit for bit, atomic failure on exhaustion, double-free rejection.
"""
from __future__ import annotations

import numpy as np

from .decoder import kv_cache_bytes

PAGE = 16
OK, E_INVALID, E_NO_PAGES = 0, -1, -3


def pages_needed(tokens: int, page: int = PAGE) -> int:
    return -(-int(tokens) // page)


def slot_of(row, pos: int, page: int = PAGE):
    """(page id, in-page offset) holding position pos of the sequence with block-table row ``row``."""
    return int(row[pos // page]), pos % page


def pool_bytes(n_layers, n_kv_heads, head_dim, num_pages, dtype_bytes=2, page=PAGE):
    """Device bytes of a pool of num_pages pages for every layer, K and V."""
    return kv_cache_bytes(n_layers, n_kv_heads, head_dim, num_pages * page, dtype_bytes)


class PagePool:
    """Free-list page allocator over page ids 0..num_pages-1."""

    def __init__(self, num_pages: int, free_order=None):
        order = list(range(num_pages)) if free_order is None else [int(p) for p in free_order]
        assert sorted(order) == list(range(num_pages)), "free order must be a permutation"
        self.num_pages = num_pages
        self._stack = order[::-1]            # top of the stack = end of the list
        self._free = set(order)

    @property
    def n_free(self):
        return len(self._stack)

    def alloc(self, tokens_needed: int, row: list, n_pages: int, max_pages: int):
        """Grow a sequence's row so it covers tokens_needed tokens; returns (status, n_pages)."""
        need = pages_needed(tokens_needed)
        if tokens_needed < 0 or n_pages < 0 or n_pages > max_pages or need > max_pages:
            return E_INVALID, n_pages
        extra = need - n_pages
        if extra <= 0:
            return OK, n_pages
        if extra > len(self._stack):
            return E_NO_PAGES, n_pages
        for i in range(extra):
            p = self._stack.pop()
            self._free.discard(p)
            row[n_pages + i] = p
        return OK, need

    def free(self, pages):
        pages = [int(p) for p in pages]
        if any(p < 0 or p >= self.num_pages or p in self._free for p in pages) or len(set(pages)) != len(pages):
            return E_INVALID
        for p in pages:
            self._stack.append(p)
            self._free.add(p)
        return OK


class PagedKV:
    """A paged mirror of the cache: per layer, K pool [num_pages][Hkv][16][D] and V pool [num_pages][Hkv][4][D][4].

    Values are float64 holding bf16 values.

    Same interface as decoder.ContiguousKV; positions are found through block-table rows.
    """

    def __init__(self, n_layers, n_kv_heads, head_dim, num_pages, block_rows: dict):
        self.L, self.H, self.D = n_layers, n_kv_heads, head_dim
        self.K = np.zeros((n_layers, num_pages, n_kv_heads, PAGE, head_dim))
        self.V = np.zeros((n_layers, num_pages, n_kv_heads, PAGE // 4, head_dim, 4))
        self.rows = block_rows          # seq id -> block-table row (list of page ids)
        self.len = {}

    def length(self, layer, seq):
        return self.len.get((layer, seq), 0)

    def store(self, layer, seq, pos, k, v):
        assert pos == self.length(layer, seq), "append out of order"
        pg, off = slot_of(self.rows[seq], pos)
        self.K[layer, pg, :, off, :] = k
        self.V[layer, pg, :, off // 4, :, off % 4] = v
        self.len[(layer, seq)] = pos + 1

    def preload(self, layer, seq, k, v):
        for p in range(k.shape[0]):
            pg, off = slot_of(self.rows[seq], p)
            self.K[layer, pg, :, off, :] = k[p]
            self.V[layer, pg, :, off // 4, :, off % 4] = v[p]
        self.len[(layer, seq)] = k.shape[0]

    def keys_values(self, layer, seq, upto):
        """Gather positions 0..upto-1 through the page index, one position at a time."""
        K = np.empty((upto, self.H, self.D))
        V = np.empty_like(K)
        for p in range(upto):
            pg, off = slot_of(self.rows[seq], p)
            K[p] = self.K[layer, pg, :, off, :]
            V[p] = self.V[layer, pg, :, off // 4, :, off % 4]
        return K, V
