"""Set-up shared by the layer-level GPU tests and the benchmark: a packed layer,
a pool holding a seeded cache history, block tables from the library's
allocator, and the matching oracle cache."""
import numpy as np

import synth
from oracle import decoder as od
from oracle import pages as op
from tests import pool_layout as pl


class LayerCase:
    """One layer, n sequences with cached histories ctxs[s], ready for a decode or prefill step.

    extra_tokens[s] = how many new tokens sequence s will append this step.
    """

    def __init__(self, L, R, shape, workload, ctxs, extra_tokens, build_oracle=True, slack_pages=0, pack=True):
        import torch
        self.L, self.R, self.shape, self.workload = L, R, shape, workload
        self.cfg = L.make_config(shape)
        self.ctxs = [int(c) for c in ctxs]
        self.extra = [int(e) for e in extra_tokens]
        H, D = shape.n_kv_heads, shape.head_dim
        self.lw = synth.layer_weights(workload, 0, shape) if pack else None
        self.packed = R.PackedLayer(self.cfg, self.lw.tensors) if pack else None
        totals = [c + e for c, e in zip(self.ctxs, self.extra)]
        self.max_pages = max(op.pages_needed(t) for t in totals) + 1
        self.num_pages = sum(op.pages_needed(t) for t in totals) + slack_pages
        order = synth.free_order(workload, self.num_pages)
        self.pool = R.Pool(self.cfg, self.num_pages, order, fill_bits=0xFFFF)
        ref_alloc = op.PagePool(self.num_pages, order)
        n = len(ctxs)
        self.bt = np.full((n, self.max_pages), -1, np.int32)
        for s, t in enumerate(totals):
            row = [-1] * self.max_pages
            got = self.pool.alloc(t, self.bt[s], 0, self.max_pages)
            st, ref_n = ref_alloc.alloc(t, row, 0, self.max_pages)
            assert st == op.OK and got == ref_n and self.bt[s].tolist() == row, "allocator differs from the oracle"
        # seeded history, written into host K/V blocks of the pool (the documented layout), then uploaded
        nblk = pl.block_elems(self.num_pages, H, D)
        kblk = np.full(nblk, 0xFFFF, np.uint16)
        vblk = np.full(nblk, 0xFFFF, np.uint16)
        self.kv = od.ContiguousKV(1, H, D) if build_oracle else None
        for s, c in enumerate(self.ctxs):
            if c == 0:
                continue
            k, v = synth.kv_history(workload, 0, s, c, H, D)
            pl.write_history(kblk, vblk, self.bt[s], k, v, H, D)
            if build_oracle:
                self.kv.preload(0, s, od.widen_bf16(k), od.widen_bf16(v))
        pl.upload_layer(self.pool, 0, kblk, vblk, H, D)
        self.kblk0, self.vblk0 = kblk, vblk
        self.bt_dev = R.dev_i32(self.bt)

    def workspace(self, max_tokens):
        return self.R.Workspace(self.L.llmdec_workspace_bytes(self.cfg, max_tokens, len(self.ctxs), self.max_pages))

    def pool_blocks(self):
        """Host copies of layer 0's K and V blocks (the documented layout: see tests/pool_layout.py)."""
        return pl.host_layer(self.pool, 0, self.shape.n_kv_heads, self.shape.head_dim)
