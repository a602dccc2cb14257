"""Set-up shared by the layer-level GPU tests and the benchmark: a packed layer,
a pool holding a seeded cache history, block tables from the library's
allocator, and the matching oracle cache."""
import numpy as np

import synth
from oracle import decoder as od
from oracle import pages as op


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
        # seeded history, written into a host image of the pool, then uploaded
        kimg = np.full((self.num_pages, H, 16, D), 0xFFFF, np.uint16)
        vimg = np.full((self.num_pages, H, D, 16), 0xFFFF, np.uint16)
        self.kv = od.ContiguousKV(1, H, D) if build_oracle else None
        for s, c in enumerate(self.ctxs):
            if c == 0:
                continue
            k, v = synth.kv_history(workload, 0, s, c, H, D)
            synth.scatter_kv_into_pool(kimg, vimg, self.bt[s], k, v)
            if build_oracle:
                self.kv.preload(0, s, od.widen_bf16(k), od.widen_bf16(v))
        kd, vd = self.pool.layer_views(0)
        kd.copy_(torch.from_numpy(kimg.view(np.int16)).to("cuda"))
        vd.copy_(torch.from_numpy(R.Pool.v_raw(vimg).view(np.int16)).to("cuda"))
        self.kimg0, self.vimg0 = kimg, vimg
        self.bt_dev = R.dev_i32(self.bt)

    def workspace(self, max_tokens):
        return self.R.Workspace(self.L.llmdec_workspace_bytes(self.cfg, max_tokens, len(self.ctxs), self.max_pages))

    def pool_images(self):
        """Host images of layer 0: K [pages][H][16][D], V [pages][H][D][16] (dim, in-page offset)."""
        k, v = self.pool.layer_views(0)
        return self.R.host_u16(k.contiguous()), self.R.Pool.v_logical(self.R.host_u16(v.contiguous()))
