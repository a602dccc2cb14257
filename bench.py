#!/usr/bin/env python3
"""Throughput of the KV-cached LLaMA-style decoder step on one MI355X.

Headline: greedy decode of the full 32-layer 7B-shaped model (hidden 4096,
32 heads x 128, intermediate 11008, vocab 32000, bf16 weights) over 64
sequences whose cached contexts are seeded uniform in [256, 2048], in a paged
KV pool of 16-token pages.  One step = one call of llmdec_model_step_greedy:
embedding, 32 x (RMSNorm, fused q/k/v projection, RoPE + paged append, paged
decode attention, o projection + residual, RMSNorm, gate/up, silu*up, down +
residual), final RMSNorm, lm_head and argmax; the step's output ids are the
next step's input ids, on the device, with no host synchronisation between
steps.  value = 64 * K / (time of K steps), tokens/s.

Also reported (sub-benchmarks, one layer each): decode at batch 1 over 2048
cached tokens (weights and cache rotated over 4 copies so the 256 MB
last-level cache does not serve them), decode over 32 sequences with contexts
uniform in [128, 4096], a 4 x 512 prefill, and the batch-1 decode again with
group-quantized matrices (8-bit and 4-bit codes, a bf16 scale and a zero point
per 128 inputs), with its four weight products also timed alone, on-device
sampling of 64 x 32000 logits, and the tiny model's decode step enqueued per
step against the same step replayed from a HIP graph.  Each gets its
algorithmic bytes or FLOPs per step and the fraction of the MI355X peak.

Inputs are seeded and synthetic: weights N(0, 0.02^2) in bf16 drawn on the
device, RMSNorm gains 1, cached K/V N(0, 1) in bf16.  Timing uses HIP events
on the stream the library launches on.  The cpu_baseline leg times the CPU
oracle (float64 NumPy) on a bounded sample of the same decode workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only c5,c2,q8,q4,sample,c1,c3,c4]

Profiling helpers (no GPU needed for the two summaries):
  python bench.py --only copy                  1 GiB device copies: calibrates the HBM counters
  python bench.py --pmc-summary FETCH WRITE    traffic summary from two rocprofv3 --pmc runs
  python bench.py --trace-summary DIR          per-kernel table from a rocprofv3 --kernel-trace run
  python bench.py --traffic-table FETCH WRITE  HBM bytes per dispatch of every kernel (two --pmc runs)
  python bench.py --mfma-summary DIR           MFMA busy fraction and issued FLOPs per kernel (one --pmc run)
The roofline's traffic field is read from the committed traffic summary, and
only while the attention sources still hash to the value recorded there.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
ATTN_SOURCES = ("kv_cached_transformer_amd/csrc/kernels_attn.hip", "kv_cached_transformer_amd/csrc/common.h")
TRAFFIC_PROFILE = "profiles/decode_attention_7B-b64-ctx256..2048_traffic.txt"
COPY_BYTES = 1 << 30
MFMA_BF16_PEAK = 2.5e15    # dense bf16 FLOP/s, MI355X
METRIC = "decode tokens/s + % peak HBM BW (7B-shaped, paged KV); prefill tok/s + % MFMA"
SEED = 20261202


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- device set-up helpers
class Dev:
    """Seeded device-side synthetic inputs and library objects for one model shape."""

    def __init__(self, torch, L, R, shape, seed):
        self.torch, self.L, self.R, self.shape = torch, L, R, shape
        self.cfg = L.make_config(shape)
        self.gen = torch.Generator(device="cuda")
        self.gen.manual_seed(seed)

    def normal_bf16(self, rows, cols, std):
        t = self.torch.randn(rows, cols, device="cuda", generator=self.gen, dtype=self.torch.float32)
        return (t * std).to(self.torch.bfloat16)

    def packed_layer(self):
        torch, s = self.torch, self.shape
        ones = torch.ones(s.hidden, device="cuda", dtype=torch.bfloat16)
        mats = {k: self.normal_bf16(r, c, 0.02) for k, (r, c) in s.matrix_shapes().items()}
        w = self.L.llmdec_layer_weights(ones.data_ptr(), mats["wq"].data_ptr(), mats["wk"].data_ptr(),
                                        mats["wv"].data_ptr(), mats["wo"].data_ptr(), ones.data_ptr(),
                                        mats["w_gate"].data_ptr(), mats["w_up"].data_ptr(), mats["w_down"].data_ptr())
        nbytes = self.L.llmdec_packed_layer_bytes(self.cfg)
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = self.L.llmdec_pack_layer(self.cfg, w, buf.data_ptr(), nbytes, self.R.stream())
        torch.cuda.synchronize()
        return buf, st

    def q_matrix(self, rows, cols, bits):
        """Seeded device draws with the host generators' distributions (synth.q8_matrix, synth.q4_matrix):
        codes uniform over their range (a uniform byte is two uniform 4-bit codes), zero points near the
        middle (112..143; 7..8), bf16 scales U(0.75, 1.25) * 0.02 / 74 (4.6 for 4-bit codes), one per 128
        columns."""
        torch = self.torch
        g = (cols + 127) // 128
        nbytes_row = cols if bits == 8 else cols // 2
        codes = torch.randint(0, 256, (rows, nbytes_row), device="cuda", generator=self.gen, dtype=torch.uint8)
        u = torch.rand(rows, g, device="cuda", generator=self.gen, dtype=torch.float32)
        scales = ((0.75 + 0.5 * u) * (0.02 / (74.0 if bits == 8 else 4.6))).to(torch.bfloat16)
        lo, hi = (112, 144) if bits == 8 else (7, 9)
        zeros = torch.randint(lo, hi, (rows, g), device="cuda", generator=self.gen, dtype=torch.uint8)
        keep = (codes, scales, zeros)
        return keep, self.L.llmdec_q8_matrix(*(t.data_ptr() for t in keep))

    def q_layer(self, bits):
        torch, s, L = self.torch, self.shape, self.L
        ones = torch.ones(s.hidden, device="cuda", dtype=torch.bfloat16)
        mats = {k: self.q_matrix(r, c, bits) for k, (r, c) in s.matrix_shapes().items()}
        w = L.llmdec_q8_layer_weights(ones.data_ptr(), *(mats[k][1] for k in ("wq", "wk", "wv", "wo")),
                                      ones.data_ptr(), *(mats[k][1] for k in ("w_gate", "w_up", "w_down")))
        size, pack = ((L.llmdec_q8_packed_layer_bytes, L.llmdec_q8_pack_layer) if bits == 8 else
                      (L.llmdec_q4_packed_layer_bytes, L.llmdec_q4_pack_layer))
        nbytes = size(self.cfg)
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        st = pack(self.cfg, w, buf.data_ptr(), nbytes, self.R.stream())
        torch.cuda.synchronize()
        return buf, st

    def packed_matrix(self, rows, cols):
        torch = self.torch
        m = self.normal_bf16(rows, cols, 0.02)
        nbytes = self.L.llmdec_packed_matrix_bytes(rows, cols)
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.L.llmdec_pack_matrix(rows, cols, m.data_ptr(), buf.data_ptr(), nbytes, self.R.stream())
        torch.cuda.synchronize()
        return buf

    def pool(self, num_pages, free_order):
        """A pool whose every K/V element is N(0,1) bf16 (a 64 MiB seeded block tiled over the buffer)."""
        torch = self.torch
        pool = self.R.Pool(self.cfg, num_pages, free_order)
        flat = pool.buf.view(torch.int16)
        blk = self.normal_bf16(1, 32 << 20, 1.0).view(torch.int16).view(-1)
        n = flat.numel()
        for o in range(0, n, blk.numel()):
            m = min(blk.numel(), n - o)
            flat[o:o + m].copy_(blk[:m])
        torch.cuda.synchronize()
        return pool


def alloc_rows(pool, totals, max_pages):
    import numpy as np
    bt = np.full((len(totals), max_pages), -1, np.int32)
    for s, t in enumerate(totals):
        pool.alloc(int(t), bt[s], 0, max_pages)
    return bt


def time_loop(torch, fn, iters, warmup):
    """Mean ms per call of fn(i) over iters calls after warmup calls, HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def time_dist(torch, fn, iters, warmup):
    """(mean, p10, median, p90) in ms of fn(i), on the current stream.  After warmup calls, the mean comes
    from iters calls between one pair of events; the percentiles from iters more calls with an event
    recorded before every call and after the last (the events between calls add a little time)."""
    import numpy as np
    mean = time_loop(torch, fn, iters, warmup)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record()
    for i in range(iters):
        fn(warmup + iters + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])
    return mean, float(np.percentile(t, 10)), float(np.median(t)), float(np.percentile(t, 90))


def dist_fields(d):
    """The p10 / median / p90 of a time_dist result as sub-benchmark fields (ms)."""
    return {"ms_p10": d[1], "ms_median": d[2], "ms_p90": d[3]}


def attn_alg_bytes(steps, warmup):
    """Algorithmic bytes of one standalone attention call on the decode cache after warmup + steps
    steps: every cached K and V element once (bf16), q read and the output written (fp32)."""
    import numpy as np
    import synth
    shape = synth.LLAMA7B
    B, h = 64, shape.hidden
    ctx = synth.context_lengths(5, B, 256, 2048)
    return float(np.sum(ctx + steps + warmup + 1)) * 2 * h * 2 + 2 * B * h * 4


# ----------------------------------------------------------------------------- the headline: 32-layer decode
def bench_model_decode(torch, L, R, steps, warmup):
    import numpy as np
    import synth
    shape = synth.LLAMA7B
    B = 64
    d = Dev(torch, L, R, shape, SEED + 5)
    log("C5: generating and packing 32 layers of 7B-shaped weights on the device")
    layers = [d.packed_layer() for _ in range(shape.n_layers)]
    embed = d.normal_bf16(shape.vocab, shape.hidden, 0.02)
    fnorm = torch.ones(shape.hidden, device="cuda", dtype=torch.bfloat16)
    head = d.packed_matrix(shape.vocab, shape.hidden)
    mw, keep = L.make_model_weights(embed.data_ptr(), [st for _, st in layers], fnorm.data_ptr(), head.data_ptr())
    ctx = synth.context_lengths(5, B, 256, 2048)
    n_iter = steps + warmup
    totals = ctx + 2 * n_iter + 1  # the eager steps, then as many replayed from a graph
    max_pages = int(max(synth.pages_for(t) for t in totals))
    num_pages = int(sum(synth.pages_for(t) for t in totals))
    log(f"C5: pool of {num_pages} pages ({L.llmdec_kv_pool_bytes(d.cfg, num_pages) / 1e9:.1f} GB), max_pages {max_pages}")
    pool = d.pool(num_pages, synth.free_order(5, num_pages))
    bt = R.dev_i32(alloc_rows(pool, totals, max_pages))
    pos = [R.dev_i32(ctx + i) for i in range(n_iter)]
    toks = [R.dev_i32(synth.first_tokens(5, B, shape.vocab)), torch.empty(B, dtype=torch.int32, device="cuda")]
    ws = R.Workspace(L.llmdec_workspace_bytes(d.cfg, B, B, max_pages))
    strm = R.stream()

    def step(i):
        L.llmdec_model_step_greedy(d.cfg, mw, B, B, 1, toks[i % 2].data_ptr(), None, pos[i].data_ptr(),
                                   bt.data_ptr(), max_pages, pool.handle, toks[(i + 1) % 2].data_ptr(), None,
                                   ws.ptr, ws.nbytes, strm)

    log(f"C5: {warmup} warm-up + {steps} timed greedy steps over {B} sequences")
    ms = time_loop(torch, step, steps, warmup)
    assert ws.error_bits() == 0, "device error word set"
    ids = toks[n_iter % 2].cpu().numpy()
    assert ids.min() >= 0 and ids.max() < shape.vocab
    # algorithmic bytes of one step: every weight once + every cached K/V read once + new K/V written
    h, I, V = shape.hidden, shape.intermediate, shape.vocab
    w_bytes = shape.n_layers * (4 * h * h + 3 * h * I + 2 * h) * 2 + V * h * 2 + h * 2 + B * h * 2
    ctx_mid = ctx + warmup + (steps - 1) / 2.0
    kv_bytes = float(np.sum(ctx_mid + 1)) * shape.n_layers * 2 * h * 2
    step_bytes = w_bytes + kv_bytes
    res = dict(ms_per_step=ms, tokens_per_s=B / (ms * 1e-3), step_bytes=step_bytes,
               hbm_frac=step_bytes / (ms * 1e-3) / HBM_PEAK, weight_bytes=w_bytes, kv_bytes=kv_bytes)

    # dominant kernel, timed on its own through its single-operation entry point on the same cache
    q = torch.randn(B, h, device="cuda", generator=d.gen, dtype=torch.float32)
    out = torch.empty(B, h, device="cuda", dtype=torch.float32)
    ctx_last = R.dev_i32(ctx + n_iter)
    attn_bytes = attn_alg_bytes(steps, warmup)

    def attn(i):
        L.llmdec_op_decode_attention(d.cfg, q.data_ptr(), B, ctx_last.data_ptr(), bt.data_ptr(), max_pages,
                                     pool.handle, i % shape.n_layers, out.data_ptr(), ws.ptr, ws.nbytes, strm)

    a_ms = time_loop(torch, attn, 64, 4)
    res["attn"] = dict(ms=a_ms, bytes=attn_bytes, gbps=attn_bytes / (a_ms * 1e-3) / 1e9)

    # the same step captured once in a HIP graph (the chosen tokens and the positions fed back on the
    # device) and replayed over the next n_iter positions of every sequence
    tok_g = toks[n_iter % 2].clone()
    nxt_g = torch.empty(B, dtype=torch.int32, device="cuda")
    pos_g = R.dev_i32(ctx + n_iter)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.llmdec_model_step_greedy(d.cfg, mw, B, B, 1, tok_g.data_ptr(), None, pos_g.data_ptr(), bt.data_ptr(),
                                   max_pages, pool.handle, nxt_g.data_ptr(), None, ws.ptr, ws.nbytes, R.stream())
        tok_g.copy_(nxt_g)
        pos_g.add_(1)
    g_ms = time_loop(torch, lambda i: g.replay(), steps, warmup)
    assert ws.error_bits() == 0, "device error word set"
    assert torch.equal(pos_g.cpu(), torch.from_numpy((ctx + 2 * n_iter).astype(np.int32))), "graph did not replay"
    res["graph"] = dict(ms_per_step=g_ms, tokens_per_s=B / (g_ms * 1e-3))
    del g
    res["ctx"] = ctx
    del pool, layers, head, embed
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- one-layer sub-benchmarks
def layer_bytes(shape):
    h, I = shape.hidden, shape.intermediate
    return (4 * h * h + 3 * h * I + 2 * h) * 2


def bench_layer_decode(torch, L, R, ctxs, copies, iters, tag, workload):
    import numpy as np
    import synth
    shape = synth.LLAMA7B_LAYER
    d = Dev(torch, L, R, shape, SEED + workload)
    B = len(ctxs)
    ctxs = np.asarray(ctxs, np.int32)
    layers = [d.packed_layer() for _ in range(copies)]
    per_copy = int(sum(synth.pages_for(c + 1) for c in ctxs))
    max_pages = int(max(synth.pages_for(c + 1) for c in ctxs))
    pool = d.pool(per_copy * copies, synth.free_order(workload, per_copy * copies))
    bts = [R.dev_i32(alloc_rows(pool, ctxs + 1, max_pages)) for _ in range(copies)]
    ctx_d = R.dev_i32(ctxs)
    x = torch.randn(B, shape.hidden, device="cuda", generator=d.gen, dtype=torch.float32)
    ws = R.Workspace(L.llmdec_workspace_bytes(d.cfg, B, B, max_pages))
    strm = R.stream()

    def step(i):
        c = i % copies
        L.llmdec_layer_decode(d.cfg, layers[c][1], 0, x.data_ptr(), B, ctx_d.data_ptr(), bts[c].data_ptr(),
                              max_pages, pool.handle, ws.ptr, ws.nbytes, strm)

    dist = time_dist(torch, step, iters, max(10, 2 * copies))
    ms = dist[0]
    assert ws.error_bits() == 0
    kv = float(np.sum(ctxs + 1)) * 2 * shape.hidden * 2
    byt = layer_bytes(shape) + kv + 2 * B * shape.hidden * 4
    log(f"{tag}: {ms * 1e3:.1f} us per layer-step (median {dist[2] * 1e3:.1f}, p10 {dist[1] * 1e3:.1f}, "
        f"p90 {dist[3] * 1e3:.1f}), {byt / (ms * 1e-3) / 1e9:.0f} GB/s")
    return dict(workload=tag, ms_per_layer_step=ms, **dist_fields(dist), layer_steps_per_s=1e3 / ms,
                tokens_per_s=B * 1e3 / ms, algorithmic_bytes=byt, hbm_frac=byt / (ms * 1e-3) / HBM_PEAK)


def q_matrix_bytes(rows, cols, bits):
    """Algorithmic bytes of a group-quantized matrix: bits/8 bytes per code, 4 per group (bf16 scale, zero
    point)."""
    return rows * cols * bits // 8 + rows * ((cols + 127) // 128) * 4


def q_layer_bytes(shape, bits):
    return sum(q_matrix_bytes(r, c, bits) for r, c in shape.matrix_shapes().values()) + 2 * shape.hidden * 2


def bench_layer_decode_q(torch, L, R, ctx, copies, iters, bits):
    """One 7B-shaped layer with group-quantized matrices (8- or 4-bit codes), one sequence, ctx cached
    tokens; weights and cache rotated over `copies` copies.  Also times the layer's four quantized
    products alone."""
    import numpy as np
    import synth
    shape = synth.LLAMA7B_LAYER
    tag = f"7B-layer-decode-q{bits}-b1-ctx{ctx}"
    d = Dev(torch, L, R, shape, SEED + 12 + bits)
    layers = [d.q_layer(bits) for _ in range(copies)]
    per_copy = synth.pages_for(ctx + 1)
    pool = d.pool(per_copy * copies, synth.free_order(12, per_copy * copies))
    bts = [R.dev_i32(alloc_rows(pool, [ctx + 1], per_copy)) for _ in range(copies)]
    ctx_d = R.dev_i32([ctx])
    x = torch.randn(1, shape.hidden, device="cuda", generator=d.gen, dtype=torch.float32)
    ws = R.Workspace(L.llmdec_workspace_bytes(d.cfg, 1, 1, per_copy))
    strm = R.stream()

    decode = L.llmdec_layer_decode_q8 if bits == 8 else L.llmdec_layer_decode_q4
    linear = L.llmdec_op_linear_q8 if bits == 8 else L.llmdec_op_linear_q4

    def step(i):
        c = i % copies
        decode(d.cfg, layers[c][1], 0, x.data_ptr(), 1, ctx_d.data_ptr(), bts[c].data_ptr(), per_copy, pool.handle,
               ws.ptr, ws.nbytes, strm)

    dist = time_dist(torch, step, iters, max(10, 2 * copies))
    ms = dist[0]
    assert ws.error_bits() == 0
    kv = float(ctx + 1) * 2 * shape.hidden * 2
    byt = q_layer_bytes(shape, bits) + kv + 2 * shape.hidden * 4
    log(f"{tag}: {ms * 1e3:.1f} us per layer-step, {byt / (ms * 1e-3) / 1e9:.0f} GB/s")

    # the four products alone (q|k|v, o, [gate; up], down), same rotation
    h, I = shape.hidden, shape.intermediate
    nqkv = 3 * h
    y = torch.randn(I, device="cuda", generator=d.gen, dtype=torch.float32)
    out = torch.empty(2 * I, device="cuda", dtype=torch.float32)

    def products(i):
        st = layers[i % copies][1]
        linear(y.data_ptr(), h, st.w_qkv, nqkv, out.data_ptr(), 0, strm)
        linear(y.data_ptr(), h, st.w_o, h, out.data_ptr(), 0, strm)
        linear(y.data_ptr(), h, st.w_gu, 2 * I, out.data_ptr(), 0, strm)
        linear(y.data_ptr(), I, st.w_down, h, out.data_ptr(), 0, strm)

    pms = time_loop(torch, products, iters, 2 * copies)
    pbyt = q_layer_bytes(shape, bits) - 2 * shape.hidden * 2
    log(f"{tag} products: {pms * 1e3:.1f} us for {pbyt / 1e6:.1f} MB, {pbyt / (pms * 1e-3) / 1e9:.0f} GB/s")
    res = dict(workload=tag, ms_per_layer_step=ms, **dist_fields(dist), layer_steps_per_s=1e3 / ms,
               tokens_per_s=1e3 / ms,
               algorithmic_bytes=byt, hbm_frac=byt / (ms * 1e-3) / HBM_PEAK,
               products=dict(us=pms * 1e3, algorithmic_bytes=pbyt, hbm_frac=pbyt / (pms * 1e-3) / HBM_PEAK))
    del layers, pool
    torch.cuda.empty_cache()
    return res


def bench_sample(torch, L, R, iters):
    """Sampling 64 rows of 32000 logits on the device (temperature 0.8, top-k 50, top-p 0.9), against the
    greedy argmax of the same rows (the choice C5 times)."""
    rows, vocab = 64, 32000
    g = torch.Generator(device="cuda")
    g.manual_seed(SEED + 13)
    logits = torch.randn(rows, vocab, device="cuda", generator=g, dtype=torch.float32) * 2.0
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    strm = R.stream()
    res = {}
    for name, (t, k, p) in (("sample_t0.8_k50_p0.9", (0.8, 50, 0.9)), ("sample_t1_p0.9", (1.0, 0, 0.9)),
                            ("greedy", (0.0, 0, 1.0))):
        def step(i, t=t, k=k, p=p):
            L.llmdec_op_sample(logits.data_ptr(), rows, vocab, L.llmdec_sampling(t, k, p, 7, i), nxt.data_ptr(), strm)
        dist = time_dist(torch, step, iters, 10)
        ms = dist[0]
        res[name] = dict(us=ms * 1e3, us_p10=dist[1] * 1e3, us_median=dist[2] * 1e3, us_p90=dist[3] * 1e3)
        log(f"{name} 64 x 32000: {ms * 1e3:.1f} us (median {dist[2] * 1e3:.1f})")
    return dict(workload="sample-64x32000", **res)


def bench_tiny_graph(torch, L, R, steps):
    """The tiny 2-layer model (C1's shape): greedy decode steps of one sequence after a 32-token prompt,
    each step enqueued from the host, against the same step captured once in a HIP graph and replayed
    (the chosen token and the next position fed back on the device).  Steps this small are bound by
    launch latency, which the graph removes from the host side."""
    import numpy as np
    import synth
    shape = synth.TINY
    d = Dev(torch, L, R, shape, SEED + 1)
    cfg = d.cfg
    layers = [d.packed_layer() for _ in range(shape.n_layers)]
    embed = d.normal_bf16(shape.vocab, shape.hidden, 0.02)
    fnorm = torch.ones(shape.hidden, device="cuda", dtype=torch.bfloat16)
    head = d.packed_matrix(shape.vocab, shape.hidden)
    mw, keep = L.make_model_weights(embed.data_ptr(), [st for _, st in layers], fnorm.data_ptr(), head.data_ptr())
    prompt, total = 32, 32 + 2 * steps + 8
    max_pages = (total + 15) // 16

    def run():
        pool = R.Pool(cfg, max_pages, synth.free_order(1, max_pages))
        row = np.full((1, max_pages), -1, np.int32)
        pool.alloc(total, row[0], 0, max_pages)
        bt = R.dev_i32(row)
        ws = R.Workspace(L.llmdec_workspace_bytes(cfg, prompt, 1, max_pages))
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        toks, cu, sp = R.dev_i32(np.arange(prompt) % shape.vocab), R.dev_i32([0, prompt]), R.dev_i32([0])
        L.llmdec_model_step_greedy(cfg, mw, 1, prompt, prompt, toks.data_ptr(), cu.data_ptr(), sp.data_ptr(),
                                   bt.data_ptr(), max_pages, pool.handle, nxt.data_ptr(), None, ws.ptr, ws.nbytes,
                                   R.stream())
        tok, pos = nxt.clone(), torch.tensor([prompt], dtype=torch.int32, device="cuda")

        def step():
            # the stream is looked up at each call: under capture it is the capturing stream
            L.llmdec_model_step_greedy(cfg, mw, 1, 1, 1, tok.data_ptr(), None, pos.data_ptr(), bt.data_ptr(),
                                       max_pages, pool.handle, nxt.data_ptr(), None, ws.ptr, ws.nbytes, R.stream())
            tok.copy_(nxt)
            pos.add_(1)
        return step, (pool, ws, bt, nxt, toks, cu, sp, tok, pos)

    step, hold = run()
    ms_eager = time_loop(torch, lambda i: step(), steps, 4)
    step2, hold2 = run()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step2()
    ms_graph = time_loop(torch, lambda i: g.replay(), steps, 4)
    # both runs took the same number of steps from the same prompt: the same tokens
    assert torch.equal(hold[3], hold2[3]) and torch.equal(hold[8], hold2[8]), "graph replays diverged from eager steps"
    log(f"tiny 2-layer decode: {ms_eager * 1e3:.1f} us per step enqueued, {ms_graph * 1e3:.1f} us replayed from a graph")
    del hold, hold2, keep, layers
    return dict(workload="tiny-2L-h256-decode-b1", us_per_step_eager=ms_eager * 1e3, us_per_step_graph=ms_graph * 1e3,
                tokens_per_s_eager=1e3 / ms_eager, tokens_per_s_graph=1e3 / ms_graph)


def bench_layer_prefill(torch, L, R, iters):
    import numpy as np
    import synth
    shape = synth.LLAMA7B_LAYER
    d = Dev(torch, L, R, shape, SEED + 4)
    n, plen = 4, 512
    T = n * plen
    keep, w = d.packed_layer()
    max_pages = plen // 16
    pool = d.pool(n * max_pages, synth.free_order(4, n * max_pages))
    bt = R.dev_i32(alloc_rows(pool, [plen] * n, max_pages))
    cu = R.dev_i32(np.arange(n + 1) * plen)
    start = R.dev_i32([0] * n)
    x = torch.randn(T, shape.hidden, device="cuda", generator=d.gen, dtype=torch.float32)
    ws = R.Workspace(L.llmdec_workspace_bytes(d.cfg, T, n, max_pages))
    strm = R.stream()

    def step(i):
        L.llmdec_layer_prefill(d.cfg, w, 0, x.data_ptr(), n, T, plen, cu.data_ptr(), start.data_ptr(), bt.data_ptr(),
                               max_pages, pool.handle, ws.ptr, ws.nbytes, strm)

    dist = time_dist(torch, step, iters, 10)
    ms = dist[0]
    assert ws.error_bits() == 0
    h, I = shape.hidden, shape.intermediate
    gemm_flops = 2.0 * T * (3 * h + h + 2 * I) * h + 2.0 * T * h * I
    attn_flops = 4.0 * n * shape.n_heads * shape.head_dim * (plen * (plen + 1) / 2)
    del keep
    log(f"C4 prefill: {ms * 1e3:.1f} us per layer, {gemm_flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s on the GEMMs")
    return dict(workload="7B-layer-prefill-4x512", ms_per_layer=ms, **dist_fields(dist), tokens_per_s=T * 1e3 / ms,
                gemm_flops=gemm_flops, attn_flops=attn_flops,
                mfma_frac=(gemm_flops + attn_flops) / (ms * 1e-3) / MFMA_BF16_PEAK)


# ----------------------------------------------------------------------------- CPU oracle baseline
def cpu_baseline(ctx):
    """The float64 oracle on a bounded sample of the headline workload: one 7B-shaped layer's decode
    step for 4 of the 64 sequences (the shortest, the longest, two seeded), plus the final norm and
    lm_head for those 4; scaled to tokens/s of the 32-layer model as 4 / (32 t_layer + t_head)."""
    import numpy as np
    import synth
    from oracle import decoder as od
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    shape = synth.LLAMA7B
    order = np.argsort(ctx, kind="stable")
    pick = [int(order[0]), int(order[-1])] + [int(i) for i in synth.rng(5, 99).choice(
        [i for i in range(len(ctx)) if i not in (order[0], order[-1])], 2, replace=False)]
    lw = synth.layer_weights(5, 0, shape)
    kv = od.ContiguousKV(1, shape.n_kv_heads, shape.head_dim)
    for j, s in enumerate(pick):
        k, v = synth.kv_history(5, 0, s, int(ctx[s]), shape.n_kv_heads, shape.head_dim)
        kv.preload(0, j, od.widen_bf16(k), od.widen_bf16(v))
    x = synth.hidden_input(5, len(pick), shape.hidden)
    head = synth.normal_bf16((5, synth.S_LMHEAD), (shape.vocab, shape.hidden), 0.02)
    fnorm = np.full(shape.hidden, synth.BF16_ONE, np.uint16)
    t0 = time.perf_counter()
    y = od.layer_step(shape, lw.tensors, 0, x, list(range(len(pick))), [int(ctx[s]) for s in pick], kv)
    t1 = time.perf_counter()
    logits = od.lm_head_logits(shape, fnorm, head, y)
    t2 = time.perf_counter()
    assert np.all(np.isfinite(logits))
    t_layer, t_head = t1 - t0, t2 - t1
    val = len(pick) / (shape.n_layers * t_layer + t_head)
    return dict(value=val, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=(f"one 7B-shaped layer decode step for 4 of the 64 sequences (contexts "
                        f"{[int(ctx[s]) for s in pick]}) took {t_layer:.2f} s, final norm + lm_head for them "
                        f"{t_head:.2f} s; tokens/s = 4 / (32 * t_layer + t_head)"))


def cpu_configs():
    """The oracle on each workload as the GPU runs it (inputs from the same seeded generators): C1 the whole
    generation (32-token prefill, 15 decode steps), C2 and C3 one layer decode step, C4 one layer prefill;
    C1 and C2 again on one BLAS thread.  Rates: generated tokens/s (C1), layer-steps/s and tokens/s (C2, C3),
    prompt tokens/s (C4)."""
    import numpy as np
    import synth
    from oracle import decoder as od
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threadpool_limits, blas = None, None

    def c1():
        mw = synth.model_weights(1, synth.TINY)
        kv = od.ContiguousKV(synth.TINY.n_layers, synth.TINY.n_kv_heads, synth.TINY.head_dim)
        t0 = time.perf_counter()
        od.greedy_generate(synth.TINY, mw, synth.prompt_ids(1, 32, synth.TINY.vocab), 16, kv)
        return time.perf_counter() - t0

    def layer(workload, ctxs, lens):
        shape = synth.LLAMA7B_LAYER
        lw = synth.layer_weights(workload, 0, shape)
        kv = od.ContiguousKV(1, shape.n_kv_heads, shape.head_dim)
        for s, c in enumerate(ctxs):
            if c:
                k, v = synth.kv_history(workload, 0, s, int(c), shape.n_kv_heads, shape.head_dim)
                kv.preload(0, s, od.widen_bf16(k), od.widen_bf16(v))
        x = synth.hidden_input(workload, int(sum(lens)), shape.hidden)
        seqs = np.repeat(np.arange(len(lens)), lens)
        pos = np.concatenate([np.arange(c, c + n) for c, n in zip(ctxs, lens)])
        t0 = time.perf_counter()
        od.layer_step(shape, lw.tensors, 0, x, seqs, pos, kv)
        return time.perf_counter() - t0

    c2 = lambda: layer(2, [2048], [1])
    ctx3 = synth.context_lengths(3, 32, 128, 4096)
    out = {"affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": blas}
    t = c1()
    out["c1"] = dict(workload="tiny-2L-h256-prefill32-greedy16", s=t, tokens_per_s=16 / t)
    t = c2()
    out["c2"] = dict(workload="7B-layer-decode-b1-ctx2048", s=t, layer_steps_per_s=1 / t)
    t = layer(3, ctx3, [1] * 32)
    out["c3"] = dict(workload="7B-layer-decode-b32-ctx128..4096", s=t, layer_steps_per_s=1 / t, tokens_per_s=32 / t)
    t = layer(4, [0] * 4, [512] * 4)
    out["c4"] = dict(workload="7B-layer-prefill-4x512", s=t, tokens_per_s=2048 / t)
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            t1, t2 = c1(), c2()
        out["c1"]["one_thread"] = dict(s=t1, tokens_per_s=16 / t1)
        out["c2"]["one_thread"] = dict(s=t2, layer_steps_per_s=1 / t2)
    return out


# ----------------------------------------------------------------------------- main
# ----------------------------------------------------------------------------- counter calibration and summaries
def bench_copy(torch):
    """Three copies of a 1 GiB float tensor: a plain stream of known bytes for the HBM counters."""
    a = torch.ones(COPY_BYTES // 4, device="cuda", dtype=torch.float32)
    b = torch.empty_like(a)
    ms = time_loop(torch, lambda i: b.copy_(a), 3, 1)
    log(f"copy: {COPY_BYTES} bytes read + written in {ms * 1e3:.1f} us ({2 * COPY_BYTES / (ms * 1e-3) / 1e9:.0f} GB/s)")


def sources_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _pmc_rows(d, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    return rows


def _per_dispatch(rows, name_part, last=64):
    """Mean counter value (KiB) over the last `last` dispatches of the named kernel (the standalone
    attention calls, which follow the model steps); None where the run has no dispatch of it."""
    sel = sorted((r for r in rows if name_part in r["Kernel_Name"]), key=lambda r: int(r["Dispatch_Id"]))[-last:]
    if not sel:
        return None
    vals = [float(r["Counter_Value"]) for r in sel]
    return sum(vals) / len(vals), len(vals), sel[-1]["Grid_Size"]


def pmc_summary(fetch_dir, write_dir):
    """Print the traffic summary committed under profiles/ from a FETCH_SIZE run and a WRITE_SIZE run of
    `bench.py --only c5,copy --no-cpu` with the default --steps 10 --warmup 3."""
    fr, wr = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")
    copy_f = max(float(r["Counter_Value"]) for r in fr if "copy" in r["Kernel_Name"].lower())
    copy_w = max(float(r["Counter_Value"]) for r in wr if "copy" in r["Kernel_Name"].lower())
    kf, kw = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
    out = ["# HBM traffic per call of llmdec_op_decode_attention on the 64-sequence decode cache (7B shapes,",
           "# contexts 256..2048 after the default 3 + 10 steps): the partition kernel, plus the combine kernel",
           "# where some sequence spans several blocks (none does at these contexts: it is not launched).",
           "# Counters are KiB per dispatch; each is scaled by what it reads for a 1 GiB device copy.",
           "# Commands (from /tmp, committed files only), then the summary:",
           "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <F> -o p -- python3 <repo>/bench.py --only c5,copy --no-cpu",
           "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <W> -o p -- python3 <repo>/bench.py --only c5,copy --no-cpu",
           "#   python3 bench.py --pmc-summary <F> <W>",
           f"sources_sha256: {sources_hash()}",
           f"copy_fetch_kib: {copy_f:.1f}  fetch_scale: {kf:.4f}",
           f"copy_write_kib: {copy_w:.1f}  write_scale: {kw:.4f}"]
    total = 0.0
    for name in ("decode_attn_kernel<128,", "decode_combine_kernel<128>"):
        pf, pw = _per_dispatch(fr, name), _per_dispatch(wr, name)
        if pf is None or pw is None:
            if name.startswith("decode_attn"):
                raise SystemExit(f"no dispatch of {name}")
            out.append(f"{name}: not launched")
            continue
        (f, nf, grid), (w, nw, _) = pf, pw
        b = f * 1024 * kf + w * 1024 * kw
        total += b
        out.append(f"{name.rstrip(',')}: grid {grid}: FETCH_SIZE {f:.1f} KiB ({nf} dispatches), WRITE_SIZE {w:.1f} KiB "
                   f"({nw}) -> {b / 1e6:.2f} MB")
    alg = attn_alg_bytes(10, 3)
    out.append(f"algorithmic_bytes_per_call: {alg:.0f}")
    out.append(f"traffic_bytes_per_call: {total:.0f}  (x{total / alg:.3f} the algorithmic bytes)")
    out.append("# Every kernel of the run with at least 1% of its traffic, bytes per dispatch (the run holds the")
    out.append("# 13 model steps, the standalone attention calls, the 13 graph-replayed steps and the weight setup):")
    out += traffic_table(fetch_dir, write_dir)[2:]  # without the calibration lines, printed above
    print("\n".join(out))


def traffic_table(fetch_dir, write_dir, min_share=0.01):
    """HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, each scaled by the 1 GiB copy's reading) of every
    kernel, grouped by name and grid, over all of a run's dispatches; kernels under min_share of the
    run's traffic are left out."""
    import collections
    fr, wr = _pmc_rows(fetch_dir, "FETCH_SIZE"), _pmc_rows(write_dir, "WRITE_SIZE")
    copy_f = max(float(r["Counter_Value"]) for r in fr if "copy" in r["Kernel_Name"].lower())
    copy_w = max(float(r["Counter_Value"]) for r in wr if "copy" in r["Kernel_Name"].lower())
    kf, kw = COPY_BYTES / (copy_f * 1024), COPY_BYTES / (copy_w * 1024)
    agg = collections.defaultdict(lambda: [0.0, 0, 0.0, 0])
    for rows, i, k in ((fr, 0, kf), (wr, 2, kw)):
        for r in rows:
            if "copy" in r["Kernel_Name"].lower():
                continue
            key = (r["Kernel_Name"].split("(")[0].replace("void ", "")[:52], r["Grid_Size"])
            agg[key][i] += float(r["Counter_Value"]) * 1024 * k
            agg[key][i + 1] += 1
    total = sum(v[0] + v[2] for v in agg.values())
    out = [f"copy_fetch_kib: {copy_f:.1f}  fetch_scale: {kf:.4f}", f"copy_write_kib: {copy_w:.1f}  write_scale: {kw:.4f}",
           f"{'kernel':52s} {'grid':>9s} {'dispatches':>10s} {'MB read':>9s} {'MB written':>10s}  (per dispatch)"]
    for (name, grid), v in sorted(agg.items(), key=lambda kv: -(kv[1][0] + kv[1][2])):
        if v[0] + v[2] < min_share * total or not v[1] or not v[3]:
            continue
        out.append(f"{name:52s} {grid:>9s} {v[1]:10d} {v[0] / v[1] / 1e6:9.2f} {v[2] / v[3] / 1e6:10.2f}")
    return out


def mfma_summary(d):
    """MFMA use per kernel from a rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16,
    SQ_INSTS_VALU_MFMA_MOPS_BF16 and GRBM_GUI_ACTIVE: busy = MFMA busy cycles / (1024 SIMDs x GUI-active
    cycles, summed over the 8 XCDs), issued FLOPs = 512 x MOPS, and the issued rate over the dispatch's
    duration."""
    import collections
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    durs = collections.defaultdict(dict)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"].split("(")[0].replace("void ", "")[:52], r["Grid_Size"])
                agg[key][r["Counter_Name"]] += float(r["Counter_Value"])
                durs[key][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    print(f"{'kernel':52s} {'grid':>9s} {'calls':>5s} {'avg us':>8s} {'MFMA busy':>9s} {'GFLOP issued':>12s} "
          f"{'TFLOP/s issued':>14s}")
    for key, c in sorted(agg.items(), key=lambda kv: -sum(durs[kv[0]].values())):
        ops = c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        n = len(durs[key])
        if not ops or not n:
            continue
        t = sum(durs[key].values()) / n
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / n
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n / (1024 * gui / 8) if gui else float("nan")
        flop = 512 * ops / n
        print(f"{key[0]:52s} {key[1]:>9s} {n:5d} {t * 1e6:8.1f} {busy:9.3f} {flop / 1e9:12.1f} {flop / t / 1e12:14.1f}")


def read_traffic(attn_bytes_now):
    """HBM bytes per attention call from the committed summary, scaled to this run's cache (the bytes
    grow with the context, which depends on --steps/--warmup), or None when the sources changed."""
    try:
        with open(os.path.join(ROOT, TRAFFIC_PROFILE)) as fh:
            kv = dict(line.split(": ", 1) for line in fh.read().splitlines() if ": " in line and not line.startswith("#"))
        if kv.get("sources_sha256", "").strip() != sources_hash():
            return None
        traffic = float(kv["traffic_bytes_per_call"].split()[0])
        alg = float(kv.get("algorithmic_bytes_per_call", "0").split()[0]) or None
        return traffic * (attn_bytes_now / alg) if alg else traffic
    except (OSError, KeyError, ValueError):
        return None


def trace_summary(d):
    """Per-kernel table (calls, mean and total time) from a rocprofv3 --kernel-trace --stats run."""
    import collections
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    agg = collections.defaultdict(list)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].split("(")[0].replace("void ", "")[:58]
                grid = f'{r["Grid_Size_X"]}x{r["Grid_Size_Y"]}x{r["Grid_Size_Z"]}'
                agg[(name, grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in agg.values())
    print(f"{'kernel':58s} {'grid':>18s} {'calls':>6s} {'avg us':>9s} {'total ms':>9s} {'%':>6s}")
    for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        if sum(v) < 0.002 * total:
            continue
        print(f"{name:58s} {grid:>18s} {len(v):6d} {sum(v) / len(v):9.1f} {sum(v) / 1e3:9.2f} {100 * sum(v) / total:6.2f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default="c5,c2,q8,q4,sample,c1,c3,c4", help="comma list of workloads to run (also: copy)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the attention traffic summary from two rocprofv3 --pmc output folders")
    ap.add_argument("--trace-summary", metavar="DIR", help="print a per-kernel table from a rocprofv3 kernel trace")
    ap.add_argument("--traffic-table", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per dispatch of every kernel from two rocprofv3 --pmc output folders")
    ap.add_argument("--mfma-summary", metavar="DIR", help="print MFMA use per kernel from a rocprofv3 --pmc run")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.traffic_table:
        print("\n".join(traffic_table(*args.traffic_table)))
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decoder step has no multi-GPU path)", file=sys.stderr, flush=True)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only; WORLD_SIZE > 1 is not supported", file=sys.stderr, flush=True)
        sys.exit(2)
    import numpy as np  # noqa: F401
    import torch
    from kv_cached_transformer_amd import llmdec as L
    from kv_cached_transformer_amd import runtime as R
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    L.lib()
    only = set(args.only.split(","))
    extra = {}
    head = None
    if "c5" in only:
        head = bench_model_decode(torch, L, R, args.steps, args.warmup)
        log(f"C5: {head['ms_per_step']:.2f} ms/step, {head['tokens_per_s']:.0f} tokens/s, "
            f"{head['hbm_frac'] * 100:.1f}% of HBM peak; decode attention {head['attn']['ms'] * 1e3:.0f} us "
            f"= {head['attn']['gbps']:.0f} GB/s; replayed from a graph {head['graph']['ms_per_step']:.2f} ms/step")
        extra["decode_step_graph"] = dict(workload="7B-32L-decode-b64-ctx256..2048, one step captured in a HIP graph",
                                          **head["graph"])
    if "c2" in only:
        extra["decode_b1_ctx2048"] = bench_layer_decode(torch, L, R, [2048], 4, 100, "7B-layer-decode-b1-ctx2048", 2)
    if "q8" in only:
        extra["decode_q8_b1_ctx2048"] = bench_layer_decode_q(torch, L, R, 2048, 4, 100, 8)
    if "q4" in only:
        extra["decode_q4_b1_ctx2048"] = bench_layer_decode_q(torch, L, R, 2048, 4, 100, 4)
    if "c1" in only:
        extra["tiny_decode_graph"] = bench_tiny_graph(torch, L, R, 20)
    if "sample" in only:
        extra["sample_64x32000"] = bench_sample(torch, L, R, 50)
    if "c3" in only:
        import synth
        extra["decode_b32_ctx128..4096"] = bench_layer_decode(torch, L, R, synth.context_lengths(3, 32, 128, 4096), 1,
                                                              50, "7B-layer-decode-b32-ctx128..4096", 3)
    if "c4" in only:
        extra["prefill_4x512"] = bench_layer_prefill(torch, L, R, 20)
    if "copy" in only:
        bench_copy(torch)
    cpu = None
    if head is not None and not args.no_cpu:
        log("cpu_baseline: timing the oracle on a 4-sequence sample")
        cpu = cpu_baseline(head["ctx"])
        log("cpu_baseline: timing the oracle on the one-layer and tiny workloads")
        cpu["configs"] = cpu_configs()
        cpu["affinity_cores"] = cpu["configs"]["affinity_cores"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"] if head else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "7B-32L-decode-b64-ctx256..2048", "layers": 32, "hidden": 4096, "heads": 32,
                   "head_dim": 128, "intermediate": 11008, "vocab": 32000, "batch": 64, "page_size": 16,
                   "ctx_range": [256, 2048]},
    }
    if head:
        a = head["attn"]
        line["hbm_frac_step"] = head["hbm_frac"]
        line["roofline"] = {"bound": "hbm",
                            "kernel": "paged decode attention, one layer, 64 sequences (partition kernel; the combine "
                                      "kernel only where a sequence spans several blocks)",
                            "achieved": a["gbps"], "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": a["gbps"] * 1e9 / HBM_PEAK, "traffic": read_traffic(a["bytes"]),
                            "algorithmic_bytes": a["bytes"], "us_per_call": a["ms"] * 1e3}
    line["cpu_baseline"] = cpu
    line["sub_benchmarks"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
