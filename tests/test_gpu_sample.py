"""Sampling on the device against oracle.sampling on the same Philox draws.

Every row's token must hold the draw: it is a kept token whose cumulative-probability interval
contains u to within MARGIN (1e-5, several times the device's fp32 summation error over 32768 terms).
Where the oracle's own decision is farther than MARGIN from every boundary that fp32 sums could cross
(u against the cumulative probabilities of the kept tokens; with top-p, the sorted cumulative sum
against p at the cut) the token must equal the oracle's exactly; with tens of thousands of tokens and
no truncation most rows lie that close to some boundary, which is why the interval check applies to
all.  The top-k set itself is exact (it compares logits, the same fp32 values on both sides), and
temperature 0 is the greedy choice, exact.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import decoder as od
from oracle import pages as op
from oracle import sampling as osm
from tests.gpu_util import assert_close, banner

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MARGIN = 1e-5


@pytest.fixture(scope="module")
def L():
    from kv_cached_transformer_amd import llmdec
    llmdec.lib()
    return llmdec


@pytest.fixture(scope="module")
def R():
    from kv_cached_transformer_amd import runtime
    return runtime


def decision_margin(z, T, top_k, top_p, u):
    """Distance of the oracle's decision from the nearest boundary that rounding could cross."""
    if T <= 0:
        return np.inf
    ids, w = osm.kept_tokens(z, T, top_k, top_p)
    m = float(np.min(np.abs(np.cumsum(w) - u)))
    if top_p < 1.0:
        zz = np.asarray(z, np.float64)
        e = np.exp((zz - zz.max()) / T)
        if 0 < top_k < zz.size:
            e = np.where(zz >= np.sort(zz)[::-1][top_k - 1], e, 0.0)
        q = np.sort(e / e.sum())[::-1]
        cum = np.cumsum(q)
        n = int(np.searchsorted(cum, top_p, side="left"))
        near = [abs(cum[n] - top_p)] + ([abs(cum[n - 1] - top_p)] if n > 0 else [])
        m = min(m, float(min(near)))
    return m


def consistent(z, T, top_k, top_p, u, tok):
    """The device's token is one whose cumulative-probability interval holds u to within MARGIN, for the
    oracle's kept set (or, near the top-p cut, the kept set of p -/+ MARGIN)."""
    if T <= 0:
        return tok == osm.sample(z, T, top_k, top_p, u)
    for pp in [top_p] + ([max(top_p - MARGIN, 1e-12), min(top_p + MARGIN, 1.0)] if top_p < 1.0 else []):
        ids, w = osm.kept_tokens(z, T, top_k, pp)
        hit = np.nonzero(ids == tok)[0]
        if hit.size:
            c = np.cumsum(w)
            j = int(hit[0])
            lo = c[j - 1] if j else 0.0
            if lo - MARGIN <= u < c[j] + MARGIN:
                return True
    return False


def check_rows(tag, logits, got, T, top_k, top_p, seed, step):
    near = 0
    for r in range(logits.shape[0]):
        u = osm.uniform(seed, step, r)
        z = logits[r].astype(np.float64)
        ref = osm.sample(z, T, top_k, top_p, u)
        tok = int(got[r])
        assert consistent(z, T, top_k, top_p, u, tok), f"{tag} row {r}: {tok} does not hold u={u} (oracle {ref})"
        if decision_margin(z, T, top_k, top_p, u) > MARGIN:
            assert tok == ref, f"{tag} row {r}: device {tok} oracle {ref} (u={u})"
        else:
            near += 1
    print(f"[parity] {tag}: {logits.shape[0]} rows, {near} within {MARGIN} of a boundary "
          f"(checked as consistent with u), the rest equal to the oracle", flush=True)


PARAMS = [(0.0, 0, 1.0), (1.0, 0, 1.0), (0.7, 40, 1.0), (1.3, 0, 0.9), (0.8, 50, 0.5), (1.0, 1, 1.0),
          (1.0, 0, 1e-6), (2.0, 1000, 0.95)]


@pytest.mark.parametrize("rows,vocab,scale", [(64, 32000, 2.0), (16, 1024, 1.0), (7, 1000, 3.0), (3, 32768, 2.0),
                                              (5, 37, 1.0), (2, 1, 1.0)])
def test_sample_matches_oracle(L, R, rows, vocab, scale):
    logits = (synth.rng(70, rows, vocab).standard_normal((rows, vocab)) * scale).astype(np.float32)
    ld = R.dev_f32(logits)
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    for i, (T, k, p) in enumerate(PARAMS):
        seed, step = 1234 + i, (i << 33) + 5
        banner(f"sample rows={rows} vocab={vocab} T={T} top_k={k} top_p={p}")
        params = L.llmdec_sampling(T, k, p, seed, step)
        L.llmdec_op_sample(ld.data_ptr(), rows, vocab, params, nxt.data_ptr(), R.stream())
        torch.cuda.synchronize()
        got = nxt.cpu().numpy()
        check_rows(f"sample {rows}x{vocab} T={T} k={k} p={p}", logits, got, T, k, p, seed, step)
        # the same call again gives the same tokens
        L.llmdec_op_sample(ld.data_ptr(), rows, vocab, params, nxt.data_ptr(), R.stream())
        torch.cuda.synchronize()
        assert np.array_equal(nxt.cpu().numpy(), got)


def test_sample_repeatable(L, R):
    """The same logits, parameters, seed and step give the same tokens on every call: the top-p cut sums
    masses in a fixed order (per-wave histograms added in wave order), as does the draw."""
    rows, vocab = 64, 32000
    logits = (synth.rng(72, rows, vocab).standard_normal((rows, vocab)) * 2.0).astype(np.float32)
    ld = R.dev_f32(logits)
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    for T, k, p in [(1.0, 0, 0.9), (0.8, 50, 0.9), (1.3, 0, 0.5)]:
        banner(f"sample repeatability T={T} top_k={k} top_p={p}")
        params = L.llmdec_sampling(T, k, p, 4242, 17)
        first = None
        for _ in range(20):
            L.llmdec_op_sample(ld.data_ptr(), rows, vocab, params, nxt.data_ptr(), R.stream())
            torch.cuda.synchronize()
            got = nxt.cpu().numpy().copy()
            if first is None:
                first = got
                check_rows(f"repeatable T={T} k={k} p={p}", logits, got, T, k, p, 4242, 17)
            assert np.array_equal(got, first)


def test_sample_ties_and_greedy_ties(L, R):
    """Three equal largest logits: greedy takes the lowest index; top_k = 2 keeps all three (ties with the
    k-th stay) and the draws over many steps reach each of them and nothing else."""
    vocab, rows = 4096, 64
    logits = (synth.rng(71).standard_normal((rows, vocab))).astype(np.float32)
    logits[:, [100, 2000, 4000]] = 9.0
    ld = R.dev_f32(logits)
    nxt = torch.empty(rows, dtype=torch.int32, device="cuda")
    L.llmdec_op_sample(ld.data_ptr(), rows, vocab, L.llmdec_sampling(0.0, 0, 1.0, 0, 0), nxt.data_ptr(), R.stream())
    torch.cuda.synchronize()
    assert np.all(nxt.cpu().numpy() == 100)
    seen = set()
    for step in range(4):
        params = L.llmdec_sampling(1.0, 2, 1.0, 99, step)
        L.llmdec_op_sample(ld.data_ptr(), rows, vocab, params, nxt.data_ptr(), R.stream())
        torch.cuda.synchronize()
        got = nxt.cpu().numpy()
        check_rows(f"ties step {step}", logits, got, 1.0, 2, 1.0, 99, step)
        seen |= set(got.tolist())
    assert seen == {100, 2000, 4000}


def test_sample_rejects_bad_parameters(L, R):
    ld = R.dev_f32(np.zeros((1, 64), np.float32))
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for params, vocab in [(L.llmdec_sampling(1.0, 0, 0.0, 0, 0), 64), (L.llmdec_sampling(1.0, 0, 1.5, 0, 0), 64),
                          (L.llmdec_sampling(float("nan"), 0, 1.0, 0, 0), 64), (L.llmdec_sampling(1.0, 0, 1.0, 0, 0),
                                                                                 40000)]:
        with pytest.raises(L.LlmdecError) as e:
            L.llmdec_op_sample(ld.data_ptr(), 1, vocab, params, nxt.data_ptr(), R.stream())
        assert e.value.status == L.LLMDEC_E_INVALID


def test_tiny_model_sampled_generation(L, R):
    """A prompt and 7 decode steps of the tiny model with llmdec_model_step_sample: the logits against the
    oracle's at every step (the oracle fed the same tokens), and each drawn token against the oracle's
    sampler applied to the device's logits with the same draw."""
    from tests.test_gpu_model import DeviceModel
    shape = dataclasses.replace(synth.TINY)
    mw = synth.model_weights(1, shape)
    dm = DeviceModel(L, R, mw)
    prompt = synth.prompt_ids(1, 32, shape.vocab)
    num_pages = max_pages = 4
    order = synth.free_order(1, num_pages)
    pool = R.Pool(dm.cfg, num_pages, order)
    row = np.full((1, max_pages), -1, np.int32)
    ws = R.Workspace(L.llmdec_workspace_bytes(dm.cfg, 32, 1, max_pages))
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(1, shape.vocab, dtype=torch.float32, device="cuda")
    kv = od.ContiguousKV(shape.n_layers, shape.n_kv_heads, shape.head_dim)
    feed, pos0, npg = list(prompt), 0, 0
    T_, k_, p_, seed = 0.9, 50, 0.9, 777
    for step in range(8):
        banner(f"tiny sampled step {step}")
        T = len(feed)
        npg = pool.alloc(pos0 + T, row[0], npg, max_pages)
        bt, toks, sp = R.dev_i32(row), R.dev_i32(feed), R.dev_i32([pos0])
        params = L.llmdec_sampling(T_, k_, p_, seed, step)
        cu = R.dev_i32([0, T]) if step == 0 else None
        L.llmdec_model_step_sample(dm.cfg, dm.struct, 1, T, T, toks.data_ptr(), cu.data_ptr() if cu is not None else None,
                                   sp.data_ptr(), bt.data_ptr(), max_pages, pool.handle, params, nxt.data_ptr(),
                                   logits.data_ptr(), ws.ptr, ws.nbytes, R.stream())
        torch.cuda.synchronize()
        ref_logits, _ = od.model_step(shape, mw, feed, [0] * T, list(range(pos0, pos0 + T)), kv)
        got = logits.cpu().numpy()
        assert_close(f"tiny sampled step {step} logits", got[0], ref_logits[0])
        tok = nxt.cpu().numpy()
        check_rows(f"tiny sampled step {step}", got, tok, T_, k_, p_, seed, step)
        pos0 += T
        feed = [int(tok[0])]
    assert ws.error_bits() == 0
    assert op.pages_needed(pos0) <= npg
