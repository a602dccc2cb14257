"""A decode step captured in a HIP graph and replayed, against the same steps run eagerly.

The library allocates nothing, never synchronises and enqueues only kernels in a step, so a caller can
capture llmdec_model_step_greedy (here with torch.cuda.graph, together with the two small torch ops
that feed the chosen token and the next position back) and replay it: generation then runs on the
device with one launch per token.  Each replay is checked against the eager step with the same
inputs, bit for bit (the same kernels in the same order), with eager work and synchronisation between
the replays.
"""
import numpy as np
import pytest

import synth
from oracle import decoder as od
from tests.gpu_util import assert_close, banner

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


class Run:
    """Prompt prefill of the tiny model into a pool, then device-resident decode inputs."""

    def __init__(self, L, R, dm, prompt, n_steps):
        shape = synth.TINY
        self.L, self.R, self.dm = L, R, dm
        total = len(prompt) + n_steps
        self.max_pages = (total + 15) // 16 + 1
        order = synth.free_order(1, self.max_pages)
        self.pool = R.Pool(dm.cfg, self.max_pages, order, fill_bits=0xFFFF)
        row = np.full((1, self.max_pages), -1, np.int32)
        self.pool.alloc(total, row[0], 0, self.max_pages)  # every page the run will need, allocated up front
        self.bt = R.dev_i32(row)
        self.ws = R.Workspace(L.llmdec_workspace_bytes(dm.cfg, len(prompt), 1, self.max_pages))
        self.nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        self.logits = torch.empty(1, shape.vocab, dtype=torch.float32, device="cuda")
        toks, cu, sp = R.dev_i32(prompt), R.dev_i32([0, len(prompt)]), R.dev_i32([0])
        L.llmdec_model_step_greedy(dm.cfg, dm.struct, 1, len(prompt), len(prompt), toks.data_ptr(), cu.data_ptr(),
                                   sp.data_ptr(), self.bt.data_ptr(), self.max_pages, self.pool.handle,
                                   self.nxt.data_ptr(), self.logits.data_ptr(), self.ws.ptr, self.ws.nbytes,
                                   R.stream())
        torch.cuda.synchronize()
        self.first_logits = self.logits.cpu().numpy()[0].copy()
        self.tok = self.nxt.clone()                               # the token fed to the next step
        self.pos = torch.tensor([len(prompt)], dtype=torch.int32, device="cuda")

    def step(self):
        """One decode step, then feed the chosen token and the next position back (all enqueued)."""
        L, R, dm = self.L, self.R, self.dm
        L.llmdec_model_step_greedy(dm.cfg, dm.struct, 1, 1, 1, self.tok.data_ptr(), None, self.pos.data_ptr(),
                                   self.bt.data_ptr(), self.max_pages, self.pool.handle, self.nxt.data_ptr(),
                                   self.logits.data_ptr(), self.ws.ptr, self.ws.nbytes, R.stream())
        self.tok.copy_(self.nxt)
        self.pos.add_(1)


def test_graph_replayed_decode_steps_match_eager(L, R):
    from tests.test_gpu_model import DeviceModel
    banner("tiny model: 12 decode steps eager vs replayed from one captured step")
    mw = synth.model_weights(1, synth.TINY)
    dm = DeviceModel(L, R, mw)
    prompt = synth.prompt_ids(1, 32, synth.TINY.vocab)
    n = 12
    eager = Run(L, R, dm, prompt, n)
    ref_logits, ref_ids = [], []
    for _ in range(n):
        eager.step()
        torch.cuda.synchronize()
        ref_logits.append(eager.logits.cpu().numpy()[0].copy())
        ref_ids.append(int(eager.nxt.cpu().numpy()[0]))
    assert eager.ws.error_bits() == 0

    run = Run(L, R, dm, prompt, n)
    assert np.array_equal(run.first_logits, eager.first_logits)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.step()
    # the capture ran nothing: the inputs still hold the first decode step's token and position
    torch.cuda.synchronize()
    assert int(run.pos.cpu().numpy()[0]) == 32
    for i in range(n):
        g.replay()
        torch.cuda.synchronize()
        got = run.logits.cpu().numpy()[0]
        assert np.array_equal(got, ref_logits[i]), f"replay {i}: logits differ from the eager step"
        assert int(run.nxt.cpu().numpy()[0]) == ref_ids[i]
        assert int(run.pos.cpu().numpy()[0]) == 33 + i
        _ = torch.ones(256, device="cuda").sum().item()  # unrelated eager work between replays
    assert run.ws.error_bits() == 0
    # and the last replay's logits against the oracle fed the same tokens
    kv = od.ContiguousKV(synth.TINY.n_layers, synth.TINY.n_kv_heads, synth.TINY.head_dim)
    feed = list(prompt)
    od.model_step(synth.TINY, mw, feed, [0] * 32, list(range(32)), kv)
    toks = [int(eager.first_logits.argmax())] + ref_ids
    for i in range(n):
        ref, _ = od.model_step(synth.TINY, mw, [toks[i]], [0], [32 + i], kv)
    assert_close("tiny graph replay, last step logits", ref_logits[-1], ref[0])
