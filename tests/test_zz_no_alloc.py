"""The greedy model step without a workspace argument (llmdec_model_step_greedy_noalloc) against the same
step with one (llmdec_model_step_greedy).

The entry point is for callers that cannot allocate: its workspace is a static device array of the
library.  Two calls in a row on the tiny 2-layer model, a 32-token prompt prefill and then a one-token
decode step (the smaller input, run on the array as the first call left it), must give the same next
tokens, the same logits and the same KV pool contents, bit for bit, as the workspace step on an
identical pool, and report no device error.  A step whose workspace would not fit the array is
refused with E_WORKSPACE before anything is launched.
"""
import numpy as np
import pytest

import synth

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


class TinyModel:
    def __init__(self, L, R, seed):
        self.shape = synth.TINY
        mw = synth.model_weights(seed, self.shape)
        self.cfg = L.make_config(self.shape)
        self.layers = [R.PackedLayer(self.cfg, lw.tensors) for lw in mw.layers]
        self.embed = R.dev_u16(mw.embed)
        self.final_norm = R.dev_u16(mw.final_norm)
        self.lm_head = R.PackedMatrix(self.shape.vocab, self.shape.hidden, mw.lm_head)
        self.struct, self._keep = L.make_model_weights(self.embed.data_ptr(), [p.struct for p in self.layers],
                                                       self.final_norm.data_ptr(), self.lm_head.ptr)


def test_noalloc_step_matches_workspace_step(L, R):
    m = TinyModel(L, R, 11)
    vocab, P = m.shape.vocab, 4
    # two identical pools, every byte preset to the same pattern so that untouched slots compare too
    pools = [R.Pool(m.cfg, P, synth.free_order(5, P), fill_bits=0x7f11) for _ in range(2)]
    rows = []
    for pool in pools:
        row = np.full((1, P), -1, np.int32)
        pool.alloc(33, row[0], 0, P)
        rows.append(row)
    assert np.array_equal(rows[0], rows[1])
    bt = R.dev_i32(rows[0])
    ws = R.Workspace(L.llmdec_workspace_bytes(m.cfg, 32, 1, P))
    err = torch.full((1,), 0x5a5a5a5a, dtype=torch.int32, device="cuda")
    prompt = synth.prompt_ids(7, 32, vocab)

    # call 1: prefill of the 32-token prompt; call 2: one decode token at position 32
    steps = [dict(n_tokens=32, max_q_len=32, tokens=prompt, cu=[0, 32], start=[0])]
    next_token = None
    for call in range(2):
        if call == 1:
            steps.append(dict(n_tokens=1, max_q_len=1, tokens=[next_token], cu=None, start=[32]))
        st = steps[call]
        print(f"[no-alloc] call {call + 1}: n_tokens={st['n_tokens']}", flush=True)
        tok = R.dev_i32(st["tokens"])
        cu = R.dev_i32(st["cu"]) if st["cu"] is not None else None
        sp = R.dev_i32(st["start"])
        out = []
        for which, pool in enumerate(pools):
            nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            lg = torch.full((1, vocab), float("nan"), dtype=torch.float32, device="cuda")
            args = (m.cfg, m.struct, 1, st["n_tokens"], st["max_q_len"], tok.data_ptr(),
                    cu.data_ptr() if cu is not None else None, sp.data_ptr(), bt.data_ptr(), P, pool.handle,
                    nxt.data_ptr(), lg.data_ptr())
            if which == 0:
                L.llmdec_model_step_greedy(*args, ws.ptr, ws.nbytes, R.stream())
            else:
                L.llmdec_model_step_greedy_noalloc(*args, err.data_ptr(), R.stream())
            out.append((nxt, lg))
        torch.cuda.synchronize()
        assert ws.error_bits() == 0
        assert int(err.cpu()[0]) == 0, "the no-alloc step reported a device error"
        assert torch.equal(out[0][1], out[1][1]), f"call {call + 1}: logits differ"
        assert torch.equal(out[0][0], out[1][0]), f"call {call + 1}: next tokens differ"
        assert torch.equal(pools[0].buf, pools[1].buf), f"call {call + 1}: KV pools differ"
        next_token = int(out[0][0].cpu()[0])
        assert 0 <= next_token < vocab


def test_noalloc_step_refuses_oversized_workspace(L, R):
    m = TinyModel(L, R, 12)
    P = 8
    need = L.llmdec_workspace_bytes(m.cfg, 100000, 1, P)
    assert need > 48 << 20
    pool = R.Pool(m.cfg, P)
    tok = R.dev_i32(np.zeros(16, np.int32))
    sp = R.dev_i32([0])
    bt = R.dev_i32(np.zeros((1, P), np.int32))
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(L.LlmdecError) as e:
        L.llmdec_model_step_greedy_noalloc(m.cfg, m.struct, 1, 100000, 100000, tok.data_ptr(), None,
                                           sp.data_ptr(), bt.data_ptr(), P, pool.handle, nxt.data_ptr(), None,
                                           None, R.stream())
    assert e.value.status == L.LLMDEC_E_WORKSPACE
    assert "static" in str(e.value)
