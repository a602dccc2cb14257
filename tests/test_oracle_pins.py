"""Pins of the CPU oracle to what the pages and mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: figures the
pages print (tests/golden/page_figures.json), closed forms, invariants, special
cases that reduce to a known answer, or an independent library routine.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import decoder as od
from oracle import pages as op

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def close(a, b, rel):
    return abs(a - b) <= rel * abs(b)


# ----------------------------------------------------------------------------- sizes
def test_param_counts_match_page_figures():
    s = GOLD["shape"]
    per = od.layer_param_counts(s["hidden"], s["intermediate"])
    assert per["attention"] == 4 * 4096 * 4096 == 67_108_864
    assert close(per["attention"], GOLD["attention_params_per_layer"]["value"], GOLD["attention_params_per_layer"]["rel_tol"])
    assert close(per["attention"] * 32, GOLD["attention_params_all_layers"]["value"], GOLD["attention_params_all_layers"]["rel_tol"])
    assert per["mlp"] == 3 * 4096 * 11008 == 135_266_304
    assert close(per["mlp"], GOLD["mlp_params_per_layer"]["value"], GOLD["mlp_params_per_layer"]["rel_tol"])
    assert close(per["mlp"] * 32, GOLD["mlp_params_all_layers"]["value"], GOLD["mlp_params_all_layers"]["rel_tol"])
    assert per["norms"] // 2 == GOLD["norm_params_per_norm"]["value"]
    emb = s["vocab"] * s["hidden"]
    assert close(emb, GOLD["embedding_params"]["value"], GOLD["embedding_params"]["rel_tol"])
    total = od.model_param_count(32, 4096, 11008, 32000, tied=False)
    assert total == 6_738_415_616
    for key, nbytes in (("weights_fp16_bytes", 2), ("weights_int8_bytes", 1), ("weights_int4_bytes", 0.5)):
        assert close(total * nbytes, GOLD[key]["value"], GOLD[key]["rel_tol"]), key


def test_kv_cache_size_formula_matches_page_example():
    g = GOLD["kv_bytes_one_request"]
    b = od.kv_cache_bytes(g["layers"], g["heads"], g["head_dim"], g["seq_len"], g["dtype_bytes"])
    assert b == 2 ** 30
    assert close(b, g["value"], g["rel_tol"])
    assert close(b * GOLD["kv_bytes_ten_requests"]["requests"], GOLD["kv_bytes_ten_requests"]["value"],
                 GOLD["kv_bytes_ten_requests"]["rel_tol"])
    # a pool of 2048/16 = 128 pages holds exactly one such request
    assert op.pool_bytes(32, 32, 128, 2048 // 16) == b
    assert 16 in GOLD["page_size_tokens"]["value"]


# ----------------------------------------------------------------------------- bf16
def test_bf16_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-20).astype(np.float32),
        (r.standard_normal(2000) * 1e20).astype(np.float32),
        # exact ties: 1 + 2^-8 (-> 1), 1 + 3*2^-8 (-> 1 + 2^-6), and negatives
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), -(1 + 3 * 2 ** -8), 0.0, -0.0], np.float32),
    ])
    ours = od.round_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert od.round_to_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    assert od.round_to_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert np.array_equal(od.bf16_bits_of(ref[:100]), torch.from_numpy(x[:100]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_f16_rounding_worked_cases():
    """fp16 keeps 11 significant bits: its spacing is 2^-10 on [1, 2), normal numbers reach down to
    2^-14 and subnormals are multiples of 2^-24 (IEEE 754 binary16).  Values past the largest finite
    one, 65504, are clipped to it (the weights article's remedy for fp16 overflow)."""
    cases = [
        (1.0 + 2.0 ** -11, 1.0),                      # halfway between 1 and 1 + 2^-10: ties to even
        (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),      # halfway between 1 + 2^-10 and 1 + 2^-9: to the even one
        (1.0 + 2.0 ** -11 + 2.0 ** -20, 1.0 + 2.0 ** -10),  # just past halfway: up
        (2049.0, 2048.0),                             # spacing 2 on [2048, 4096): tie to even
        (2051.0, 2052.0),
        (65504.0, 65504.0), (65519.0, 65504.0), (70000.0, 65504.0), (-1e9, -65504.0),
        (2.0 ** -14, 2.0 ** -14),                     # smallest normal
        (2.0 ** -24, 2.0 ** -24),                     # smallest subnormal
        (2.0 ** -25, 0.0),                            # halfway to zero: ties to even (zero)
        (3 * 2.0 ** -25, 2.0 ** -23),                 # halfway between 1 and 2 units of 2^-24: to 2
        (-0.1, -0.0999755859375),                     # 0.1 = 1.6 * 2^-4: 1638.4 / 2^14 -> 1638 / 2^14
    ]
    x = np.array([c[0] for c in cases])
    assert np.array_equal(od.round_to_f16(x), np.array([c[1] for c in cases]))
    # random values: within half a spacing, where the spacing is 2^(e-10) for |x| in [2^e, 2^(e+1))
    rng = np.random.default_rng(11)
    v = rng.standard_normal(10000) * np.exp2(rng.integers(-12, 14, 10000))
    e = np.floor(np.log2(np.abs(v)))
    assert np.all(np.abs(od.round_to_f16(v) - v) <= np.exp2(np.maximum(e, -14) - 11))
    # the pair: hi + lo carries 22 bits (lo rounds the remainder, which is below half hi's spacing)
    w = rng.standard_normal(10000)
    assert np.all(np.abs(od.f16_pair(w) - w) <= np.abs(w) * 2.0 ** -21 + 2.0 ** -25)
    assert np.array_equal(od.f16_pair(od.round_to_f16(w)), od.round_to_f16(w))


def test_lm_head_logits_closed_form():
    """Final norm, then lm_head ("企业官网建设流程全解析" §1.1: the last RMSNorm precedes the output head;
    "大模型推理全流程解析" §2.2.3: logits = hidden . lm_head^T).  With lm_head row j = 2 e_{d_j} (a one-hot
    row, [out][in] layout), logit j is 2 x[d_j] gamma[d_j] / sqrt(mean(x^2) + eps): a missing final norm,
    a transposed head or an ignored gain each changes it."""
    class S:
        rms_eps = 1e-6
    h, V = 64, 48
    rng = np.random.default_rng(5)
    x = 3.0 * rng.standard_normal((2, h))
    gamma = od.bf16_bits_of(od.round_to_bf16(0.5 + rng.random(h)))
    d = rng.permutation(h)[:V]
    head = np.zeros((V, h), np.uint16)
    head[np.arange(V), d] = 0x4000  # bf16 2.0
    got = od.lm_head_logits(S, gamma, head, x)
    g = od.widen_bf16(gamma)
    for r in range(2):
        inv = 1.0 / np.sqrt(sum(v * v for v in x[r]) / h + 1e-6)
        for j in range(V):
            assert abs(got[r, j] - 2.0 * x[r, d[j]] * g[d[j]] * inv) <= 1e-12 * (1 + abs(got[r, j]))
    # a constant row: the norm maps c * 1 to c / sqrt(c^2 + eps) * 1, so the logits are 2 gamma[d_j] c / |c|
    c = np.full((1, h), -4.0)
    assert np.allclose(od.lm_head_logits(S, gamma, head, c)[0], -2.0 * g[d] * 4.0 / np.sqrt(16.0 + 1e-6), rtol=1e-13)


def test_widen_bf16_exact():
    assert od.widen_bf16(np.array([0x3F80, 0xBF80, 0x4049, 0x0000], np.uint16)).tolist() == [1.0, -1.0, 3.140625, 0.0]


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_forms():
    eps = 1e-6
    h = 64
    for c in (0.5, 3.0, -7.25):
        y = od.rms_norm(np.full(h, c), np.ones(h), eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)
    # (3, 4): mean square 12.5
    y = od.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(y, [3 / math.sqrt(12.5), 2 * 4 / math.sqrt(12.5)], rtol=1e-15)
    # homogeneity: scaling x by c and eps by c^2 leaves the output unchanged
    x = np.random.default_rng(1).standard_normal(h)
    assert np.allclose(od.rms_norm(1e3 * x, np.ones(h), 1e6 * eps), od.rms_norm(x, np.ones(h), eps), rtol=1e-13)


def test_rmsnorm_eps_inside_the_root():
    # x = 1e-3 * ones, eps = 1e-6: eps inside gives 1e-3/sqrt(2e-6) = 0.7071; eps added
    # after the root would give 1e-3/(1e-3 + 1e-6) = 0.999.  [E] §4.2 puts it inside.
    y = od.rms_norm(np.full(16, 1e-3), np.ones(16), 1e-6)
    assert np.allclose(y, 1 / math.sqrt(2), rtol=1e-12)
    assert not np.allclose(y, 1e-3 / (1e-3 + 1e-6), rtol=1e-3)


# ----------------------------------------------------------------------------- RoPE
def test_rope_closed_form_angles():
    # D = 2: one pair with frequency theta^0 = 1, so position p rotates by p radians
    for p in (0, 1, 5, 1000):
        r = od.apply_rope(np.array([[[1.0, 0.0]]]), np.array([p]), 10000.0)[0, 0]
        assert np.allclose(r, [math.cos(p), math.sin(p)], atol=1e-12)
        r = od.apply_rope(np.array([[[0.0, 1.0]]]), np.array([p]), 10000.0)[0, 0]
        assert np.allclose(r, [-math.sin(p), math.cos(p)], atol=1e-12)
    # D = 4: the second pair turns at 10000^(-2/4) = 1/100 rad per position
    r = od.apply_rope(np.array([[[0.0, 0.0, 1.0, 0.0]]]), np.array([300]), 10000.0)[0, 0]
    assert np.allclose(r, [0, 0, math.cos(3.0), math.sin(3.0)], atol=1e-12)
    assert np.allclose(od.rope_inv_freq(128, 10000.0)[[0, 1, 63]], [1.0, 10000 ** (-2 / 128), 10000 ** (-126 / 128)])


def test_rope_invariants():
    r = np.random.default_rng(2)
    D, H = 64, 3
    q = r.standard_normal((1, H, D))
    k = r.standard_normal((1, H, D))
    # identity at position 0
    assert np.array_equal(od.apply_rope(q, np.array([0]), 1e4), q)
    # every pair keeps its length
    qr = od.apply_rope(q, np.array([777]), 1e4)
    assert np.allclose(np.hypot(qr[..., 0::2], qr[..., 1::2]), np.hypot(q[..., 0::2], q[..., 1::2]), rtol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    dots = [np.sum(od.apply_rope(q, np.array([m]), 1e4) * od.apply_rope(k, np.array([m - 5]), 1e4), axis=-1)
            for m in (5, 17, 300, 4000)]
    for d in dots[1:]:
        assert np.allclose(d, dots[0], rtol=1e-10, atol=1e-10)
    # R_a R_b = R_(a+b)
    ab = od.apply_rope(od.apply_rope(q, np.array([11]), 1e4), np.array([29]), 1e4)
    assert np.allclose(ab, od.apply_rope(q, np.array([40]), 1e4), atol=1e-12)


# ----------------------------------------------------------------------------- attention
def test_attention_special_cases():
    r = np.random.default_rng(3)
    D, n = 64, 37
    K, V = r.standard_normal((n, D)), r.standard_normal((n, D))
    # q = 0: every key weighs the same, output is the mean of V
    assert np.allclose(od.attend(np.zeros(D), K, V), V.mean(0), rtol=1e-13, atol=1e-15)
    # a single key returns its value exactly
    assert np.array_equal(od.attend(r.standard_normal(D), K[:1], V[:1]), V[0])
    # a dominant key returns (almost exactly) its value
    q = 50.0 * K[7] / np.linalg.norm(K[7]) * math.sqrt(D)
    K2 = K.copy()
    K2[7] *= 10
    assert np.allclose(od.attend(q, K2, V), V[7], atol=1e-12)


def test_attention_two_keys_sigmoid_form():
    # two keys: weight of key 1 is sigmoid((s1 - s2)/sqrt(D)), which pins the 1/sqrt(D) scale
    r = np.random.default_rng(4)
    D = 128
    q, K, V = r.standard_normal(D), r.standard_normal((2, D)), r.standard_normal((2, D))
    a = 1.0 / (1.0 + math.exp(-(q @ K[0] - q @ K[1]) / math.sqrt(D)))
    assert np.allclose(od.attend(q, K, V), a * V[0] + (1 - a) * V[1], rtol=1e-12)


def test_attention_is_a_convex_combination():
    r = np.random.default_rng(5)
    K, V = r.standard_normal((50, 16)), r.standard_normal((50, 16))
    o = od.attend(3 * r.standard_normal(16), K, V)
    assert np.all(o <= V.max(0) + 1e-12) and np.all(o >= V.min(0) - 1e-12)
    perm = r.permutation(50)
    assert np.allclose(od.attend(o, K[perm], V[perm]), od.attend(o, K, V), rtol=1e-12)


# ----------------------------------------------------------------------------- SwiGLU / argmax
def test_silu_closed_forms():
    assert od.silu(0.0) == 0.0
    assert abs(od.silu(1.0) - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(od.silu(40.0) - 40.0) < 1e-12
    assert abs(od.silu(-40.0)) < 1e-15
    assert abs(od.silu(-1.0) + math.exp(-1) / (1 + math.exp(-1))) < 1e-16


def test_argmax_lowest_index_on_ties():
    assert od.greedy_token([1.0, 3.0, 3.0, 2.0]) == 1
    assert od.greedy_token([5.0, 5.0, 5.0]) == 0
    x = np.random.default_rng(6).standard_normal(32000)
    x[31999] = 10.0
    assert od.greedy_token(x) == 31999
    x[12345] = 10.0
    assert od.greedy_token(x) == 12345
    assert od.top2_gap([1.0, 4.0, 2.5]) == 1.5


# ----------------------------------------------------------------------------- layer special cases
class _Shape:
    def __init__(self, h, H, D, I, theta=10000.0, eps=1e-6, L=1, V=16):
        self.hidden, self.n_heads, self.n_kv_heads, self.head_dim, self.intermediate = h, H, H, D, I
        self.rope_theta, self.rms_eps, self.n_layers, self.vocab = theta, eps, L, V


def _rand_layer(r, s, scale=0.1):
    h, I = s.hidden, s.intermediate
    return {"attn_norm": np.ones(h), "mlp_norm": np.ones(h),
            "wq": scale * r.standard_normal((h, h)), "wk": scale * r.standard_normal((h, h)),
            "wv": scale * r.standard_normal((h, h)), "wo": scale * r.standard_normal((h, h)),
            "w_gate": scale * r.standard_normal((I, h)), "w_up": scale * r.standard_normal((I, h)),
            "w_down": scale * r.standard_normal((h, I))}


def test_layer_identity_when_output_projections_vanish():
    r = np.random.default_rng(7)
    s = _Shape(16, 2, 8, 24)
    w = _rand_layer(r, s)
    w["wo"][:] = 0
    w["w_down"][:] = 0
    x = r.standard_normal((5, 16))
    kv = od.ContiguousKV(1, 2, 8)
    out = od.layer_step(s, w, 0, x, [0] * 5, list(range(5)), kv)
    assert np.array_equal(out, x)
    # the cache still received the rotated keys, rounded to bf16
    y = od.rms_norm(x, np.ones(16), s.rms_eps)
    k = od.apply_rope((y @ w["wk"].T).reshape(5, 2, 8), np.arange(5), s.rope_theta)
    assert np.array_equal(kv.k[(0, 0)], od.round_to_bf16(k))


def test_layer_value_path_orientation():
    # One token at position 0 attends only to itself, so o = bf16(v) with v = y Wv^T.
    # With Wv a cyclic shift and Wo diagonal, x_out = x + d * bf16(roll(y, -1)); a transposed
    # Wv would give roll(y, +1) and a transposed Wo cannot hide behind the diagonal.
    r = np.random.default_rng(8)
    h = 16
    s = _Shape(h, 2, 8, 24)
    w = _rand_layer(r, s)
    w["wv"] = np.roll(np.eye(h), 1, axis=1)          # row i has its 1 at column i+1: v_i = y_{i+1}
    d = r.uniform(0.5, 2.0, h)
    w["wo"] = np.diag(d)
    w["w_down"][:] = 0
    x = r.standard_normal((1, h))
    out = od.layer_step(s, w, 0, x, [0], [0], od.ContiguousKV(1, 2, 8))
    y = od.rms_norm(x, np.ones(h), s.rms_eps)
    assert np.allclose(out, x + d * od.round_to_bf16(np.roll(y, -1, axis=1)), rtol=1e-14, atol=1e-15)


def test_layer_query_zero_gives_prefix_mean_of_values():
    r = np.random.default_rng(9)
    h, T = 16, 6
    s = _Shape(h, 2, 8, 24)
    w = _rand_layer(r, s)
    w["wq"][:] = 0
    w["w_down"][:] = 0
    x = r.standard_normal((T, h))
    kv = od.ContiguousKV(1, 2, 8)
    out = od.layer_step(s, w, 0, x, [0] * T, list(range(T)), kv)
    V = kv.v[(0, 0)].reshape(T, h)
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, T + 1)[:, None]
    assert np.allclose(out, x + prefix_mean @ w["wo"].T, rtol=1e-12, atol=1e-14)


def test_grouped_kv_heads_equal_repeated_kv_heads():
    """Grouped-query attention ([W] §5.1: k/v projections of n_kv_heads * head_dim rows; [E] §4.3: K/V
    reshaped to n_kv_heads heads): query head h reads K/V head h // (n_heads / n_kv_heads).  That equals
    plain multi-head attention whose k/v projections repeat each K/V head's rows for its group.  Pairing
    the heads any other way (h % n_kv_heads) gives a different layer output."""
    r = np.random.default_rng(12)
    h, H, Hk, D, T = 32, 4, 2, 8, 5
    g = H // Hk
    s_mha = _Shape(h, H, D, 24)
    s_gqa = _Shape(h, H, D, 24)
    s_gqa.n_kv_heads = Hk
    w = _rand_layer(r, s_mha)
    w["wk"] = 0.3 * r.standard_normal((Hk * D, h))
    w["wv"] = 0.3 * r.standard_normal((Hk * D, h))
    x = r.standard_normal((T, h))
    out_g = od.layer_step(s_gqa, w, 0, x, [0] * T, list(range(T)), od.ContiguousKV(1, Hk, D))

    def mha_with(head_map):
        rows = np.concatenate([np.arange(D) + head_map(hh) * D for hh in range(H)])
        w_m = dict(w, wk=w["wk"][rows], wv=w["wv"][rows])
        return od.layer_step(s_mha, w_m, 0, x, [0] * T, list(range(T)), od.ContiguousKV(1, H, D))

    assert np.allclose(out_g, mha_with(lambda hh: hh // g), rtol=1e-12, atol=1e-14)
    assert not np.allclose(out_g, mha_with(lambda hh: hh % Hk), rtol=1e-3, atol=1e-3)


def test_mlp_path_closed_form():
    # attention off (Wo = 0); gate and up diagonal, down a permutation: the MLP output
    # is silu(a*y) * (b*y) routed through the permutation.
    r = np.random.default_rng(10)
    h = 16
    s = _Shape(h, 2, 8, h)
    w = _rand_layer(r, s)
    w["wo"][:] = 0
    a, b = r.uniform(0.5, 2, h), r.uniform(0.5, 2, h)
    w["w_gate"], w["w_up"] = np.diag(a), np.diag(b)
    P = np.roll(np.eye(h), 3, axis=1)
    w["w_down"] = P
    x = r.standard_normal((2, h))
    out = od.layer_step(s, w, 0, x, [0, 0], [0, 1], od.ContiguousKV(1, 2, 8))
    y = od.rms_norm(x, np.ones(h), s.rms_eps)
    m = od.silu(a * y) * (b * y)
    assert np.allclose(out, x + np.roll(m, -3, axis=1), rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------------------- cache checks
def _tiny_model(seed=11, L=2, h=32, H=2, D=16, I=48, V=64):
    r = np.random.default_rng(seed)

    class M:
        pass
    s = _Shape(h, H, D, I, L=L, V=V)
    m = M()
    bf = lambda a: od.round_to_bf16(a)
    m.embed = bf(0.5 * r.standard_normal((V, h)))
    m.layers = [{k: bf(v) for k, v in _rand_layer(r, s, 0.2).items()} for _ in range(L)]
    m.final_norm = np.ones(h)
    m.lm_head = bf(0.2 * r.standard_normal((V, h)))
    return s, m


def test_cached_decode_equals_full_recompute():
    # [E] §5.2: with the cache turned off and the whole sequence recomputed each step,
    # the outputs must agree with the cached run.
    s, m = _tiny_model()
    prompt = [3, 17, 42, 5, 9, 60, 1]
    ids, logits = od.greedy_generate(s, m, prompt, 12, od.ContiguousKV(s.n_layers, 2, 16))
    full = od.full_recompute_logits(s, m, prompt + ids[:-1])
    for i, lg in enumerate(logits):
        ref = full[len(prompt) - 1 + i]
        assert np.allclose(lg, ref, rtol=1e-9, atol=1e-12), f"step {i}"
        assert od.greedy_token(ref) == ids[i]


def test_prefill_in_one_pass_equals_token_by_token():
    s, m = _tiny_model(seed=12)
    ids = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18]
    kv1 = od.ContiguousKV(s.n_layers, 2, 16)
    lg_once, _ = od.model_step(s, m, ids, [0] * len(ids), list(range(len(ids))), kv1)
    kv2 = od.ContiguousKV(s.n_layers, 2, 16)
    for p, t in enumerate(ids):
        lg_step, _ = od.model_step(s, m, [t], [0], [p], kv2)
    assert np.allclose(lg_once, lg_step, rtol=1e-9, atol=1e-12)
    for l in range(s.n_layers):
        assert np.array_equal(kv1.k[(l, 0)], kv2.k[(l, 0)]) or np.allclose(kv1.k[(l, 0)], kv2.k[(l, 0)], atol=2 ** -7)


def test_paged_equals_contiguous_bitwise():
    s, m = _tiny_model(seed=13)
    prompt = list(range(5, 25))
    n_new = 14
    total = len(prompt) + n_new
    npg = op.pages_needed(total) + 3
    pool = op.PagePool(npg, np.random.default_rng(14).permutation(npg))
    row = [-1] * npg
    st, n = pool.alloc(total, row, 0, npg)
    assert st == op.OK
    paged = op.PagedKV(s.n_layers, 2, 16, npg, {0: row})
    ids_c, lg_c = od.greedy_generate(s, m, prompt, n_new, od.ContiguousKV(s.n_layers, 2, 16))
    ids_p, lg_p = od.greedy_generate(s, m, prompt, n_new, paged)
    assert ids_c == ids_p
    assert all(np.array_equal(a, b) for a, b in zip(lg_c, lg_p))


# ----------------------------------------------------------------------------- page allocator
def test_slot_formula_against_page_walk():
    row = [7, 2, 9, 0]
    walk = [(pg, off) for pg in row for off in range(16)]
    for p in range(64):
        assert op.slot_of(row, p) == walk[p]


def test_pool_alloc_free_semantics():
    pool = op.PagePool(6, [4, 1, 5, 0, 3, 2])
    row = [-1] * 4
    assert pool.alloc(17, row, 0, 4) == (op.OK, 2) and row[:2] == [4, 1]
    assert pool.alloc(32, row, 2, 4) == (op.OK, 2)          # already covered
    assert pool.alloc(33, row, 2, 4) == (op.OK, 3) and row[2] == 5
    row2 = [-1] * 4
    assert pool.alloc(64, row2, 0, 4) == (op.E_NO_PAGES, 0) and row2 == [-1] * 4 and pool.n_free == 3
    assert pool.alloc(65, row2, 0, 4)[0] == op.E_INVALID     # more than max_pages
    assert pool.free([4, 1]) == op.OK
    assert pool.free([1]) == op.E_INVALID                      # double free
    assert pool.free([6]) == op.E_INVALID                      # foreign id
    assert pool.alloc(16, row2, 0, 4) == (op.OK, 1) and row2[0] == 1   # last returned is reused first


# ----------------------------------------------------------------------------- group-quantized weights
def test_dequantize_worked_example():
    """A 1 x 256 row, two groups ([W] §4.2: 128 elements per group, a scale and a zero point each):
    group 0 scale 0.5, zero 128; group 1 scale 2, zero 3.  Values worked by hand."""
    from oracle import quant as oq
    codes = np.zeros((1, 256), np.uint8)
    codes[0, [0, 1, 127]] = [0, 255, 128]
    codes[0, [128, 129, 255]] = [3, 4, 0]
    w = oq.dequantize(codes, np.array([[0.5, 2.0]]), np.array([[128, 3]], np.uint8))
    assert w[0, 0] == -64.0 and w[0, 1] == 63.5 and w[0, 127] == 0.0
    assert w[0, 128] == 0.0 and w[0, 129] == 2.0 and w[0, 255] == -6.0
    assert w[0, 2] == -64.0 and w[0, 130] == -6.0      # untouched codes (0) in each group


def test_dequantize_group_boundaries_and_laws():
    """Each scale and zero point reaches exactly its own 128 columns of its own row; equal codes and
    zeros give 0; shifting codes and zeros together changes nothing; doubling a scale doubles its group."""
    from oracle import quant as oq
    r = np.random.default_rng(31)
    rows, cols = 3, 512
    codes = r.integers(60, 256, (rows, cols)).astype(np.uint8)
    scales = r.uniform(0.01, 0.1, (rows, cols // 128))
    zeros = r.integers(100, 156, (rows, cols // 128)).astype(np.uint8)
    w = oq.dequantize(codes, scales, zeros)
    for row in range(rows):
        for g in range(cols // 128):
            s2 = scales.copy()
            s2[row, g] *= 2
            d = oq.dequantize(codes, s2, zeros) - w
            changed = np.zeros((rows, cols), bool)
            changed[row, 128 * g:128 * (g + 1)] = True
            assert np.allclose(d[changed], w[changed]) and np.all(d[~changed] == 0)
    assert np.all(oq.dequantize(np.repeat(zeros, 128, axis=1), scales, zeros) == 0)
    c1, z1 = codes - np.uint8(50), zeros - np.uint8(50)   # both shifted down, still in range
    assert np.array_equal(oq.dequantize(c1, scales, z1), w)
    unit = oq.dequantize(codes, np.ones_like(scales), np.zeros_like(zeros))
    assert np.array_equal(unit, codes.astype(np.float64))


def test_linear_q8_matches_dense_product_of_dequantized_rows():
    """The quantized product is the plain product with the dequantized [out][in] matrix: row j of the
    output is x . w_j, checked one output element at a time with a Python sum."""
    from oracle import quant as oq
    r = np.random.default_rng(32)
    codes = r.integers(0, 256, (4, 256)).astype(np.uint8)
    scales = r.uniform(0.01, 0.05, (4, 2))
    zeros = r.integers(120, 136, (4, 2)).astype(np.uint8)
    x = r.standard_normal((2, 256))
    y = oq.linear_q8(x, codes, scales, zeros)
    for i in range(2):
        for j in range(4):
            ref = sum(float(x[i, c]) * (int(codes[j, c]) - int(zeros[j, c // 128])) * float(scales[j, c // 128])
                      for c in range(256))
            assert abs(y[i, j] - ref) <= 1e-12 * (1 + abs(ref))


def test_dequantize_short_last_group():
    """A 1 x 130 row is a full group of 128 and a group of 2 with their own scale and zero point
    (values worked by hand): group 0 scale 0.25 zero 10, group 1 scale 3 zero 7."""
    from oracle import quant as oq
    codes = np.full((1, 130), 10, np.uint8)
    codes[0, 0], codes[0, 127], codes[0, 128], codes[0, 129] = 14, 2, 9, 7
    w = oq.dequantize(codes, np.array([[0.25, 3.0]]), np.array([[10, 7]], np.uint8))
    assert w.shape == (1, 130)
    assert w[0, 0] == 1.0 and w[0, 127] == -2.0 and w[0, 1] == 0.0
    assert w[0, 128] == 6.0 and w[0, 129] == 0.0
    with pytest.raises(AssertionError):   # a missing group's scale is an error, not a silent reuse
        oq.dequantize(codes, np.array([[0.25]]), np.array([[10]], np.uint8))


# ----------------------------------------------------------------------------- sampling
GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_philox_known_answers():
    """Philox4x32-10 reproduces the generator's published known-answer vectors."""
    from oracle import sampling as osm
    with open(os.path.join(GOLDEN_DIR, "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        got = osm.philox4x32_10([int(x, 16) for x in v["counter"]], [int(x, 16) for x in v["key"]])
        assert got == tuple(int(x, 16) for x in v["out"])


def test_uniform_draw_range_and_keying():
    """u is a multiple of 2^-24 in [0, 1), and rows, steps and seeds give different draws."""
    from oracle import sampling as osm
    us = [osm.uniform(7, 3, r) for r in range(64)]
    assert all(0.0 <= u < 1.0 and float(u * 2 ** 24).is_integer() for u in us)
    assert len(set(us)) == 64
    assert osm.uniform(7, 3, 0) != osm.uniform(7, 4, 0) != osm.uniform(8, 3, 0)
    assert osm.uniform(7, 1 << 33, 0) != osm.uniform(7, 0, 0)     # the step's high word is used


def test_sample_worked_example():
    """Logits ln 1, ln 2, ln 3, ln 4 at T = 1 give p = (1, 2, 3, 4) / 10.  top_k = 3 keeps tokens 1..3
    (2, 3, 4)/9; top_p = 0.7 then keeps 3 (4/9) and 2 (4/9 + 3/9 = 7/9 >= 0.7), renormalised to
    3/7 for token 2 and 4/7 for token 3, taken in increasing id: u < 3/7 gives 2, else 3.  Worked by hand."""
    from oracle import sampling as osm
    z = np.log([1.0, 2.0, 3.0, 4.0])
    ids, w = osm.kept_tokens(z, 1.0, 3, 0.7)
    assert ids.tolist() == [2, 3] and np.allclose(w, [3 / 7, 4 / 7], rtol=0, atol=1e-15)
    assert osm.sample(z, 1.0, 3, 0.7, 0.42) == 2 and osm.sample(z, 1.0, 3, 0.7, 0.43) == 3
    ids, w = osm.kept_tokens(z, 1.0, 3, 1.0)
    assert ids.tolist() == [1, 2, 3] and np.allclose(w, [2 / 9, 3 / 9, 4 / 9], rtol=0, atol=1e-15)
    # no truncation: u in [0, 0.1) -> 0, [0.1, 0.3) -> 1, [0.3, 0.6) -> 2, [0.6, 1) -> 3
    assert [osm.sample(z, 1.0, 0, 1.0, u) for u in (0.05, 0.15, 0.35, 0.65)] == [0, 1, 2, 3]


def test_sample_limits_reduce_to_argmax():
    """Temperature 0, top_k = 1 and a top_p below every probability all give the argmax for any u."""
    from oracle import sampling as osm
    r = np.random.default_rng(41)
    for _ in range(20):
        z = r.standard_normal(500) * 3
        am = int(np.argmax(z))
        for u in (0.0, 0.3, 0.999999):
            assert osm.sample(z, 0.0, 0, 1.0, u) == am
            assert osm.sample(z, 0.8, 1, 1.0, u) == am
            assert osm.sample(z, 1.3, 0, 1e-9, u) == am


def test_sample_measure_matches_probabilities():
    """Without truncation a fine grid of u gives each token a share equal to softmax(z / T); the ratio of
    two tokens' probabilities is exp((z_i - z_j) / T)."""
    from oracle import sampling as osm
    r = np.random.default_rng(42)
    z = r.standard_normal(12)
    T = 0.7
    ids, w = osm.kept_tokens(z, T, 0, 1.0)
    assert ids.tolist() == list(range(12))
    for i in range(12):
        assert abs(w[i] / w[0] - math.exp((z[i] - z[0]) / T)) < 1e-12 * math.exp((z[i] - z[0]) / T)
    grid = (np.arange(200000) + 0.5) / 200000
    counts = np.bincount([osm.sample(z, T, 0, 1.0, u) for u in grid], minlength=12) / grid.size
    assert np.allclose(counts, w, atol=1e-5)


def test_sample_truncation_sets():
    """top_k keeps exactly the k largest logits (and ties with the k-th); top_p keeps the smallest prefix
    of the sorted probabilities whose sum reaches p; both are checked by brute force over subsets."""
    from oracle import sampling as osm
    r = np.random.default_rng(43)
    z = r.standard_normal(9)
    for k in range(1, 9):
        ids, _ = osm.kept_tokens(z, 1.0, k, 1.0)
        assert set(ids.tolist()) == set(np.argsort(-z)[:k].tolist())
    zt = np.array([0.0, 1.0, 1.0, 0.5])               # a tie at the 2nd largest logit
    assert osm.kept_tokens(zt, 1.0, 2, 1.0)[0].tolist() == [1, 2]
    assert osm.kept_tokens(zt, 1.0, 1, 1.0)[0].tolist() == [1, 2]
    p = np.exp(z - z.max())
    p /= p.sum()
    for top_p in (0.05, 0.3, 0.5, 0.8, 0.95):
        ids, _ = osm.kept_tokens(z, 1.0, 0, top_p)
        # brute force: the fewest tokens whose mass reaches top_p, and of those sets the most probable one
        best = None
        for mask in range(1, 1 << 9):
            sel = [i for i in range(9) if mask >> i & 1]
            if p[sel].sum() >= top_p and (best is None or (len(sel), -p[sel].sum()) < (len(best), -p[best].sum())):
                best = sel
        assert sorted(ids.tolist()) == sorted(best)


def test_unpack_nibbles_worked_example():
    """Two 4-bit codes per byte, column 2j in the low nibble of byte j: bytes 0x21, 0xF0, 0x3C are columns
    1, 2, 0, 15, 12, 3 (worked by hand); an odd column count takes the last byte's low nibble only."""
    from oracle import quant as oq
    assert oq.unpack_nibbles(np.array([[0x21, 0xF0, 0x3C]], np.uint8), 6).tolist() == [[1, 2, 0, 15, 12, 3]]
    assert oq.unpack_nibbles(np.array([[0x21, 0xF0, 0x3C]], np.uint8), 5).tolist() == [[1, 2, 0, 15, 12]]


def test_synthetic_4bit_codes_follow_the_storage_convention():
    """The seeded 4-bit generator packs what the oracle unpacks: re-packing the oracle's columns by the
    stated convention gives back the generator's bytes, and the codes span 0..15."""
    import synth
    from oracle import quant as oq
    codes, scales, zeros = synth.q4_matrix(5, 0, 0, 8, 256)
    c = oq.unpack_nibbles(codes, 256)
    assert c.min() == 0 and c.max() == 15 and scales.shape == (8, 2) and zeros.shape == (8, 2)
    repacked = np.array([[int(c[r, 2 * j]) + 16 * int(c[r, 2 * j + 1]) for j in range(128)] for r in range(8)])
    assert np.array_equal(repacked, codes)
