"""Plain float64 model of one KV-cached decoder step (test infrastructure only).

Everything here is the definition written out with NumPy primitives; matrix
products are ``numpy.matmul`` in float64.  The only roundings that belong to
the problem itself are (a) weights are bf16 and are widened exactly, and (b)
K and V are stored in a bf16 cache, rounded to nearest-even when appended.
Nothing is blocked, fused or reordered beyond that.

Readings taken where the pages are silent or garbled (each also listed in the
design notes):

* pre-norm blocks with two RMSNorm gains per layer, x += Attn(N1(x)),
  x += MLP(N2(x))  ([W] §1.1 "interleaved" norms and residuals);
* eps is added to the mean square inside the reciprocal square root
  ([E] §4.2, stated in the prose after the RMSNorm class);
* rotary embedding on adjacent pairs (x[2i], x[2i+1]) with angle
  p * theta^(-2i/D), rotating (a, b) to (a cos - b sin, a sin + b cos),
  applied per head to q and k before the cache update ([E] §4.3 code order);
* causal attention over keys 0..p inclusive, scores scaled by 1/sqrt(D)
  ([E] §4.3, mask slice start_pos:start_pos+seq_len);
* SwiGLU as down(silu(gate(y)) * up(y)) with silu(z) = z / (1 + e^-z)
  ([W] §1.2 gate/up/down; [E] §4.2 "SwiGLU, three linear layers");
* greedy: argmax of the last position's logits, lowest index on ties
  ([F] §2.2.3, §4; [E] §4.4).

Parity pins (tests/test_oracle_pins.py): bf16 rounding against torch's cast;
RMSNorm closed forms and the eps-placement discriminator; RoPE identity at 0,
norm preservation, relative-position and composition laws, closed-form angles
for D = 2 and D = 4; attention special cases (q = 0 gives the mean of V,
single key, dominant key, the two-key sigmoid form that fixes the 1/sqrt(D)
scale, convexity); SwiGLU closed forms; argmax ties; layer special cases (zero
output projections give the identity, a cyclic-shift value projection exposes
a transposed operand, q = 0 gives prefix means of V, diagonal gate/up give the
MLP in closed form);
cached decode equal to a full no-cache recompute ([E] §5.2); paged storage
equal to contiguous storage bit for bit.  The end-to-end model has no printed
worked example on the pages: beyond these pins it is parity unpinned.
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- bf16 handling
def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: a bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even; returns float64.

    bf16 keeps 8 significant bits and float32's exponent range.  Working on the
    float64 encoding, that means keeping the top 7 of the 52 stored fraction
    bits: drop 45 bits with round-half-to-even.  Values used here are far from
    the bf16 overflow and subnormal ranges, which is asserted.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.all((a == 0) | ((a > 1e-37) & (a < 3e38))), "value outside the modelled bf16 range"
    u = x.view(np.uint64)
    drop = np.uint64(45)
    half = np.uint64(1) << (drop - np.uint64(1))
    lsb = (u >> drop) & np.uint64(1)
    u = (u + (half - np.uint64(1)) + lsb) >> drop << drop
    return u.view(np.float64)


F16_MAX = 65504.0


def round_to_f16(x) -> np.ndarray:
    """Round to the nearest IEEE binary16 value, ties to even; returns float64.

    The pages' minimal engine computes in fp16 ("为什么要自己动手写一个LLM推理引擎" §4.1), and
    the weights article recommends clipping values beyond fp16's range instead of letting them
    overflow to infinity; magnitudes above 65504 (the largest finite binary16) are clipped to it
    first.  The rounding itself is numpy's float16 conversion.  Used to state what a product sees
    when its activation is carried in fp16.
    """
    x = np.clip(np.asarray(x, dtype=np.float64), -F16_MAX, F16_MAX)
    return x.astype(np.float16).astype(np.float64)


def f16_pair(x) -> np.ndarray:
    """hi + lo with hi = fp16(x), lo = fp16(x - hi): x carried in two fp16 parts (about 22 bits)."""
    x = np.asarray(x, dtype=np.float64)
    hi = round_to_f16(x)
    return hi + round_to_f16(x - hi)


def bf16_bits_of(x) -> np.ndarray:
    """Bit pattern of values that are already bf16-representable."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)), "not bf16-representable"
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------- building blocks
def rms_norm(x, gamma, eps):
    """y = x * (mean(x^2) + eps)^(-1/2) * gamma over the last axis ([E] §4.2)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta^(-2i/D) for pair i = 0..D/2-1 (rotary embedding of [E] §4.2-4.3)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def apply_rope(x, pos, theta: float):
    """Rotate adjacent pairs of the last axis of x[..., n_heads, D] by pos * inv_freq.

    ``pos`` has x's shape without the last two axes (one position per token).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * rope_inv_freq(D, theta)  # [..., 1, D/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def attend(q, K, V):
    """softmax(K q / sqrt(D)) V for one query vector q[D] over keys K[n][D] ([E] §4.3)."""
    q = np.asarray(q, dtype=np.float64)
    scores = (np.asarray(K, dtype=np.float64) @ q) / np.sqrt(q.shape[-1])
    w = np.exp(scores - scores.max())
    w /= w.sum()
    return w @ np.asarray(V, dtype=np.float64)


def greedy_token(logits) -> int:
    """Index of the largest logit; the lowest index wins a tie ([F] §4; [E] §4.4)."""
    logits = np.asarray(logits)
    return int(np.flatnonzero(logits == logits.max())[0])


def top2_gap(logits) -> float:
    s = np.sort(np.asarray(logits, dtype=np.float64))
    return float(s[-1] - s[-2])


# ----------------------------------------------------------------------------- sizes
def layer_param_counts(hidden: int, intermediate: int, n_kv_heads: int = None, head_dim: int = None):
    """Parameters per layer by group, as [W] §1.2 counts them (q/k/v/o; gate/up/down; norms)."""
    kv = hidden if n_kv_heads is None else n_kv_heads * head_dim
    attn = hidden * hidden * 2 + hidden * kv * 2
    mlp = 3 * hidden * intermediate
    return {"attention": attn, "mlp": mlp, "norms": 2 * hidden}


def model_param_count(n_layers, hidden, intermediate, vocab, tied=False):
    per = layer_param_counts(hidden, intermediate)
    total = n_layers * (per["attention"] + per["mlp"] + per["norms"]) + vocab * hidden + hidden
    return total + (0 if tied else vocab * hidden)


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, seq_len, dtype_bytes):
    """layers x 2 (K and V) x heads x head_dim x tokens x bytes ([E] §3.4)."""
    return n_layers * 2 * n_kv_heads * head_dim * seq_len * dtype_bytes


# ----------------------------------------------------------------------------- caches
class ContiguousKV:
    """Per (layer, sequence) growing arrays of stored (bf16-rounded) K and V: [n][Hkv][D].

    This is the concatenating cache of [E] §4.3, kept as the oracle's primary store.
    """

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int):
        self.L, self.H, self.D = n_layers, n_kv_heads, head_dim
        self.k = {}
        self.v = {}

    def length(self, layer, seq):
        return 0 if (layer, seq) not in self.k else self.k[(layer, seq)].shape[0]

    def preload(self, layer, seq, k, v):
        """Install an existing history (values must already be bf16-representable)."""
        self.k[(layer, seq)] = np.array(k, dtype=np.float64)
        self.v[(layer, seq)] = np.array(v, dtype=np.float64)

    def store(self, layer, seq, pos, k, v):
        n = self.length(layer, seq)
        assert pos == n, f"append out of order: position {pos}, cache holds {n}"
        z = np.zeros((0, self.H, self.D))
        self.k[(layer, seq)] = np.concatenate([self.k.get((layer, seq), z), k[None]], axis=0)
        self.v[(layer, seq)] = np.concatenate([self.v.get((layer, seq), z), v[None]], axis=0)

    def keys_values(self, layer, seq, upto):
        """K and V for positions 0..upto-1."""
        return self.k[(layer, seq)][:upto], self.v[(layer, seq)][:upto]


def _w(x):
    return x if x.dtype == np.float64 else widen_bf16(x)


def layer_step(shape, weights, layer: int, x, seqs, pos, kv):
    """One decoder layer on T new tokens; returns the new residual stream [T][h].

    weights: mapping with attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down
    as bf16 bit arrays ([out][in]) or float64 arrays.  seqs[t], pos[t]: sequence id
    and absolute position of token t.  kv: a cache with store/keys_values.
    """
    H, Hk, D = shape.n_heads, shape.n_kv_heads, shape.head_dim
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    seqs = np.asarray(seqs)
    pos = np.asarray(pos)

    y = rms_norm(x, _w(weights["attn_norm"]), shape.rms_eps)
    q = (y @ _w(weights["wq"]).T).reshape(T, H, D)
    k = (y @ _w(weights["wk"]).T).reshape(T, Hk, D)
    v = (y @ _w(weights["wv"]).T).reshape(T, Hk, D)
    q = apply_rope(q, pos, shape.rope_theta)
    k = apply_rope(k, pos, shape.rope_theta)

    # the cache is updated before attention, as in [E] §4.3
    k_st, v_st = round_to_bf16(k), round_to_bf16(v)
    for t in range(T):
        kv.store(layer, int(seqs[t]), int(pos[t]), k_st[t], v_st[t])

    group = H // Hk
    o = np.empty((T, H, D))
    for t in range(T):
        K, V = kv.keys_values(layer, int(seqs[t]), int(pos[t]) + 1)
        for hh in range(H):
            o[t, hh] = attend(q[t, hh], K[:, hh // group], V[:, hh // group])
    x = x + o.reshape(T, H * D) @ _w(weights["wo"]).T

    y2 = rms_norm(x, _w(weights["mlp_norm"]), shape.rms_eps)
    gate = y2 @ _w(weights["w_gate"]).T
    up = y2 @ _w(weights["w_up"]).T
    return x + (silu(gate) * up) @ _w(weights["w_down"]).T


def lm_head_logits(shape, final_norm, lm_head, x_last):
    """logits = RMSNorm(x_last) lm_head^T ([W] §1.1; [F] §2.2.3)."""
    z = rms_norm(np.asarray(x_last, dtype=np.float64), _w(final_norm), shape.rms_eps)
    return z @ _w(lm_head).T


def model_step(shape, mw, tokens, seqs, pos, kv, layer_hook=None):
    """Embed the new tokens, run every layer, return (logits of each sequence's last new token, seq order).

    mw: object with embed, layers (list of layer weight mappings), final_norm, lm_head.
    Returns logits [n_seqs_in_step][V] in order of first appearance of each sequence id.
    """
    tokens = np.asarray(tokens)
    x = _w(np.asarray(mw.embed)[tokens])                    # [F] §2.2.1 row lookup
    for l in range(shape.n_layers):
        x = layer_step(shape, mw.layers[l], l, x, seqs, pos, kv)
        if layer_hook is not None:
            layer_hook(l, x)
    seqs = np.asarray(seqs)
    order, last = [], {}
    for t, s in enumerate(seqs):
        if s not in last:
            order.append(int(s))
        last[int(s)] = t
    rows = [last[s] for s in order]
    return lm_head_logits(shape, mw.final_norm, mw.lm_head, x[rows]), order


def greedy_generate(shape, mw, prompt, new_tokens: int, kv, seq: int = 0, step_hook=None):
    """Prefill the whole prompt, then feed one token per step ([F] §4 loop).

    Returns (generated ids, per-step logits).  There is no end-of-sequence stop:
    the model has random weights and no tokenizer.
    """
    prompt = [int(t) for t in prompt]
    out_ids, all_logits = [], []
    logits, _ = model_step(shape, mw, prompt, [seq] * len(prompt), list(range(len(prompt))), kv)
    nxt = greedy_token(logits[0])
    out_ids.append(nxt)
    all_logits.append(logits[0])
    if step_hook:
        step_hook(0, logits[0], nxt)
    for i in range(1, new_tokens):
        p = len(prompt) + i - 1
        logits, _ = model_step(shape, mw, [out_ids[-1]], [seq], [p], kv)
        nxt = greedy_token(logits[0])
        out_ids.append(nxt)
        all_logits.append(logits[0])
        if step_hook:
            step_hook(i, logits[0], nxt)
    return out_ids, all_logits


def full_recompute_logits(shape, mw, ids):
    """No-cache forward of the whole sequence: logits at every position ([E] §5.2 check).

    Uses a fresh cache for one pass over all tokens; every position attends its
    prefix, so row i equals what step i of cached generation should produce.
    """
    ids = [int(t) for t in ids]
    n = len(ids)
    kv = ContiguousKV(shape.n_layers, shape.n_kv_heads, shape.head_dim)
    x = _w(np.asarray(mw.embed)[ids])
    for l in range(shape.n_layers):
        x = layer_step(shape, mw.layers[l], l, x, [0] * n, list(range(n)), kv)
    return lm_head_logits(shape, mw.final_norm, mw.lm_head, x)
