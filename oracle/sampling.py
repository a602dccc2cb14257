"""Sampling the next token with temperature, top-k and top-p, and the counter-based generator that
supplies its uniform draw (test infrastructure only: the tests, the smoke check and the benchmark's
CPU baseline use it).

The pages describe the strategies ("为什么要自己动手写一个LLM推理引擎" §3.5; "大模型推理全流程解析" §2.2.3):
temperature divides the logits before the softmax; top-k keeps the k most probable tokens and
renormalises; top-p keeps the smallest set of most probable tokens whose cumulative probability
reaches p; in combination the distribution is first adjusted by temperature, then truncated, then
sampled.  Readings taken where the pages stop (the same on the device):
  * top-k is applied before top-p, and top-p works on the distribution renormalised over the top-k
    set; top_k <= 0 and top_p >= 1 turn the truncations off; temperature <= 0 is greedy (argmax,
    lowest index on ties);
  * a token tied with the last one a truncation keeps is kept too (ties at the k-th largest logit,
    or at the probability where the top-p sum reaches p);
  * the draw: u in [0, 1) from Philox4x32-10 (below); the token is the first kept token, in
    increasing token id, whose cumulative renormalised probability exceeds u.

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC 2011): ten rounds over a 4 x 32-bit counter with a 2 x 32-bit key.
Each round multiplies counter words 0 and 2 by two fixed odd constants into 64-bit products and
mixes the halves with words 1 and 3 and the key; the key is bumped by two Weyl constants between
rounds.  Here the counter is (row, step low, step high, 0) and the key (seed low, seed high); u is
the top 24 bits of the first output word times 2^-24, exact in float32 and float64.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57          # round multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85          # key increments between rounds
MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Four 32-bit counter words and two key words -> four 32-bit output words (Python ints)."""
    c0, c1, c2, c3 = (int(v) & MASK for v in counter)
    k0, k1 = (int(v) & MASK for v in key)
    for r in range(10):
        if r:
            k0, k1 = (k0 + W0) & MASK, (k1 + W1) & MASK
        p0 = M0 * c0            # 64-bit products
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK, p1 & MASK, ((p0 >> 32) ^ c3 ^ k1) & MASK, p0 & MASK
    return c0, c1, c2, c3


def uniform(seed: int, step: int, row: int) -> float:
    """The draw for one row of one step: top 24 bits of Philox word 0, times 2^-24, in [0, 1)."""
    w = philox4x32_10((row, step & MASK, (step >> 32) & MASK, 0), (seed & MASK, (seed >> 32) & MASK))[0]
    return (w >> 8) * 2.0 ** -24


def kept_tokens(logits, temperature: float, top_k: int, top_p: float):
    """(ids of the kept tokens in increasing order, their probabilities renormalised over the kept set),
    in float64, for temperature > 0."""
    z = np.asarray(logits, dtype=np.float64)
    e = np.exp((z - z.max()) / temperature)
    keep = np.ones(z.size, bool)
    if 0 < top_k < z.size:
        kth = np.sort(z)[::-1][top_k - 1]
        keep &= z >= kth                          # ties with the k-th largest logit stay
    if top_p < 1.0:
        q = np.where(keep, e, 0.0)
        q = q / q.sum()
        order = np.argsort(-q, kind="stable")
        cum = np.cumsum(q[order])
        n = int(np.searchsorted(cum, top_p, side="left"))   # first place the sum reaches top_p
        n = min(n, z.size - 1)
        tau = q[order[n]]
        keep &= q >= tau                          # ties with the last kept probability stay
    ids = np.nonzero(keep)[0]
    w = e[ids] / e[ids].sum()
    return ids, w


def sample(logits, temperature: float, top_k: int, top_p: float, u: float) -> int:
    """The sampled token id for one row of logits and the draw u in [0, 1)."""
    z = np.asarray(logits, dtype=np.float64)
    if temperature <= 0:
        return int(np.argmax(z))                  # lowest index on ties
    ids, w = kept_tokens(z, temperature, top_k, top_p)
    cum = np.cumsum(w)
    j = int(np.searchsorted(cum, u, side="right"))         # first cumulative value > u
    return int(ids[min(j, ids.size - 1)])
