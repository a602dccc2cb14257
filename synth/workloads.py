"""Model shapes and seeded synthetic inputs for the five decoder workloads.

Every array is drawn from NumPy's PCG64 keyed by
``SeedSequence([20261202, workload_id, stream_id, *sub_keys])``, so each tensor
(and each row chunk of a large tensor) has its own independent stream and the
result does not depend on thread count or generation order.  Floating-point
values are drawn in float32 and rounded to bfloat16 with round-to-nearest-even;
they are returned as raw ``uint16`` bit patterns, which is how both the device
path and the oracle receive weights and cache contents.

Workloads (sizes follow the pages' LLaMA-7B description: hidden 4096, 32 heads,
intermediate 11008, vocab 32000, 16-token pages):

* 1  tiny: 2 layers, hidden 256, 4 x 64 heads, intermediate 688, vocab 1024;
      batch 1, 32-token prompt, 16 greedy tokens.
* 2  one 7B layer, decode, batch 1, 2048 cached tokens.
* 3  one 7B layer, decode, 32 sequences, context lengths uniform in [128, 4096].
* 4  one 7B layer, prefill, 4 x 512 tokens at positions 0..511.
* 5  32-layer 7B model, decode, 64 sequences, context in [256, 2048], vocab 32000.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED = 20261202
PAGE = 16

# stream ids (second key after the workload id)
S_EMBED, S_LMHEAD, S_HIDDEN, S_CTX, S_KV, S_PROMPT, S_FREE, S_TOKENS, S_LAYER = 1, 2, 3, 4, 5, 6, 7, 8, 100
S_FINAL_NORM = 9
LAYER_TENSORS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
NORMS = ("attn_norm", "mlp_norm")
BF16_ONE = np.uint16(0x3F80)
WEIGHT_STD = 0.02


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    page_size: int = PAGE
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    def matrix_shapes(self):
        """[out][in] shape of each per-layer matrix (nn.Linear convention)."""
        h, kv, i = self.hidden, self.n_kv_heads * self.head_dim, self.intermediate
        return {"wq": (h, h), "wk": (kv, h), "wv": (kv, h), "wo": (h, h),
                "w_gate": (i, h), "w_up": (i, h), "w_down": (h, i)}


TINY = ModelShape(n_layers=2, hidden=256, n_heads=4, n_kv_heads=4, head_dim=64,
                  intermediate=688, vocab=1024)
LLAMA7B = ModelShape(n_layers=32, hidden=4096, n_heads=32, n_kv_heads=32, head_dim=128,
                     intermediate=11008, vocab=32000)
LLAMA7B_LAYER = ModelShape(n_layers=1, hidden=4096, n_heads=32, n_kv_heads=32, head_dim=128,
                           intermediate=11008, vocab=32000)


def rng(*keys) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, *keys])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        n = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count())
        _POOL = ThreadPoolExecutor(max(1, n))
    return _POOL


def normal_bf16(keys: tuple, shape: tuple, std: float, chunk_rows: int = 512) -> np.ndarray:
    """Seeded N(0, std^2) draws rounded to bf16, generated in row chunks in parallel.

    Chunk c of the leading dimension uses the stream ``keys + (c,)``.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    flat = out.reshape(rows, -1)
    cols = flat.shape[1]

    def fill(c):
        r0, r1 = c * chunk_rows, min(rows, (c + 1) * chunk_rows)
        x = rng(*keys, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        flat[r0:r1] = f32_to_bf16_bits(x)

    n_chunks = (rows + chunk_rows - 1) // chunk_rows
    list(_pool().map(fill, range(n_chunks)))
    return out


@dataclass
class LayerWeights:
    """bf16 bit patterns, each matrix [out][in]; norms [hidden]."""
    tensors: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.tensors[k]


def layer_weights(workload: int, layer: int, shape: ModelShape, norm_gamma: str = "ones") -> LayerWeights:
    """Matrices ~ N(0, 0.02^2); RMSNorm gains are 1.0 (the pages' initial value)."""
    t = {}
    for idx, name in enumerate(LAYER_TENSORS):
        t[name] = normal_bf16((workload, S_LAYER + 16 * layer + idx), shape.matrix_shapes()[name], WEIGHT_STD)
    for idx, name in enumerate(NORMS):
        if norm_gamma == "ones":
            t[name] = np.full(shape.hidden, BF16_ONE, dtype=np.uint16)
        else:  # literal variant: every parameter ~ N(0, 0.02^2)
            t[name] = normal_bf16((workload, S_LAYER + 16 * layer + 8 + idx), (shape.hidden,), WEIGHT_STD)
    return LayerWeights(t)


@dataclass
class ModelWeights:
    shape: ModelShape
    embed: np.ndarray           # [V][h] bf16 bits
    layers: list                # [LayerWeights]
    final_norm: np.ndarray      # [h]
    lm_head: np.ndarray         # [V][h]


def model_weights(workload: int, shape: ModelShape, norm_gamma: str = "ones") -> ModelWeights:
    """norm_gamma = "ones": every RMSNorm gain 1.0; "literal": gains ~ N(0, 0.02^2) like every other
    parameter (the final norm's from its own stream)."""
    final = (np.full(shape.hidden, BF16_ONE, dtype=np.uint16) if norm_gamma == "ones" else
             normal_bf16((workload, S_FINAL_NORM), (shape.hidden,), WEIGHT_STD))
    return ModelWeights(
        shape=shape,
        embed=normal_bf16((workload, S_EMBED), (shape.vocab, shape.hidden), WEIGHT_STD),
        layers=[layer_weights(workload, l, shape, norm_gamma) for l in range(shape.n_layers)],
        final_norm=final,
        lm_head=normal_bf16((workload, S_LMHEAD), (shape.vocab, shape.hidden), WEIGHT_STD),
    )


# group-quantized matrices: codes uniform over the 8-bit range, zero points near its middle, bf16 scales
# sized so that (code - zero) * scale spreads like the N(0, 0.02^2) bf16 matrices (codes uniform on
# 0..255 around a zero near 128 have a standard deviation of about 74)
S_QUANT = 1000
QGROUP = 128


def q8_matrix(workload: int, layer: int, idx: int, rows: int, cols: int):
    """(codes uint8 [rows][cols], scales bf16 bits [rows][g], zeros uint8 [rows][g]), g = ceil(cols / 128)."""
    g = (cols + QGROUP - 1) // QGROUP
    key = (workload, S_QUANT + 16 * layer + idx)
    codes = rng(*key, 0).integers(0, 256, (rows, cols), dtype=np.uint8)
    scales = f32_to_bf16_bits(rng(*key, 1).uniform(0.75, 1.25, (rows, g)).astype(np.float32)
                              * np.float32(WEIGHT_STD / 74.0))
    zeros = rng(*key, 2).integers(112, 144, (rows, g), dtype=np.uint8)
    return codes, scales, zeros


def q4_matrix(workload: int, layer: int, idx: int, rows: int, cols: int):
    """4-bit codes: (codes uint8 [rows][cols/2], two per byte, column 2j in the low nibble of byte j;
    scales bf16 bits [rows][g]; zeros uint8 [rows][g] in 7..8), g = ceil(cols / 128); scales sized so
    that (code - zero) * scale spreads like N(0, 0.02^2) (codes uniform on 0..15 have a standard
    deviation of about 4.6)."""
    g = (cols + QGROUP - 1) // QGROUP
    key = (workload, S_QUANT + 16 * layer + idx, 4)
    c = rng(*key, 0).integers(0, 16, (rows, cols), dtype=np.uint8)
    codes = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    scales = f32_to_bf16_bits(rng(*key, 1).uniform(0.75, 1.25, (rows, g)).astype(np.float32)
                              * np.float32(WEIGHT_STD / 4.6))
    zeros = rng(*key, 2).integers(7, 9, (rows, g), dtype=np.uint8)
    return codes, scales, zeros


def q_matrix(bits: int, workload: int, layer: int, idx: int, rows: int, cols: int):
    return (q8_matrix if bits == 8 else q4_matrix)(workload, layer, idx, rows, cols)


def q_layer_weights(bits: int, workload: int, layer: int, shape: ModelShape) -> dict:
    """Quantized matrices of one layer by name (as q_matrix), plus the two norm gains (1.0)."""
    t = {name: q_matrix(bits, workload, layer, idx, *shape.matrix_shapes()[name])
         for idx, name in enumerate(LAYER_TENSORS)}
    for name in NORMS:
        t[name] = np.full(shape.hidden, BF16_ONE, dtype=np.uint16)
    return t


def q8_layer_weights(workload: int, layer: int, shape: ModelShape) -> dict:
    """Quantized matrices of one layer by name (as q8_matrix), plus the two norm gains (1.0)."""
    t = {name: q8_matrix(workload, layer, idx, *shape.matrix_shapes()[name]) for idx, name in enumerate(LAYER_TENSORS)}
    for name in NORMS:
        t[name] = np.full(shape.hidden, BF16_ONE, dtype=np.uint16)
    return t


def free_order(workload: int, num_pages: int) -> np.ndarray:
    """Seeded permutation of page ids: the initial order of the pool's free list."""
    return rng(workload, S_FREE).permutation(num_pages).astype(np.int32)


def pages_for(tokens: int, page: int = PAGE) -> int:
    return (int(tokens) + page - 1) // page


def hidden_input(workload: int, tokens: int, hidden: int) -> np.ndarray:
    """Layer input ~ N(0,1), bf16-representable values stored as float32 [T][h]."""
    return bf16_bits_to_f32(normal_bf16((workload, S_HIDDEN), (tokens, hidden), 1.0))


def kv_history(workload: int, layer: int, seq: int, n_tokens: int, n_kv_heads: int, head_dim: int):
    """Cached (already rotated) K and V for positions 0..n_tokens-1 ~ N(0,1) bf16: [n][Hkv][D] each."""
    k = normal_bf16((workload, S_KV, layer, seq, 0), (n_tokens, n_kv_heads, head_dim), 1.0, chunk_rows=1024)
    v = normal_bf16((workload, S_KV, layer, seq, 1), (n_tokens, n_kv_heads, head_dim), 1.0, chunk_rows=1024)
    return k, v


def context_lengths(workload: int, n: int, lo: int, hi: int) -> np.ndarray:
    return rng(workload, S_CTX).integers(lo, hi + 1, n).astype(np.int32)


def prompt_ids(workload: int, n: int, vocab: int) -> np.ndarray:
    return rng(workload, S_PROMPT).integers(0, vocab, n).astype(np.int32)


def first_tokens(workload: int, n: int, vocab: int) -> np.ndarray:
    return rng(workload, S_TOKENS).integers(0, vocab, n).astype(np.int32)


# --- workload recipes -------------------------------------------------------------------------
WORKLOADS = {
    1: dict(name="tiny-2L-h256-prefill32-greedy16", shape=TINY, batch=1, prompt=32, new_tokens=16),
    2: dict(name="7B-layer-decode-b1-ctx2048", shape=LLAMA7B_LAYER, batch=1, ctx=2048),
    3: dict(name="7B-layer-decode-b32-ctx128..4096", shape=LLAMA7B_LAYER, batch=32, ctx_lo=128, ctx_hi=4096),
    4: dict(name="7B-layer-prefill-4x512", shape=LLAMA7B_LAYER, batch=4, prompt=512),
    5: dict(name="7B-32L-decode-b64-ctx256..2048", shape=LLAMA7B, batch=64, ctx_lo=256, ctx_hi=2048),
}
