"""Helpers for the GPU parity tests (tolerances, layout decoding, host pool images)."""
import os
import sys

import numpy as np

MAX_ABS = 2e-2    # hidden states and logits: max abs error
REL_L2 = 5e-3     # and relative L2 error, against the oracle fed the same bf16 weights


def report(tag, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    mx = float(np.abs(d).max()) if d.size else 0.0
    rl = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0
    print(f"[parity] {tag}: max_abs={mx:.3e} rel_l2={rl:.3e} n={d.size}", flush=True)
    return mx, rl


def assert_close(tag, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2):
    assert np.all(np.isfinite(got)), f"{tag}: non-finite values"
    mx, rl = report(tag, got, ref)
    assert mx <= max_abs and rl <= rel_l2, f"{tag}: max_abs {mx:.3e} (<= {max_abs}) rel_l2 {rl:.3e} (<= {rel_l2})"


def unpack_tiled(buf_u16: np.ndarray, rows: int, cols: int, kpad: int) -> np.ndarray:
    """Read a [rows][cols] matrix out of the 16 x 32 tile layout (lane l: row l%16, cols 8(l/16)..+7)."""
    kt = kpad // 32
    rb = (rows + 15) // 16
    t = buf_u16[: rb * kt * 512].reshape(rb, kt, 4, 16, 8)   # [row block][k tile][col group][row][8]
    m = t.transpose(0, 3, 1, 2, 4).reshape(rb * 16, kt * 32)
    return m[:rows, :cols]


def f32_from_bf16(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()
