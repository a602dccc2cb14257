"""libllmdec: KV-cached LLaMA-style decoder step over a paged KV cache on MI355X (gfx950).

The compute path is the HIP library built from ``csrc/`` (``build.py``);
``llmdec`` is its ctypes binding and ``runtime`` holds device-memory plumbing
(torch allocations and streams) for callers that use PyTorch.
"""
from . import llmdec  # noqa: F401
