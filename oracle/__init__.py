"""CPU oracle for the KV-cached LLaMA-style decoder step.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The product path (the HIP library and its Python
binding) never imports, calls or links it, and it shares no code with that
path: it receives inputs as plain arrays (bf16 bit patterns, int32 ids and
tables) and computes everything itself, in float64.

Pages it follows (cited by tag throughout):

[W] "企业官网建设流程全解析" (www.dpshk.com/news/4990443): the weights article;
    §1.1 forward skeleton, §1.2 where the parameters live.
[F] "大模型推理全流程解析：从权重加载到文本生成的工程实践"
    (www.stapisi.com/news/4049481): §2.2.1 embedding, §2.2.2 attention and the
    KV cache, §2.2.3 lm_head and greedy choice, §4 the cached greedy loop.
[E] "为什么要自己动手写一个LLM推理引擎" (www.wzjinhao.cn/news/61427): §3.4 KV
    cache sizing and paging, §3.5 sampling, §4.2 RMSNorm, §4.3 attention
    forward with the cache, §4.4 the generate loop, §5.2 turning the cache off
    as a check, §5.3 preallocated cache pool.

Parity status per function is recorded in each module's header.
"""
from . import decoder, pages  # noqa: F401
