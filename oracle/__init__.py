"""Float64 CPU oracle for paged KV-cache decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The
product (``paged_kv_cache_368_amd``) never imports it, and this package imports
nothing from the product: the two share no kernels, headers, helpers or
constants.  Only the seeded input generators in ``workloads`` serve both.

Sources (cited by short key throughout):

* P1 -- "大模型部署中的PagedAttention：KV Cache显存管理突破" (PagedAttention in
  LLM deployment: a breakthrough in KV-cache memory management),
  blog.csdn.net/qq_22409661/article/details/146144360.
* P2 -- "大模型推理优化：KV Cache与PagedAttention技术详解" (LLM inference
  optimisation: KV cache and PagedAttention explained),
  intelliparadigm.com/article/weixin_32678995/2221576.
* P3 -- "LLM 推理中的 PageAttention 实现原理：虚拟内存管理在 KV Cache 中的创新应用"
  (How PageAttention works in LLM inference: virtual-memory management applied
  to the KV cache), www.dpshk.com/news/3461484/.

Pins: every function in ``oracle.paged`` is pinned by CPU tests in
``tests/test_oracle_pins.py`` to facts the pages or the mathematics fix, and
``tests/test_oracle_mutations.py`` shows that plausible mistakes planted in the
oracle fail those pins.  Parity unpinned: none of the functions; the grouped
query head mapping (query head h reads kv head h // (H / Hkv)) is a convention
the pages do not state, pinned only by its reduction to the library routine
with repeated kv heads and by G = 1 reducing to multi-head attention.
"""
from . import paged  # noqa: F401
