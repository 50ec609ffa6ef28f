"""CPU oracle for paged attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The
product path (``paged_kv_cache_57_amd``) never does, and this package never
imports the product path: the two share no code.

Everything here is plain and slow on purpose: numpy in float64, one step of
the method per line, citing the passage of the source pages it follows.
Page titles used in citations:

* "大模型部署.md" (WeThinkIn AIGC-Interview-Book), §2.1 vLLM, item 3 "vLLM 调度策略与显存块管理"
  (BlockSpaceManagerV1) and item 4 "PageAttention 内存管理技术详解"; §4.1 item 4 "MQA 与 GQA".
* "【自用】AI infra相关", part 一 (prefill / decode) and part 二.2(1) "Paged Attention".
* "DeepSpeed-FastGen 深度解析", §3.1-§3.2 (Dynamic SplitFuse), §6 (blocked KV cache).
* "第7章：大模型部署实战", §2.1 (KV-cache size), §2.2.1 (block allocation),
  §2.2.2 (attention over blocks), §2.3 (BlockManager).
* "第 15 章：推理引擎与部署", §15.1 "算法详解" (online softmax) and its Python
  simulation, §15.3 (RoPE fused with attention), §15.4 (Attention Sink,
  StreamingLLM), §15.6 "PagedAttention：分页 KV Cache", "KV Cache 大小计算",
  "两阶段与 Chunked Prefill".
* "大模型部署.md" §2.1 item 3 also for CachedBlockAllocator and LRUEvictor, and
  "【自用】AI infra相关" part 二.4(2) (prefix caching by block hashes).

Parity status of each function is stated in its module header.
"""
from . import layout, attention, online_softmax, cache_ops, allocator, sizes, rope, splitfuse  # noqa: F401
