"""Reference oracle for hybrid sliding-window / full GQA attention over a
dual-pool KV cache.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``hybrid_sliding_window_gqa_amd``) never imports, calls or links anything
here, and nothing here imports the product path.

It is a plain, slow, obviously-correct float64 NumPy model of what the method
computes, written from the following web pages (cited by title and section):

* [HTX]   htx.com news, "Xiaomi MiMo's 99% price cut is not marketing --
          Luo Fuli posts ...", sections 工程一 (KV memory compressed to 1/7),
          工程二 (dual pool), 工程三 (window-safe prefix reuse).
* [YLY]   youleyou.com, "小米MiMo首次公开模型推理系统全链路优化降价99%",
          section 1 "为什么选择 Hybrid SWA 架构" and section 2 sub-section
          "KVCache系统重构：让缓存真正省下来".
* [HD9]   blog.hotdry.top 2026-06-09, "MiMo-V2.5 ultra-speed inference
          architecture", sections "Hybrid SWA：用 1/7 计算量捕获长程依赖" and
          "三层 KVCache 系统".
* [HD12]  blog.hotdry.top 2026-06-12, "MiMo inference optimization / edge
          deployment", sections "架构层面的 KV Cache 压缩" and
          "双池分治与三级缓存的工程实现".

Modules
-------
attention   masked softmax attention (SWA window / full causal), GQA, LSE.
indexing    ring-buffer slot model (SWA pool) and page model (Full pool).
window_safe brute-force "window-safe length" prefix match.
accounting  visible-pair and KV-size counts (the pages' 1/7 figures).

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library routines, brute force or the pages' printed figures. See the module
docstrings for which pin covers which function.
"""

from . import accounting, attention, indexing, window_safe  # noqa: F401
