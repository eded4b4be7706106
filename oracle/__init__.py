"""Plain CPU oracle for the CSA2 sparse-decode step.  TEST INFRASTRUCTURE.

This package is the checker, not the product.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path (no kernels, headers,
helpers, tables or layout code) and never imports it; its only inputs are
the host arrays made by ``harness.gen``.

Arithmetic: real numbers in float64, integers in int64 / Python int.  Where
the method reaches exactly a result that has a plain definition (indexer
scores, Top-K, softmax attention) the oracle writes that definition out;
the FP4 codec is an encoding, so it is spelled out as a nearest-value search
over the format's value table.

Sources (cited by page title and section throughout):

* neodrop.ai, "DeepSeek 首次公开 V4.1-Flash 技术报告 ... KV 缓存压至 890 字节",
  section "架构拆解" item 2 (CSA2 modes, shared main KV and indexer K,
  reused Top-K indices, hierarchical sparse indexer) and item 3 (FP4 main KV:
  E2M1 with one E4M3 scale per 16 channels).
* blog.zulogic.cn, "DeepSeek V4 1-Flash 架构拆解：CED、CSA2、Engram、mHC 与 DSp",
  section 3 (mode table Full / Reindex / Reuse and the owner/consumer state
  diagram) and section 4 (global KV plus a 128-token local window per layer).
* infernews.com, "DeepSeek V4.1 Flash 模型架構與推論優化技術規格剖析",
  section 2 (128-token sliding window, global cache merged with the window
  cache before decoding) and the section 4 table (CSA 2 row).
"""
from . import formats, cache, select, attention  # noqa: F401
