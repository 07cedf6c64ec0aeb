"""CPU oracle for hybrid compressed attention (CSA + HCA).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.

It is a plain, slow, obviously-correct numpy implementation in float64 of what
the GPU library computes. Every input is decoded exactly from the bytes the GPU
sees (bf16 / e4m3fn / e2m1 + e8m0 / f32) and no output is rounded.

Sources (cited by page title and section; see each module):
  [P1] "DeepSeek V4 重磅開源！首次打通華為Ascend，也沒丟掉英偉達，百萬上下文奪回國產模型話語權"
       (InfoQ article, 69574.cn mirror), section 拆解關鍵技術創新:
       混合注意力機制 (CSA, HCA, partial RoPE, sliding window, attention sink),
       FP4 量化 (fp4 indexer QK, FP4->FP8 dequantisation without loss).
  [P3] 智猩猩 digest of "DeepSeek-V4: Towards Highly Efficient Million-Token
       Context Intelligence" (aiorang.com), section 01 架构与基础设施优化.
  [P5] "DeepSeek V4 重磅开源！百万上下文+双算力兼容，国产大模型正式迈入新时代"
       (gitcode.csdn.net), sections 3 混合注意力机制 and 4 FP4 量化训练.
  [P1] also, section 確定性內核: a deterministic attention backward (no
       split-KV, fixed accumulation order) for training;
  [P1] also, section 框架層優化: the state cache (window tokens plus tokens of
       the incomplete block) kept apart from the compressed KV cache.

The pages name the compressor and the Lightning Indexer without defining them;
the forms implemented here are the plain readings listed in each module.

Parity status: every function here is pinned by tests in
tests/test_oracle_*.py against closed forms, brute force, library routines or
format tables; none is "parity unpinned" with respect to these readings.
"""
from . import formats, rope, compress, indexer, topk, attention, attention_bwd, state  # noqa: F401
