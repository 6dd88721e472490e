"""Plain, slow CPU oracle for the DFlash drafter hot path (fp64 NumPy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The GPU
library never calls it and shares no code, headers, tables or constants with
it; the two meet only in the seeded input generators of ``synth/``.

What it computes, and which passage each part follows:

  [P1] "LLM的推理加速-DFlash" (wnma3mz.github.io blog)
       sections headed "关键创新" (Steps 1-3), "核心推理伪代码" and "验证".
  [P2] "一次前向，白赚 4 个 token：DFlash 2 块扩散投机解码技术详解" (forceinjection.github.io)
       §2.1 (anchor + masks), §2.2 (shared embedding x input_embedding_scale,
       fc + RMSNorm over concatenated target layers, per-position logits),
       §2.3 (rejection sampling, bonus token, greedy prefix match),
       §4.2 (fallback to p when the residual is exhausted).
  [P3] "DFlash：块扩散 + KV 注入，让投机解码的草稿不再串行" (rainlin-top.pages.dev)
       §四 (immediate materialisation: project context K/V with norm + RoPE
       before the draft forward).
  [P4] "【大模型】DFlash：把串行 Draft 变成并行“填空”" (developer.horizon.auto)
       §4 (1 anchor + K masks; K+1 queries, K outputs), §4.1 (positions),
       §5.1 (normalise, K/V projection, RoPE, write into the drafter cache),
       §5.3 table (non-causal attention in the block).
  [P5] "DDTree 深度解析:从 Block Diffusion 到 Diffusion Draft Tree" (zhichai.net)
       §2.1-2.3 (Prop. 1, Prop. 2, Lemma 1, best-first heap over rank tuples),
       §3.2 (softmax then top-k), §3.3 (ancestor-only mask).

Parity status per function is listed in ``oracle/PINS.md``-style form in the
module docstrings: every function is pinned by a ``-m "not gpu"`` test except
the forward's numeric values, which no page prints ("parity unpinned" for
absolute values; pinned only through library special cases and invariants).
"""
from . import philox, select, verify, tree, drafter  # noqa: F401
