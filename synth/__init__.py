"""Seeded synthetic workloads for the DFlash drafter hot path.

This package only *describes* workloads (model shapes, batch/context mixes) and
draws seeded random inputs for them (weights, target hidden states, ids,
noise).  It contains none of the method's arithmetic: both the CPU oracle
(``oracle/``) and the GPU library's tests/benchmarks consume what it produces.

Public sources the workloads follow (cited by key elsewhere):
  [P1] "LLM的推理加速-DFlash" (wnma3mz.github.io blog)
  [P2] "一次前向，白赚 4 个 token：DFlash 2 块扩散投机解码技术详解" (forceinjection.github.io)
  [P3] "DFlash：块扩散 + KV 注入，让投机解码的草稿不再串行" (rainlin-top.pages.dev)
  [P4] "【大模型】DFlash：把串行 Draft 变成并行“填空”" (developer.horizon.auto)
  [P5] "DDTree 深度解析:从 Block Diffusion 到 Diffusion Draft Tree" (zhichai.net)
"""
from .configs import CONFIGS, DrafterConfig, Workload, get_workload  # noqa: F401
from . import gen  # noqa: F401
