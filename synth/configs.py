"""Drafter shapes and workload mixes.

Shapes: a Qwen3-style drafter (GQA decoder layers, SwiGLU MLP, q/k head norms)
whose context K/V are projected from hidden states of several target layers
[P1 "关键创新" Steps 1-3; P2 §2.2].  The block is one anchor plus K masks
[P2 §2.1; P4 §4], so a block has R = K + 1 query rows and K output rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class DrafterConfig:
    dtype: str                 # "f32" or "bf16": weights, activations fed to GEMMs, KV cache
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_target_layers: int
    target_hidden: int
    mask_token_id: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    input_embedding_scale: float = 1.0
    target_layer_ids: Tuple[int, ...] = ()
    conv_group: int = 0        # DFlash 2 dynamic conv: channels per kernel-correction group (0 = no conv)
    sel_rank: int = 0          # DFlash 2 path selector: codebook rank (0 = no selector)
    sel_cands: int = 16        # candidates per position kept by the selector
    causal_block: bool = False  # block rows attend to the context and to block rows up to their own

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def feat_dim(self) -> int:
        return self.n_target_layers * self.target_hidden

    def layer_params(self) -> int:
        h = self.hidden
        return h * (self.q_dim + 2 * self.kv_dim) + self.q_dim * h + 3 * h * self.ffn

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def kv_bytes_per_token(self) -> int:
        return self.n_layers * 2 * self.kv_dim * self.elem_bytes


@dataclass(frozen=True)
class Workload:
    name: str
    model: DrafterConfig
    batch: int
    K: int
    ctx: int                              # fixed context length (or the mean if ragged)
    ctx_range: Optional[Tuple[int, int]] = None   # ragged: uniform integers in [lo, hi]
    ctx_seed: int = 7
    temperature: float = 0.0
    sigma: float = 1.5                    # target logits = drafter logits + sigma * N(0,1)
    steps: int = 1
    top_k: int = 0
    tree_budget: int = 0
    philox_seed: int = 99
    notes: str = ""

    def ctx_lengths(self):
        import numpy as np
        if self.ctx_range is None:
            return [self.ctx] * self.batch
        rng = np.random.default_rng(self.ctx_seed)
        lo, hi = self.ctx_range
        return [int(x) for x in rng.integers(lo, hi + 1, size=self.batch)]

    def max_ctx_needed(self) -> int:
        base = max(self.ctx_lengths())
        return base + (self.K + 1) * max(self.steps, 1) + 1


TINY = DrafterConfig(dtype="f32", n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                     ffn=512, vocab=1024, n_target_layers=3, target_hidden=256, mask_token_id=1023)

QWEN3_8B_SHAPED = DrafterConfig(dtype="bf16", n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8,
                                head_dim=128, ffn=12288, vocab=151936, n_target_layers=5,
                                target_hidden=4096, mask_token_id=151935)

H5120 = DrafterConfig(dtype="bf16", n_layers=5, hidden=5120, n_q_heads=64, n_kv_heads=8, head_dim=128,
                      ffn=17408, vocab=151936, n_target_layers=5, target_hidden=5120,
                      mask_token_id=151935, target_layer_ids=(5, 19, 33, 47, 61))

CONFIGS = {
    # tiny fp32 drafter, ctx 128, K=4, batch 1; greedy and T=1 verify
    "tiny": Workload("tiny", TINY, batch=1, K=4, ctx=128, sigma=1.0, steps=4),
    # Qwen3-8B-shaped bf16 drafter, batch 1, ctx 2048, K=16, greedy
    "b1_ctx2k": Workload("b1_ctx2k", QWEN3_8B_SHAPED, batch=1, K=16, ctx=2048, sigma=1.5, steps=100),
    # same drafter, batch 32, ragged ctx U[512, 8192], K=16, greedy verify, 100 steps
    "b32_ragged4k": Workload("b32_ragged4k", QWEN3_8B_SHAPED, batch=32, K=16, ctx=4352,
                             ctx_range=(512, 8192), sigma=1.5, steps=100),
    # long context: batch 4, 32768-token prompts in one injection, 50 steps at T=1 (rejection verify)
    "b4_ctx32k": Workload("b4_ctx32k", QWEN3_8B_SHAPED, batch=4, K=16, ctx=32768, temperature=1.0,
                          sigma=1.5, steps=50, philox_seed=99),
    # larger drafter, batch 64, ctx 8192, K=16, top-64 + best-first tree B=64
    "b64_tree": Workload("b64_tree", H5120, batch=64, K=16, ctx=8192, temperature=1.0, sigma=1.5,
                         steps=1, top_k=64, tree_budget=64),
}


def get_workload(name: str, **overrides) -> Workload:
    w = CONFIGS[name]
    return replace(w, **overrides) if overrides else w


def scaled_model(base: DrafterConfig, **kw) -> DrafterConfig:
    """A smaller model of the same family (used by tests to span tiles cheaply)."""
    return replace(base, **kw)
