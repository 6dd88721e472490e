"""Seeded random inputs.

Everything here is a deterministic function of (seed, name, index) so that the
CPU oracle and the GPU library see identical values.  Generation is chunked
(fixed 4 Mi-element chunks, each with its own torch.Generator) so the result
does not depend on the number of worker threads.

Recipe (stated once, used everywhere):
  * every weight matrix ~ N(0, 0.02^2), rounded to the model dtype;
  * RMSNorm gains are 1 ("ones"), or 1 + 0.1 N(0,1) when a test asks for
    "random" gains so that a misapplied gain cannot hide;
  * target hidden rows ~ N(0, 1); row (slot, position) depends only on
    (seed, slot, position), so incremental and from-scratch injection of the
    same positions see identical rows;
  * anchor ids are uniform on [0, vocab-2] (never the mask id vocab-1);
  * synthetic target logits = drafter logits + sigma * N(0, 1) noise.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List

import numpy as np
import torch

from .configs import DrafterConfig

CHUNK = 1 << 22
_ROW_CHUNK = 64          # hidden rows are drawn per (slot, 64-position block)


def _seed_of(*parts) -> int:
    h = hashlib.sha256(("/".join(str(p) for p in parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def torch_dtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal(shape, std: float, dtype: str, *key) -> torch.Tensor:
    """N(0, std^2) tensor of `shape`, rounded to `dtype`, deterministic in `key`."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch_dtype(dtype))
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        g = torch.Generator().manual_seed(_seed_of(*key, c))
        sl = out[c * CHUNK:min(n, (c + 1) * CHUNK)]
        tmp = torch.empty(sl.numel(), dtype=torch.float32)
        tmp.normal_(0.0, 1.0, generator=g)
        sl.copy_(tmp.mul_(std))

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.view(*shape)


def weights(cfg: DrafterConfig, seed: int = 1234, gains: str = "ones",
            lm_head_std: float = 0.02) -> Dict[str, object]:
    """All drafter weights as CPU tensors in the model dtype.

    Linear layers use the [out_features, in_features] row-major convention.
    Returns a dict with the shared tensors and a list `layers` of per-layer dicts.
    """
    dt = cfg.dtype
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab

    def gain(n, *key):
        if gains == "ones":
            return torch.ones(n, dtype=torch_dtype(dt))
        return (1.0 + normal((n,), 0.1, "f32", seed, *key)).to(torch_dtype(dt))

    w = {
        "embed": normal((V, H), 0.02, dt, seed, "embed"),
        "lm_head": normal((V, H), lm_head_std, dt, seed, "lm_head"),
        "fc": normal((H, cfg.feat_dim), 0.02, dt, seed, "fc"),
        "hidden_norm": gain(H, "hidden_norm"),
        "final_norm": gain(H, "final_norm"),
        "layers": [],
    }
    for l in range(cfg.n_layers):
        w["layers"].append({
            "in_norm": gain(H, l, "in_norm"),
            "q_w": normal((cfg.q_dim, H), 0.02, dt, seed, l, "q"),
            "k_w": normal((cfg.kv_dim, H), 0.02, dt, seed, l, "k"),
            "v_w": normal((cfg.kv_dim, H), 0.02, dt, seed, l, "v"),
            "o_w": normal((H, cfg.q_dim), 0.02, dt, seed, l, "o"),
            "q_norm": gain(cfg.head_dim, l, "q_norm"),
            "k_norm": gain(cfg.head_dim, l, "k_norm"),
            "post_norm": gain(H, l, "post_norm"),
            "gate_w": normal((F, H), 0.02, dt, seed, l, "gate"),
            "up_w": normal((F, H), 0.02, dt, seed, l, "up"),
            "down_w": normal((H, F), 0.02, dt, seed, l, "down"),
        })
    return w


def dflash2_weights(cfg: DrafterConfig, seed: int = 4321, conv_base_std: float = 0.3, conv_proj_std: float = 0.002,
                    codebook_std: float = 0.2, sel_hidden_std: float = 0.02, post: bool = True) -> Dict[str, object]:
    """Weights of the DFlash 2 modules, in the model dtype, as CPU tensors.

    The pages describe the convolution's kernel as a learned base plus a small
    correction derived from the hidden state: the correction projection is drawn
    at std 0.002, so that on unit-RMS rows at hidden 4096 a correction has std
    about 0.13 against base taps around 1 and 0 (std 0.3).

    Per layer (when cfg.conv_group > 0): attn_conv_base / mlp_conv_base [2, H]
    (tap 0 drawn around 1, tap 1 around 0), attn_conv_proj / mlp_conv_proj
    [2 * H / conv_group, H] for the convolutions before the sub-layers and, with
    post=True, attn_conv_post_* / mlp_conv_post_* for those after them (same recipe).  Shared (when cfg.sel_rank > 0): sel_pred and sel_succ
    [V, rank] codebooks, sel_hidden [rank, H].  Returns {"layers": [...], ...} to
    merge into the dict of `weights`.
    """
    dt = cfg.dtype
    H, V = cfg.hidden, cfg.vocab
    out: Dict[str, object] = {"layers": [{} for _ in range(cfg.n_layers)]}
    if cfg.conv_group > 0:
        G = cfg.conv_group
        names = ("attn", "mlp", "attn_post", "mlp_post") if post else ("attn", "mlp")
        for l in range(cfg.n_layers):
            for name in names:
                base = normal((2, H), conv_base_std, "f32", seed, l, name, "conv_base")
                base[0] += 1.0
                key = name.replace("_post", "_conv_post") if name.endswith("_post") else f"{name}_conv"
                out["layers"][l][f"{key}_base"] = base.to(torch_dtype(dt))
                out["layers"][l][f"{key}_proj"] = normal((2 * H // G, H), conv_proj_std, dt, seed, l, name,
                                                         "conv_proj")
    if cfg.sel_rank > 0:
        r = cfg.sel_rank
        out["sel_pred"] = normal((V, r), codebook_std, dt, seed, "sel_pred")
        out["sel_succ"] = normal((V, r), codebook_std, dt, seed, "sel_succ")
        out["sel_hidden"] = normal((r, H), sel_hidden_std, dt, seed, "sel_hidden")
    return out


def merge_weights(w: Dict[str, object], extra: Dict[str, object]) -> Dict[str, object]:
    """w with the entries of dflash2_weights(...) added (per-layer dicts merged)."""
    out = dict(w)
    out["layers"] = [dict(a, **b) for a, b in zip(w["layers"], extra["layers"])]
    for k, v in extra.items():
        if k != "layers":
            out[k] = v
    return out


def hidden_rows(cfg: DrafterConfig, slot: int, pos0: int, n: int, seed: int = 2024) -> torch.Tensor:
    """Target hidden states for positions [pos0, pos0+n) of request `slot`.

    Returns [n, n_target_layers, target_hidden] (layer-major per row) in the
    model dtype; row (slot, p) depends only on (seed, slot, p).
    """
    width = cfg.n_target_layers * cfg.target_hidden
    out = torch.empty((n, width), dtype=torch_dtype(cfg.dtype))
    if n == 0:
        return out.view(0, cfg.n_target_layers, cfg.target_hidden)
    c_lo, c_hi = pos0 // _ROW_CHUNK, (pos0 + n - 1) // _ROW_CHUNK

    def fill(c):
        g = torch.Generator().manual_seed(_seed_of(seed, "hidden", slot, c))
        blk = torch.empty((_ROW_CHUNK, width), dtype=torch.float32)
        blk.normal_(0.0, 1.0, generator=g)
        lo = max(pos0, c * _ROW_CHUNK)
        hi = min(pos0 + n, (c + 1) * _ROW_CHUNK)
        out[lo - pos0:hi - pos0].copy_(blk[lo - c * _ROW_CHUNK:hi - c * _ROW_CHUNK])

    chunks = list(range(c_lo, c_hi + 1))
    if len(chunks) <= 2:
        for c in chunks:
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
    return out.view(n, cfg.n_target_layers, cfg.target_hidden)


def anchor_ids(cfg: DrafterConfig, n: int, seed: int, step: int = 0) -> np.ndarray:
    rng = np.random.default_rng(_seed_of(seed, "anchor", step) & 0xFFFFFFFF)
    return rng.integers(0, cfg.vocab - 1, size=n, dtype=np.int64).astype(np.int32)


def logits_like(shape, std: float, seed: int, *key) -> torch.Tensor:
    """fp32 N(0, std^2) logits, e.g. synthetic draft/target rows for verify tests."""
    return normal(shape, std, "f32", seed, "logits", *key)


def noise(shape, seed: int, *key) -> torch.Tensor:
    return normal(shape, 1.0, "f32", seed, "noise", *key)
