"""Drafter context injection and block forward (oracle side, fp64).

Injection [P1 "关键创新" Steps 2-3; P2 §2.2; P3 §四; P4 §5.1]: for every new
context row, concatenate the selected target layers' hidden states (ascending
layer order), project with fc, apply one RMSNorm (gain gamma_h) to get the
fused feature g, then for every drafter layer project g with that layer's own
W_k / W_v, RMS-normalise each k head (gain gamma_k of the layer), apply RoPE at
the row's absolute position and store (k, v) in the drafter cache.  Hidden
states themselves are not kept (immediate materialisation, [P3 §四]).

Block forward [P2 §2.1-2.2; P4 §4, §4.1-4.4; P1 "关键创新" Step 3]: the block
is [anchor | mask x K] embedded with the shared embedding times
input_embedding_scale at positions C..C+K (C = context length of the request).
Each Qwen3-style layer: RMSNorm, q/k/v projections, per-head RMSNorm of q and
k, RoPE, attention of the block queries over [context K/V ; block K/V] with no
mask inside the block (non-causal, [P4 §5.3 table; P1 training paragraph]),
output projection + residual, RMSNorm, SwiGLU MLP + residual.  A final
RMSNorm and the shared LM head give logits for the K mask rows only [P4 §4.3].

Readings (silent points): no biases; RMSNorm y = x / sqrt(mean(x^2) + eps) * g
with eps = 1e-6; rotate-half RoPE pairing (i, i + d/2) with inv_freq_i =
theta^(-2i/d); attention scale 1/sqrt(d); q head h uses kv head h // (n_q/n_kv);
a final RMSNorm precedes the LM head; the fused feature g is shared by all
layers (one RMSNorm after fc, no per-layer norm on g).

DFlash 2 dynamic convolution [P2 §3.2.3], when the
layer carries conv weights: a two-tap depthwise convolution over the block's
rows, y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}, where each tap's kernel is a
learned per-channel base plus a correction projected linearly from x_t and
shared by every group of conv_group channels; the row before the anchor is zero
(block-local, zero padding).  Readings: the pages put one convolution before
and one after each of the attention and MLP sub-layers, four per layer, which
is also what their parameter count needs (+16.5M for the 5-layer drafter at
hidden 2560 with groups of 16: 20 convolutions of 2*H/16*H + 2*H weights each;
two per layer would be 8.2M).  A "before" convolution acts on the sub-layer's
input, the RMS-normalised rows that feed q/k/v or gate/up; an "after" one acts
on the sub-layer's output (after o, after down) before it is added to the
residual stream.  Each convolution's correction is projected from its own
input rows.  Weights: attn_conv_* / mlp_conv_* (before) and attn_conv_post_* /
mlp_conv_post_* (after); a layer may carry either pair alone.  The correction
projection has no bias, its output rows [0, H/G) correct tap 0 and rows
[H/G, 2H/G) tap 1, channel c using group c // G; context rows are untouched
(their K/V come from the fused target feature).

Variants [P2 §2.2; P4 §5.2]: a causal-in-block flag (block
row i attends to the context and to block rows j <= i; the pages disagree on the
block-internal mask, non-causal is the default); the logits' output multiplier
and softcap z -> c * tanh(z / c) applied in that order; a mask-embedding
override, a trained vector that replaces the embedding row of mask_token_id at
the mask positions (the input_embedding_scale still applies to it).

Parity of absolute forward values is unpinned by the pages (no page prints an
activation or a logit); the pieces are pinned against library routines and the
invariants listed in tests/test_oracle_drafter.py.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np


def as64(t) -> np.ndarray:
    """Widen a tensor/array (fp32/bf16 torch or numpy) to fp64 numpy exactly."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to(torch.float64).cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2, last axis) + eps) * gain."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * gain


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE on the last axis (size d) of x[..., n, heads, d] with positions pos[n]."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]        # [n, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, group: int, causal_from=None) -> np.ndarray:
    """q [R, n_q, d]; keys/vals [S, n_kv, d]; softmax(q k^T / sqrt d) v.

    causal_from = (C, rows): the last keys are the block's, key C + j is hidden
    from query row i when j > rows[i] (block-internal causal mask); None: no mask.
    """
    R, nq, d = q.shape
    out = np.zeros_like(q)
    for h in range(nq):
        kv = h // group
        s = q[:, h, :] @ keys[:, kv, :].T / np.sqrt(d)
        if causal_from is not None:
            C, rows = causal_from
            for i in range(R):
                s[i, C + rows[i] + 1:] = -np.inf
        s = s - s.max(axis=-1, keepdims=True)
        a = np.exp(s)
        a /= a.sum(axis=-1, keepdims=True)
        out[:, h, :] = a @ vals[:, kv, :]
    return out


def dynamic_conv(x: np.ndarray, base: np.ndarray, proj: np.ndarray, group: int) -> np.ndarray:
    """Two-tap dynamic depthwise conv over the rows of one block, x [R, H] (row 0 = anchor).

    base [2, H] per-channel kernels of the taps; proj [2*H/group, H] projects each
    row to its per-group kernel corrections (tap 0 groups first, then tap 1).
    """
    x = np.asarray(x, dtype=np.float64)
    R, H = x.shape
    ng = H // group
    corr = x @ np.asarray(proj, dtype=np.float64).T                    # [R, 2 * ng]
    k0 = base[0][None, :] + np.repeat(corr[:, :ng], group, axis=1)
    k1 = base[1][None, :] + np.repeat(corr[:, ng:], group, axis=1)
    prev = np.concatenate([np.zeros((1, H)), x[:-1]], axis=0)           # zero row before the anchor
    return k0 * x + k1 * prev


class DrafterOracle:
    """fp64 drafter with its own per-slot context K/V cache."""

    def __init__(self, cfg, weights: Dict, pos_offset: int = 0, output_multiplier: float = 1.0,
                 logit_softcap: float = 0.0):
        self.cfg = cfg
        self.output_multiplier = float(output_multiplier)
        self.logit_softcap = float(logit_softcap)
        self.mask_embedding = as64(weights["mask_embedding"]) if "mask_embedding" in weights else None
        self.pos_offset = pos_offset          # added to every absolute position (tests only)
        c = cfg
        self.embed = as64(weights["embed"])
        self.lm_head = as64(weights["lm_head"])
        self.fc = as64(weights["fc"])
        self.hidden_norm = as64(weights["hidden_norm"])
        self.final_norm = as64(weights["final_norm"])
        self.layers = [{k: as64(v) for k, v in lw.items()} for lw in weights["layers"]]
        self.cache: Dict[int, List] = {}      # slot -> per layer [k (C, n_kv, d), v (C, n_kv, d)]
        self.d = c.head_dim

    # ---- context ----
    def ctx_len(self, slot: int) -> int:
        return 0 if slot not in self.cache else self.cache[slot][0][0].shape[0]

    def reset(self, slot: int):
        self.cache.pop(slot, None)

    def project_context(self, feats: np.ndarray, pos: np.ndarray):
        """feats [n, L_t, H_t] -> per layer (k [n, n_kv, d], v [n, n_kv, d]) at positions pos."""
        c = self.cfg
        x = as64(feats).reshape(feats.shape[0], -1)           # concat over selected layers
        g = rms_norm(x @ self.fc.T, self.hidden_norm, c.rms_eps)
        out = []
        for lw in self.layers:
            k = (g @ lw["k_w"].T).reshape(-1, c.n_kv_heads, self.d)
            v = (g @ lw["v_w"].T).reshape(-1, c.n_kv_heads, self.d)
            k = rope(rms_norm(k, lw["k_norm"], c.rms_eps), pos, c.rope_theta)
            out.append((k, v))
        return out

    def inject(self, slot: int, feats) -> None:
        """Append rows for `slot` at positions ctx_len..ctx_len+n-1."""
        n = feats.shape[0]
        c0 = self.ctx_len(slot)
        kv = self.project_context(feats, np.arange(c0, c0 + n) + self.pos_offset)
        if slot not in self.cache:
            self.cache[slot] = [[k, v] for k, v in kv]
        else:
            for l, (k, v) in enumerate(kv):
                self.cache[slot][l][0] = np.concatenate([self.cache[slot][l][0], k], axis=0)
                self.cache[slot][l][1] = np.concatenate([self.cache[slot][l][1], v], axis=0)

    # ---- block forward ----
    def block_hidden(self, slot: int, anchor: int, K: int, single_query: bool = False):
        """Residual stream after all layers for the R = K+1 block rows.

        single_query=True evaluates each row's attention separately against the
        same keys (the block-parallel invariant's other side).
        """
        c = self.cfg
        R = K + 1
        C = self.ctx_len(slot)
        ids = np.array([anchor] + [c.mask_token_id] * K)
        X = self.embed[ids] * c.input_embedding_scale
        if self.mask_embedding is not None:
            X[1:] = self.mask_embedding * c.input_embedding_scale
        pos = np.arange(C, C + R) + self.pos_offset
        for l, lw in enumerate(self.layers):
            h = rms_norm(X, lw["in_norm"], c.rms_eps)
            if "attn_conv_base" in lw:
                h = dynamic_conv(h, lw["attn_conv_base"], lw["attn_conv_proj"], c.conv_group)
            q = (h @ lw["q_w"].T).reshape(R, c.n_q_heads, self.d)
            k = (h @ lw["k_w"].T).reshape(R, c.n_kv_heads, self.d)
            v = (h @ lw["v_w"].T).reshape(R, c.n_kv_heads, self.d)
            q = rope(rms_norm(q, lw["q_norm"], c.rms_eps), pos, c.rope_theta)
            k = rope(rms_norm(k, lw["k_norm"], c.rms_eps), pos, c.rope_theta)
            if C > 0:
                keys = np.concatenate([self.cache[slot][l][0], k], axis=0)
                vals = np.concatenate([self.cache[slot][l][1], v], axis=0)
            else:
                keys, vals = k, v
            causal = getattr(c, "causal_block", False)
            if single_query:
                o = np.concatenate([attention(q[i:i + 1], keys, vals, c.group,
                                             (C, [i]) if causal else None) for i in range(R)], axis=0)
            else:
                o = attention(q, keys, vals, c.group, (C, list(range(R))) if causal else None)
            o = o.reshape(R, c.q_dim) @ lw["o_w"].T
            if "attn_conv_post_base" in lw:      # after the attention sub-layer, before the residual add
                o = dynamic_conv(o, lw["attn_conv_post_base"], lw["attn_conv_post_proj"], c.conv_group)
            X = X + o
            h = rms_norm(X, lw["post_norm"], c.rms_eps)
            if "mlp_conv_base" in lw:
                h = dynamic_conv(h, lw["mlp_conv_base"], lw["mlp_conv_proj"], c.conv_group)
            m = (silu(h @ lw["gate_w"].T) * (h @ lw["up_w"].T)) @ lw["down_w"].T
            if "mlp_conv_post_base" in lw:       # after the MLP sub-layer, before the residual add
                m = dynamic_conv(m, lw["mlp_conv_post_base"], lw["mlp_conv_post_proj"], c.conv_group)
            X = X + m
        return X

    def block_logits(self, slot: int, anchor: int, K: int, single_query: bool = False) -> np.ndarray:
        """Logits [K, V] of the mask rows (block positions 1..K)."""
        return self.block_final(slot, anchor, K, single_query)[0]

    def block_final(self, slot: int, anchor: int, K: int, single_query: bool = False):
        """(logits [K, V], final-normalised hidden rows [K, H]) of the mask rows."""
        X = self.block_hidden(slot, anchor, K, single_query)
        h = rms_norm(X[1:], self.final_norm, self.cfg.rms_eps)
        z = (h @ self.lm_head.T) * self.output_multiplier
        if self.logit_softcap > 0:
            z = self.logit_softcap * np.tanh(z / self.logit_softcap)
        return z, h
