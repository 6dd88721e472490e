"""Shared helpers of the GPU parity tests: build a library drafter and the oracle
from the same seeded synthetic inputs, and feed both the same rows."""
from __future__ import annotations

import numpy as np
import torch

from oracle import drafter as od
from synth import gen


def to_cuda(w):
    out = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: v.cuda() for k, v in lw.items()} for lw in w["layers"]]
    return out


def make_pair(cfg, *, max_batch, max_ctx, max_k, max_inject_rows=4096, max_top_k=0, max_tree=0, gains="random",
              seed=1234, lm_head_std=0.02, conv_post=True, **kw):
    """conv_post: with DFlash 2 convolutions, also those after the sub-layers (True), none of
    them (False), or a function editing the merged weights (e.g. dropping one layer's pair)."""
    import block_diffusion_drafter_kv_amd as dk
    w = gen.weights(cfg, seed=seed, gains=gains, lm_head_std=lm_head_std)
    if cfg.conv_group or cfg.sel_rank:
        w = gen.merge_weights(w, gen.dflash2_weights(cfg, seed=seed + 1, post=conv_post is not False))
    if callable(conv_post):
        conv_post(w)
    drafter = dk.Drafter(cfg, to_cuda(w), max_batch=max_batch, max_ctx=max_ctx, max_k=max_k,
                         max_inject_rows=max_inject_rows, max_top_k=max_top_k, max_tree=max_tree, **kw)
    return drafter, od.DrafterOracle(cfg, w), w


def inject_both(drafter, oracle, cfg, slots, counts, pos0, seed=2024):
    """Inject counts[i] rows at positions pos0[i].. for slots[i] into both implementations."""
    rows = [gen.hidden_rows(cfg, s, p, c, seed=seed) for s, p, c in zip(slots, pos0, counts)]
    allrows = torch.cat(rows, dim=0) if sum(counts) else rows[0]
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int32)
    dev = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")
    drafter.inject(dev(slots), dev(starts), dev(counts), int(sum(counts)), allrows.cuda().contiguous())
    for s, r in zip(slots, rows):
        if r.shape[0]:
            oracle.inject(s, r)


def assert_close_report(got, want, atol, rtol=0.0, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: got {got[i]} "
                             f"want {want[i]} (max abs err {err.max():.3e})")
    return float(err.max())
