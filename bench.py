#!/usr/bin/env python3
"""Benchmark of the DFlash drafter hot path on one MI355X.

Workload (default "b32_ragged4k"): a 5-layer Qwen3-8B-shaped bf16 drafter
(hidden 4096, 32/8 heads, SwiGLU 12288, vocab 151936, 5 x 4096 target
features), batch 32 with ragged context lengths uniform in [512, 8192]
(seed 7, mean ~4.3K), K = 16.  One step = the whole hot path over the batch:
  dflash_inject_context (the out_len committed rows of every request),
  dflash_draft_block (K+1 rows per request, greedy),
  dflash_verify (greedy) against synthetic target logits
  (drafter logits + sigma * N(0,1), generated between draft and verify by a
  helper kernel that stands in for the target model and is not timed).
Inputs are synthetic and seeded (weights N(0, 0.02^2) in bf16, target hidden
states N(0, 1) in bf16), resident in HBM before timing starts.  The library
computes with fp16 operands and fp32 accumulation (weights converted once, at
handle creation, to exactly equal fp16 copies scaled by a power of two); the fc
product takes the bf16 operands as given.

Prints one JSON line (see the keys below).  --gpus N > 1 is not supported: the
path runs on one GPU (requests shard across GPUs with no exchange).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_16B_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 MFMA, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_weights(cfg, seed):
    """Seeded N(0, 0.02^2) bf16 weights generated on the GPU (gains 1)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    dt = torch.bfloat16
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab

    def n(*shape):
        return (torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32) * 0.02).to(dt)

    ones = lambda k: torch.ones(k, device="cuda", dtype=dt)
    w = {"embed": n(V, H), "lm_head": n(V, H), "fc": n(H, cfg.feat_dim), "hidden_norm": ones(H),
         "final_norm": ones(H), "layers": []}
    for _ in range(cfg.n_layers):
        w["layers"].append({"in_norm": ones(H), "q_w": n(cfg.q_dim, H), "k_w": n(cfg.kv_dim, H),
                            "v_w": n(cfg.kv_dim, H), "o_w": n(H, cfg.q_dim), "q_norm": ones(cfg.head_dim),
                            "k_norm": ones(cfg.head_dim), "post_norm": ones(H), "gate_w": n(F, H),
                            "up_w": n(F, H), "down_w": n(H, F)})
    return w


def phase_work(cfg, B, K, sum_ctx):
    """Algorithmic flops / bytes per launch of each draft phase (one layer for per-layer phases)."""
    R = K + 1
    M = B * R
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    e = 2
    per_layer_w = cfg.layer_params() * e
    return {
        "qkv": ("mfma", 2.0 * M * H * (cfg.q_dim + 2 * cfg.kv_dim)),
        "o": ("mfma", 2.0 * M * cfg.q_dim * H),
        "gate_up": ("mfma", 2.0 * M * H * 2 * F),
        "down": ("mfma", 2.0 * M * F * H),
        "lm_head": ("mfma", 2.0 * B * K * H * V),
        # one launch reads every context K/V element of one layer once (+ the block's own K/V)
        "attn": ("hbm", float((sum_ctx + B * R) * cfg.kv_dim * 2 * e)),
        "_weights_bytes": ("hbm", float(per_layer_w * cfg.n_layers + V * H * e)),
    }


def cpu_baseline(cfg, K, ctx, sigma, seconds_budget=25.0):
    """The oracle, as it stands, on the host: one request's step (inject 5 rows + draft + verify)."""
    import numpy as np
    import torch

    from oracle import drafter as od
    from oracle import verify as ov
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.time()
    w = gpu_weights(cfg, seed=4321)
    wc = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in w.items() if k != "layers"}
    wc["layers"] = [{k: v.cpu() for k, v in lw.items()} for lw in w["layers"]]
    del w
    torch.cuda.empty_cache()
    orc = od.DrafterOracle(cfg, wc)
    del wc
    rng = np.random.default_rng(0)
    # a context of `ctx` positions already materialised (random K/V, values do not affect timing)
    orc.cache[0] = [[rng.standard_normal((ctx, cfg.n_kv_heads, cfg.head_dim)),
                     rng.standard_normal((ctx, cfg.n_kv_heads, cfg.head_dim))] for _ in range(cfg.n_layers)]
    setup = time.time() - t0
    feats = rng.standard_normal((5, cfg.n_target_layers, cfg.target_hidden))
    times = []
    t_start = time.time()
    while True:
        t1 = time.perf_counter()
        orc.inject(0, feats)
        z = orc.block_logits(0, 7, K)
        t = np.concatenate([z, np.zeros((1, cfg.vocab))]) + sigma * rng.standard_normal((K + 1, cfg.vocab))
        ov.verify_greedy(z.argmax(axis=1), t)
        times.append(time.perf_counter() - t1)
        if time.time() - t_start > seconds_budget or len(times) >= 5:
            break
    per = statistics.median(times)
    return {"value": K / per, "unit": "draft tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} step(s) of one request (ctx {ctx}: inject 5 rows + draft K={K} + greedy "
                      f"verify) in fp64 NumPy; per-request throughput equals whole-batch throughput of a "
                      f"sequential CPU run; setup {setup:.1f}s untimed",
            "seconds_per_request_step": per,
            "host_cpu": _cpu_model(), "os_cpu_count": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = os.path.join(ROOT, "block_diffusion_drafter_kv_amd", "csrc")


def kernel_source_hash():
    """SHA-256 over the HIP sources, so that recorded counter traffic is only used for the code it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCES)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(phase, workload):
    """HBM bytes per launch of a phase's kernel from the FETCH_SIZE / WRITE_SIZE counter runs (profiles/traffic.json,
    calibrated against a plain device copy), or None when absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(phase)
    return None if k is None else k.get("bytes_per_launch")


def copy_calibration():
    """A plain device-to-device copy of a known size, for calibrating FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


def idle_weights(cfg):
    """Zero bf16 weights of the right shapes, one set shared by all layers: a handle that only
    runs selection and verification needs valid weight pointers it never reads."""
    import torch
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    H, F = cfg.hidden, cfg.ffn
    lw = {"in_norm": z(H), "q_w": z(cfg.q_dim, H), "k_w": z(cfg.kv_dim, H), "v_w": z(cfg.kv_dim, H),
          "o_w": z(H, cfg.q_dim), "q_norm": z(cfg.head_dim), "k_norm": z(cfg.head_dim), "post_norm": z(H),
          "gate_w": z(F, H), "up_w": z(F, H), "down_w": z(H, F)}
    return {"embed": z(cfg.vocab, H), "lm_head": z(cfg.vocab, H), "fc": z(H, cfg.feat_dim), "hidden_norm": z(H),
            "final_norm": z(H), "layers": [lw] * cfg.n_layers}


def inject_prompt_measure(w, reps=3):
    """dflash_inject_context at the long-context shape: 4 requests x 32768-row prompts in one call
    (131072 rows of 5 x 4096 bf16 target features, N(0,1)), into an emptied cache each time.

    Algorithmic work per call: fc 2 * N * (L_t * H_t) * H flops, the 5-layer K/V product
    2 * N * H * (L_d * 2 * kv_dim) flops; the per-phase times come from the library's events.
    """
    import numpy as np
    import torch

    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload

    wl = get_workload("b4_ctx32k")
    cfg, B, C = wl.model, wl.batch, wl.ctx
    N = B * C
    dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=C + 64, max_k=wl.K, max_inject_rows=N)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    rows = torch.empty((N, cfg.n_target_layers, cfg.target_hidden), dtype=torch.bfloat16, device="cuda")
    for s0 in range(0, N, 8192):
        rows[s0:s0 + 8192] = torch.randn((8192, cfg.n_target_layers, cfg.target_hidden), generator=g,
                                         device="cuda").to(torch.bfloat16)
    slots, starts, counts = i32(np.arange(B)), i32(np.arange(B) * C), i32(np.full(B, C))
    stream = torch.cuda.current_stream()
    totals, phase_acc = [], {}
    for i in range(reps + 1):
        dr.reset(slots)
        if i > 0:
            dr.profile(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dr.inject(slots, starts, counts, N, rows)
        e1.record(stream)
        torch.cuda.synchronize()
        if i > 0:
            for ph, (ms, n) in dr.profile_read().items():
                phase_acc.setdefault(ph, []).append(ms)
            dr.profile(False)
            totals.append(e0.elapsed_time(e1))
    assert dr.get_error() == 0
    dr.close()
    del rows
    torch.cuda.empty_cache()
    fc_flops = 2.0 * N * cfg.feat_dim * cfg.hidden
    kv_flops = 2.0 * N * cfg.hidden * cfg.n_layers * 2 * cfg.kv_dim
    ph = {k: statistics.median(v) for k, v in phase_acc.items()}
    fc_ms, kv_ms, tot = ph.get("inject_fc", float("nan")), ph.get("inject_kv", float("nan")), statistics.median(totals)
    return {"workload": wl.name, "rows": N, "features": cfg.feat_dim, "reps": reps,
            "ms_per_call": round(tot, 3), "phase_ms": {k: round(v, 3) for k, v in sorted(ph.items())},
            "fc": {"flops": fc_flops, "tflops": round(fc_flops / (fc_ms * 1e-3) / 1e12, 1),
                   "mfma_frac": round(fc_flops / (fc_ms * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4)},
            "kv": {"flops": kv_flops, "tflops": round(kv_flops / (kv_ms * 1e-3) / 1e12, 1),
                   "mfma_frac": round(kv_flops / (kv_ms * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4)},
            "gemm_mfma_frac": round((fc_flops + kv_flops) / ((fc_ms + kv_ms) * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4),
            "call_mfma_frac": round((fc_flops + kv_flops) / (tot * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4)}


def dflash2_measure(w, ctx, steps=10, warmup=2):
    """Draft steps of the same batch-32 workload with the DFlash 2 modules on: dynamic
    convolutions in every layer (group 16) and the path selector (16 candidates, rank 256),
    greedy.  Reports the draft time, the two modules' per-step time from the library's events and
    the overhead against the plain draft; the selector's walk is one work-group per request."""
    import numpy as np
    import torch

    import block_diffusion_drafter_kv_amd as dk
    from synth import gen
    from synth.configs import get_workload, scaled_model

    wl = get_workload("b32_ragged4k")
    cfg = scaled_model(wl.model, conv_group=16, sel_rank=256, sel_cands=16)
    B, K = wl.batch, wl.K
    extra = gen.dflash2_weights(cfg, seed=77)
    dev = lambda t: t.cuda()
    w2 = dict(w)
    w2["layers"] = [dict(a, **{k: dev(v) for k, v in b.items()}) for a, b in zip(w["layers"], extra["layers"])]
    for k in ("sel_pred", "sel_succ", "sel_hidden"):
        w2[k] = dev(extra[k])
    dr = dk.Drafter(cfg, w2, max_batch=B, max_ctx=max(ctx) + 64, max_k=K, max_inject_rows=8192)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(2024)
    for r, c in enumerate(ctx):
        for s0 in range(0, c, 8192):
            n = min(8192, c - s0)
            rows = torch.randn((n, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                               dtype=torch.float32).to(torch.bfloat16)
            dr.inject(i32([r]), i32([0]), i32([n]), n, rows)
    slots = i32(np.arange(B))
    anchors = i32(np.random.default_rng(3).integers(0, cfg.vocab - 1, B))
    stream = torch.cuda.current_stream()
    logits = torch.empty((B, K, cfg.vocab), dtype=torch.float32, device="cuda")   # as the plain draft above
    for _ in range(warmup):
        dr.draft(slots, anchors, K, want_stats=False, logits_out=logits)
    torch.cuda.synchronize()
    marks = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dr.draft(slots, anchors, K, want_stats=False, logits_out=logits)
        e1.record(stream)
        marks.append((e0, e1))
    torch.cuda.synchronize()
    # per-phase breakdown in a separate pass (the events between phases cost time of their own)
    dr.profile(True)
    for _ in range(steps):
        dr.draft(slots, anchors, K, want_stats=False, logits_out=logits)
    torch.cuda.synchronize()
    ph = dr.profile_read()
    dr.profile(False)
    assert dr.get_error() == 0
    dr.close()
    torch.cuda.empty_cache()
    us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in marks)
    per_step = {k: round(v[0] / steps, 4) for k, v in ph.items() if v[1]}
    return {"workload": wl.name, "conv_group": 16, "sel_rank": 256, "sel_cands": 16, "steps": steps,
            "draft_us_median": round(us, 1), "draft_tokens_per_s": round(B * K / (us * 1e-6), 1),
            "conv_ms_per_step": per_step.get("conv"), "selector_ms_per_step": per_step.get("selector"),
            "phase_ms_per_step": dict(sorted(per_step.items(), key=lambda x: -x[1]))}


def inject_rows_measure(w, reps=10):
    """Per-step injection on the batch-32 workload at 1, 5 and 17 committed rows per request (5 is
    the middle of the pages' 4-6 accepted tokens; random weights commit about one): median us per
    call of dflash_inject_context with the row counts on the device and the same bound (B * (K+1))."""
    import numpy as np
    import torch
    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload
    wl = get_workload("b32_ragged4k")
    cfg, B, K = wl.model, wl.batch, wl.K
    R = K + 1
    ctx0 = 4096
    dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=ctx0 + 3 * (reps + 2) * R + 64, max_k=K, max_inject_rows=8192)
    _fill_prompts(dr, cfg, [ctx0] * B, 2026)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(78)
    pool = torch.randn((B * R, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)
    slots, row_start = i32(np.arange(B)), i32(np.arange(B) * R)
    out = {}
    for n in (1, 5, 17):
        counts = i32(np.full(B, n))
        out["rows_%d" % n] = round(_timed(lambda: dr.inject(slots, row_start, counts, B * R, pool), reps), 1)
    assert dr.get_error() == 0
    dr.close()
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": B, "row_bound": B * R, "reps": reps, "us_per_call": out}


def dflash2_b1_measure(w, steps=20):
    """The DFlash 2 modules at the pages' scale: batch 1, context 2048, K = 16, greedy; the plain
    draft and the draft with both modules (conv group 16, 16 candidates, rank 256) on handles that
    differ only in the modules, timed alternately on the same device."""
    import numpy as np
    import torch
    import block_diffusion_drafter_kv_amd as dk
    from synth import gen
    from synth.configs import get_workload, scaled_model
    wl = get_workload("b1_ctx2k")
    cfg, B, K = wl.model, wl.batch, wl.K
    cfg2 = scaled_model(cfg, conv_group=16, sel_rank=256, sel_cands=16)
    extra = gen.dflash2_weights(cfg2, seed=77)
    dev = lambda t: t.cuda()
    w2 = dict(w)
    w2["layers"] = [dict(a, **{k: dev(v) for k, v in b.items()}) for a, b in zip(w["layers"], extra["layers"])]
    for k in ("sel_pred", "sel_succ", "sel_hidden"):
        w2[k] = dev(extra[k])
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    handles = []
    for c, ww in ((cfg, w), (cfg2, w2)):
        dr = dk.Drafter(c, ww, max_batch=B, max_ctx=wl.ctx + 64, max_k=K, max_inject_rows=8192)
        _fill_prompts(dr, c, [wl.ctx], 2025)
        handles.append(dr)
    slots = i32(np.arange(B))
    anchors = i32(np.random.default_rng(3).integers(0, cfg.vocab - 1, B))
    logits = torch.empty((B, K, cfg.vocab), dtype=torch.float32, device="cuda")
    times = []
    for dr in handles:
        times.append(_timed(lambda: dr.draft(slots, anchors, K, want_stats=False, logits_out=logits), steps))
    # a second round in the opposite order, against drift of the clocks
    for i, dr in reversed(list(enumerate(handles))):
        times[i] = min(times[i], _timed(lambda: dr.draft(slots, anchors, K, want_stats=False, logits_out=logits),
                                        steps))
    for dr in handles:
        assert dr.get_error() == 0
        dr.close()
    del w2, extra
    torch.cuda.empty_cache()
    return {"workload": wl.name, "batch": B, "ctx": wl.ctx, "steps": steps, "draft_plain_us": round(times[0], 1),
            "draft_dflash2_us": round(times[1], 1), "overhead_vs_plain_draft": round(times[1] / times[0] - 1.0, 4)}


def _timed(fn, steps, warmup=2):
    """Median microseconds of fn() over `steps` calls on torch's current stream (after `warmup`)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    marks = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        marks.append((e0, e1))
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in marks)


def variants_measure(w, ctx, steps=10):
    """The sampling and attention variants on the batch-32 workload: the draft with the
    causal-in-block mask, and with a paged cache (256-position pages scattered over the pool by
    a shuffled table), against the plain draft; sampled drafting (T = 1) and
    rejection verification (T = 1, K = 16, V = 151936) without and with symmetric truncation
    (top_k 50, top_p 0.9).  Verification bytes: one read of the K+1 target and K draft fp32 rows
    per request."""
    import numpy as np
    import torch

    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload, scaled_model

    wl = get_workload("b32_ragged4k")
    B, K, V = wl.batch, wl.K, wl.model.vocab
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    out = {"workload": wl.name, "steps": steps}
    slots = i32(np.arange(B))
    anchors = i32(np.random.default_rng(3).integers(0, V - 1, B))
    logits = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    page = 256
    for mode in ("plain", "causal", "paged"):
        causal = mode == "causal"
        cfg = scaled_model(wl.model, causal_block=causal)
        mctx = max(ctx) + 64
        kw = {}
        if mode == "paged":   # 256-position pages, each request's pages scattered over the pool
            per_slot = -(-mctx // page)
            kw = {"page_size": page, "num_pages": B * per_slot}
        dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=mctx, max_k=K, max_inject_rows=8192, **kw)
        if mode == "paged":
            perm = np.random.default_rng(11).permutation(B * per_slot).astype(np.int32)
            dr.set_page_table(torch.tensor(perm.reshape(B, per_slot), device="cuda"))
        g = torch.Generator(device="cuda").manual_seed(2024)
        for r, c in enumerate(ctx):
            for s0 in range(0, c, 8192):
                n = min(8192, c - s0)
                rows = torch.randn((n, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                                   dtype=torch.float32).to(torch.bfloat16)
                dr.inject(i32([r]), i32([0]), i32([n]), n, rows)
        us = _timed(lambda: dr.draft(slots, anchors, K, want_stats=False, logits_out=logits), steps)
        out[f"draft_{mode}_us"] = round(us, 1)
        if mode != "plain":
            assert dr.get_error() == 0
            dr.close()
            continue
        # sampled drafting and verification on this drafter's logits (drafts drawn under each mode)
        dr.draft(slots, anchors, K, want_stats=False, logits_out=logits)
        gt = torch.Generator(device="cuda").manual_seed(7)
        target = torch.cat([logits, torch.zeros((B, 1, V), device="cuda")], dim=1)
        target += torch.randn(target.shape, generator=gt, device="cuda") * 0.5
        vb = (B * (2 * K + 1) * V * 4)
        for name, (tk, tp) in (("plain", (0, 1.0)), ("trunc_k50_p0.9", (50, 0.9))):
            dr.set_sampling(tk, tp)
            d_ids = dr.draft(slots, anchors, K, temperature=1.0, seed=1, step=0, want_stats=False,
                             logits_out=logits)["draft_ids"].clone()
            res = {}
            res["draft_t1_us"] = round(_timed(lambda: dr.draft(slots, anchors, K, temperature=1.0, seed=1, step=0,
                                                                want_stats=False, logits_out=logits), steps), 1)
            vo = dr.verify(slots, d_ids, logits, target, temperature=1.0, seed=2, step=0)
            us = _timed(lambda: dr.verify(slots, d_ids, logits, target, temperature=1.0, seed=2, step=0, out=vo),
                        steps)
            res["verify_t1_us"] = round(us, 1)
            res["verify_algorithmic_bytes"] = vb
            res["verify_hbm_frac"] = round(vb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            res["mean_committed"] = round(float(vo["out_len"].float().mean().item()), 3)
            out[name] = res
        dr.set_sampling(0, 1.0)
        assert dr.get_error() == 0
        dr.close()
        del target
    torch.cuda.empty_cache()
    out["causal_overhead_vs_plain"] = round(out["draft_causal_us"] / out["draft_plain_us"] - 1.0, 4)
    out["paged_overhead_vs_plain"] = round(out["draft_paged_us"] / out["draft_plain_us"] - 1.0, 4)
    out["page_size"] = page
    return out


def tree_verify_measure(reps=20):
    """dflash_verify_tree at the batch-64 tree shape (64 requests, 65-node best-first trees from
    top-64 marginals, K = 16, V = 151936), greedy and T = 1.

    Trees: the library's builder over peaked synthetic marginals (N(0,1) plus 12.5 on one token per
    position), which gives a deep spine beside bushy first levels.  Target rows: scale * N(0,1) plus a
    bump on one token per node (a child's token with probability 0.8, the first-popped child two times
    in three; else a random token), scale 1 / bump 6 for greedy, 3 / 20 for sampling.  The walk reads
    one fp32 row per visited node (out_len rows per request); algorithmic bytes = rows read * V * 4.
    """
    import numpy as np
    import torch

    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload

    wl = get_workload("b64_tree")
    cfg, B, K, V, Bt = wl.model, wl.batch, wl.K, wl.model.vocab, wl.tree_budget
    nn = Bt + 1
    dr = dk.Drafter(cfg, idle_weights(cfg), max_batch=B, max_ctx=64, max_k=K, max_inject_rows=64,
                    max_top_k=wl.top_k, max_tree=Bt)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(52)
    z = torch.randn((B, K, V), generator=g, device="cuda")
    hot = torch.randint(0, V, (B, K, 1), generator=g, device="cuda")
    z.scatter_add_(2, hot, torch.full((B, K, 1), 12.5, device="cuda"))
    slots = i32(np.arange(B))
    o = dr.select_from_logits(slots, i32(np.arange(B) + 7), z, temperature=1.0, seed=1, step=0, top_k=wl.top_k,
                              tree_budget=Bt)
    del z
    tok, par = o["tree_tokens"].cpu().numpy(), o["tree_parents"].cpu().numpy()
    rng = np.random.default_rng(53)
    bump_tok = np.empty((B, nn), np.int64)
    for r in range(B):
        for u in range(nn):
            kids = [int(tok[r, c]) for c in range(nn) if par[r, c] == u]
            if kids and rng.random() < 0.8:
                bump_tok[r, u] = kids[0] if rng.random() < 2 / 3 else kids[rng.integers(0, len(kids))]
            else:
                bump_tok[r, u] = rng.integers(0, V)
    idx = torch.tensor(bump_tok, device="cuda")[..., None]
    stream = torch.cuda.current_stream()
    out = {}
    for T, scale, bump in ((0.0, 1.0, 6.0), (1.0, 3.0, 20.0)):
        t = torch.randn((B, nn, V), generator=g, device="cuda") * scale
        t.scatter_add_(2, idx, torch.full((B, nn, 1), bump, device="cuda"))
        marks, lens, res = [], [], None
        for i in range(reps + 3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            res = dr.verify_tree(slots, K, o["tree_tokens"], o["tree_parents"], t, temperature=T, seed=4, step=i,
                                 out=res)
            e1.record(stream)
            marks.append((e0, e1))
            lens.append(res["out_len"].clone())
        torch.cuda.synchronize()
        assert dr.get_error() == 0
        us = [a.elapsed_time(b) * 1e3 for a, b in marks[3:]]
        ls = [x.cpu().numpy() for x in lens[3:]]
        med = statistics.median(us)
        rows = float(np.mean([x.sum() for x in ls]))
        deepest = float(np.mean([x.max() for x in ls]))
        nbytes = rows * V * 4
        out["greedy" if T == 0.0 else "t1"] = {
            "us_median": round(med, 1), "rows_read_per_call": round(rows, 1),
            "mean_out_len": round(rows / B, 3), "deepest_walk_rows": round(deepest, 2),
            "algorithmic_bytes": round(nbytes), "achieved_GBs": round(nbytes / (med * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "us_per_row_of_deepest_walk": round(med / deepest, 2)}
        del t
    dr.close()
    torch.cuda.empty_cache()
    return {"workload": "b64_tree", "batch": B, "nodes": nn, "K": K, "vocab": V, "reps": reps,
            "target_rows_bytes_if_all_read": B * nn * V * 4, **out}


def _draft_bytes_flops(cfg, B, K, sum_ctx):
    """Algorithmic bytes (weights once, context K/V once per layer) and flops of one draft step."""
    R = K + 1
    w = phase_work(cfg, B, K, sum_ctx)
    nbytes = w["_weights_bytes"][1] + w["attn"][1] * cfg.n_layers
    layer_flops = w["qkv"][1] + w["o"][1] + w["gate_up"][1] + w["down"][1]
    attn_flops = 4.0 * cfg.n_q_heads * R * cfg.head_dim * (sum_ctx + B * R)
    flops = cfg.n_layers * (layer_flops + attn_flops) + w["lm_head"][1]
    return nbytes, flops


def _fill_prompts(dr, cfg, ctx, seed, chunk=8192):
    """Untimed prompt injection of every request (rows N(0,1) drawn on the GPU)."""
    import numpy as np
    import torch
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed)
    for r, c in enumerate(ctx):
        for s0 in range(0, c, chunk):
            n = min(chunk, c - s0)
            rows = torch.randn((n, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                               dtype=torch.float32).to(torch.bfloat16)
            dr.inject(i32([r]), i32([0]), i32([n]), n, rows)


def _loop(dr, cfg, B, K, steps, temperature, sigma, seed, pool_seed, warmup=2):
    """The decode cycle chained on the device, as in main(): inject the out_len committed rows of each
    request, draft at the next anchor, synthetic target (drafter logits + sigma N(0,1), not timed),
    verify (greedy, or rejection sampling at `temperature`).  Per-call medians (us), mean out_len."""
    import numpy as np
    import torch
    import ctypes
    import block_diffusion_drafter_kv_amd as dk
    R = K + 1
    V = cfg.vocab
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(pool_seed)
    pool = torch.randn((B * R, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)
    slots, row_start = i32(np.arange(B)), i32(np.arange(B) * R)
    logits = torch.empty((B, K, V), dtype=torch.float32, device="cuda")
    target = torch.empty((B, R, V), dtype=torch.float32, device="cuda")
    vout = {"out_tokens": torch.empty((B, R), dtype=torch.int32, device="cuda"), "out_len": i32(np.ones(B)),
            "accept_len": torch.empty((B,), dtype=torch.int32, device="cuda"),
            "next_anchor": i32(np.random.default_rng(3).integers(0, V - 1, B))}
    stream = torch.cuda.current_stream()
    cs = ctypes.c_void_p(stream.cuda_stream)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks, lens = [], []
    for i in range(warmup + steps):
        e = [ev() for _ in range(6)]
        e[0].record(stream)
        dr.inject(slots, row_start, vout["out_len"], B * R, pool)
        e[1].record(stream)
        o = dr.draft(slots, vout["next_anchor"], K, temperature=temperature, seed=seed, step=i, want_stats=False,
                     logits_out=logits)
        e[2].record(stream)
        dk.dflash_synth_target_logits(cs, B, K, V, logits.data_ptr(), sigma, seed + 1, i, target.data_ptr())
        e[3].record(stream)
        dr.verify(slots, o["draft_ids"], logits if temperature > 0 else None, target, temperature=temperature,
                  seed=seed, step=i, out=vout)
        e[4].record(stream)
        if i >= warmup:
            marks.append(e)
            lens.append(vout["out_len"].clone())
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    med = lambda a, b: round(statistics.median(m[a].elapsed_time(m[b]) * 1e3 for m in marks), 1)
    mean_len = float(torch.stack(lens).float().mean().item())
    inj, dra, ver = med(0, 1), med(1, 2), med(3, 4)
    return {"steps": steps, "temperature": temperature, "sigma": sigma, "inject_us": inj, "draft_us": dra,
            "verify_us": ver, "step_us": round(inj + dra + ver, 1), "mean_committed_per_verify": round(mean_len, 3),
            "committed_tokens_per_s": round(B * mean_len / ((inj + dra + ver) * 1e-6), 1)}


def c2_measure(w, steps=20):
    """Batch 1, context 2048, K = 16, greedy: the weight-streaming draft step."""
    import numpy as np
    import torch
    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload
    wl = get_workload("b1_ctx2k")
    cfg, B, K = wl.model, wl.batch, wl.K
    dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=wl.ctx + (steps + 4) * (K + 1) + 64, max_k=K,
                    max_inject_rows=8192)
    _fill_prompts(dr, cfg, [wl.ctx], 2025)
    res = _loop(dr, cfg, B, K, steps, 0.0, wl.sigma, 11, 31)
    sum_ctx = dr.ctx_lens()[:B].sum().item()
    nbytes, flops = _draft_bytes_flops(cfg, B, K, sum_ctx)
    t = res["draft_us"] * 1e-6
    res.update({"workload": wl.name, "batch": B, "ctx": wl.ctx, "draft_tokens_per_s": round(B * K / t, 1),
                "draft_algorithmic_bytes": nbytes, "draft_hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                "draft_mfma_frac": round(flops / t / 1e12 / PEAK_16B_TFLOPS, 4)})
    dr.close()
    torch.cuda.empty_cache()
    return res


def c4_measure(w, steps=50):
    """Batch 4: 32768-row prompts injected in one call (timed), then 50 cycles with T = 1 drafting and
    rejection-sampling verification (Philox seed 99)."""
    import numpy as np
    import torch
    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload
    wl = get_workload("b4_ctx32k")
    cfg, B, K, C = wl.model, wl.batch, wl.K, wl.ctx
    N = B * C
    dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=C + (steps + 4) * (K + 1) + 64, max_k=K, max_inject_rows=N)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(78)
    rows = torch.empty((N, cfg.n_target_layers, cfg.target_hidden), dtype=torch.bfloat16, device="cuda")
    for s0 in range(0, N, 8192):
        rows[s0:s0 + 8192] = torch.randn((8192, cfg.n_target_layers, cfg.target_hidden), generator=g,
                                         device="cuda").to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    dr.inject(i32(np.arange(B)), i32(np.arange(B) * C), i32(np.full(B, C)), N, rows)
    e1.record(stream)
    torch.cuda.synchronize()
    inject_ms = e0.elapsed_time(e1)
    del rows
    torch.cuda.empty_cache()
    res = _loop(dr, cfg, B, K, steps, wl.temperature, wl.sigma, wl.philox_seed, 32)
    sum_ctx = dr.ctx_lens()[:B].sum().item()
    nbytes, flops = _draft_bytes_flops(cfg, B, K, sum_ctx)
    t = res["draft_us"] * 1e-6
    inj_flops = 2.0 * N * cfg.feat_dim * cfg.hidden + 2.0 * N * cfg.hidden * cfg.n_layers * 2 * cfg.kv_dim
    res.update({"workload": wl.name, "batch": B, "prompt": C, "prompt_inject_ms": round(inject_ms, 3),
                "prompt_inject_mfma_frac": round(inj_flops / (inject_ms * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4),
                "draft_tokens_per_s": round(B * K / t, 1), "draft_algorithmic_bytes": nbytes,
                "draft_hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
                "verify_algorithmic_bytes": B * (2 * K + 1) * cfg.vocab * 4})
    res["verify_hbm_frac"] = round(res["verify_algorithmic_bytes"] / (res["verify_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    dr.close()
    torch.cuda.empty_cache()
    return res


def c5_measure(steps=10):
    """The larger drafter (hidden 5120, 64/8 heads, SwiGLU 17408, fc 25600 -> 5120), batch 64 at
    context 8192: a T = 1 draft with per-position top-64 and the best-first B = 64 tree + mask."""
    import numpy as np
    import torch
    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload
    wl = get_workload("b64_tree")
    cfg, B, K, C = wl.model, wl.batch, wl.K, wl.ctx
    w = gpu_weights(cfg, seed=4321)
    dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=C + 64, max_k=K, max_inject_rows=32768, max_top_k=wl.top_k,
                    max_tree=wl.tree_budget)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(79)
    per = 32768 // C
    stream = torch.cuda.current_stream()
    inj_ms = 0.0
    for r0 in range(0, B, per):
        rows = torch.randn((per * C, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                           dtype=torch.float32).to(torch.bfloat16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dr.inject(i32(np.arange(r0, r0 + per)), i32(np.arange(per) * C), i32(np.full(per, C)), per * C, rows)
        e1.record(stream)
        torch.cuda.synchronize()
        inj_ms += e0.elapsed_time(e1)
        del rows
    assert dr.get_error() == 0
    slots = i32(np.arange(B))
    anchors = i32(np.random.default_rng(5).integers(0, cfg.vocab - 1, B))
    us = _timed(lambda: dr.draft(slots, anchors, K, temperature=1.0, seed=1, step=0, top_k=wl.top_k,
                                 tree_budget=wl.tree_budget, want_stats=False), steps)
    us_plain = _timed(lambda: dr.draft(slots, anchors, K, temperature=1.0, seed=1, step=0, want_stats=False), steps)
    assert dr.get_error() == 0
    nbytes, flops = _draft_bytes_flops(cfg, B, K, B * C)
    N = B * C
    inj_flops = 2.0 * N * cfg.feat_dim * cfg.hidden + 2.0 * N * cfg.hidden * cfg.n_layers * 2 * cfg.kv_dim
    dr.close()
    del w
    torch.cuda.empty_cache()
    t = us * 1e-6
    return {"workload": wl.name, "batch": B, "ctx": C, "hidden": cfg.hidden, "top_k": wl.top_k,
            "tree_budget": wl.tree_budget, "steps": steps, "draft_topk_tree_us": round(us, 1),
            "draft_only_us": round(us_plain, 1), "draft_tokens_per_s": round(B * K / t, 1),
            "draft_algorithmic_bytes": nbytes, "draft_flops": flops,
            "draft_hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4),
            "draft_mfma_frac": round(flops / t / 1e12 / PEAK_16B_TFLOPS, 4),
            "setup_inject_rows": N, "setup_inject_ms": round(inj_ms, 2),
            "setup_inject_mfma_frac": round(inj_flops / (inj_ms * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b32_ragged4k")
    ap.add_argument("--sigma", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tree", action="store_true", help="skip the tree verifier walk measurement")
    ap.add_argument("--no-inject", action="store_true", help="skip the long-prompt injection measurement")
    ap.add_argument("--no-dflash2", action="store_true", help="skip the DFlash 2 modules measurement")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the causal-mask / sampled / truncated draft and verify measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (batch 1 / batch 4 long context / larger drafter) and the sigma sweep")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the drafter hot path shards by request with no exchange "
              "between GPUs; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_diffusion_drafter_kv_amd as dk
    from synth.configs import get_workload

    wl = get_workload(args.workload)
    cfg = wl.model
    B, K = wl.batch, wl.K
    R = K + 1
    sigma = wl.sigma if args.sigma is None else args.sigma
    if wl.temperature != 0.0 or wl.tree_budget:
        print(f"workload {wl.name} is a parity configuration; bench.py times the greedy hot path",
              file=sys.stderr)
    dk.load()
    torch.cuda.set_device(0)
    ctx = wl.ctx_lengths()
    sweep = [0.5, 1.5, 3.0, 0.1] if not args.no_configs else []
    sweep_steps = 15
    total_steps = args.warmup + args.steps + 4 + len(sweep) * (sweep_steps + 2)
    max_ctx = max(ctx) + total_steps * R + 64
    log(f"[bench] workload {wl.name}: B={B} K={K} ctx mean {np.mean(ctx):.0f} (sum {sum(ctx)}), sigma {sigma}")

    t0 = time.time()
    w = gpu_weights(cfg, seed=1234)
    dr = dk.Drafter(cfg, w, max_batch=B, max_ctx=max_ctx, max_k=K, max_inject_rows=8192)
    i32 = lambda a: torch.tensor(np.asarray(a), dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(2024)
    # prompt injection, untimed (one call per request, rows generated on the GPU)
    for r, c in enumerate(ctx):
        for s0 in range(0, c, 8192):
            n = min(8192, c - s0)
            rows = torch.randn((n, cfg.n_target_layers, cfg.target_hidden), generator=gen, device="cuda",
                               dtype=torch.float32).to(torch.bfloat16)
            dr.inject(i32([r]), i32([0]), i32([n]), n, rows)
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    log(f"[bench] setup (weights + {sum(ctx)} prompt rows injected) {time.time() - t0:.1f}s")

    # per-step inputs: a pool of target hidden rows for the committed positions (N(0,1))
    pool = torch.randn((B * R, cfg.n_target_layers, cfg.target_hidden), generator=gen, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)
    slots = i32(np.arange(B))
    row_start = i32(np.arange(B) * R)
    anchors = i32(np.random.default_rng(3).integers(0, cfg.vocab - 1, B))
    out_len = i32(np.ones(B))           # the first step commits the anchor row of every request
    logits = torch.empty((B, K, cfg.vocab), dtype=torch.float32, device="cuda")
    target = torch.empty((B, R, cfg.vocab), dtype=torch.float32, device="cuda")
    vout = {"out_tokens": torch.empty((B, R), dtype=torch.int32, device="cuda"), "out_len": out_len,
            "accept_len": torch.empty((B,), dtype=torch.int32, device="cuda"),
            "next_anchor": anchors}
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(i, marks=None):
        e = [ev() for _ in range(6)] if marks is not None else None
        if e: e[0].record(stream)
        dr.inject(slots, row_start, vout["out_len"], B * R, pool)
        if e: e[1].record(stream)
        if e: e[2].record(stream)
        o = dr.draft(slots, vout["next_anchor"], K, temperature=0.0, logits_out=logits, want_stats=False)
        if e: e[3].record(stream)
        dk.dflash_synth_target_logits(ctypes_stream(), B, K, cfg.vocab, logits.data_ptr(), sigma, 99, i,
                                      target.data_ptr())
        if e: e[4].record(stream)
        dr.verify(slots, o["draft_ids"], None, target, temperature=0.0, out=vout)
        if e: e[5].record(stream)
        if marks is not None:
            marks.append(e)

    def ctypes_stream():
        import ctypes
        return ctypes.c_void_p(stream.cuda_stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ctx_before = dr.ctx_lens()[:B].sum().item()

    # phase breakdown (separate, untimed pass over 3 steps with per-phase events)
    dr.profile(True)
    for i in range(3):
        step(args.warmup + i)
    torch.cuda.synchronize()
    phases = dr.profile_read()
    dr.profile(False)
    ctx_before = dr.ctx_lens()[:B].sum().item()

    # timed region
    marks = []
    accepted = []
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + 3 + i, marks)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ctx_after = dr.ctx_lens()[:B].sum().item()
    assert dr.get_error() == 0
    inj = [m[0].elapsed_time(m[1]) for m in marks]
    dra = [m[2].elapsed_time(m[3]) for m in marks]
    ver = [m[4].elapsed_time(m[5]) for m in marks]
    per_step = [a + b + c for a, b, c in zip(inj, dra, ver)]
    ms_step = statistics.mean(per_step)
    mean_out_len = (ctx_after - ctx_before) / (B * args.steps)   # rows committed per request per step

    # dominant kernel phase and its roofline
    n_steps_prof = 3
    sum_ctx_mid = (ctx_before + ctx_after) / 2.0
    work = phase_work(cfg, B, K, sum_ctx_mid)
    per_launch = {p: (ms / max(n, 1), n) for p, (ms, n) in phases.items() if n}
    totals = {p: ms / n_steps_prof for p, (ms, n) in phases.items() if n}
    dom = max((p for p in totals if p in work), key=lambda p: totals[p])
    bound, amount = work[dom]
    avg_ms = per_launch[dom][0]
    if bound == "mfma":
        achieved = amount / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_16B_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_16B_TFLOPS, 4), "traffic": recorded_traffic(dom, wl.name),
                "algorithmic_per_launch": amount, "avg_launch_ms": round(avg_ms, 4)}
    else:
        achieved = amount / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(dom, wl.name),
                "algorithmic_per_launch": amount, "avg_launch_ms": round(avg_ms, 4)}

    # whole-step HBM roofline of the draft (algorithmic bytes: weights once + context K/V once per layer)
    draft_bytes, draft_flops = _draft_bytes_flops(cfg, B, K, sum_ctx_mid)
    draft_ms = statistics.median(dra)
    # phase-wise floor: each phase at the larger of its HBM time (bytes / 8 TB/s) and MFMA time (flops / 2.5 PF)
    pw = phase_work(cfg, B, K, sum_ctx_mid)
    lw_bytes = cfg.layer_params() * 2
    gemm_fl = pw["qkv"][1] + pw["o"][1] + pw["gate_up"][1] + pw["down"][1]
    attn_fl = 4.0 * cfg.n_q_heads * R * cfg.head_dim * (sum_ctx_mid + B * R)
    phase_floor_us = 1e6 * (cfg.n_layers * (max(lw_bytes / (PEAK_HBM_GBS * 1e9), gemm_fl / (PEAK_16B_TFLOPS * 1e12))
                                            + max(pw["attn"][1] / (PEAK_HBM_GBS * 1e9),
                                                  attn_fl / (PEAK_16B_TFLOPS * 1e12)))
                            + max(cfg.vocab * cfg.hidden * 2 / (PEAK_HBM_GBS * 1e9),
                                  pw["lm_head"][1] / (PEAK_16B_TFLOPS * 1e12)))
    result = {
        "metric": "draft tokens/s (5-layer, K=16, ctx 4K, B=32)",
        "value": round(B * K / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,0.02^2) bf16 weights, N(0,1) bf16 target features; fp16 operands, "
                "fp32 accumulation; target logits = drafter logits + sigma*N(0,1))",
        "config": {"workload": wl.name, "batch": B, "K": K, "ctx": "uniform[512,8192] seed 7",
                   "mean_ctx_start": round(sum(ctx) / B, 1), "layers": cfg.n_layers, "hidden": cfg.hidden,
                   "heads": f"{cfg.n_q_heads}/{cfg.n_kv_heads}x{cfg.head_dim}", "ffn": cfg.ffn,
                   "vocab": cfg.vocab, "target_features": f"{cfg.n_target_layers}x{cfg.target_hidden}",
                   "verify": "greedy", "sigma": sigma, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "draft_step": {"us_median": round(draft_ms * 1e3, 1),
                       "hbm_roofline_frac": round(draft_bytes / (draft_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                       "algorithmic_bytes": draft_bytes, "algorithmic_flops": draft_flops,
                       "mfma_roofline_frac": round(draft_flops / (draft_ms * 1e-3) / 1e12 / PEAK_16B_TFLOPS, 4),
                       "phase_floor_us": round(phase_floor_us, 1),
                       "frac_of_phase_floor": round(phase_floor_us / (draft_ms * 1e3), 4)},
        "draft_us_median": round(draft_ms * 1e3, 1),
        "draft_only_tokens_per_s": round(B * K / (draft_ms * 1e-3), 1),
        "draft_hbm_roofline_frac": round(draft_bytes / (draft_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "draft_algorithmic_bytes": draft_bytes,
        "inject_us_median": round(statistics.median(inj) * 1e3, 1),
        "verify_us_median": round(statistics.median(ver) * 1e3, 1),
        "cycle_ms_wall_incl_synthetic_target": round(t_wall / args.steps * 1e3, 4),
        "mean_committed_per_verify": round(mean_out_len, 3),
        "phase_ms_per_step": {p: round(t, 4) for p, t in sorted(totals.items(), key=lambda x: -x[1])},
    }
    # the batch-32 workload at the configuration's other noise levels, and at a noise level calibrated so that
    # a verify commits the pages' 4-6 tokens (random weights accept far less at sigma 1.5)
    if sweep:
        log("[bench] sigma sweep on the batch-32 workload ...")
        result["sigma_sweep"] = [_loop(dr, cfg, B, K, sweep_steps, 0.0, sg, 21 + j, 40 + j)
                                 for j, sg in enumerate(sweep)]
    dr.close()
    torch.cuda.empty_cache()
    if not args.no_configs:
        log("[bench] batch 1, context 2048 ...")
        result.setdefault("configs", {})["b1_ctx2k"] = c2_measure(w)
        log("[bench] batch 4, 32768-row prompts in one call, 50 T=1 cycles ...")
        result["configs"]["b4_ctx32k"] = c4_measure(w)
    if not args.no_inject:
        log("[bench] prompt injection (4 x 32768 rows, one call) ...")
        result["inject_prompt"] = inject_prompt_measure(w)
        log("[bench] per-step injection at 1, 5 and 17 rows per request ...")
        result["inject_step_rows"] = inject_rows_measure(w)
    if not args.no_dflash2:
        log("[bench] DFlash 2 modules (conv + selector) on the same workload ...")
        d2 = dflash2_measure(w, ctx)
        d2["overhead_vs_plain_draft"] = round(d2["draft_us_median"] / (draft_ms * 1e3) - 1.0, 4)
        log("[bench] DFlash 2 modules at batch 1 (context 2048) ...")
        d2["b1_ctx2k"] = dflash2_b1_measure(w)
        result["dflash2"] = d2
    if not args.no_variants:
        log("[bench] sampling and attention variants on the same workload ...")
        result["variants"] = variants_measure(w, ctx)
    del w
    torch.cuda.empty_cache()
    if not args.no_configs:
        log("[bench] larger drafter, batch 64, context 8192, top-64 + tree ...")
        result.setdefault("configs", {})["b64_tree"] = c5_measure()
    if not args.no_tree:
        log("[bench] tree verify walk (batch 64, 65-node trees) ...")
        result["tree_verify"] = tree_verify_measure()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(cfg, K, ctx=4096, sigma=sigma)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
