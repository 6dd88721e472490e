"""The decode cycle over several steps, chained on the device [P2 §2.1 steps 1-6;
P4 §4.2, §5.6]: verify -> inject the committed rows (row count = verify's out_len,
a device array) -> draft at the next anchor (verify's last emitted token, a
device array), with no host round trip between the calls.

The oracle follows sampled requests step by step with the same seeded inputs:
the same prompt rows, the same hidden rows for each step's committed positions,
and the same fp32 target logits.  Target logits are built on the host from the
oracle's own logits and decisions (never from the library's outputs), with a
planned acceptance length per request and step, so that the cycle's outcome
(out_len, the emitted tokens, the next anchor, ctx_len) is unique whatever the
library's rounding does at near-ties:
  * greedy: the target's argmax at block row i-1 is the oracle's draft d_i for
    i <= a (only where the oracle's top-2 margin clears twice the logit
    tolerance, so the library must draft the same id), then a token x outside
    the top-2 of the next position (a rejection whichever near-tied id the
    library drafted);
  * T = 1 rejection sampling (Philox): rows i-1 <= a equal the oracle's drafter
    logits (p / q within exp(+-4e-2) for every token, so with the accept test's
    uniform below 0.85 -- known from the Philox stream -- every drafted token is
    accepted), then a row holding a bump of 60 on x (every drafted token is
    rejected, and the residual, or the bonus row, puts all its mass on x).
Each request-step checks the logits against the oracle forward (2e-2, max error
logged), the out_len, the emitted tokens (the accepted drafts against the
oracle's wherever its decision is clear of the tolerance), the next anchor and
the context length after the injection.
"""
import numpy as np
import pytest
import torch

from oracle import drafter as od
from oracle import philox
from oracle import select as osel
from synth import gen
from synth.configs import get_workload

from gpu_helpers import assert_close_report, to_cuda
from parity_checks import Tally

pytestmark = pytest.mark.gpu

LOGIT_TOL = 2e-2


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _gpu_rows(cfg, n, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn((n, cfg.n_target_layers, cfg.target_hidden), generator=g, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)


def _plan_greedy(z, rng, V):
    """Planned acceptance for a greedy step from the oracle's logits z [K, V]."""
    K = z.shape[0]
    d, decided = [], 0
    for j in range(K):
        top, margin = osel.argmax_with_margin(z[j])
        d.append(top)
        if decided == j and margin > 2 * LOGIT_TOL:
            decided += 1
    a = int(min(decided, rng.integers(2, 8)))
    x = int(rng.integers(0, V - 1))
    if a < K:   # every id the library may draft at position a + 1 (within twice the tolerance of the max)
        excl = set(int(i) for i in np.nonzero(z[a] >= z[a].max() - 2 * LOGIT_TOL)[0])
        while x in excl:
            x = int(rng.integers(0, V - 1))
    return a, d, x


def _plan_rejection(z, rng, V, seed, slot, step):
    """Planned acceptance for a T = 1 step: accept tests whose Philox uniform is below 0.85."""
    K = z.shape[0]
    a = 0
    cap = int(rng.integers(1, 4))
    while a < min(K, cap) and philox.uniform(seed, slot, step, a + 1, philox.PURPOSE_ACCEPT) < 0.85:
        a += 1
    return a, int(rng.integers(0, V - 1))


def _run_cycle(gpu_lib, wl, ctx, followed, steps, T, one_call_prompt):
    cfg, K, B, V = wl.model, wl.K, wl.batch, wl.model.vocab
    R = K + 1
    import block_diffusion_drafter_kv_amd as dk
    w = gen.weights(cfg, seed=1234, gains="ones")
    max_ctx = max(ctx) + (steps + 1) * R + 64
    dr = dk.Drafter(cfg, to_cuda(w), max_batch=B, max_ctx=max_ctx, max_k=K,
                    max_inject_rows=max(B * R, sum(ctx) if one_call_prompt else 8192))
    orc = od.DrafterOracle(cfg, w)
    del w
    # prompts: followed requests from the seeded CPU generator, the others drawn on the GPU
    rows = {r: gen.hidden_rows(cfg, r, 0, ctx[r]) for r in followed}
    if one_call_prompt:
        allrows = torch.cat([rows[r].cuda() if r in rows else _gpu_rows(cfg, ctx[r], 500 + r) for r in range(B)])
        starts = np.concatenate([[0], np.cumsum(ctx)[:-1]])
        dr.inject(_dev(np.arange(B)), _dev(starts), _dev(ctx), int(sum(ctx)), allrows.contiguous())
        del allrows
    else:
        for r in range(B):
            for s0 in range(0, ctx[r], 8192):
                n = min(8192, ctx[r] - s0)
                x = rows[r][s0:s0 + n].cuda() if r in rows else _gpu_rows(cfg, n, 7000 + r * 97 + s0)
                dr.inject(_dev([r]), _dev([0]), _dev([n]), n, x.contiguous())
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    for r in followed:
        orc.inject(r, rows[r])
    del rows

    rng = np.random.default_rng(11)
    slots = _dev(np.arange(B))
    row_start = _dev(np.arange(B) * R)
    anchors_host = gen.anchor_ids(cfg, B, seed=3)
    vout = {"out_tokens": torch.empty((B, R), dtype=torch.int32, device="cuda"),
            "out_len": torch.empty((B,), dtype=torch.int32, device="cuda"),
            "accept_len": torch.empty((B,), dtype=torch.int32, device="cuda"),
            "next_anchor": _dev(anchors_host)}
    o_anchor = {r: int(anchors_host[r]) for r in followed}
    o_ctx = {r: ctx[r] for r in followed}
    cases = Tally(f"cycle request-steps ({'greedy' if T == 0 else f'T={T}'})")
    drafts = Tally("accepted drafts against the oracle's")
    max_err = 0.0
    seed = wl.philox_seed
    for s in range(steps):
        print(f"[cycle] step {s}", flush=True)
        o = dr.draft(slots, vout["next_anchor"], K, temperature=T, seed=seed, step=s, want_logits=True)
        torch.cuda.synchronize()
        assert dr.get_error() == 0
        # target logits: oracle-planned rows for the followed requests, seeded noise elsewhere
        t = rng.standard_normal((B, R, V), dtype=np.float32)
        plans = {}
        for r in followed:
            z = orc.block_logits(r, o_anchor[r], K)
            err = assert_close_report(o["logits"][r].cpu().numpy(), z, LOGIT_TOL, what=f"step {s} req {r} logits")
            max_err = max(max_err, err)
            if T == 0:
                a, d, x = _plan_greedy(z, rng, V)
                for i in range(1, a + 1):
                    t[r, i - 1, d[i - 1]] += 8.0          # argmax of row i-1 is d_i
                t[r, a, x] += 8.0                          # argmax of row a is x (rejection or bonus)
            else:
                a, x = _plan_rejection(z, rng, V, seed, r, s)
                d = None
                t[r, :a] = z[:a].astype(np.float32)        # p = q up to the forward's rounding
                t[r, a] = rng.standard_normal(V, dtype=np.float32)
                t[r, a, x] += 60.0                         # all mass on x: rejection and draw, or the bonus
            plans[r] = (a, d, x, z)
        tt = torch.from_numpy(t).cuda()
        dr.verify(slots, o["draft_ids"], o["logits"] if T > 0 else None, tt, temperature=T, seed=seed, step=s,
                  out=vout)
        # committed rows of this step: positions ctx..ctx+K of every request
        lens_before = dr.ctx_lens()[:B].cpu().numpy()
        pool = []
        step_rows = {}
        for r in range(B):
            if r in followed:
                x = gen.hidden_rows(cfg, r, o_ctx[r], R)
                step_rows[r] = x
                pool.append(x.cuda())
            else:
                pool.append(_gpu_rows(cfg, R, 90000 + 131 * s + r))
        dr.inject(slots, row_start, vout["out_len"], B * R, torch.cat(pool).contiguous())
        torch.cuda.synchronize()
        assert dr.get_error() == 0
        out_len = vout["out_len"].cpu().numpy()
        out_tok = vout["out_tokens"].cpu().numpy()
        nxt = vout["next_anchor"].cpu().numpy()
        ids = o["draft_ids"].cpu().numpy()
        lens_after = dr.ctx_lens()[:B].cpu().numpy()
        # every request: the cycle's bookkeeping
        assert np.array_equal(lens_after, lens_before + out_len), f"step {s}: ctx_len"
        for r in range(B):
            L = int(out_len[r])
            assert 1 <= L <= R and list(out_tok[r, :L - 1]) == list(ids[r, :L - 1]) and nxt[r] == out_tok[r, L - 1]
        # followed requests: the planned outcome, and the oracle's state advanced by it
        for r in followed:
            a, d, x, z = plans[r]
            assert out_len[r] == a + 1, f"step {s} req {r}: out_len {out_len[r]}, planned {a + 1}"
            assert out_tok[r, a] == x and nxt[r] == x, f"step {s} req {r}: emitted {out_tok[r, a]}, planned {x}"
            if d is not None:
                assert list(out_tok[r, :a]) == d[:a], f"step {s} req {r}: accepted drafts"
                for _ in range(a):
                    drafts.add(True)
            cases.add(True)
            orc.inject(r, step_rows[r][:a + 1])
            o_ctx[r] += a + 1
            o_anchor[r] = x
            assert lens_after[r] == o_ctx[r] == orc.ctx_len(r)
    print(f"[cycle] max |logit - oracle| over {steps} steps: {max_err:.3e}", flush=True)
    if T == 0:
        drafts.report()
    cases.assert_floor(1.0, min_total=len(followed) * steps)
    dr.close()


@pytest.mark.timeout(900)
def test_cycle_greedy_b32(gpu_lib):
    """The batch-32 workload (contexts U[512, 8192], K = 16), six greedy cycles chained on the
    device; the oracle follows the four requests with the shortest contexts."""
    wl = get_workload("b32_ragged4k")
    ctx = wl.ctx_lengths()
    followed = [int(i) for i in np.argsort(ctx)[:4]]
    _run_cycle(gpu_lib, wl, ctx, followed, steps=6, T=0.0, one_call_prompt=False)


@pytest.mark.timeout(900)
def test_cycle_rejection_b4(gpu_lib):
    """The long-context workload's shape (batch 4, K = 16, T = 1 drafting and rejection
    verification with Philox seed 99), prompts of 4096 rows injected in one call (not the
    workload's 32768, to keep the oracle's fp64 prompt injection within the test's time),
    four cycles chained on the device; the oracle follows requests 0 and 2."""
    wl = get_workload("b4_ctx32k")
    ctx = [4096] * wl.batch
    _run_cycle(gpu_lib, wl, ctx, [0, 2], steps=4, T=1.0, one_call_prompt=True)
