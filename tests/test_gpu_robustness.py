"""Numeric robustness of the bf16 drafter on the GPU (fp16 operands and stores):

* per-group weight scales: each group of weight matrices that one product reads
  is converted to fp16 with its own power of two, so a very large matrix (here
  the LM head at 2^12 times the others) leaves a very small one (every k
  projection at 2^-20) exact: the K cache and the logits still match the oracle;
* out-of-range 16-bit stores: an activation or cache value beyond fp16's range
  sets DFLASH_DEV_NONFINITE and is stored saturated, so the outputs stay finite.
"""
import numpy as np
import pytest
import torch

from oracle import drafter as od
from synth import gen
from synth.configs import QWEN3_8B_SHAPED, scaled_model

from gpu_helpers import assert_close_report, inject_both, to_cuda

pytestmark = pytest.mark.gpu

SMALL_BF16 = scaled_model(QWEN3_8B_SHAPED, n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128,
                          ffn=384, vocab=1000, n_target_layers=2, target_hidden=192, mask_token_id=999)
NONFINITE = 32
CACHE_ATOL, CACHE_RTOL = 3e-3, 2.0 ** -10


def _dev(a, dtype=torch.int32):
    return torch.tensor(np.asarray(a), dtype=dtype, device="cuda")


def _pair(cfg, w, **kw):
    import block_diffusion_drafter_kv_amd as dk
    dr = dk.Drafter(cfg, to_cuda(w), max_batch=3, max_ctx=256, max_k=8, max_inject_rows=1024, **kw)
    return dr, od.DrafterOracle(cfg, w)


def test_per_group_weight_scales(gpu_lib):
    cfg = SMALL_BF16
    w = gen.weights(cfg, seed=1234, gains="random")
    big, small = 2.0 ** 12, 2.0 ** -20             # powers of two: exact in bf16
    w["lm_head"] = w["lm_head"] * big
    for lw in w["layers"]:
        lw["k_w"] = lw["k_w"] * small
    dr, orc = _pair(cfg, w)
    slots, counts = [0, 2], [90, 33]
    inject_both(dr, orc, cfg, slots, counts, [0, 0])
    assert dr.get_error() == 0
    for s in slots:
        for layer in range(cfg.n_layers):
            k, v = dr.copy_cache(layer, s, 0, orc.ctx_len(s))
            kw_, vw_ = orc.cache[s][layer]
            assert_close_report(k.float().cpu().numpy(), kw_, CACHE_ATOL, CACHE_RTOL, f"K slot {s} layer {layer}")
            assert_close_report(v.float().cpu().numpy(), vw_, CACHE_ATOL, CACHE_RTOL, f"V slot {s} layer {layer}")
    K, anchors = 6, [11, 400]
    o = dr.draft(_dev(slots), _dev(anchors), K, want_logits=True)
    torch.cuda.synchronize()
    assert dr.get_error() == 0
    z = o["logits"].cpu().numpy()
    for i, (s, a) in enumerate(zip(slots, anchors)):
        want = orc.block_logits(s, a, K)
        # the LM head is 2^12 larger: compare on the unscaled axis
        err = assert_close_report(z[i] / big, want / big, atol=2e-2, what=f"logits req {i} / 2^12")
        print(f"[robustness] per-group scales: logits / 2^12 max error {err:.3e}", flush=True)
    dr.close()


def test_out_of_range_activation_sets_nonfinite_bit(gpu_lib):
    cfg = SMALL_BF16
    w = gen.weights(cfg, seed=1234)
    w["layers"][0]["up_w"] = w["layers"][0]["up_w"] * 2.0 ** 22   # SwiGLU products far beyond 65504
    dr, orc = _pair(cfg, w)
    inject_both(dr, orc, cfg, [1], [40], [0])
    assert dr.get_error() == 0                                    # injection does not touch the MLP
    o = dr.draft(_dev([1]), _dev([5]), 5, want_logits=True)
    torch.cuda.synchronize()
    assert dr.get_error() & NONFINITE
    assert torch.isfinite(o["logits"]).all()
    # the flag is sticky until read, then clear; a normal handle never raises it
    assert dr.get_error() == 0
    dr.close()


def test_out_of_range_cache_value_sets_nonfinite_bit(gpu_lib):
    cfg = SMALL_BF16
    w = gen.weights(cfg, seed=1234)
    w["layers"][1]["v_w"] = w["layers"][1]["v_w"] * 2.0 ** 20     # |v| ~ 3e5 in layer 1
    dr, orc = _pair(cfg, w)
    inject_both(dr, orc, cfg, [0], [70], [0])
    assert dr.get_error() & NONFINITE
    _, v = dr.copy_cache(1, 0, 0, 70)
    vv = v.float().cpu().numpy()
    assert np.isfinite(vv).all() and np.abs(vv).max() == 65504.0
    k0, v0 = dr.copy_cache(0, 0, 0, 70)                          # layer 0 unaffected and exact
    assert_close_report(v0.float().cpu().numpy(), orc.cache[0][0][1], CACHE_ATOL, CACHE_RTOL, "V layer 0")
    dr.close()
