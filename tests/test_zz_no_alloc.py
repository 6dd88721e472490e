"""dflash_verify_noalloc (the verification for callers that cannot allocate) against
dflash_verify on a handle, through the C ABI: greedy and rejection sampling, two
calls in a row on the same GPU (the second smaller), outputs equal bit for bit;
sizes beyond its limits are refused."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import select as osel
from synth import gen
from synth.configs import QWEN3_8B_SHAPED, scaled_model

pytestmark = pytest.mark.gpu


def _idle_weights(cfg):
    """Zero device weights of the right shapes (a handle that only verifies never reads them)."""
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    H, F = cfg.hidden, cfg.ffn
    lw = {"in_norm": z(H), "q_w": z(cfg.q_dim, H), "k_w": z(cfg.kv_dim, H), "v_w": z(cfg.kv_dim, H),
          "o_w": z(H, cfg.q_dim), "q_norm": z(cfg.head_dim), "k_norm": z(cfg.head_dim), "post_norm": z(H),
          "gate_w": z(F, H), "up_w": z(F, H), "down_w": z(H, F)}
    return {"embed": z(cfg.vocab, H), "lm_head": z(cfg.vocab, H), "fc": z(H, cfg.feat_dim), "hidden_norm": z(H),
            "final_norm": z(H), "layers": [lw] * cfg.n_layers}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _case(n, K, V, seed):
    z = gen.logits_like((n, K, V), 2.0, seed, "na_draft").numpy().astype(np.float32)
    t = np.concatenate([z, np.zeros((n, 1, V), np.float32)], axis=1) + \
        gen.logits_like((n, K + 1, V), 1.0, seed + 1, "na_target").numpy().astype(np.float32)
    slots = np.arange(n, dtype=np.int32)[::-1].copy()
    d = np.stack([osel.select_block(z[i], 1.0, 0, 5, int(slots[i]), 3)["draft_ids"] for i in range(n)])
    # a bump on the drafted token at the first half of the positions: acceptances there, rejections after
    bump = np.where(np.arange(K) < K // 2, 6.0, 0.5).astype(np.float32)
    t[:, :K][np.arange(n)[:, None], np.arange(K)[None, :], d] += bump[None, :]
    return (torch.tensor(z, device="cuda"), torch.tensor(t, device="cuda"), torch.tensor(d, dtype=torch.int32,
            device="cuda"), torch.tensor(slots, device="cuda"))


def _noalloc(dk, n, K, V, slots, d, z, t, T, seed, step):
    dev = torch.device("cuda")
    out = {"out_tokens": torch.full((n, K + 1), -7, dtype=torch.int32, device=dev),
           "out_len": torch.full((n,), -7, dtype=torch.int32, device=dev),
           "accept_len": torch.full((n,), -7, dtype=torch.int32, device=dev),
           "next_anchor": torch.full((n,), -7, dtype=torch.int32, device=dev)}
    dk.dflash_verify_noalloc(_stream(), n, K, V, slots.data_ptr(), d.data_ptr(), z.data_ptr(), t.data_ptr(),
                             float(T), seed, step, out["out_tokens"].data_ptr(), out["out_len"].data_ptr(),
                             out["accept_len"].data_ptr(), out["next_anchor"].data_ptr())
    return out


@pytest.mark.parametrize("V", [1000, 151936])
def test_verify_noalloc_equals_verify(gpu_lib, V):
    dk = gpu_lib
    cfg = scaled_model(QWEN3_8B_SHAPED, n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=256,
                       vocab=V, n_target_layers=1, target_hidden=256, mask_token_id=V - 1)
    dr = dk.Drafter(cfg, _idle_weights(cfg), max_batch=16, max_ctx=64, max_k=16, max_inject_rows=64)
    for T in (0.0, 1.0, 0.6):
        # two calls in a row on the one array: the second with fewer requests and a shorter block
        for n, K, seed in ((16, 16, 31), (5, 7, 37)):
            z, t, d, slots = _case(n, K, V, seed)
            ref = dr.verify(slots, d, z if T > 0 else None, t, temperature=T, seed=5, step=3)
            got = _noalloc(dk, n, K, V, slots, d, z, t, T, 5, 3)
            torch.cuda.synchronize()
            for k in ("out_tokens", "out_len", "accept_len", "next_anchor"):
                assert torch.equal(got[k], ref[k]), f"T {T} n {n} K {K}: {k}"
            print(f"[no-alloc] V {V} T {T} n {n} K {K}: out_len {got['out_len'].tolist()}", flush=True)
    assert dr.get_error() == 0
    dr.close()


def test_verify_noalloc_limits(gpu_lib):
    dk = gpu_lib
    z, t, d, slots = _case(2, 4, 1000, 41)
    for n, K, V in ((257, 4, 1000), (2, 32, 1000), (2, 4, 262145)):
        with pytest.raises(dk.DflashError) as e:
            _noalloc(dk, n, K, V, slots, d, z, t, 1.0, 5, 3)
        assert e.value.code == -3
    with pytest.raises(dk.DflashError):   # sampling needs the draft logits
        dk.dflash_verify_noalloc(_stream(), 2, 4, 1000, slots.data_ptr(), d.data_ptr(), None, t.data_ptr(), 1.0,
                                 5, 3, d.data_ptr(), d.data_ptr(), d.data_ptr(), None)
