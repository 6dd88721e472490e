"""Python binding of the MI355X DFlash drafter library (libdflash_amd.so).

Argument marshalling only: every function here forwards to the C ABI declared
in include/dflash.h under the same name.  There is no Python or CPU fallback:
if the shared library is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_uint32, c_uint64, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdflash_amd.so")
_lib = None

DFLASH_F32 = 0
DFLASH_BF16 = 1
STATUS = {0: "ok", -1: "invalid argument", -2: "out of device memory", -3: "capacity exceeded",
          -4: "unsupported shape", -5: "HIP runtime error"}


class DflashError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({STATUS.get(code, 'unknown')})")
        self.code = code


class dflash_config(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("n_layers", c_int32), ("hidden", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32), ("vocab", c_int32),
                ("n_target_layers", c_int32), ("target_hidden", c_int32), ("mask_token_id", c_int32),
                ("rms_eps", c_float), ("rope_theta", c_float), ("input_embedding_scale", c_float),
                ("output_multiplier", c_float), ("logit_softcap", c_float), ("max_batch", c_int32),
                ("max_ctx", c_int32), ("max_k", c_int32), ("max_inject_rows", c_int32), ("max_top_k", c_int32),
                ("max_tree", c_int32), ("conv_group", c_int32), ("sel_rank", c_int32), ("sel_cands", c_int32),
                ("causal_block", c_int32), ("page_size", c_int32), ("num_pages", c_int32)]


class dflash_layer_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("in_norm", "q_w", "k_w", "v_w", "o_w", "q_norm", "k_norm", "post_norm",
                                        "gate_w", "up_w", "down_w", "attn_conv_base", "attn_conv_proj",
                                        "mlp_conv_base", "mlp_conv_proj", "attn_conv_post_base",
                                        "attn_conv_post_proj", "mlp_conv_post_base", "mlp_conv_post_proj")]


class dflash_weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("fc", c_void_p), ("hidden_norm", c_void_p),
                ("final_norm", c_void_p), ("n_layers", c_int32), ("layers", POINTER(dflash_layer_weights)),
                ("sel_pred", c_void_p), ("sel_succ", c_void_p), ("sel_hidden", c_void_p),
                ("mask_embedding", c_void_p)]


class dflash_draft_params(ctypes.Structure):
    _fields_ = [("K", c_int32), ("temperature", c_float), ("seed", c_uint64), ("step", c_uint64),
                ("top_k", c_int32), ("tree_budget", c_int32)]


class dflash_draft_outputs(ctypes.Structure):
    _fields_ = [("draft_ids", c_void_p), ("topk_ids", c_void_p), ("topk_probs", c_void_p), ("row_max", c_void_p),
                ("row_lse", c_void_p), ("logits", c_void_p), ("tree_tokens", c_void_p), ("tree_parents", c_void_p),
                ("tree_depth", c_void_p), ("tree_mask", c_void_p), ("cand_ids", c_void_p),
                ("cand_probs", c_void_p), ("hidden", c_void_p)]


_SIGS = {
    "dflash_create": ([POINTER(dflash_config), POINTER(dflash_weights), POINTER(c_void_p)], c_int32),
    "dflash_destroy": ([c_void_p], c_int32),
    "dflash_reset_slots": ([c_void_p, c_void_p, c_int32, c_void_p], c_int32),
    "dflash_inject_context": ([c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int64,
                               POINTER(c_void_p), c_int64], c_int32),
    "dflash_draft_block": ([c_void_p, c_void_p, c_int32, c_void_p, c_void_p, POINTER(dflash_draft_params),
                            POINTER(dflash_draft_outputs)], c_int32),
    "dflash_select_from_logits": ([c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                   POINTER(dflash_draft_params), POINTER(dflash_draft_outputs)], c_int32),
    "dflash_verify": ([c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                       c_uint64, c_uint64, c_void_p, c_void_p, c_void_p, c_void_p], c_int32),
    "dflash_verify_noalloc": ([c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                               c_uint64, c_uint64, c_void_p, c_void_p, c_void_p, c_void_p], c_int32),
    "dflash_verify_tree": ([c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_float, c_uint64, c_uint64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p], c_int32),
    "dflash_inject_tree_path": ([c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int64,
                                 POINTER(c_void_p), c_int64], c_int32),
    "dflash_select_path": ([c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                            c_uint64, c_uint64, c_void_p, c_void_p, c_void_p], c_int32),
    "dflash_verify_subset": ([c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_float, c_uint64, c_uint64, c_void_p, c_void_p, c_void_p, c_void_p], c_int32),
    "dflash_set_sampling": ([c_void_p, c_int32, c_float], c_int32),
    "dflash_set_page_table": ([c_void_p, c_void_p], c_int32),
    "dflash_profile": ([c_void_p, c_int32], c_int32),
    "dflash_profile_read": ([c_void_p, c_int32, POINTER(ctypes.c_double), POINTER(c_int32)], c_int32),
    "dflash_get_error": ([c_void_p, c_void_p, POINTER(c_int32)], c_int32),
    "dflash_status_str": ([c_int32], ctypes.c_char_p),
    "dflash_ctx_lens": ([c_void_p, c_void_p, c_void_p], c_int32),
    "dflash_copy_cache": ([c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p], c_int32),
    "dflash_synth_target_logits": ([c_void_p, c_int32, c_int32, c_int32, c_void_p, c_float, c_uint64, c_uint64,
                                    c_void_p], c_int32),
    "dflash_philox_uniforms": ([c_void_p, c_int32, c_uint64, c_uint32, c_uint64, c_uint32, c_void_p], c_int32),
}
EXPORTS = tuple(_SIGS)


def load(path: str = LIB_PATH):
    """Load the shared library (raises OSError if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} not found: build it with `python -m block_diffusion_drafter_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(name, rc):
    if rc != 0:
        raise DflashError(name, rc)
    return rc


def _call(name, *args):
    return _check(name, getattr(load(), name)(*args))


# ---- thin wrappers, same names as the C ABI ----

def dflash_create(cfg: dflash_config, weights: dflash_weights) -> c_void_p:
    h = c_void_p()
    _call("dflash_create", ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h))
    return h


def dflash_destroy(h):
    return _call("dflash_destroy", h)


def dflash_reset_slots(h, stream, n, slots_ptr):
    return _call("dflash_reset_slots", h, stream, n, slots_ptr)


def dflash_inject_context(h, stream, n_req, slots, row_start, row_count, rows_upper_bound, layer_ptrs, row_stride):
    arr = (c_void_p * len(layer_ptrs))(*layer_ptrs)
    return _call("dflash_inject_context", h, stream, n_req, slots, row_start, row_count, rows_upper_bound, arr,
                 row_stride)


def dflash_draft_block(h, stream, n_req, slots, anchors, params: dflash_draft_params, outs: dflash_draft_outputs):
    return _call("dflash_draft_block", h, stream, n_req, slots, anchors, ctypes.byref(params), ctypes.byref(outs))


def dflash_select_from_logits(h, stream, n_req, slots, anchors, logits, params, outs):
    return _call("dflash_select_from_logits", h, stream, n_req, slots, anchors, logits, ctypes.byref(params),
                 ctypes.byref(outs))


def dflash_verify(h, stream, n_req, K, slots, draft_ids, draft_logits, target_logits, temperature, seed, step,
                  out_tokens, out_len, accept_len, next_anchor=None):
    return _call("dflash_verify", h, stream, n_req, K, slots, draft_ids, draft_logits, target_logits, temperature,
                 seed, step, out_tokens, out_len, accept_len, next_anchor)


def dflash_verify_noalloc(stream, n_req, K, vocab, slots, draft_ids, draft_logits, target_logits, temperature, seed,
                          step, out_tokens, out_len, accept_len, next_anchor=None):
    return _call("dflash_verify_noalloc", stream, n_req, K, vocab, slots, draft_ids, draft_logits, target_logits,
                 temperature, seed, step, out_tokens, out_len, accept_len, next_anchor)


def dflash_verify_tree(h, stream, n_req, K, n_nodes, slots, tree_tokens, tree_parents, target_logits, temperature,
                       seed, step, out_tokens, out_len, accept_len, next_anchor=None, path_nodes=None):
    return _call("dflash_verify_tree", h, stream, n_req, K, n_nodes, slots, tree_tokens, tree_parents, target_logits,
                 temperature, seed, step, out_tokens, out_len, accept_len, next_anchor, path_nodes)


def dflash_inject_tree_path(h, stream, n_req, slots, path_nodes, path_len, max_path, tree_stride, rows_upper_bound,
                            layer_ptrs, row_stride):
    arr = (c_void_p * len(layer_ptrs))(*layer_ptrs)
    return _call("dflash_inject_tree_path", h, stream, n_req, slots, path_nodes, path_len, max_path, tree_stride,
                 rows_upper_bound, arr, row_stride)


def dflash_select_path(h, stream, n_req, K, slots, anchors, logits, hidden, temperature, seed, step, draft_ids,
                       cand_ids, cand_probs):
    return _call("dflash_select_path", h, stream, n_req, K, slots, anchors, logits, hidden, temperature, seed, step,
                 draft_ids, cand_ids, cand_probs)


def dflash_verify_subset(h, stream, n_req, K, C, slots, draft_ids, cand_ids, cand_probs, target_logits, temperature,
                         seed, step, out_tokens, out_len, accept_len, next_anchor=None):
    return _call("dflash_verify_subset", h, stream, n_req, K, C, slots, draft_ids, cand_ids, cand_probs,
                 target_logits, temperature, seed, step, out_tokens, out_len, accept_len, next_anchor)


def dflash_set_page_table(h, table_ptr):
    return _call("dflash_set_page_table", h, table_ptr)


def dflash_set_sampling(h, top_k, top_p):
    return _call("dflash_set_sampling", h, int(top_k), float(top_p))


PHASES = ("inject_prep", "inject_fc", "inject_norm", "inject_kv", "embed", "qkv", "attn", "attn_combine", "o",
          "norm", "gate_up", "down", "lm_head", "select", "verify", "attn_plan", "conv", "selector")


def dflash_profile(h, enable: bool):
    return _call("dflash_profile", h, 1 if enable else 0)


def dflash_profile_read(h):
    """Accumulated (ms, launches) per phase since the last read, as a dict keyed by phase name."""
    n = len(PHASES)
    ms = (ctypes.c_double * n)()
    cnt = (c_int32 * n)()
    _call("dflash_profile_read", h, n, ms, cnt)
    return {p: (ms[i], cnt[i]) for i, p in enumerate(PHASES)}


def dflash_get_error(h, stream) -> int:
    code = c_int32(0)
    _call("dflash_get_error", h, stream, ctypes.byref(code))
    return code.value


def dflash_status_str(code: int) -> str:
    return load().dflash_status_str(code).decode()


def dflash_ctx_lens(h, stream, out_ptr):
    return _call("dflash_ctx_lens", h, stream, out_ptr)


def dflash_copy_cache(h, stream, layer, slot, start, n, k_out, v_out):
    return _call("dflash_copy_cache", h, stream, layer, slot, start, n, k_out, v_out)


def dflash_synth_target_logits(stream, n_req, K, vocab, draft_logits, sigma, seed, step, out):
    return _call("dflash_synth_target_logits", stream, n_req, K, vocab, draft_logits, sigma, seed, step, out)


def dflash_philox_uniforms(stream, n, seed, slot, step, purpose, out):
    return _call("dflash_philox_uniforms", stream, n, seed, slot, step, purpose, out)


from .drafter import Drafter  # noqa: E402,F401
