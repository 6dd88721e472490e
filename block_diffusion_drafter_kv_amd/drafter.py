"""Convenience wrapper holding one library handle and its borrowed torch tensors.

PyTorch supplies device memory and the current HIP stream; all computation is
done by the library's kernels through the C ABI.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import torch

from . import (DFLASH_BF16, DFLASH_F32, dflash_config, dflash_copy_cache, dflash_create, dflash_ctx_lens,
               dflash_destroy, dflash_draft_block, dflash_draft_outputs, dflash_draft_params, dflash_get_error,
               dflash_inject_context, dflash_layer_weights, dflash_profile, dflash_profile_read, dflash_reset_slots,
               dflash_select_from_logits, dflash_verify, dflash_verify_tree, dflash_inject_tree_path,
               dflash_weights, dflash_select_path, dflash_verify_subset, dflash_set_sampling,
               dflash_set_page_table)

_LAYER_KEYS = ("in_norm", "q_w", "k_w", "v_w", "o_w", "q_norm", "k_norm", "post_norm", "gate_w", "up_w", "down_w")
_CONV_KEYS = ("attn_conv_base", "attn_conv_proj", "mlp_conv_base", "mlp_conv_proj")
_CONV_POST_KEYS = ("attn_conv_post_base", "attn_conv_post_proj", "mlp_conv_post_base", "mlp_conv_post_proj")
_SEL_KEYS = ("sel_pred", "sel_succ", "sel_hidden")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Drafter:
    def __init__(self, model, weights: Dict, *, max_batch: int, max_ctx: int, max_k: int, max_inject_rows: int,
                 max_top_k: int = 0, max_tree: int = 0, output_multiplier: float = 1.0, logit_softcap: float = 0.0,
                 page_size: int = 0, num_pages: int = 0):
        self.model = model
        self.dtype = torch.float32 if model.dtype == "f32" else torch.bfloat16
        self._w = weights                       # keep the borrowed tensors alive
        for k in ("embed", "lm_head", "fc", "hidden_norm", "final_norm"):
            t = weights[k]
            if not t.is_cuda or t.dtype != self.dtype or not t.is_contiguous():
                raise ValueError(f"weight {k}: need a contiguous {self.dtype} CUDA tensor")
        cfg = dflash_config()
        cfg.dtype = DFLASH_F32 if model.dtype == "f32" else DFLASH_BF16
        for f in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "n_target_layers",
                  "target_hidden", "mask_token_id"):
            setattr(cfg, f, int(getattr(model, f)))
        cfg.rms_eps = float(model.rms_eps)
        cfg.rope_theta = float(model.rope_theta)
        cfg.input_embedding_scale = float(model.input_embedding_scale)
        cfg.output_multiplier = float(output_multiplier)
        cfg.logit_softcap = float(logit_softcap)
        cfg.max_batch, cfg.max_ctx, cfg.max_k = max_batch, max_ctx, max_k
        cfg.max_inject_rows, cfg.max_top_k, cfg.max_tree = max_inject_rows, max_top_k, max_tree
        cfg.conv_group = int(getattr(model, "conv_group", 0))
        cfg.sel_rank = int(getattr(model, "sel_rank", 0))
        cfg.sel_cands = int(getattr(model, "sel_cands", 16)) if cfg.sel_rank else 0
        cfg.causal_block = 1 if getattr(model, "causal_block", False) else 0
        cfg.page_size, cfg.num_pages = int(page_size), int(num_pages)
        self.pages_per_slot = -(-max_ctx // page_size) if page_size else 0
        self._page_table = None
        self.cfg = cfg
        layers = (dflash_layer_weights * model.n_layers)()
        for l, lw in enumerate(weights["layers"]):
            post = tuple(k for k in _CONV_POST_KEYS if k in lw) if cfg.conv_group else ()
            for k in _LAYER_KEYS + (_CONV_KEYS if cfg.conv_group else ()) + post:
                t = lw[k]
                if not t.is_cuda or t.dtype != self.dtype or not t.is_contiguous():
                    raise ValueError(f"layer {l} weight {k}: need a contiguous {self.dtype} CUDA tensor")
                setattr(layers[l], k, t.data_ptr())
        self._layers = layers
        w = dflash_weights()
        w.embed, w.lm_head, w.fc = _ptr(weights["embed"]), _ptr(weights["lm_head"]), _ptr(weights["fc"])
        w.hidden_norm, w.final_norm = _ptr(weights["hidden_norm"]), _ptr(weights["final_norm"])
        w.n_layers = model.n_layers
        w.layers = layers
        if "mask_embedding" in weights:
            t = weights["mask_embedding"]
            if not t.is_cuda or t.dtype != self.dtype or not t.is_contiguous() or t.shape != (model.hidden,):
                raise ValueError(f"mask_embedding: need a contiguous {self.dtype} CUDA tensor [hidden]")
            w.mask_embedding = t.data_ptr()
        if cfg.sel_rank:
            for k in _SEL_KEYS:
                t = weights[k]
                if not t.is_cuda or t.dtype != self.dtype or not t.is_contiguous():
                    raise ValueError(f"weight {k}: need a contiguous {self.dtype} CUDA tensor")
                setattr(w, k, t.data_ptr())
        self._wstruct = w
        self.handle = dflash_create(cfg, w)

    def close(self):
        if self.handle is not None:
            dflash_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- calls ----
    def reset(self, slots: torch.Tensor):
        dflash_reset_slots(self.handle, _stream(), slots.numel(), slots.data_ptr())

    def inject(self, slots: torch.Tensor, row_start: torch.Tensor, row_count: torch.Tensor, rows_upper_bound: int,
               hidden):
        """hidden: [N, L_t, H_t] tensor, or a list of L_t tensors [N, H_t] sharing one row stride."""
        tensors = [hidden] if isinstance(hidden, torch.Tensor) else list(hidden)
        for t in tensors:
            if not t.is_cuda or t.dtype != self.dtype:
                raise ValueError(f"hidden states must be {self.dtype} CUDA tensors")
        for t in (slots, row_start, row_count):
            if not t.is_cuda or t.dtype != torch.int32:
                raise ValueError("slots / row_start / row_count must be int32 CUDA tensors")
        if isinstance(hidden, torch.Tensor):
            n, lt, ht = hidden.shape
            if not hidden.is_contiguous():
                raise ValueError("hidden must be contiguous")
            es = hidden.element_size()
            ptrs = [hidden.data_ptr() + l * ht * es for l in range(lt)]
            stride = lt * ht
        else:
            ptrs = [t.data_ptr() for t in hidden]
            stride = hidden[0].stride(0)
        dflash_inject_context(self.handle, _stream(), slots.numel(), slots.data_ptr(), row_start.data_ptr(),
                              row_count.data_ptr(), int(rows_upper_bound), ptrs, stride)

    def _outputs(self, n, K, top_k, tree_budget, logits, want_stats, want_hidden=False):
        dev = torch.device("cuda")
        o = {"draft_ids": torch.empty((n, K), dtype=torch.int32, device=dev)}
        if self.cfg.sel_rank:
            C = self.cfg.sel_cands
            o["cand_ids"] = torch.empty((n, K, C), dtype=torch.int32, device=dev)
            o["cand_probs"] = torch.empty((n, K, C), dtype=torch.float32, device=dev)
        if want_hidden:
            o["hidden"] = torch.empty((n, K, self.model.hidden), dtype=torch.float32, device=dev)
        if top_k:
            o["topk_ids"] = torch.empty((n, K, top_k), dtype=torch.int32, device=dev)
            o["topk_probs"] = torch.empty((n, K, top_k), dtype=torch.float32, device=dev)
        if want_stats:
            o["row_max"] = torch.empty((n, K), dtype=torch.float32, device=dev)
            o["row_lse"] = torch.empty((n, K), dtype=torch.float32, device=dev)
        if logits is not None:
            o["logits"] = logits
        if tree_budget:
            B = tree_budget
            o["tree_tokens"] = torch.empty((n, B + 1), dtype=torch.int32, device=dev)
            o["tree_parents"] = torch.empty((n, B + 1), dtype=torch.int32, device=dev)
            o["tree_depth"] = torch.empty((n, B + 1), dtype=torch.int32, device=dev)
            o["tree_mask"] = torch.empty((n, B + 1, (B + 64) // 64), dtype=torch.int64, device=dev)
        s = dflash_draft_outputs()
        for k, v in o.items():
            setattr(s, k, v.data_ptr())
        return o, s

    def draft(self, slots, anchors, K, temperature=0.0, seed=0, step=0, top_k=0, tree_budget=0,
              want_logits=False, logits_out: Optional[torch.Tensor] = None, want_stats=True, want_hidden=False):
        n = slots.numel()
        if want_logits and logits_out is None:
            logits_out = torch.empty((n, K, self.model.vocab), dtype=torch.float32, device="cuda")
        o, s = self._outputs(n, K, top_k, tree_budget, logits_out, want_stats, want_hidden)
        p = dflash_draft_params(K, float(temperature), seed, step, top_k, tree_budget)
        dflash_draft_block(self.handle, _stream(), n, slots.data_ptr(), anchors.data_ptr(), p, s)
        return o

    def select_from_logits(self, slots, anchors, logits, temperature=0.0, seed=0, step=0, top_k=0, tree_budget=0):
        n, K, _ = logits.shape
        o, s = self._outputs(n, K, top_k, tree_budget, None, True)
        p = dflash_draft_params(K, float(temperature), seed, step, top_k, tree_budget)
        dflash_select_from_logits(self.handle, _stream(), n, slots.data_ptr(),
                                  anchors.data_ptr() if anchors is not None else None, logits.data_ptr(), p, s)
        return o

    def verify(self, slots, draft_ids, draft_logits, target_logits, temperature=0.0, seed=0, step=0, out=None):
        n, K = draft_ids.shape
        dev = torch.device("cuda")
        if out is None:
            out = {"out_tokens": torch.empty((n, K + 1), dtype=torch.int32, device=dev),
                   "out_len": torch.empty((n,), dtype=torch.int32, device=dev),
                   "accept_len": torch.empty((n,), dtype=torch.int32, device=dev),
                   "next_anchor": torch.empty((n,), dtype=torch.int32, device=dev)}
        dflash_verify(self.handle, _stream(), n, K, slots.data_ptr(), draft_ids.data_ptr(),
                      _ptr(draft_logits), target_logits.data_ptr(), float(temperature), seed, step,
                      out["out_tokens"].data_ptr(), out["out_len"].data_ptr(), out["accept_len"].data_ptr(),
                      _ptr(out.get("next_anchor")))
        return out

    def set_page_table(self, table: torch.Tensor):
        """Paged cache: the device page table [max_batch, pages_per_slot] int32 (borrowed; kept alive here)."""
        if not table.is_cuda or table.dtype != torch.int32 or not table.is_contiguous() \
                or tuple(table.shape) != (self.cfg.max_batch, self.pages_per_slot):
            raise ValueError(f"page table: need a contiguous int32 CUDA tensor [{self.cfg.max_batch}, "
                             f"{self.pages_per_slot}]")
        self._page_table = table
        dflash_set_page_table(self.handle, table.data_ptr())

    def set_sampling(self, top_k=0, top_p=1.0):
        """Symmetric top-k / top-p truncation of later sampled drafts and verifications (dflash_set_sampling)."""
        dflash_set_sampling(self.handle, top_k, top_p)

    def select_path(self, slots, anchors, logits, hidden, temperature=0.0, seed=0, step=0):
        """DFlash 2 path selector alone (dflash_select_path) from fp32 logits [n, K, V] and hidden [n, K, H]."""
        n, K, _ = logits.shape
        for t in (logits, hidden):
            if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("logits / hidden must be contiguous fp32 CUDA tensors")
        C = self.cfg.sel_cands
        dev = torch.device("cuda")
        o = {"draft_ids": torch.empty((n, K), dtype=torch.int32, device=dev),
             "cand_ids": torch.empty((n, K, C), dtype=torch.int32, device=dev),
             "cand_probs": torch.empty((n, K, C), dtype=torch.float32, device=dev)}
        dflash_select_path(self.handle, _stream(), n, K, slots.data_ptr(), anchors.data_ptr(), logits.data_ptr(),
                           hidden.data_ptr(), float(temperature), seed, step, o["draft_ids"].data_ptr(),
                           o["cand_ids"].data_ptr(), o["cand_probs"].data_ptr())
        return o

    def verify_subset(self, slots, draft_ids, cand_ids, cand_probs, target_logits, temperature=0.0, seed=0, step=0,
                      out=None):
        """Rejection verification against candidate-subset draft distributions (dflash_verify_subset)."""
        n, K = draft_ids.shape
        C = cand_ids.shape[-1]
        dev = torch.device("cuda")
        if out is None:
            out = {"out_tokens": torch.empty((n, K + 1), dtype=torch.int32, device=dev),
                   "out_len": torch.empty((n,), dtype=torch.int32, device=dev),
                   "accept_len": torch.empty((n,), dtype=torch.int32, device=dev),
                   "next_anchor": torch.empty((n,), dtype=torch.int32, device=dev)}
        dflash_verify_subset(self.handle, _stream(), n, K, C, _ptr(slots), draft_ids.data_ptr(), _ptr(cand_ids),
                             _ptr(cand_probs), target_logits.data_ptr(), float(temperature), seed, step,
                             out["out_tokens"].data_ptr(), out["out_len"].data_ptr(), out["accept_len"].data_ptr(),
                             _ptr(out.get("next_anchor")))
        return out

    def verify_tree(self, slots, K, tree_tokens, tree_parents, target_logits, temperature=0.0, seed=0, step=0,
                    out=None):
        """Verifier walk down each request's draft tree (dflash_verify_tree)."""
        n, n_nodes = tree_tokens.shape
        for t in (tree_tokens, tree_parents):
            if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous() or t.shape != (n, n_nodes):
                raise ValueError("tree_tokens / tree_parents must be contiguous int32 CUDA tensors [n, B+1]")
        if target_logits.shape != (n, n_nodes, self.model.vocab) or target_logits.dtype != torch.float32 \
                or not target_logits.is_contiguous():
            raise ValueError("target_logits must be contiguous fp32 [n, B+1, vocab]")
        dev = torch.device("cuda")
        if out is None:
            out = {"out_tokens": torch.empty((n, K + 1), dtype=torch.int32, device=dev),
                   "out_len": torch.empty((n,), dtype=torch.int32, device=dev),
                   "accept_len": torch.empty((n,), dtype=torch.int32, device=dev),
                   "next_anchor": torch.empty((n,), dtype=torch.int32, device=dev),
                   "path_nodes": torch.empty((n, K + 1), dtype=torch.int32, device=dev)}
        dflash_verify_tree(self.handle, _stream(), n, K, n_nodes, _ptr(slots), tree_tokens.data_ptr(),
                           tree_parents.data_ptr(), target_logits.data_ptr(), float(temperature), seed, step,
                           out["out_tokens"].data_ptr(), out["out_len"].data_ptr(), out["accept_len"].data_ptr(),
                           _ptr(out.get("next_anchor")), _ptr(out.get("path_nodes")))
        return out

    def inject_tree_path(self, slots, path_nodes, path_len, tree_stride, rows_upper_bound, hidden):
        """Inject the accepted path rows: row i of request r is hidden row r * tree_stride + path_nodes[r, i]
        (hidden: [n * tree_stride, n_target_layers, target_hidden] contiguous)."""
        for t in (slots, path_nodes, path_len):
            if not t.is_cuda or t.dtype != torch.int32:
                raise ValueError("slots / path_nodes / path_len must be int32 CUDA tensors")
        if not path_nodes.is_contiguous() or path_nodes.dim() != 2:
            raise ValueError("path_nodes must be a contiguous [n, max_path] tensor")
        if not hidden.is_contiguous() or hidden.dim() != 3:
            raise ValueError("hidden must be contiguous [rows, n_target_layers, target_hidden]")
        _, lt, ht = hidden.shape
        es = hidden.element_size()
        ptrs = [hidden.data_ptr() + l * ht * es for l in range(lt)]
        dflash_inject_tree_path(self.handle, _stream(), slots.numel(), slots.data_ptr(), path_nodes.data_ptr(),
                                path_len.data_ptr(), path_nodes.shape[1], int(tree_stride), int(rows_upper_bound),
                                ptrs, lt * ht)

    def profile(self, enable: bool = True):
        dflash_profile(self.handle, enable)

    def profile_read(self):
        return dflash_profile_read(self.handle)

    # ---- inspection ----
    def ctx_lens(self) -> torch.Tensor:
        out = torch.empty(self.cfg.max_batch, dtype=torch.int32, device="cuda")
        dflash_ctx_lens(self.handle, _stream(), out.data_ptr())
        return out

    def copy_cache(self, layer, slot, start, n):
        m = self.model
        # cache element type: fp32, or fp16 for a bf16 drafter (fp16 operands)
        ct = torch.float32 if self.dtype == torch.float32 else torch.float16
        k = torch.empty((n, m.n_kv_heads, m.head_dim), dtype=ct, device="cuda")
        v = torch.empty_like(k)
        dflash_copy_cache(self.handle, _stream(), layer, slot, start, n, k.data_ptr(), v.data_ptr())
        return k, v

    def get_error(self) -> int:
        return dflash_get_error(self.handle, _stream())
