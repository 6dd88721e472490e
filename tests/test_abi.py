"""The C ABI library loads and exports every entry point include/dflash.h declares (no GPU needed)."""
import ctypes
import os
import re

import pytest

import block_diffusion_drafter_kv_amd as dk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls():
    names = _declared()
    for n in ("dflash_inject_context", "dflash_draft_block", "dflash_verify", "dflash_create", "dflash_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(dk.LIB_PATH):
        pytest.skip("library not built")
    lib = ctypes.CDLL(dk.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding wraps each of them under the same name
    assert sorted(dk.EXPORTS) == _declared()
    for n in _declared():
        assert callable(getattr(dk, n))


def test_status_strings_and_host_validation_without_gpu():
    if not os.path.exists(dk.LIB_PATH):
        pytest.skip("library not built")
    dk.load()
    assert dk.dflash_status_str(0) == "ok"
    assert dk.dflash_status_str(-3) == "capacity exceeded"
    # invalid configurations are rejected before any device work
    cfg = dk.dflash_config()
    w = dk.dflash_weights()
    h = ctypes.c_void_p()
    assert dk.load().dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -1
    cfg.dtype, cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads = 1, 1, 256, 4, 2
    cfg.head_dim, cfg.ffn, cfg.vocab, cfg.n_target_layers, cfg.target_hidden = 96, 512, 1024, 1, 256
    cfg.mask_token_id, cfg.rms_eps, cfg.rope_theta = 1023, 1e-6, 1e4
    cfg.max_batch, cfg.max_ctx, cfg.max_k, cfg.max_inject_rows = 1, 16, 4, 16
    assert dk.load().dflash_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) == -4   # head_dim 96
    # null handle / null pointers
    assert dk.load().dflash_verify(None, None, 1, 4, None, None, None, None, 0.0, 0, 0, None, None, None,
                                   None) == -1
    assert dk.load().dflash_profile(None, 1) == -1
    assert dk.load().dflash_draft_block(None, None, 1, None, None, None, None) == -1


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU (requests shard across GPUs with no exchange): bench.py --gpus 2 exits
    with status 2 and says so, before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _header_structs():
    """{struct name: [field names in order]} of every typedef struct the header defines."""
    src = open(os.path.join(ROOT, "include", "dflash.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for name, body in re.findall(r"typedef struct (\w+) \{(.*?)\}\s*\1\s*;", src, flags=re.S):
        fields = []
        for decl in body.split(";"):
            decl = decl.strip()
            if not decl:
                continue
            # "const void* a" / "int32_t a, b" / "const dflash_layer_weights* layers"
            head, *rest = decl.split(",")
            fields.append(re.findall(r"(\w+)\s*$", head)[0])
            fields += [r.strip().lstrip("*").strip() for r in rest]
        out[name] = fields
    return out


@pytest.mark.parametrize("name", ["dflash_config", "dflash_layer_weights", "dflash_weights", "dflash_draft_params",
                                  "dflash_draft_outputs"])
def test_ctypes_structs_mirror_the_header(name):
    structs = _header_structs()
    assert name in structs
    assert [f for f, _ in getattr(dk, name)._fields_] == structs[name]
