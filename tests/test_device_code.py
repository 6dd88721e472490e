"""Checks on the library's own gfx950 device code (no GPU needed).

The direct global -> LDS copies set M0 themselves and declare it clobbered
instead of saving and restoring it, which is only sound while no other
instruction of the library's kernels keeps a value in M0: the compiler reads
M0 for indirect register moves, add-tid LDS operations, messages, GWS and
ordered-count operations, interpolation and buffer-to-LDS loads.  This test
unpacks the code objects the built library carries and disassembles them
(llvm-objdump from the ROCm toolchain) to check that none of those
instructions occurs and that every M0 write feeds an LDS-DMA copy (or restores
M0 right after one, in the copy that saves it).
"""
import os
import re
import struct
import subprocess

import pytest

import block_diffusion_drafter_kv_amd as dk

OBJCOPY = "/opt/rocm/llvm/bin/llvm-objcopy"
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# mnemonic fragments of the instructions that read M0 implicitly (other than the LDS-DMA copies)
M0_READERS = ("movrel", "addtid", "sendmsg", "ds_gws", "ordered_count", "v_interp", "s_ttracedata")


def _code_objects(tmp_path):
    fat = tmp_path / "fat.bin"
    subprocess.run([OBJCOPY, "--dump-section", ".hip_fatbin=%s" % fat, dk.LIB_PATH], check=True,
                   capture_output=True)
    d = fat.read_bytes()
    objs, pos = [], 0
    while True:
        i = d.find(MAGIC, pos)
        if i < 0:
            break
        n = struct.unpack_from("<Q", d, i + 24)[0]
        p = i + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", d, p)
            p += 24
            triple = d[p:p + tl].decode()
            p += tl
            if "gfx950" in triple:
                objs.append(d[i + off:i + off + size])
        pos = i + len(MAGIC)
    return objs


def test_m0_is_written_only_for_lds_dma_copies(tmp_path):
    if not os.path.exists(dk.LIB_PATH):
        pytest.skip("library not built")
    if not (os.access(OBJCOPY, os.X_OK) and os.access(OBJDUMP, os.X_OK)):
        pytest.skip("ROCm llvm tools not found")
    objs = _code_objects(tmp_path)
    assert objs, "no gfx950 code object in the library"
    readers, orphan_writes, copies = [], 0, 0
    for k, o in enumerate(objs):
        path = tmp_path / ("co%d.o" % k)
        path.write_bytes(o)
        out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(path)], check=True, capture_output=True,
                             text=True).stdout
        ins = [ln.split()[0] for ln in out.splitlines() if re.match(r"^\s+[a-z_][a-z0-9_]*\s", ln)]
        ins_lines = [ln.strip() for ln in out.splitlines() if re.match(r"^\s+[a-z_][a-z0-9_]*\s", ln)]
        for j, (op, line) in enumerate(zip(ins, ins_lines)):
            if any(r in op for r in M0_READERS):
                readers.append(line)
            if op.startswith("global_load_lds"):        # the library's own copies (inline asm)
                copies += 1
            elif op.startswith("buffer_load") and " lds" in line:
                readers.append(line)
            if op == "s_mov_b32" and line.split()[1].rstrip(",") == "m0":
                # a copy sets M0 (s_mov_b32 m0, sX; s_nop 0; global_load_lds_*), or one
                # that saved M0 restores it right after its load
                nxt = ins[j + 1:j + 3]
                sets = len(nxt) == 2 and nxt[0] == "s_nop" and nxt[1].startswith("global_load_lds")
                restores = j > 0 and ins[j - 1].startswith("global_load_lds")
                if not (sets or restores):
                    orphan_writes += 1
    assert copies > 0
    assert not readers, readers[:5]
    assert orphan_writes == 0
