"""Checks on the gfx950 code this repository builds (no GPU needed).

The decode kernels stream every cache byte once per call, so their K/V
loads carry the non-temporal hint.  A select between a non-temporal and a
plain load of the same address is folded by the compiler into a single
plain load; that once removed the hint from every decode kernel without any
test noticing (about 10 % slower launches).  This disassembles the device
code objects inside the built libpa.so and counts the hinted loads per
kernel.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_attention_kv_block_amd", "libpa.so")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"

pytestmark = pytest.mark.skipif(not (os.path.exists(OBJDUMP) and os.path.exists(LIB)),
                                reason="needs llvm-objdump and a built libpa.so")


def _kernels(tmp_path):
    """{kernel symbol: its disassembly} over every gfx950 code object."""
    lib = tmp_path / "libpa.so"
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", str(lib)], check=True, capture_output=True)
    out = {}
    for f in sorted(tmp_path.iterdir()):
        if "amdgcn-amd-amdhsa--gfx950" not in f.name:
            continue
        asm = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", str(f)], check=True,
                             capture_output=True, text=True).stdout
        parts = re.split(r"^[0-9a-f]+ <([^>]+)>:\s*$", asm, flags=re.M)
        for name, body in zip(parts[1::2], parts[2::2]):
            out[name] = body
    return out


def _nt_loads(body):
    return sum(1 for line in body.splitlines()
               if re.match(r"\s*(global|buffer)_load_\w+\s.*\bnt\b", line))


def test_decode_kernels_keep_nontemporal_kv_loads(tmp_path):
    ks = _kernels(tmp_path)
    decode = {n: b for n, b in ks.items() if n.startswith("_ZN2pa13decode_kernel")}
    assert len(decode) >= 40, sorted(ks)[:10]
    for name, body in decode.items():
        # last template argument: ordinary loads for shared column groups
        shared = name.endswith("Lb1EEEvNS_12DecodeParamsE")
        n = _nt_loads(body)
        if shared:
            assert n == 0, (name, n)
        else:
            assert n >= 8, (name, n)
    varlen = {n: b for n, b in ks.items() if n.startswith("_ZN2pa13varlen_kernel")}
    assert varlen and all(_nt_loads(b) >= 8 for b in varlen.values())
