"""Checks on the gfx950 assembly of the kernels (compiled here on the CPU, no GPU needed).

Inline-assembly blocks that issue several scalar loads before one wait must not give a load's
destination a register that a later load of the same block reads as its address: the data
may land before that load issues. (The outputs of such blocks are early-clobber; this test
keeps them so.)"""
import os
import re
import shutil
import subprocess

import pytest

from exact_softmax_attention_paged_amd import build as B

SOURCES = ["prefill_bf16.hip", "decode_bf16.hip"]


def _sgprs(tok):
    """Register numbers named by an operand like s14 or s[60:61]."""
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def _asm_blocks(text):
    for blk in re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", text, flags=re.S):
        yield [ln.strip() for ln in blk.splitlines() if ln.strip()]


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("isa")
    for src in SOURCES:
        dst = d / (src + ".s")
        cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", B.INCLUDE, "-I", B.CSRC, os.path.join(B.CSRC, src), "-o", str(dst)]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert res.returncode == 0, res.stderr[-2000:]
        out[src] = dst.read_text()
    return out


@pytest.mark.parametrize("src", SOURCES)
def test_scalar_loads_in_asm_do_not_overwrite_later_addresses(isa, src):
    checked = 0
    for blk in _asm_blocks(isa[src]):
        loads = []
        for ln in blk:
            m = re.match(r"s_load_dword\w*\s+(s\d+|s\[\d+:\d+\]),\s*(s\[\d+:\d+\])", ln)
            if m:
                loads.append((_sgprs(m.group(1)), _sgprs(m.group(2))))
        for i, (dst, _) in enumerate(loads):
            for _, later_addr in loads[i + 1:]:
                assert not (dst & later_addr), f"{src}: {blk}"
        checked += len(loads) > 1
    if src == "prefill_bf16.hip":
        assert checked > 0, "no multi-load asm block found: the check would test nothing"
