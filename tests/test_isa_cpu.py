"""ISA checks of the hand-pipelined kernels (compiled here for gfx950, no GPU).

The HBM -> LDS copies set m0 in inline assembly; that is only sound if the
compiler itself never keeps a value in m0 in those kernels.  Also checks that
the kernels fit their register budgets without spilling.
"""

import os
import re
import subprocess

import pytest

from conftest import build_module

B = build_module()

COPY_SRC = ["decode_mfma.hip", "absorb_mfma.hip", "gemm_mfma.hip", "prefill_mfma.hip", "stream_probe.hip"]   # HBM -> LDS copies
SRC = COPY_SRC + ["combine.hip"]


def _asm(name, tmp_path):
    out = tmp_path / (name + ".s")
    cmd = [B.HIPCC, *B.COMMON, "-x", "hip", "-S", "--cuda-device-only", os.path.join(B.CSRC, name), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out.read_text()


@pytest.mark.parametrize("name", COPY_SRC)
def test_m0_only_set_by_the_copy_sequences(name, tmp_path):
    text = _asm(name, tmp_path)
    lines = [ln.strip() for ln in text.splitlines() if re.search(r"\bm0\b", ln) and not ln.strip().startswith(";")]
    assert lines, "expected the copy sequences to set m0"
    others = [ln for ln in lines if not ln.startswith("s_mov_b32 m0,")]
    assert not others, f"compiler-generated uses of m0: {others[:5]}"
    # every m0 write comes from an SGPR (the text form would print a VGPR for
    # an "s" operand the compiler kept in a VGPR, which does not assemble) and
    # is immediately followed by an LDS copy
    body = [ln.strip() for ln in text.splitlines()]
    for i, ln in enumerate(body):
        if ln.startswith("s_mov_b32 m0,"):
            assert re.match(r"s_mov_b32 m0, s\d+$", ln), ln
            assert body[i + 1].startswith("global_load_lds_dword"), body[i + 1]


def _spills(text):
    names = re.findall(r"\.name:\s+(\S+)", text)
    spills = [int(v) for v in re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)]
    kernels = [n for n in names if "kernel" in n]
    assert len(kernels) == len(spills), (kernels, spills)
    return dict(zip(kernels, spills))


@pytest.mark.parametrize("name", SRC)
def test_no_spills(name, tmp_path):
    """Every hot kernel fits its register budget: every latent-attention
    variant (16, 32 and 64-head groupings, gathered or not, packed cache or
    separate arrays), the absorb, GEMM, flash-attention, merge and probe kernels."""
    sp = _spills(_asm(name, tmp_path))
    hot = {n: s for n, s in sp.items()
           if any(k in n for k in ("decode_mfma", "absorb", "gemm", "flash", "combine", "stream_probe"))}
    assert hot and max(hot.values()) == 0, hot


def test_every_attention_grouping_is_built(tmp_path):
    """The no-spill check above covers all 12 attention variants
    <NW, GATHER, PACKED> (NW = 1, 2, 4)."""
    sp = _spills(_asm("decode_mfma.hip", tmp_path))
    seen = set()
    for n in sp:
        m = re.search(r"decode_mfma_kernelILi(\d)ELb(\d)ELb(\d)E", n)
        if m:
            seen.add(tuple(int(v) for v in m.groups()))
    assert seen == {(nw, g, pk) for nw in (1, 2, 4) for g in (0, 1) for pk in (0, 1)}, seen
