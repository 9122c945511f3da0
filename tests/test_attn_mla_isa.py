"""Checks on the gfx950 code hipcc builds here for csrc/attn_mla.hip (CPU only;
needs hipcc).  The MLA attention issues its Q.K MFMAs as inline assembly with
the S^T accumulator in VGPRs, so the compiler's hazard recognizer does not see
them; the kernel relies on:
  - every source operand of those MFMAs coming from memory loads (LDS or
    global), whose waits the compiler inserts, never from a VALU instruction
    just before the MFMA;
  - no instance needing scratch memory (a spill would also cost the
    no-allocation entry point its promise).
Both are properties of the built code, checked here on the same flags the
library is built with."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "sparse_attention_04_amd"))


def _asm(tmp_path):
    import build as B
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "attn_mla.s"
    flags = dict(B.SOURCES)["attn_mla.hip"]
    cmd = [hipcc, *B.COMMON, *flags, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(B.CSRC, "attn_mla.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(text):
    """{kernel symbol: [instruction lines]} for the attention kernels."""
    ks, name, body = {}, None, []
    for line in text.splitlines():
        m = re.match(r"^(_ZN\S*sparse_attn_mla_kernel\S*):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        s = line.strip()
        if s.startswith(".Lfunc_end"):
            ks[name] = body
            name = None
            continue
        if s and not s.startswith((";", ".")):
            body.append(s)
    return ks


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _asm(tmp_path_factory.mktemp("isa"))


def test_no_scratch(asm):
    sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)]
    assert sizes and all(s == 0 for s in sizes), sizes


def test_inline_mfma_sources_not_written_by_valu(asm):
    ks = _kernels(asm)
    assert len(ks) == 6, sorted(ks)                       # 32/64/128 heads, split and unsplit
    for name, body in ks.items():
        n = 0
        for i, ins in enumerate(body):
            if not ins.startswith("v_mfma_f32_32x32x16_bf16 v["):
                continue
            n += 1
            ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
            src = _regs(ops[1]) | _regs(ops[2])
            for prev in body[max(0, i - 6):i]:
                if prev.startswith("v_") and not prev.startswith("v_mfma"):
                    dst = prev.split(None, 1)[1].split(",")[0].strip()
                    assert not (_regs(dst) & src), f"{name}: '{prev}' writes a source of '{ins}'"
        assert n >= 36, (name, n)                          # the Q.K chain of every chunk


def test_wait_states_after_the_chain(asm):
    """The two s_nop 7 and one s_nop 3 (20 wait states) follow the Q.K chain in
    every instance, before S^T is read."""
    for name, body in _kernels(asm).items():
        text = "\n".join(body)
        assert "s_nop 7\ns_nop 7\ns_nop 3" in text, name
