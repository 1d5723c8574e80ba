"""Static check of the gfx950 assembly of the MFMA kernels (CPU only; needs hipcc).

On gfx950 an MFMA may take as its accumulator (SrcC) the register block the
previous MFMA just wrote, back to back.  With two different shapes in such a chain
(a 16x16x32 bf16 product followed by a 16x16x16 bf16 product on one accumulator)
the second product read stale rows when only 1 to 3 plain VALU instructions
separated them (rows 4g and 4g+1 of lane groups g = 0, 1 came out wrong, in both the
VGPR-form and the AGPR-form builds of the chunked state kernel at d_k = 64); builds
where a wait on an LDS read or well over a hundred instructions separated them were
exact.  The compiler schedules such chains as if no wait were needed.  The kernels
therefore keep one shape per accumulator chain, and this test compiles each MFMA
source to assembly and fails if any accumulator chain mixes two shapes with fewer
than MIN_GAP instructions between writer and reader (counted without credit for
waits, so a conservative floor rather than the hardware's exact threshold).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_sequence_mixing_amd", "csrc")
MIN_GAP = 8
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc is not installed")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return [(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    m = re.match(r"([va])(\d+)$", tok)
    return [(m.group(1), int(m.group(2)))] if m else []


def _functions(asm):
    cur, body = None, []
    for ln in asm.splitlines():
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            if cur:
                yield cur, body
            cur, body = m.group(1), []
            continue
        s = ln.split(";")[0].strip()
        if s and not s.startswith((".", "//")) and not s.endswith(":"):
            body.append(s)
    if cur:
        yield cur, body


def mixed_chain_gaps(asm):
    """[(kernel, wait states, writer shape, reader shape)] for every MFMA whose SrcC
    was last written by an MFMA of another opcode, counted within straight-line
    order of the listing (s_nop n counts n + 1)."""
    out = []
    for name, body in _functions(asm):
        last = {}
        for i, ins in enumerate(body):
            op = ins.split()[0]
            if not op.startswith("v_mfma"):
                continue
            args = [a.strip() for a in ins[len(op):].split(",")]
            prev = [last[r] for r in (_regs(args[3]) if len(args) > 3 else []) if r in last]
            if prev:
                j, pop = max(prev)
                if pop != op:
                    gap = sum(int(x.split()[1], 0) + 1 if x.split()[0] == "s_nop" else 1 for x in body[j + 1:i])
                    out.append((name, gap, pop, op))
            for r in _regs(args[0]):
                last[r] = (i, op)
    return out


def _flags(src):
    sys_path = list(os.sys.path)
    try:
        os.sys.path.insert(0, ROOT)
        from attention_sequence_mixing_amd import build
        return build.FLAGS + build.EXTRA.get(os.path.basename(src), [])
    finally:
        os.sys.path[:] = sys_path


@pytest.mark.parametrize("name", ["ham_rnn_chunked.hip", "ham_attn.hip", "ham_bwd.hip"])
def test_no_short_mixed_shape_accumulator_chains(name, tmp_path):
    src = os.path.join(CSRC, name)
    out = tmp_path / (name + ".s")
    cmd = [HIPCC] + _flags(src) + ["-x", "hip", "--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    chains = mixed_chain_gaps(out.read_text())
    short = [c for c in chains if c[1] < MIN_GAP]
    assert not short, "MFMA accumulator chains mixing shapes too closely:\n" + "\n".join(
        f"  {k[:80]}: {w} wait states, {a} -> {b}" for k, w, a, b in short[:20])


def test_the_scanner_finds_a_short_chain():
    """The scanner itself: a 16x16x32 result read as SrcC by a 16x16x16 product two
    instructions later is reported with its gap; an unrelated accumulator is not."""
    asm = "\n".join([
        "_Zkernel:",
        "  v_mfma_f32_16x16x32_bf16 v[4:7], v[0:3], v[8:11], v[4:7]",
        "  v_add_f32 v20, v21, v22",
        "  s_nop 0",
        "  v_mfma_f32_16x16x16_bf16 v[4:7], v[12:13], v[14:15], v[4:7]",
        "  v_mfma_f32_16x16x16_bf16 v[30:33], v[12:13], v[14:15], v[40:43]",
    ])
    assert mixed_chain_gaps(asm) == [("_Zkernel", 2, "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16")]
