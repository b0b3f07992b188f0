"""Instruction-level checks on the gfx950 assembly of every kernel source (CPU only).

A vector-memory store of more than 8 bytes reads its data registers after it issues, so
those registers must not be rewritten for two wait states. The compiler adds the wait
states itself only when the store's uniform offset field is not a register; with a
register there it once let the next VALU or MFMA instruction overwrite the data at once,
which on gfx950 corrupted what the store wrote (the segmented state kernel's recorded
states, in some workgroups and runs only). Every kernel now stores 16 bytes with a
constant uniform offset; this test keeps it that way by scanning the assembly that
build() writes next to the objects.
"""
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASM = sorted(glob.glob(os.path.join(ROOT, "state_space_sequence_chunk_amd", "_build", "*.hip.s")))
WIDE = ("dwordx3", "dwordx4")
NEED = 2  # wait states between such a store and a write of its data registers

pytestmark = pytest.mark.skipif(not ASM, reason="no kernel assembly (run __graft_entry__.build())")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return m.group(1), set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = re.match(r"([va])(\d+)$", tok)
    return (m.group(1), {int(m.group(2))}) if m else (None, set())


def wide_store_overwrites(text, need=NEED):
    """(kernel, line, store, overwriting instruction) for every store of 12 or 16 bytes whose
    data registers a vector instruction rewrites after fewer than `need` wait states (each
    instruction counts one, s_nop n counts n + 1)."""
    lines = text.splitlines()
    kern, hits = None, []
    for i, line in enumerate(lines):
        if re.match(r"^_Z\S+:", line):
            kern = line.split(":")[0]
        s = line.strip()
        m = re.match(r"(buffer|global|flat|scratch)_store_(\w+)", s)
        if not m or m.group(2) not in WIDE:
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        kind, data = _regs(ops[0] if m.group(1) == "buffer" else ops[1])
        waits = 0
        for t in (x.strip() for x in lines[i + 1:i + 16]):
            if not t or t.startswith((";", ".")) or t.endswith(":"):
                continue
            if t.startswith("s_nop"):
                waits += int(t.split()[1], 0) + 1
            elif t.startswith("v_"):
                k2, dst = _regs(t.split(None, 1)[1].split(",")[0].strip())
                if k2 == kind and dst & data:
                    if waits < need:
                        hits.append((kern, i + 1, s, t))
                    break
                waits += 1
            else:
                waits += 1
            if waits >= need:
                break
    return hits


def test_scanner_flags_the_pattern():
    bad = ("_Zk:\n  buffer_store_dwordx4 v[4:7], v1, s[0:3], s8 offen\n"
           "  v_mov_b32_e32 v5, 0\n")
    ok_nop = ("_Zk:\n  buffer_store_dwordx4 v[4:7], v1, s[0:3], 0 offen\n  s_nop 1\n"
              "  v_mov_b32_e32 v5, 0\n")
    ok_narrow = "_Zk:\n  buffer_store_dword v4, v1, s[0:3], s8 offen\n  v_mov_b32_e32 v4, 0\n"
    assert len(wide_store_overwrites(bad)) == 1
    assert not wide_store_overwrites(ok_nop) and not wide_store_overwrites(ok_narrow)


@pytest.mark.parametrize("path", ASM, ids=[os.path.basename(p) for p in ASM])
def test_no_wide_store_data_overwritten_early(path):
    hits = wide_store_overwrites(open(path).read())
    assert not hits, "\n".join(f"{os.path.basename(path)}:{ln}: {s} -> {t} ({k[:60]})"
                               for k, ln, s, t in hits[:10])


def test_log2_decay_is_never_fused():
    """G = log2(e) * (running sum of A dt) is a rounded product wherever it is formed: the
    cumulative-decay kernel stores it, and the output kernels that form it themselves
    subtract it (G_e - G_j). Had the compiler fused that multiply into the subtraction (one
    FMA with -log2(e)), the in-kernel G would skip a rounding the stored one has, and the
    fused forward would no longer give the staged entry points' bits. No kernel may carry
    log2(e) (0x3fb8aa3b, negated 0xbfb8aa3b) as an FMA operand."""
    hits = []
    for path in ASM:
        for n, line in enumerate(open(path).read().splitlines(), 1):
            if re.match(r"\s*v_fma", line) and re.search(r"0x[3b]fb8aa3b", line):
                hits.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not hits, "\n".join(hits[:10])
