"""Instruction-level checks on the gfx950 assembly of every kernel source (CPU only).

A vector-memory store of more than 8 bytes reads its data registers after it issues, so
those registers must not be rewritten for two wait states. The compiler adds the wait
states itself only when the store's uniform offset field is not a register; with a
register there it once let the next VALU or MFMA instruction overwrite the data at once,
which on gfx950 corrupted what the store wrote (the segmented state kernel's recorded
states, in some workgroups and runs only). Every kernel now stores 16 bytes with a
constant uniform offset; this test keeps it that way by scanning the assembly that
build() writes next to the objects. The same scans check that no kernel carries log2(e)
as an FMA operand and that the segmented state kernel's step loop issues no load under
an exec mask.
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


def mfma_loop_masked_loads(text, name_pat):
    """(kernel, masked vector loads) for each kernel matching name_pat: the vector-memory
    loads under an exec mask in the kernel's loops that hold MFMA instructions.
    A masked region starts at s_and_saveexec; its body is the straight-line code after a
    following s_cbranch_execz, or the block that a following s_cbranch_execnz jumps to,
    up to the next label or branch."""
    out = []
    for blk in re.split(r"\n(?=_Z\S+:)", text):
        m = re.match(r"(_Z\S+):", blk)
        if not m or not re.search(name_pat, m.group(1)):
            continue
        code = [l.strip() for l in blk.split(".Lfunc_end")[0].splitlines()
                if l.strip() and not l.strip().startswith(";")]
        labels = {x[:-1]: i for i, x in enumerate(code) if re.match(r"\.LBB\d+_\d+:$", x)}
        # the span of every backward branch whose range holds MFMA instructions (the
        # loop nest, with the out-of-line blocks the compiler lays out inside it)
        best = None
        for i, x in enumerate(code):
            if x.startswith(("s_cbranch", "s_branch")):
                t = x.split()[-1]
                if t in labels and labels[t] < i and any("mfma" in y for y in code[labels[t]:i]):
                    best = (labels[t], i) if best is None else (min(best[0], labels[t]), max(best[1], i))
        if best is None:
            continue

        def body_loads(k):  # loads from line k up to the next label or branch
            n = 0
            while k < len(code) and not code[k].endswith(":") and not code[k].startswith(("s_cbranch", "s_branch")):
                n += bool(re.match(r"(buffer|global)_load", code[k]))
                k += 1
            return n

        n = 0
        for i in range(best[0], best[1] + 1):
            if not code[i].startswith("s_and_saveexec") or i + 1 >= len(code):
                continue
            br = code[i + 1]
            if br.startswith("s_cbranch_execz"):
                n += body_loads(i + 2)
            elif br.startswith("s_cbranch_execnz") and br.split()[-1] in labels:
                n += body_loads(labels[br.split()[-1]] + 1)
        out.append((m.group(1), n))
    return out


def test_state_step_loads_are_unmasked():
    """The segmented state kernel issues every load of its step loop on every lane and
    path: a load under an exec mask made the compiler's counted waits for the later loads
    conservative (the LDS write of rows loaded two steps earlier waited for the loads the
    step had just issued). Each instance's step loop must hold no masked load."""
    path = os.path.join(ROOT, "state_space_sequence_chunk_amd", "_build", "k_state_seg_bf16.hip.s")
    found = mfma_loop_masked_loads(open(path).read(), r"state_seg_kernel")
    assert len(found) >= 9, found
    bad = [(k[:70], n) for k, n in found if n]
    assert not bad, bad


def test_masked_load_scanner():
    loop = ("_Zk:\n.LBB0_1:\n  s_and_saveexec_b64 s[2:3], vcc\n  s_cbranch_execz .LBB0_2\n"
            "  buffer_load_dwordx4 v[0:3], v4, s[8:11], 0 offen\n.LBB0_2:\n"
            "  s_or_b64 exec, exec, s[2:3]\n  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
            "  s_cbranch_scc1 .LBB0_1\n.Lfunc_end0:\n")
    assert mfma_loop_masked_loads(loop, "_Zk") == [("_Zk", 1)]
    assert mfma_loop_masked_loads(loop.replace("s_and_saveexec_b64 s[2:3], vcc\n", ""), "_Zk") == [("_Zk", 0)]
    # the same load in an out-of-line block entered with execnz
    ool = ("_Zk:\n.LBB0_1:\n  s_and_saveexec_b64 s[2:3], vcc\n  s_cbranch_execnz .LBB0_3\n.LBB0_2:\n"
           "  s_or_b64 exec, exec, s[2:3]\n  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]\n"
           "  s_cbranch_scc1 .LBB0_1\n  s_endpgm\n.LBB0_3:\n  buffer_load_dwordx4 v[0:3], v4, s[8:11], 0 offen\n"
           "  s_branch .LBB0_2\n.Lfunc_end0:\n")
    assert mfma_loop_masked_loads(ool, "_Zk") == [("_Zk", 1)]
