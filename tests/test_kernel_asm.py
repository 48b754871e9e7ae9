"""Checks on the gfx950 assembly of the split kernel (CPU only: hipcc
cross-compiles, nothing runs).

The PV waves issue their LDS reads as inline asm and wait for them with
hand-counted lgkmcnt values, so the compiler does not know when those
registers are written.  If it ever copies such a register (a phi move at a
branch join, a spill) between the read and its wait, the copy holds stale
data and the results are silently wrong.  This test compiles the kernel
exactly as the library build does and scans the PV key loop for any move
that reads the destination of an LDS read not yet covered by an
lgkmcnt(0); it also checks that no VGPR spills to scratch memory.
"""

import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_tree_verify_amd import build as vbuild

CSRC = vbuild.CSRC


def _hipcc():
    try:
        return vbuild.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    cc = _hipcc()
    if cc is None or shutil.which(cc) is None and not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "split.s"
    flags = [f for f in vbuild.HIP_FLAGS if f not in ("-fPIC",)]
    cmd = [cc, *flags, "--cuda-device-only", "-S", "-I", vbuild.INCLUDE, "-I", CSRC, "-o", str(out),
           os.path.join(CSRC, "prefix_splitkv.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _function(asm, name):
    """Lines of the kernel whose symbol contains `name`, from its label to
    its end marker."""
    lines = asm.splitlines()
    start = next(i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + name + r"\S*:", l))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


def _pv_loop(lines):
    """Line range of the PV waves' key loop: the innermost loop holding the
    32x32x16 MFMAs, from its header label to its back-edge branch."""
    idx = [i for i, l in enumerate(lines) if "v_mfma_f32_32x32x16" in l]
    assert idx, "no 32x32x16 MFMA in the kernel"
    a = max(i for i in range(idx[0]) if lines[i].startswith(".LBB") and "Parent Loop" in lines[i])
    b = min(i for i in range(idx[-1], len(lines)) if "s_cbranch_execz" in lines[i])
    return a, b


def test_no_copies_of_lds_reads_in_flight(asm):
    lines = _function(asm, "prefix_splitkv_kernel")
    a, b = _pv_loop(lines)
    inflight, bad, n_reads = set(), [], 0
    for i in range(a, b + 1):
        s = lines[i].strip()
        if not s or s.startswith((";", ".")):
            continue
        op = s.split()[0]
        if op.startswith("ds_read"):
            inflight |= _regs(s.split()[1].rstrip(","))
            n_reads += 1
            continue
        if op == "s_waitcnt" and "lgkmcnt(0)" in s:
            inflight = set()
            continue
        if op.startswith(("v_mov", "v_cndmask", "v_accvgpr", "v_perm", "v_writelane")):
            srcs = set()
            for t in s.split()[2:]:
                srcs |= _regs(t.rstrip(","))
            if srcs & inflight:
                bad.append(f"line {i + 1}: {s}")
    assert n_reads >= 16, "PV loop not found where expected"
    assert not bad, "registers of LDS reads still in flight are copied:\n" + "\n".join(bad[:10])


def test_no_vgpr_spills(asm):
    spills = [int(v) for v in re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm)]
    scratch = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)]
    assert spills and max(spills) == 0
    assert scratch and max(scratch) == 0


def _blocks(lines):
    """Basic blocks of the kernel's assembly: (label or None, [(line number,
    instruction, inside inline asm)], successor labels, falls through).
    Numeric local labels inside inline asm (`1:`, branched to as `1f` /
    `1b`) are given unique names."""
    # name every numeric local label by its line, and resolve 1f / 1b
    local = {}
    for i, raw in enumerate(lines):
        m = re.match(r"^\s*(\d+):\s*$", raw)
        if m:
            local.setdefault(m.group(1), []).append(i)

    def resolve(tok, i):
        m = re.match(r"^(\d+)([fb])$", tok)
        if not m or m.group(1) not in local:
            return tok
        cands = local[m.group(1)]
        j = min((c for c in cands if c > i), default=None) if m.group(2) == "f" else \
            max((c for c in cands if c < i), default=None)
        return f".L_local_{j}" if j is not None else tok

    blocks, cur, label, in_asm = [], [], None, False

    def close(succ, falls):
        blocks.append((label, cur, succ, falls))

    for i, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^(\.LBB\w+):", s)
        n = re.match(r"^(\d+):$", s)
        if m or n:
            if cur or label is not None:
                close([], True)
            cur, label = [], (m.group(1) if m else f".L_local_{i}")
            continue
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        cur.append((i, s, in_asm))
        op = s.split()[0]
        if op.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
            tgt = resolve(s.split()[1], i) if len(s.split()) > 1 and op != "s_endpgm" else None
            close([tgt] if tgt and tgt.startswith(".L") else [], op.startswith("s_cbranch"))
            cur, label = [], None
    if cur:
        close([], False)
    return blocks


def _reads_before_wait(lines, is_load, clears, allowed):
    """Forward dataflow over the basic blocks of `lines`: registers written by
    an async load (is_load(op)) are pending until a wait (clears(s)); every
    instruction that reads a pending register must satisfy allowed(op, next
    instruction).  Returns (loads seen, violations)."""
    blocks = _blocks(lines)
    index = {b[0]: k for k, b in enumerate(blocks) if b[0]}
    succ = []
    for k, (_, _, tg, falls) in enumerate(blocks):
        nxt = [index[x] for x in tg if x in index]
        if falls and k + 1 < len(blocks):
            nxt.append(k + 1)
        succ.append(nxt)
    n_loads = sum(1 for b in blocks for _, s, a in b[1] if a and is_load(s.split()[0]))
    entry = [frozenset() for _ in blocks]
    bad = set()
    work = list(range(len(blocks)))
    while work:
        k = work.pop()
        pend = set(entry[k])
        ins = blocks[k][1]
        for j, (i, s, in_asm) in enumerate(ins):
            op = s.split()[0]
            if in_asm and is_load(op):
                pend |= _regs(s.split()[1].rstrip(","))
                continue
            if clears(s):
                pend = set()
                continue
            if pend:
                srcs = set()
                for tok in s.split()[2:]:
                    srcs |= _regs(tok.rstrip(","))
                if op.startswith(("v_mfma", "v_smfmac")) and len(s.split()) > 2:
                    srcs |= _regs(s.split()[1].rstrip(","))          # accumulator in/out
                if srcs & pend:
                    nxt = ins[j + 1][1] if j + 1 < len(ins) else ""
                    if not allowed(op, nxt):
                        bad.add(f"line {i + 1}: {s} (next: {nxt or 'end of block'})")
            if op.startswith("v_") and not op.startswith(("v_cmp", "v_cmpx", "v_mfma")) and len(s.split()) > 1:
                pend -= _regs(s.split()[1].rstrip(","))
        out = frozenset(pend)
        for n in succ[k]:
            merged = entry[n] | out
            if merged != entry[n]:
                entry[n] = merged
                work.append(n)
    return n_loads, sorted(bad)


def test_slot_loads_read_only_after_their_wait(asm):
    """The PV waves load the slot indices of a tile ahead with an asm
    `global_load_dword` and name the register in the asm `s_waitcnt vmcnt`
    that ends the iteration.  A read of that register before a wait sees
    stale data.  Over every path of the compiled kernel (a forward dataflow
    over its basic blocks), the only read allowed before the wait is a move
    directly in front of a `vmcnt(0)` wait: the path that waits for
    everything is the one on which no gather follows in the item, so the
    slot value is dead there; on the path that gathers again (`vmcnt(9)`)
    the register must be read after the wait."""
    n_loads, bad = _reads_before_wait(
        _function(asm, "prefix_splitkv_kernel"),
        is_load=lambda op: op == "global_load_dword",
        clears=lambda s: s.startswith("s_waitcnt") and "vmcnt" in s,
        allowed=lambda op, nxt: op.startswith("v_mov") and nxt.startswith("s_waitcnt") and "vmcnt(0)" in nxt)
    assert n_loads >= 1, "no asm slot load found"
    assert not bad, "slot-load registers read before their wait:\n" + "\n".join(bad[:10])


def _asm_segments(lines):
    """(first, last) line numbers of every inline-asm statement."""
    segs, start = [], None
    for i, raw in enumerate(lines):
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            start = i
        elif s.startswith(";;#ASMEND") and start is not None:
            segs.append((start, i))
            start = None
    return segs


def _pending_at(lines, starts, clears, sinks):
    """Forward dataflow over the basic blocks of `lines`: a flag is raised at
    the line numbers in `starts`, dropped by an instruction with clears(s);
    returns the instructions with sinks(s) that some path reaches with the
    flag raised."""
    blocks = _blocks(lines)
    index = {b[0]: k for k, b in enumerate(blocks) if b[0]}
    succ = []
    for k, (_, _, tg, falls) in enumerate(blocks):
        nxt = [index[x] for x in tg if x in index]
        if falls and k + 1 < len(blocks):
            nxt.append(k + 1)
        succ.append(nxt)
    entry = [False] * len(blocks)
    seen = [False] * len(blocks)
    bad = set()
    work = list(range(len(blocks)))
    while work:
        k = work.pop()
        flag = entry[k]
        seen[k] = True
        for i, s, _ in blocks[k][1]:
            if i in starts:
                flag = True
            elif clears(s):
                flag = False
            elif flag and sinks(s):
                bad.add(f"line {i + 1}: {s}")
        for n in succ[k]:
            if flag and not entry[n]:
                entry[n] = True
                work.append(n)
    return sorted(bad)


def test_staged_query_rows_land_before_the_barrier(asm):
    """A row tile of more than 16 rows stages its query rows in ring slots 2
    and 3 with single LDS-DMAs (one per inline-asm statement, unlike the
    nine-DMA tile gathers), and the QK waves read them after the next
    barrier.  Every path from such a DMA must wait for all vector memory
    (`vmcnt(0)`) before it reaches a barrier, or a wave could read a row the
    other wave of its pair has not yet copied."""
    lines = _function(asm, "prefix_splitkv_kernel")
    starts = set()
    for a, b in _asm_segments(lines):
        dmas = [i for i in range(a, b + 1) if lines[i].strip().startswith("global_load_lds_dwordx4")]
        if len(dmas) == 1:
            starts.add(dmas[0])
    assert starts, "no single-DMA query staging found"
    bad = _pending_at(lines, starts,
                      clears=lambda s: s.startswith("s_waitcnt") and "vmcnt(0)" in s,
                      sinks=lambda s: s.startswith("s_barrier"))
    assert not bad, "barrier reached with query-row DMAs in flight:\n" + "\n".join(bad[:10])
