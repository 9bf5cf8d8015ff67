"""Checks on the gfx950 assembly of the library's own product kernels (built
here from source; no device needed).

The staged product tile ends each 64-wide chunk with a barrier that waits
only until at most NF LDS operations of the wave are outstanding (NF = the
wave's fragment reads of the next chunk, 12 with two activation terms, 8
with one). LDS operations of a wave complete in order, so that wait implies
that the wave's LDS writes of the chunk are complete -- provided that, on
every path into the barrier, at least NF LDS reads follow the last LDS
write. The kernel asks the scheduler for that order; this test reads the
compiler's output and checks it on the control-flow graph of every
instantiation, so a compiler change cannot break the barrier's meaning
unnoticed. The tile that copies its chunks straight into LDS is checked
likewise for its memory waits: each chunk's closing barrier may leave only
the copy issued in that chunk in flight."""
import os
import re
import shutil
import subprocess

import pytest

from stateful_sequence_model_amd import build as B


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "k_gemm.s")
    flags = [f for f in B._flags() if f != "-fPIC"]
    cmd = [B.hipcc()] + flags + ["-x", "hip", "--cuda-device-only", "-S", os.path.join(B.CSRC, "k_gemm.hip"),
                                 "-o", out]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return open(out).read().split("\n")


def _kernels(lines, pattern):
    for i, l in enumerate(lines):
        m = re.match(r"^(%s):" % pattern, l)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            yield m.group(1), lines[i + 1:end]


def _blocks(body):
    """Basic blocks: (label, [instructions]) in layout order, and each
    block's predecessors."""
    blocks, cur, label = [], [], "entry"
    for l in body:
        m = re.match(r"^(\.LBB\w+):", l)
        if m:
            blocks.append((label, cur))
            label, cur = m.group(1), []
            continue
        ins = l.split(";")[0].strip()
        if ins and not ins.startswith("."):
            cur.append(ins)
            if ins.startswith("s_branch") or ins.startswith("s_cbranch") or ins.startswith("s_endpgm"):
                blocks.append((label, cur))
                label, cur = "%s+" % label, []
    blocks.append((label, cur))
    index = {lab: k for k, (lab, _) in enumerate(blocks)}
    preds = {k: [] for k in range(len(blocks))}
    for k, (_, ins) in enumerate(blocks):
        last = ins[-1] if ins else ""
        target = re.search(r"(\.LBB\w+)", last) if last.startswith(("s_branch", "s_cbranch")) else None
        if target:
            preds[index[target.group(1)]].append(k)
        if not last.startswith(("s_branch", "s_endpgm")) and k + 1 < len(blocks):
            preds[k + 1].append(k)
    return blocks, preds


def _min_reads_after_last_write(blocks, preds, k, pos, nf):
    """Walking back from instruction pos of block k over every path: the
    fewest LDS reads between the last LDS write and that point (nf or more
    counts as enough; a path reaching a barrier or the entry first has no
    write since, which is safe)."""
    best, seen, stack = nf, set(), [(k, pos, 0)]
    while stack:
        b, p, reads = stack.pop()
        ins = blocks[b][1]
        hit = False
        for q in range(p - 1, -1, -1):
            x = ins[q]
            if x.startswith("s_barrier"):
                hit = True
                break
            if x.startswith("ds_write"):
                best = min(best, reads)
                hit = True
                break
            if x.startswith("ds_read"):
                reads += 1
                if reads >= nf:
                    hit = True
                    break
        if hit:
            continue
        for pb in preds[b]:
            key = (pb, reads)
            if key not in seen:
                seen.add(key)
                stack.append((pb, len(blocks[pb][1]), reads))
    return best


def test_staged_tile_barrier_waits_cover_the_lds_writes(gemm_asm):
    seen = 0
    for name, body in _kernels(gemm_asm, r"_ZN3rlt14k_gemm_bf16_ltILi\dELb\dELi\dEEEvNS_8GemmArgsENS_3EpiItEE"):
        two = re.search(r"ILi\dELb(\d)", name).group(1) == "1"
        nf = 4 * (3 if two else 2)
        blocks, preds = _blocks(body)
        relaxed = 0
        for k, (_, ins) in enumerate(blocks):
            for p, x in enumerate(ins):
                if x.startswith("s_barrier") and p > 0 and ins[p - 1] == "s_waitcnt lgkmcnt(%d)" % nf:
                    relaxed += 1
                    r = _min_reads_after_last_write(blocks, preds, k, p - 1, nf)
                    assert r >= nf, (name, "a path with only %d LDS reads after the last write" % r)
        assert relaxed >= 2, (name, "relaxed chunk barriers not found")
        seen += 1
    assert seen == 16  # Q in 1, 2, 4, 8 with one and two activation terms, 128 x 64 and 64 x 128 tiles


def _min_vmem_since_barrier(blocks, preds, k, pos, need):
    """Walking back from instruction pos of block k over every path to the
    previous barrier: the fewest memory instructions (global/buffer loads,
    stores and LDS copies) issued on the way (need or more counts as
    enough)."""
    best, seen, stack = need, set(), [(k, pos, 0)]
    while stack:
        b, p, n = stack.pop()
        ins = blocks[b][1]
        hit = False
        for q in range(p - 1, -1, -1):
            x = ins[q]
            if x.startswith("s_barrier"):
                best = min(best, n)
                hit = True
                break
            if x.startswith(("global_", "buffer_")):
                n += 1
                if n >= need:
                    hit = True
                    break
        if hit:
            continue
        if not preds[b]:
            best = min(best, n)
        for pb in preds[b]:
            key = (pb, n)
            if key not in seen:
                seen.add(key)
                stack.append((pb, len(blocks[pb][1]), n))
    return best


def test_copied_staged_tile_barriers_leave_only_this_chunks_copy_in_flight(gemm_asm):
    """The tile that copies its chunks straight into LDS closes each chunk
    with s_waitcnt vmcnt(x), lgkmcnt(NF), s_barrier: the copy of the chunk
    whose fragments the next chunk reads was issued before the previous
    barrier, so it has landed once at most x memory operations remain -- as
    long as, on every path from the previous barrier, at least x memory
    instructions were issued (the copy issued in this chunk)."""
    seen = 0
    for name, body in _kernels(gemm_asm, r"_ZN3rlt15k_gemm_bf16_ltdILi\dELb\dEEEvNS_8GemmArgsENS_3EpiItEE"):
        two = re.search(r"ILi\dELb(\d)", name).group(1) == "1"
        nf = 4 * (3 if two else 2)
        blocks, preds = _blocks(body)
        closing = 0
        for k, (_, ins) in enumerate(blocks):
            for p, x in enumerate(ins):
                if x.startswith("s_barrier") and p > 1 and ins[p - 1] == "s_waitcnt lgkmcnt(%d)" % nf:
                    m = re.match(r"s_waitcnt vmcnt\((\d+)\)$", ins[p - 2])
                    assert m, (name, "no vmcnt wait before a chunk barrier", ins[p - 2])
                    x_left = int(m.group(1))
                    closing += 1
                    if x_left:
                        r = _min_vmem_since_barrier(blocks, preds, k, p - 2, x_left)
                        assert r >= x_left, (name, "a path with only %d memory operations since the last barrier" % r)
        assert closing >= 2, (name, "chunk barriers not found")
        seen += 1
    assert seen == 8  # Q in 1, 2, 4, 8 with one and two activation terms


def test_checker_finds_a_short_path():
    """The path walk itself: a loop whose header (laid out after the body)
    holds the LDS writes, once with enough reads after them and once with a
    side entry that skips two of the reads."""
    def listing(side_entry):
        return [
            "\ts_branch .LBB0_2",
            ".LBB0_1:",
            "\tds_read_b128 v[0:3], v9",
            "\tds_read_b128 v[4:7], v9 offset:16",
            ".LBB0_3:" if side_entry else "\ts_nop 0",
            "\tds_read_b128 v[8:11], v9 offset:32",
            "\tds_read_b128 v[12:15], v9 offset:48",
            "\ts_waitcnt lgkmcnt(4)",
            "\ts_barrier",
            "\ts_cbranch_scc1 .LBB0_4",
            ".LBB0_2:",
            "\tds_write_b128 v9, v[16:19]",
            "\ts_cbranch_scc0 .LBB0_3" if side_entry else "\ts_nop 0",
            "\ts_branch .LBB0_1",
            ".LBB0_4:",
            "\ts_endpgm",
        ]
    for side, want in ((False, 4), (True, 2)):
        blocks, preds = _blocks(listing(side))
        k, p = next((k, p) for k, (_, ins) in enumerate(blocks) for p, x in enumerate(ins) if x == "s_barrier")
        assert _min_reads_after_last_write(blocks, preds, k, p - 1, 4) == want


def test_memory_count_walk_finds_a_short_path():
    """The memory-operation walk: four copies between two barriers, once on
    every path and once with a branch around two of them."""
    def listing(skip):
        return [
            "\ts_barrier",
            "\tglobal_load_lds_dwordx4 v[0:1], off",
            "\tglobal_load_lds_dwordx4 v[2:3], off",
            "\ts_cbranch_scc1 .LBB0_1" if skip else "\ts_nop 0",
            "\tglobal_load_lds_dwordx4 v[4:5], off nt",
            "\tglobal_load_lds_dwordx4 v[6:7], off nt",
            ".LBB0_1:",
            "\ts_waitcnt vmcnt(4)",
            "\ts_waitcnt lgkmcnt(12)",
            "\ts_barrier",
            "\ts_endpgm",
        ]
    for skip, want in ((False, 4), (True, 2)):
        blocks, preds = _blocks(listing(skip))
        k, p = next((k, p) for k, (_, ins) in enumerate(blocks) for p, x in enumerate(ins)
                    if x == "s_waitcnt vmcnt(4)")
        assert _min_vmem_since_barrier(blocks, preds, k, p, 4) == want
