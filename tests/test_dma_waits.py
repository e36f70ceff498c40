"""LDS-DMA ordering guard (CPU only). The Int4 prefill GEMM moves A into LDS
with buffer loads whose destination is the LDS; the compiler does not order
those writes against later LDS reads, so the kernel waits for them with
explicit vmcnt counts that assume a fixed issue order of its loads. This test
compiles the kernel to assembly and replays the main loop's vector-memory
queue (loads complete in issue order; `s_waitcnt vmcnt(n)` leaves at most n
outstanding) to check, for every instantiation:
  - at every LDS read, only the DMA groups of the tiles that may still be
    filling are outstanding (at most A_TILES - 1 of the newest groups);
  - at every explicit wait for the next block's tile, at most A_TILES - 2
    groups are outstanding.
A compiler that moved a load across the wait would make a count too small
and fail here instead of racing on the GPU."""
import os
import re
import shutil
import subprocess

import pytest

from weight_quantized_gemm_amd import build_lib

HIPCC = build_lib.HIPCC

# (BM, BN) -> (A_TILES, A_PIECES, A_WAIT); mirrors TileCfg in gemm_int4.hip
TILES = {(128, 64): (2, 16, 2), (64, 128): (4, 8, 36), (128, 128): (2, 16, 4)}


def _asm(tmpdir: str) -> str:
    out = os.path.join(tmpdir, "gemm_int4.s")
    cmd = [HIPCC, *build_lib.COMMON, *build_lib.HIP_FLAGS, "-x", "hip", "-S",
           os.path.join(build_lib.CSRC, "gemm_int4.hip"), "-o", out, "--offload-device-only"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _loops(asm: str, kernel: str = "gemm_int4b64_kernel"):
    """(kernel name, loop body lines in execution order) for every such
    kernel's first loop: the header's block and the loop blocks after it in
    file order, then the loop's blocks placed before the header (a latch)."""
    lines = asm.splitlines()
    starts = [i for i, ln in enumerate(lines) if re.match(r"^(_Z\w*" + kernel + r"\w*):", ln)]
    for k, st in enumerate(starts):
        name = re.match(r"^(_Z\w*):", lines[st]).group(1)
        end = next((i for i in range(st, len(lines)) if "s_endpgm" in lines[i]), len(lines))
        # blocks: (label line index, label, comment)
        blocks = [(i, ln) for i in range(st, end) for ln in [lines[i]] if re.match(r"^\.LBB\w+:", ln)]
        hdr = next((b for b in blocks if "Loop Header" in b[1]), None)
        if hdr is None:
            continue
        hname = "BB" + re.match(r"^\.LBB(\w+):", hdr[1]).group(1)
        member = lambda ln: ln is hdr[1] or ("Header=" + hname + " ") in ln + " "
        def block_lines(idx):
            nxt = next((b[0] for b in blocks if b[0] > idx), end)
            return lines[idx:nxt]
        body = []
        after = [b for b in blocks if b[0] >= hdr[0]]
        for b in after:
            if not member(b[1]):
                break
            body += block_lines(b[0])
        for b in blocks:
            if b[0] < hdr[0] and member(b[1]):
                body += block_lines(b[0])
        yield name, body


def _replay(body, a_tiles, a_pieces, a_wait):
    """Runs the loop body twice over an empty queue; returns violations of the
    second pass."""
    queue = []          # outstanding loads: DMA group id, or None for a plain load
    ndma = 0
    bad = []
    for rep in range(2):
        for ln in body:
            t = ln.strip()
            if re.match(r"(buffer|global)_load", t):
                if t.endswith(" lds"):
                    queue.append(ndma // a_pieces)
                    ndma += 1
                else:
                    queue.append(None)
            elif t.startswith("s_waitcnt") and "vmcnt(" in t:
                n = int(re.search(r"vmcnt\((\d+)\)", t).group(1))
                while len(queue) > n:
                    queue.pop(0)
                groups = {g for g in queue if g is not None}
                if n == a_wait and rep == 1 and len(groups) > a_tiles - 2:
                    bad.append(f"{t}: {len(groups)} DMA groups outstanding")
            elif t.startswith("ds_read") and rep == 1:
                groups = {g for g in queue if g is not None}
                if len(groups) > a_tiles - 1:
                    bad.append(f"{t}: {len(groups)} DMA groups outstanding")
    return bad, ndma


@pytest.mark.skipif(not (shutil.which(HIPCC) or os.path.exists(HIPCC)), reason="hipcc not found")
def test_int4_gemm_dma_waits_cover_every_lds_read(tmp_path):
    asm = _asm(str(tmp_path))
    seen = 0
    problems = []
    for name, body in _loops(asm):
        m = re.search(r"TileCfgILi(\d+)ELi(\d+)E", name)
        assert m, name
        a_tiles, a_pieces, a_wait = TILES[(int(m.group(1)), int(m.group(2)))]
        bad, ndma = _replay(body, a_tiles, a_pieces, a_wait)
        assert ndma == 2 * 4 * a_pieces, f"{name}: {ndma // 2} DMA loads per unrolled loop"
        problems += [f"{name[:80]}: {b}" for b in bad]
        seen += 1
    assert seen >= 6, f"only {seen} kernel loops found"
    assert not problems, "\n".join(problems[:20])


def _prologues(asm: str, kernel: str = "gemm_int4b64_kernel"):
    """(kernel name, lines from the kernel's entry to its first loop header)."""
    lines = asm.splitlines()
    for st, ln in enumerate(lines):
        m = re.match(r"^(_Z\w*" + kernel + r"\w*):", ln)
        if not m:
            continue
        hdr = next(i for i in range(st, len(lines)) if "Loop Header" in lines[i])
        yield m.group(1), lines[st:hdr]


def _replay_prologue(lines):
    """DMA loads still outstanding at each LDS read before the main loop
    (the prologue waits for all of its DMAs before the first read)."""
    queue = []
    bad = []
    for ln in lines:
        t = ln.strip()
        if re.match(r"(buffer|global)_load", t):
            queue.append(t.endswith(" lds"))
        elif t.startswith("s_waitcnt") and "vmcnt(" in t:
            n = int(re.search(r"vmcnt\((\d+)\)", t).group(1))
            while len(queue) > n:
                queue.pop(0)
        elif t.startswith("ds_read") and any(queue):
            bad.append(f"{t}: {sum(queue)} DMA loads outstanding")
    return bad


@pytest.mark.skipif(not (shutil.which(HIPCC) or os.path.exists(HIPCC)), reason="hipcc not found")
def test_int4_gemm_prologue_waits_for_its_dma(tmp_path):
    """The prologue's explicit wait leaves block 0's neighbours' B loads in
    flight; it must still cover every DMA issued before it, whatever order
    the compiler gave the loads."""
    asm = _asm(str(tmp_path))
    seen = 0
    problems = []
    for name, lines in _prologues(asm):
        assert any(ln.strip().endswith(" lds") for ln in lines), f"{name}: no DMA in the prologue"
        problems += [f"{name[:80]}: {b}" for b in _replay_prologue(lines)]
        seen += 1
    assert seen >= 6
    assert not problems, "\n".join(problems[:20])
    moved = ["buffer_load_dwordx4 v1, s[0:3], 0 offen lds"] * 4 + ["s_waitcnt vmcnt(2)",
             "buffer_load_dwordx4 v[2:5], v0, s[4:7], 0 offen", "ds_read_b128 v[10:13], v20"]
    assert _replay_prologue(moved)


def test_replay_catches_a_load_moved_below_the_wait():
    """The replay itself: a B load issued after the wait leaves the DMA group
    outstanding at the next LDS read."""
    good = ["buffer_load_dwordx4 v1, s[0:3], 0 offen lds"] * 16 + \
           ["buffer_load_dwordx4 v[2:5], v0, s[4:7], 0 offen", "buffer_load_dwordx4 v[6:9], v0, s[4:7], 0 offen",
            "s_waitcnt vmcnt(2)", "ds_read_b128 v[10:13], v20"]
    assert _replay(good * 4, 2, 16, 2)[0] == []
    moved = ["buffer_load_dwordx4 v1, s[0:3], 0 offen lds"] * 16 + \
            ["s_waitcnt vmcnt(2)", "buffer_load_dwordx4 v[2:5], v0, s[4:7], 0 offen",
             "buffer_load_dwordx4 v[6:9], v0, s[4:7], 0 offen", "ds_read_b128 v[10:13], v20"]
    assert _replay(moved * 4, 2, 16, 2)[0]


# skinny kernel (M <= 64): DMA loads per wave and pass (either row count)
SKINNY_NDMA = 8


@pytest.mark.skipif(not (shutil.which(HIPCC) or os.path.exists(HIPCC)), reason="hipcc not found")
def test_int4_skinny_dma_waits_cover_every_lds_read(tmp_path):
    """The skinny kernel double-buffers A in passes: at every LDS read only
    the next pass's DMA group may be outstanding."""
    asm = _asm(str(tmp_path))
    seen = 0
    problems = []
    for name, body in _loops(asm, "gemm_int4b64_skinny_kernel"):
        bad, n = _replay(body, 2, SKINNY_NDMA, -1)
        assert n >= 2 * 2 * SKINNY_NDMA and n % SKINNY_NDMA == 0, f"{name}: {n // 2} DMA loads per round"
        problems += [f"{name[:80]}: {b}" for b in bad]
        seen += 1
    assert seen == 21, f"{seen} skinny kernel loops found"   # (RF, NB) x 3 pair layouts
    assert not problems, "\n".join(problems[:20])
