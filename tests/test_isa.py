"""Code-generation checks on our own gfx950 assembly (compile only, no GPU).

The pages assess the hoisting by the generated code (ROCm/iris #626,
"Assembly" table; ROCm/iris #594, "Compiler inspection and grouping"):
heap-base loads precede the tile loop, the only load inside it is the input
tile, no destination store is preceded by a full drain, the destination
loop has no back-edge, and VGPR/SGPR/spill counts are reported.  These tests
compile the kernels with hipcc for gfx950 and check the same properties.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_all_gather_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = {}
    d = tmp_path_factory.mktemp("isa")
    for src in ("ag_copy.hip", "ag_gemm.hip"):
        s = str(d / (src + ".s"))
        cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}", "--cuda-device-only", "-S",
               "-o", s, os.path.join(CSRC, src)]
        subprocess.run(cmd, check=True, capture_output=True)
        out[src] = open(s).read()
    return out


def _kernel_body(text, pattern):
    """Instructions of the first kernel whose symbol matches pattern (comments dropped)."""
    m = re.search(r"^(_Z\S*" + pattern + r"\S*):", text, re.M)
    assert m, pattern
    start = m.end()
    end = text.index("s_endpgm", start)
    lines = []
    for ln in text[start:end].splitlines():
        ln = ln.split(";", 1)[0].rstrip()
        if ln.strip():
            lines.append(ln.strip())
    return m.group(1), lines


def _meta(text, symbol):
    m = re.search(r"\.amdhsa_kernel " + re.escape(symbol) + r"\n(.*?)\.end_amdhsa_kernel", text, re.S)
    body = m.group(1)
    g = lambda k: int(re.search(r"\." + k + r" (\d+)", body).group(1))
    return {"vgpr": g("amdhsa_next_free_vgpr"), "sgpr": g("amdhsa_next_free_sgpr"),
            "scratch": g("amdhsa_private_segment_fixed_size"), "lds": g("amdhsa_group_segment_fixed_size"),
            "agpr_offset": g("amdhsa_accum_offset")}


def _loops(lines):
    """(header_index, backedge_index) of every loop: a branch to a label defined earlier."""
    labels = {ln[:-1]: i for i, ln in enumerate(lines) if ln.endswith(":")}
    out = []
    for i, ln in enumerate(lines):
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\S+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            out.append((labels[m.group(1)], i))
    return out


def _outermost(loops):
    return max(loops, key=lambda x: x[1] - x[0])


# (vector bytes, W, vectors per thread, partitioned); the partitioned kernel (one destination per program,
# also the all-to-all's partitioned schedule) has W = 1
COPY_CASES = [("16", "8", "1", "0"), ("16", "8", "2", "0"), ("8", "8", "2", "0"), ("16", "4", "1", "0"),
              ("4", "2", "4", "0"), ("16", "1", "1", "1"), ("16", "1", "2", "1")]


@pytest.mark.parametrize("vec,w,vpt,part", COPY_CASES)
def test_copy_kernel_hoists_bases_and_never_drains_before_a_store(asm, vec, w, vpt, part):
    sym, lines = _kernel_body(asm["ag_copy.hip"], f"ag_copy_kernelILi{vec}ELi{w}ELi{vpt}ELi0ELb{part}E")
    W, VPT = int(w), int(vpt)
    loops = _loops(lines)
    assert loops, "tile loop not found"
    h, b = _outermost(loops)
    body = lines[h:b + 1]
    prologue = lines[:h]
    # the heap-base table is read once, before the tile loop: one vector load
    # of the W entries (then readlane), issued just ahead of the first tiles'
    assert not any(ln.startswith("s_load") for ln in body), "scalar load inside the tile loop"
    table = [i for i, ln in enumerate(prologue) if ln.startswith("global_load_dwordx2")]
    assert len(table) == 1, table
    assert sum(ln.startswith("v_readlane_b32") for ln in prologue) >= 2 * W
    tiles = [i for i, ln in enumerate(prologue) if ln.startswith("buffer_load")]
    assert len(tiles) == 2 * VPT and table[0] < tiles[0], "table, then the first two tiles"
    # waiting for the table, then for the first tile, never waits for the prefetched second tile
    first_store = next(i for i, ln in enumerate(prologue) if ln.startswith("buffer_store"))
    counts = [int(re.search(r"vmcnt\((\d+)\)", ln).group(1)) for ln in prologue[tiles[-1]:first_store]
              if ln.startswith("s_waitcnt") and "vmcnt" in ln]
    assert counts and min(counts) >= VPT, counts
    # the only loads in the loop are the input tile's (two tiles per unrolled loop trip)
    loads = [ln for ln in body if re.match(r"(buffer|global|flat)_load", ln)]
    assert len(loads) == 2 * VPT, loads
    stores = [i for i, ln in enumerate(body) if ln.startswith("buffer_store")]
    assert len(stores) == 2 * W * VPT
    # no store is preceded (since the previous store) by a wait that drains the memory counter
    prev = 0
    for i in stores:
        waits = [ln for ln in body[prev:i] if ln.startswith("s_waitcnt") and "vmcnt(0)" in ln]
        assert not waits, f"drain before a store: {waits}"
        prev = i
    # the destination stores of one tile are straight-line code: no branch between them
    for first, last in ((stores[0], stores[W * VPT - 1]), (stores[W * VPT], stores[-1])):
        assert not any(re.match(r"s_(cbranch|branch)", ln) for ln in body[first:last]), "destination loop back-edge"
    meta = _meta(asm["ag_copy.hip"], sym)
    assert meta["scratch"] == 0, meta


@pytest.mark.parametrize("kernel", ["ag_copy_kernelILi16ELi8ELi1ELi0ELb0E", "ag_copy_kernelILi8ELi4ELi2ELi0ELb0E",
                                    "ag_copy_kernelILi16ELi1ELi1ELi0ELb1E", "ag_a2a_kernelILi16ELi8ELi2E"])
def test_copy_store_policy(asm, kernel):
    """Destination stores stream (nt); the wide variant (launches on at least half the CUs, never
    waited for) adds system scope (sc1), the other keeps nt alone."""
    for wide, want in (("0", {"nt"}), ("1", {"sc1", "nt"})):
        _, lines = _kernel_body(asm["ag_copy.hip"], f"{kernel}Lb{wide}E")
        stores = [ln for ln in lines if ln.startswith("buffer_store")]
        assert stores
        for ln in stores:
            bits = set(ln.split()) & {"sc0", "sc1", "nt"}
            assert bits == want, (wide, ln)


def test_grouped_copy_kernels_keep_plain_streaming_stores(asm):
    _, lines = _kernel_body(asm["ag_copy.hip"], "ag_copy_kernelILi16ELi8ELi1ELi2ELb0ELb0E")
    stores = [ln for ln in lines if ln.startswith("buffer_store")]
    assert stores and all((set(ln.split()) & {"sc0", "sc1", "nt"}) == {"nt"} for ln in stores)
    assert not re.search(r"ag_copy_kernelILi16ELi8ELi1ELi2ELb0ELb1E", asm["ag_copy.hip"]), "no wide grouped kernel"


@pytest.mark.parametrize("w,g", [(8, 1), (8, 2), (8, 4), (3, 2), (5, 4)])
def test_grouped_copy_waits_once_per_destination_group(asm, w, g):
    """dest_group G: after every G destinations' stores one wait retires what precedes them
    (at most G stores stay in flight), and there is no other wait among the stores."""
    sym, lines = _kernel_body(asm["ag_copy.hip"], f"ag_copy_kernelILi16ELi{w}ELi1ELi{g}ELb0E")
    h, b = _outermost(_loops(lines))
    body = lines[h:b + 1]
    stores = [i for i, ln in enumerate(body) if ln.startswith("buffer_store")]
    assert len(stores) == 2 * w
    for first, last in ((stores[0], stores[w - 1]), (stores[w], stores[-1])):
        waits = [ln for ln in body[first:last] if ln.startswith("s_waitcnt")]
        assert len(waits) == (w - 1) // g, waits
        assert all(f"vmcnt({g})" in ln for ln in waits), waits
    assert not any(ln.startswith("s_load") for ln in body)


@pytest.mark.parametrize("vec,w,vpt", [(16, 8, 1), (16, 8, 2), (16, 4, 1), (16, 2, 2), (8, 8, 4), (2, 3, 8)])
def test_all_to_all_kernel_hoists_bases_and_pipelines_tiles(asm, vec, w, vpt):
    """The W chunk copies as one sequence of tiles: one chunk tile loaded and stored per step, two steps
    per unrolled trip, the next tile's load ahead of the current tile's stores, no drain before a store.
    The table is read once before the loop; in the loop each stored tile reads its destination base from
    the lanes that hold them (two readlanes with a scalar lane index), never from memory."""
    sym, lines = _kernel_body(asm["ag_copy.hip"], f"ag_a2a_kernelILi{vec}ELi{w}ELi{vpt}E")
    loops = _loops(lines)
    assert loops, "tile loop not found"
    h, b = _outermost(loops)
    body, prologue = lines[h:b + 1], lines[:h]
    assert not any(ln.startswith("s_load") for ln in body), "scalar load inside the tile loop"
    assert not any(re.match(r"(global|flat)_load", ln) for ln in body), "table read inside the tile loop"
    assert sum(ln.startswith("global_load_dwordx2") for ln in prologue) == 1     # the table, once
    loads = [ln for ln in body if ln.startswith("buffer_load")]
    stores = [i for i, ln in enumerate(body) if ln.startswith("buffer_store")]
    assert len(loads) == 2 * vpt and len(stores) == 2 * vpt   # one chunk tile per step, two steps per trip
    reads = [ln for ln in body if ln.startswith("v_readlane_b32")]
    assert len(reads) == 4 and all(re.fullmatch(r"v_readlane_b32 s\d+, v\d+, s\d+", ln) for ln in reads), reads
    prev = 0
    for i in stores:
        assert not [ln for ln in body[prev:i] if ln.startswith("s_waitcnt") and "vmcnt(0)" in ln]
        prev = i
    assert _meta(asm["ag_copy.hip"], sym)["scratch"] == 0


@pytest.mark.parametrize("w,vpt,g,wide,drain", [("8", "1", "3", "1", "1"), ("8", "2", "2", "1", "1"),
                                                ("8", "1", "4", "1", "1"), ("8", "1", "4", "1", "0"),
                                                ("8", "1", "8", "1", "0"), ("8", "1", "16", "0", "0"),
                                                ("8", "2", "8", "0", "0"), ("4", "1", "4", "1", "1"),
                                                ("1", "2", "4", "1", "0")])
def test_ticket_kernel_hoists_bases_and_never_drains_before_a_store(asm, w, vpt, g, wide, drain):
    """Ticket order: the table is read once before the tile loop; the counter is an atomic increment
    (not an add, which the compiler would wait for at once); no store within a ticket's G*W stores is
    preceded by a full drain, and between tickets there is one only where the launch asks for it."""
    sym, lines = _kernel_body(asm["ag_copy.hip"],
                              f"ag_copy_ticket_kernelILi16ELi{w}ELi{vpt}ELi{g}ELb{wide}ELb{drain}E")
    W, VPT, G = int(w), int(vpt), int(g)
    h, b = _outermost(_loops(lines))
    body, prologue = lines[h:b + 1], lines[:h]
    assert sum(ln.startswith("global_load_dwordx2") for ln in prologue) == 1      # the table, once
    assert not any(ln.startswith("global_load") for ln in body)
    # the only scalar loads the loop may hold re-read kernel arguments (the counter's address, at
    # offset 0x60 of the argument block) where the compiler rematerialises instead of keeping a register
    assert all(re.match(r"s_load_dwordx2 s\[\d+:\d+\], s\[\d+:\d+\], 0x60$", ln)
               for ln in body if ln.startswith("s_load")), [ln for ln in body if ln.startswith("s_load")]
    assert sum(ln.startswith("v_readlane_b32") for ln in prologue) >= 2 * W
    incs = [ln for ln in lines if ln.startswith("global_atomic_inc")]
    assert len(incs) >= 3 and not any(ln.startswith("global_atomic_add ") and "offset:4" not in ln for ln in lines)
    loads = [ln for ln in body if re.match(r"buffer_load", ln)]
    stores = [i for i, ln in enumerate(body) if ln.startswith("buffer_store")]
    assert len(loads) == 2 * G * VPT and len(stores) == 2 * G * W * VPT    # two batches per unrolled trip
    per_batch = G * W * VPT
    drains = [i for i, ln in enumerate(body) if ln.startswith("s_waitcnt") and "vmcnt(0)" in ln]
    if drain == "0":                           # no store of the loop is preceded by a full drain
        assert not [i for i in drains if i < stores[-1]], [body[i] for i in drains]
    else:
        # one drain per ticket, each the wait for the ticket's atomic, and between two drains (the loop
        # body read cyclically, as blocks laid out ahead of the latch run after it) exactly one batch
        # of stores, none of them behind a drain of its own
        assert len(drains) == 2, [body[i] for i in drains]
        assert all(any(ln.startswith("global_atomic_inc") for ln in body[i - 3:i]) for i in drains)
        between = sum(drains[0] < i < drains[1] for i in stores)
        assert between == per_batch and len(stores) - between == per_batch, (between, len(stores))
    assert not _sign_extended_lane_reads(lines)
    assert _meta(asm["ag_copy.hip"], sym)["scratch"] == 0


@pytest.mark.parametrize("w,vpt,g,wide,drain", [("8", "1", "16", "1", "1"), ("8", "2", "8", "1", "1"),
                                                ("8", "1", "16", "0", "0"), ("3", "2", "8", "1", "0")])
def test_all_to_all_ticket_kernel_reads_bases_from_lanes(asm, w, vpt, g, wide, drain):
    """The all-to-all in ticket order: the table is read once before the tile loop; each tile has one
    load and one store per vector (two batches of G tiles per unrolled trip); its destination base comes
    from the lanes that hold the translated bases (two readlanes with a scalar lane index), never from
    memory; no store is preceded by a full drain except after each ticket's atomic where the launch asks."""
    sym, lines = _kernel_body(asm["ag_copy.hip"], f"ag_a2a_ticket_kernelILi{w}ELi{vpt}ELi{g}ELb{wide}ELb{drain}E")
    G, VPT = int(g), int(vpt)
    h, b = _outermost(_loops(lines))
    body, prologue = lines[h:b + 1], lines[:h]
    assert sum(ln.startswith("global_load_dwordx2") for ln in prologue) == 1      # the table, once
    assert not any(ln.startswith("global_load") for ln in body)
    assert all(re.match(r"s_load_dwordx2 s\[\d+:\d+\], s\[\d+:\d+\], 0x60$", ln)
               for ln in body if ln.startswith("s_load")), [ln for ln in body if ln.startswith("s_load")]
    assert any(ln.startswith("global_atomic_inc") for ln in lines)
    loads = [ln for ln in body if ln.startswith("buffer_load")]
    stores = [i for i, ln in enumerate(body) if ln.startswith("buffer_store")]
    assert len(loads) == 2 * G * VPT and len(stores) == 2 * G * VPT
    # (readlanes with a constant lane index are the compiler's scalar spills to vector lanes)
    reads = [ln for ln in body if re.fullmatch(r"v_readlane_b32 s\d+, v\d+, s\d+", ln)]
    assert len(reads) == 2 * 2 * G, len(reads)
    drains = [i for i, ln in enumerate(body) if ln.startswith("s_waitcnt") and "vmcnt(0)" in ln]
    if drain == "0":
        assert not [i for i in drains if i < stores[-1]], [body[i] for i in drains]
    else:
        assert len(drains) == 2 and all(any(ln.startswith("global_atomic_inc") for ln in body[i - 3:i]) for i in drains)
    assert not _sign_extended_lane_reads(lines)
    assert _meta(asm["ag_copy.hip"], sym)["scratch"] == 0


_SIGN_OPS = ("s_ashr_i32", "s_ashr_i64", "s_bfe_i32", "s_bfe_i64", "s_sext_i32_i8", "s_sext_i32_i16",
             "v_ashrrev_i32", "v_ashrrev_i64", "v_bfe_i32")


def _sregs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _sign_extended_lane_reads(lines):
    """Instructions that sign-propagate a 32-bit half read out of a lane (v_readlane / v_readfirstlane).

    A 64-bit address assembled from two 32-bit halves must zero-extend its low
    half; a sign extension (s_ashr / s_bfe_i* / sext of that register) turns
    the upper word into all ones whenever bit 31 of the low half is set.
    Checked from the first lane read to the first store.
    """
    halves, bad, seen = set(), [], False
    for ln in lines:
        if ln.startswith("buffer_store") or ln.startswith("global_store"):
            if seen:
                break
        m = re.match(r"v_read(?:first)?lane_b32\s+(s\d+)", ln)
        if m:
            halves |= _sregs(m.group(1))
            seen = True
            continue
        if not seen or " " not in ln:
            continue
        op, rest = ln.split(None, 1)
        ops = [o.strip() for o in rest.split(",")]
        dst = _sregs(ops[0])
        if op.split("_e32")[0].split("_e64")[0] in _SIGN_OPS and any(_sregs(o) & halves for o in ops[1:]):
            bad.append(ln)
        halves -= dst                                  # a half overwritten by something else is no longer one
    return bad


@pytest.mark.parametrize("vec,w,vpt,part", COPY_CASES)
def test_copy_kernel_bases_are_zero_extended(asm, vec, w, vpt, part):
    """The 64-bit destination bases built from readlane halves never sign-extend a half."""
    for wide in ("0", "1"):
        pat = f"ag_copy_kernelILi{vec}ELi{w}ELi{vpt}ELi0ELb{part}ELb{wide}E"
        if not re.search(r"^_Z\S*" + pat, asm["ag_copy.hip"], re.M):
            continue
        _, lines = _kernel_body(asm["ag_copy.hip"], pat)
        assert sum(ln.startswith("v_readlane_b32") for ln in lines) >= 2 * int(w)
        assert not _sign_extended_lane_reads(lines), _sign_extended_lane_reads(lines)


@pytest.mark.parametrize("w,vpt", [("8", "2"), ("4", "1")])
def test_all_to_all_bases_are_zero_extended(asm, w, vpt):
    for wide in ("0", "1"):
        _, lines = _kernel_body(asm["ag_copy.hip"], f"ag_a2a_kernelILi16ELi{w}ELi{vpt}ELb{wide}E")
        assert not _sign_extended_lane_reads(lines), _sign_extended_lane_reads(lines)


_LANE_BASE_SNIPPET = r"""
#include <hip/hip_runtime.h>
#include <stdint.h>
__global__ void zext_base(const uint64_t* t, uint64_t* out) {
    const uint64_t v = t[threadIdx.x & 63];
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const uint64_t b = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, 3))) << 32) |
                       static_cast<uint32_t>(__builtin_amdgcn_readlane(lo, 3));
    out[threadIdx.x] = b + 4096;
}
__global__ void sext_base(const uint64_t* t, uint64_t* out) {
    const uint64_t v = t[threadIdx.x & 63];
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const uint64_t b = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(hi, 3))) << 32) |
                       static_cast<uint64_t>(static_cast<int64_t>(__builtin_amdgcn_readlane(lo, 3)));
    out[threadIdx.x] = b + 4096;
}
"""


def test_sign_extension_check_catches_a_sign_extended_half(tmp_path):
    """The checker itself, on a compiled snippet: a low half widened through int64_t is flagged, the
    zero-extended one is not."""
    src = tmp_path / "lane_base.hip"
    src.write_text(_LANE_BASE_SNIPPET)
    out = tmp_path / "lane_base.s"
    subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O3", "--cuda-device-only", "-S", "-o", str(out), str(src)],
                   check=True, capture_output=True)
    text = out.read_text()
    _, good = _kernel_body(text, "zext_base")
    _, bad = _kernel_body(text, "sext_base")
    assert any(ln.startswith("v_readlane_b32") for ln in bad)
    assert not _sign_extended_lane_reads(good)
    assert _sign_extended_lane_reads(bad)


# (tile, B N-contiguous): the 256x256 kernel takes B K-contiguous only
GEMM_CFGS = [("256ELi224", "0"), ("256ELi224", "1"), ("256ELi256", "0"), ("128ELi128", "0"), ("128ELi128", "1")]


def _gemm_pattern(dt, w, cfg, bt):
    return rf"ag_gemm_kernelI{dt}ELi{w}ENS_8gemm_cfg3CfgILi{cfg}E\S*ELb{bt}EEEv"


@pytest.mark.parametrize("cfg,bt", GEMM_CFGS)
@pytest.mark.parametrize("dt", ["Lb0", "Lb1"])
def test_gemm_kernel_structure(asm, cfg, bt, dt):
    sym, lines = _kernel_body(asm["ag_gemm.hip"], _gemm_pattern(dt, "8", cfg, bt))
    first_barrier = next(i for i, ln in enumerate(lines) if ln.startswith("s_barrier"))
    # heap-base loads: all W of them before any tile or K-loop code (block layout may reorder the rest)
    assert sum(ln.startswith("s_load_dwordx2") for ln in lines[:first_barrier]) >= 8
    assert not any(ln.startswith("s_load_dwordx2") for ln in lines[first_barrier:])
    # K loop: between the first and the last MFMA of every straight-line stretch there is no
    # wait, spill or store (the next stage's loads and fragment reads overlap the MFMAs)
    runs, i = [], 0
    while i < len(lines):
        if lines[i].startswith("v_mfma"):
            j, last = i, i
            while j < len(lines) and not lines[j].endswith(":") and not re.match(r"s_(cbranch|branch|barrier)", lines[j]):
                if lines[j].startswith("v_mfma"):
                    last = j
                j += 1
            runs.append((i, last + 1))   # first to last MFMA of a straight-line stretch
            i = j
        i += 1
    mfma = [ln for ln in lines if ln.startswith("v_mfma")]
    assert mfma and all(ln.startswith("v_mfma_f32_16x16x32_" + ("bf16" if dt == "Lb1" else "f16")) for ln in mfma)
    big = [(a, b) for a, b in runs if sum(lines[k].startswith("v_mfma") for k in range(a, b)) >= 8]
    assert big, "no MFMA run found"
    for a, b in big:
        seg = lines[a:b]
        assert not any(ln.startswith(("scratch_", "buffer_store", "s_waitcnt")) for ln in seg), seg[:5]
    assert any(re.match(r"buffer_load_dwordx4 .* lds", ln) for ln in lines)
    # B fragments: 16-byte reads of a K-contiguous stage, transposing 8-byte reads of an N-contiguous one
    assert any(ln.startswith("ds_read_b64_tr_b16") for ln in lines) == (bt == "1")
    # epilogue: the W destination stores of a tile form one straight run with no drain inside
    stores = [i for i, ln in enumerate(lines) if ln.startswith("buffer_store_dwordx4")]
    assert stores
    seg = lines[stores[0]:stores[-1]]
    assert not any(ln.startswith("s_waitcnt") and "vmcnt(0)" in ln for ln in seg)
    assert not any(re.match(r"s_(cbranch|branch)", ln) for ln in seg)


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _unguarded_fragment_uses(lines):
    """Vector instructions that read a register an LDS read may still be writing.

    Walks the code in layout order (the fall-through path, which is how the
    unrolled K loop is laid out): every ds_read joins a queue of pending
    destination registers, s_waitcnt lgkmcnt(n) retires all but the newest n,
    and no MFMA or other vector instruction may read a register still in the
    queue (the two halves of a transposed B fragment may be moved into place
    before the MFMA).  The hardware
    does not interlock on LDS results, and the compiler does not count the
    fragment reads written as inline assembly, so the kernel has to wait
    explicitly.
    """
    pending, bad = [], []
    for i, ln in enumerate(lines):
        if ln.startswith("s_branch "):   # the code after an unconditional branch is not its fall-through
            pending = []
        elif ln.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", ln)
            if m:
                del pending[:max(0, len(pending) - int(m.group(1)))]
        elif ln.startswith("ds_read"):
            pending.append(_vregs(ln.split()[1].rstrip(",")))
        elif ln.startswith("v_") and " " in ln:
            ops = [o.strip() for o in ln.split(None, 1)[1].split(",")]
            src = set().union(*(_vregs(o) for o in ops[1:])) if len(ops) > 1 else set()
            if any(p & src for p in pending):
                bad.append((i, ln))
    return bad


@pytest.mark.parametrize("cfg,bt", GEMM_CFGS)
@pytest.mark.parametrize("dt", ["Lb0", "Lb1"])
@pytest.mark.parametrize("w", ["1", "8"])
def test_gemm_fragments_waited_before_mfma(asm, cfg, bt, dt, w):
    _, lines = _kernel_body(asm["ag_gemm.hip"], _gemm_pattern(dt, w, cfg, bt))
    assert any(ln.startswith("ds_read_b128") for ln in lines)
    bad = _unguarded_fragment_uses(lines)
    assert not bad, bad[:3]


def test_fragment_hazard_check_catches_a_missing_wait():
    """The checker itself: a read consumed without a wait is flagged, a waited one is not."""
    racy = ["ds_read_b128 v[2:5], v1", "ds_read_b128 v[6:9], v1 offset:64",
            "v_mfma_f32_16x16x32_f16 v[10:13], v[2:5], v[6:9], v[10:13]"]
    assert _unguarded_fragment_uses(racy)
    partial = racy[:2] + ["s_waitcnt lgkmcnt(1)"] + racy[2:]
    assert _unguarded_fragment_uses(partial)          # v[6:9] may still be landing
    ok = racy[:2] + ["s_waitcnt lgkmcnt(0)"] + racy[2:]
    assert not _unguarded_fragment_uses(ok)
    newer = racy[:2] + ["s_waitcnt lgkmcnt(0)", "ds_read_b128 v[20:23], v1"] + racy[2:]
    assert not _unguarded_fragment_uses(newer)         # an unrelated newer read may stay in flight


def test_report_registers(asm, capsys):
    """Print VGPR/AGPR/SGPR/scratch/LDS per instantiation (reported next to timings)."""
    rows = []
    for src, pat in (("ag_copy.hip", r"ag_(copy|a2a|copy_ticket|a2a_ticket)_kernel\S+"), ("ag_gemm.hip", r"ag_gemm_kernel\S+")):
        for sym in re.findall(r"^\s*\.amdhsa_kernel (\S+)\s*$", asm[src], re.M):
            if re.search(pat, sym):
                rows.append((sym, _meta(asm[src], sym)))
    assert rows
    # the instantiations the benchmark workloads run, then a summary over all of them
    bench = [r"ag_copy_ticket_kernelILi16ELi8ELi1ELi3ELb1ELb1E", r"ag_copy_ticket_kernelILi16ELi8ELi1ELi4ELb1ELb1E",
             r"ag_copy_ticket_kernelILi16ELi8ELi1ELi8ELb1ELb0E",
             r"ag_copy_ticket_kernelILi16ELi8ELi1ELi16ELb0ELb0E", r"ag_copy_ticket_kernelILi16ELi8ELi2ELi2ELb1ELb1E",
             r"ag_copy_ticket_kernelILi16ELi8ELi2ELi4ELb1ELb1E", r"ag_copy_ticket_kernelILi16ELi8ELi2ELi8ELb1ELb1E",
             r"ag_copy_ticket_kernelILi16ELi8ELi2ELi8ELb0ELb0E",
             r"ag_copy_kernelILi16ELi8ELi1ELi0ELb0ELb1E", r"ag_copy_kernelILi16ELi8ELi1ELi0ELb0ELb0E",
             r"ag_copy_kernelILi16ELi8ELi2ELi0ELb0ELb1E",
             r"ag_copy_kernelILi16ELi8ELi1ELi1ELb0ELb0E", r"ag_copy_kernelILi16ELi8ELi1ELi2ELb0ELb0E",
             r"ag_copy_kernelILi16ELi8ELi1ELi4ELb0ELb0E", r"ag_copy_kernelILi16ELi1ELi1ELi0ELb1ELb1E",
             r"ag_a2a_kernelILi16ELi8ELi2ELb1E", r"ag_a2a_ticket_kernelILi8ELi2ELi8ELb1ELb1E",
             r"ag_a2a_ticket_kernelILi8ELi2ELi8ELb1ELb0E",
             r"ag_gemm_kernelILb0ELi8E\S*CfgILi256ELi256E\S*ELb0EEEv", r"ag_gemm_kernelILb1ELi8E\S*CfgILi256ELi256E\S*ELb0EEEv",
             r"ag_gemm_kernelILb0ELi8E\S*CfgILi256ELi224E\S*ELb0EEEv", r"ag_gemm_kernelILb1ELi8E\S*CfgILi256ELi224E\S*ELb0EEEv",
             r"ag_gemm_kernelILb0ELi8E\S*CfgILi128ELi128E\S*ELb0EEEv", r"ag_gemm_kernelILb0ELi1E\S*CfgILi256ELi224E\S*ELb0EEEv",
             r"ag_gemm_kernelILb0ELi8E\S*CfgILi256ELi224E\S*ELb1EEEv", r"ag_gemm_kernelILb0ELi8E\S*CfgILi128ELi128E\S*ELb1EEEv"]
    with capsys.disabled():
        print()
        for pat in bench:
            for sym, m in rows:
                if re.search(pat, sym):
                    print(f"{sym[:104]:104s} vgpr={m['vgpr']} agpr_offset={m['agpr_offset']} sgpr={m['sgpr']} "
                          f"scratch={m['scratch']} lds={m['lds']}")
                    break
        print(f"{len(rows)} instantiations: max vgpr {max(m['vgpr'] for _, m in rows)}, "
              f"max sgpr {max(m['sgpr'] for _, m in rows)}, total scratch {sum(m['scratch'] for _, m in rows)}")
    # no kernel spills to scratch
    assert all(m["scratch"] == 0 for s, m in rows), [s for s, m in rows if m["scratch"]][:3]
