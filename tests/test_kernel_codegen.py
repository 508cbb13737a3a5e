"""Code-generation checks of the decode kernels (CPU only: hipcc cross-compiles).

A register spill reloaded inside a tile loop waits behind the tile loads in
flight (vector-memory counters retire in order) and costs a memory latency per
reload; one such regression made the 128-head INT4 kernel six times slower with
every parity test still passing.  This test compiles decode_attn.hip to gfx950
assembly and checks that no hot loop of any decode kernel (a loop holding more
than 30 matrix instructions, innermost) reads scratch memory, and that every decode kernel
uses no private scratch arrays beyond a few spilled values.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KDIR = os.path.join(ROOT, "mla_absorbed_latent_amd", "csrc", "kernels")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

pytestmark = pytest.mark.skipif(HIPCC is None, reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "decode_attn.s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + KDIR, "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", out, os.path.join(KDIR, "decode_attn.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return open(out).read().split("\n")


def _kernels(lines):
    starts = [(i, m.group(1)) for i, l in enumerate(lines) for m in [re.match(r"^(_ZN3mla\d+decode_h\w+):", l)] if m]
    assert len(starts) == 16, starts         # decode_h128v2 (bf16), decode_h128 x 7 quantised formats, decode_h16 x 8
    for st, name in starts:
        # the whole function (a kernel may hold several s_endpgm)
        en = next(i for i in range(st, len(lines)) if lines[i].startswith(".Lfunc_end"))
        yield name, lines[st:en]


def _hot_loops(body):
    """Innermost loops holding more than 30 matrix instructions (the tile loops)."""
    labels = {}
    for i, l in enumerate(body):
        m = re.match(r"^(\.LBB\d+_\d+):", l)
        if m:
            labels[m.group(1)] = i
    loops = []
    for i, l in enumerate(body):
        m = re.search(r"s_(?:c)?branch\w*\s+(\.LBB\d+_\d+)$", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a, b = labels[m.group(1)], i
            if sum("v_mfma" in body[j] for j in range(a, b)) > 30:
                loops.append((a, b))
    for a, b in loops:
        if not any(a <= c and d <= b and (c, d) != (a, b) for c, d in loops):
            yield a, b


def test_no_scratch_reads_in_tile_loops(asm):
    for name, body in _kernels(asm):
        loops = list(_hot_loops(body))
        assert loops, name
        for a, b in loops:
            reloads = sum("scratch_load" in body[j] for j in range(a, b))
            assert reloads == 0, (name, a, b, reloads)


def test_no_scratch_reads_in_staging_loops(asm):
    """The 16-head kernels' staging loops (no matrix instructions, so not covered
    above) must not reload spills either: a reload waits behind the tile loads
    the loop keeps in flight."""
    checked = 0
    for name, body in _kernels(asm):
        if "decode_h16" not in name:
            continue
        for hdr, seg in _staging_loops(body):
            assert not any("scratch_load" in x for x in seg), (name, hdr)
            checked += 1
    assert checked >= 9, checked


def test_scratch_stays_small(asm):
    text = "\n".join(asm)
    for m in re.finditer(r"\.name:\s+(_ZN3mla\d+decode_h\S+)\s*\n(?:.*\n){0,80}?\s+\.private_segment_fixed_size:\s+(\d+)", text):
        assert int(m.group(2)) <= 128, (m.group(1), m.group(2))


@pytest.mark.parametrize("src", ["prefill.hip", "front.hip"])
def test_prompt_path_kernels_use_no_scratch(src, tmp_path):
    """The prompt-path kernels (K/V expansion, prefill attention, projections)
    are sized to fit their registers; a spill there would be a silent
    regression of the same kind as in the decode kernels."""
    out = str(tmp_path / (src + ".s"))
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + KDIR, "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", out, os.path.join(KDIR, src)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    text = open(out).read()
    sizes = re.findall(r"\.name:\s+(_ZN\S+)\s*\n(?:.*\n){0,80}?\s+\.private_segment_fixed_size:\s+(\d+)", text)
    assert sizes, src
    for name, size in sizes:
        assert int(size) == 0, (name, size)


def test_expansion_keeps_stages_in_flight(tmp_path):
    """The K/V expansion keeps two 32-channel stages of direct-to-LDS loads in
    flight: each stage waits only until the later stage's loads (6 a wave) are
    left, before a bare s_barrier.  A workgroup fence (as in __syncthreads)
    would add vmcnt(0) before every barrier and drain the pipeline with every
    parity test still passing; so each of the two stage sequences (the K_nope
    and the V^T instance) must wait vmcnt(6) 15 times, then vmcnt(0), and
    nothing else; its barriers are the 16 stages' and the two around the
    output tile staged in LDS."""
    out = str(tmp_path / "prefill.s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I" + KDIR, "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           "-o", out, os.path.join(KDIR, "prefill.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    lines = open(out).read().split("\n")
    st = next(i for i, l in enumerate(lines) if "expand_kv_kernel" in l and re.match(r"^_Z\S+:", l))
    en = next(i for i in range(st, len(lines)) if lines[i].startswith(".Lfunc_end"))
    waits = [int(m.group(1)) for l in lines[st:en] for m in [_WAIT_VM.search(l)] if m]
    assert waits == ([6] * 15 + [0]) * 2, waits
    assert sum("s_barrier" in l for l in lines[st:en]) == (16 + 2) * 2


_VMEM = re.compile(r"^\s*(global_load|global_store|buffer_load|buffer_store|global_atomic)\w*\s+(v\[(\d+):(\d+)\]|v(\d+))")
_WAIT_VM = re.compile(r"s_waitcnt\s+vmcnt\((\d+)\)")
_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(line):
    out = set()
    for m in _VREG.finditer(line.split(";")[0]):
        if m.group(1) is not None:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _loop_bodies(body):
    """Lines of every loop, keyed by its header block, from the compiler's block
    annotations: a block belongs to the innermost loop named in its comment
    ("in Loop: Header=BBx_y") or heads one ("Loop Header" / "Parent Loop").
    Blocks are returned in layout order; the compiler lays a loop out so that
    this order, taken cyclically, is the order of execution."""
    blocks = []   # (header or None, [lines])
    for l in body:
        m = re.match(r"^(?:\.L(BB\d+_\d+)|; %bb\.\d+):(.*)$", l)
        if m:
            own, note = m.group(1), m.group(2)
            h = re.search(r"in Loop: Header=(BB\d+_\d+)", note)
            if h:
                hdr = h.group(1)
            elif own and ("Loop Header" in note or "Parent Loop" in note):
                hdr = own
            else:
                hdr = None
            blocks.append((hdr, [l]))
        elif blocks:
            blocks[-1][1].append(l)
    loops = {}
    for hdr, lines in blocks:
        if hdr is not None:
            loops.setdefault(hdr, []).extend(lines)
    return loops


def _staging_loops(body):
    """Innermost loops that issue non-temporal tile loads, write LDS, hold no
    matrix instruction and wait with vmcnt(N > 0): the 16-head kernels'
    staging waves."""
    out = []
    for hdr, seg in _loop_bodies(body).items():
        if any(" nt" in x and "global_load" in x for x in seg) and any("ds_write" in x for x in seg) \
                and not any("v_mfma" in x for x in seg) \
                and any(int(m.group(1)) > 0 for x in seg for m in [_WAIT_VM.search(x)] if m):
            out.append((hdr, seg))
    return out


def _inflight_hazards(seg):
    """Simulate a staging loop, taken cyclically twice, against the in-order
    vector-memory counter: a load joins the queue, s_waitcnt vmcnt(N) retires all
    but the youngest N.  In the second pass (the queue then holds what the loop
    keeps in flight across its back edge) return every instruction that touches
    a register some queued load still writes."""
    bad = []
    q = []
    for second in (False, True):
        for i, l in enumerate(seg):
            m = _WAIT_VM.search(l)
            if m:
                del q[:max(0, len(q) - int(m.group(1)))]
                continue
            inflight = set().union(*q) if q else set()
            if _VMEM.match(l):
                ops = l.split(";")[0].split(",")
                srcs = set().union(*(_regs(o) for o in ops[1:])) if len(ops) > 1 else set()
                if second and srcs & inflight:
                    bad.append((i, l.strip()))
                q.append(_regs(ops[0]))
            elif second and _regs(l) & inflight:
                bad.append((i, l.strip()))
    return bad


def test_staging_waits_match_the_loads_left_in_flight(asm):
    """The 16-head staging waves load tiles with inline assembly the compiler
    does not count, and wait for them with hand-written vmcnt(N) values (N = the
    loads of the tiles that stay in flight: one other tile, or the rest of a ring
    of tiles).  In each staging loop, no instruction may touch a destination
    register of a load that a wait has not retired (the vector-memory counter
    retires loads in order, oldest first)."""
    checked = 0
    for name, body in _kernels(asm):
        if "decode_h16" not in name:
            continue
        loops = _staging_loops(body)
        assert loops, name
        for hdr, seg in loops:
            bad = _inflight_hazards(seg)
            assert not bad, (name, hdr, bad[:3])
            checked += 1
    assert checked >= 9, checked


def test_inflight_check_catches_a_short_wait():
    """The check above on a hand-written loop: one tied load per step and a wait
    that leaves the other step's load in flight passes; a wait that leaves both in
    flight fails."""
    good = ["global_load_dwordx4 v[0:3], v[20:21], off nt", "s_waitcnt vmcnt(1)", "ds_write_b128 v30, v[4:7]",
            "global_load_dwordx4 v[4:7], v[22:23], off nt", "s_waitcnt vmcnt(1)", "ds_write_b128 v30, v[0:3]"]
    assert not _inflight_hazards(good)
    short = [l.replace("vmcnt(1)", "vmcnt(2)") for l in good]
    assert _inflight_hazards(short)
