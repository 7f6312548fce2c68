"""CPU checks of the hand-counted memory-counter waits against the compiled gfx950 code.

The grouped-GEMM and router kernels issue their operand loads as buffer->LDS
DMA from inline assembly and wait for them with explicit `s_waitcnt vmcnt(N)`
(the compiler keeps no count for those loads).  A wait is correct when, with
memory operations retiring in issue order, "at most N outstanding" implies that
every DMA of the stage about to be read has landed; it is tight when one more
outstanding operation would not.  These checks compile the kernels to gfx950
assembly on the CPU (hipcc, no GPU), read the DMA and wait sequence the
compiler actually emitted, replay it against a FIFO model of the issue order
the kernels document, and require every wait to be correct and tight:

* grouped GEMM, narrow ring (K steps of 32), steady state: each K step issues
  one step's DMA (ND instructions, half before and half after the wait); the
  wait before the barrier leaves only the steps newer than the one about to be
  read in flight;
* grouped GEMM, wide ring (K blocks of 64, five regions): the prologue loads
  A and B of blocks 0 and 1; block j issues block j + 2's A before its wait
  and block j + 2's B after it, and the wait must leave only that A in flight;
* grouped GEMM, tile change: the next tile's prologue is issued before the
  current tile's epilogue, so the first wait of the next K loop counts the
  epilogue's vector memory instructions too.  Their number in the compiled
  epilogue (stores, and the g/u loads of the down data gradient, the scale
  loads of the FP8 kernels) must equal the constant the wait is built from;
* router: each wave's private ring of W_r stages (one per 16-row step) and x
  stages (one per four steps), with the prologue and refill order of the
  kernel; every wait before a step's fragment reads must cover both stages.
"""
import importlib.util
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_expert_layer_router_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
VMCNT_MAX = 63


def _build_flags():
    """The library's own compile flags (moe_expert_layer_router_amd/build.py), minus linking."""
    spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "moe_expert_layer_router_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [f for f in mod.FLAGS if f not in ("-shared", "-fPIC")]


def _asm(src):
    out = os.path.join(tempfile.mkdtemp(prefix="moe_isa_"), os.path.basename(src) + ".s")
    cmd = [HIPCC, *_build_flags(), "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read().split("\n")


@pytest.fixture(scope="module")
def gemm_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    return _asm(os.path.join(CSRC, "gemm.hip"))


@pytest.fixture(scope="module")
def route_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    return _asm(os.path.join(CSRC, "route.hip"))


def _functions(lines, pattern):
    """{mangled name: body lines} of the kernels whose symbol matches pattern."""
    out = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*" + pattern + r"\S*):", l)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].strip().startswith(".Lfunc_end"))
            out[m.group(1)] = lines[i:end]
    return out


def _events(body):
    """The kernel's DMA issues ('D'), vmcnt waits (int) and loop headers ('L')."""
    ev = []
    for l in body:
        t = l.strip()
        if t.startswith("buffer_load_dwordx4") and " lds" in t:
            ev.append("D")
        elif t.startswith("s_waitcnt") and "vmcnt(" in t:
            ev.append(int(re.search(r"vmcnt\((\d+)\)", t).group(1)))
        elif "Loop Header" in t:
            ev.append("L")
    return ev


def _epilogue_ops(body):
    """Vector memory instructions other than the DMA: buffer stores and plain buffer loads."""
    n = 0
    for l in body:
        t = l.strip()
        if re.match(r"buffer_(store|load)_\w+", t) and " lds" not in t:
            n += 1
    return n


class Fifo:
    """Outstanding memory operations in issue order, each labelled."""

    def __init__(self):
        self.q = []

    def issue(self, label, n=1):
        self.q += [label] * n

    def wait(self, n):
        """s_waitcnt vmcnt(n): the oldest operations retire until at most n remain."""
        if len(self.q) > n:
            self.q = self.q[len(self.q) - n:]

    def pending(self, label):
        return label in self.q


# gemm_kernel<KIND, BM, FP8, WIDE>: KIND 0 gate/up, 1 down, 2 down data gradient,
# 3 gate/up data gradient, 4 weight gradient, 5 FP8 weight gradient, 6 router
# input gradient; the bf16 M-grouped products (KIND 0-3) and the router
# product run on the wide ring.  Per-lane
# vector memory instructions of one epilogue, as the kernel counts them (stores
# per 16-row half pass, times 2 MI passes), and the FP8 scale loads of the next
# tile.  The FP8 weight gradient does not count its epilogue (None): its first
# wait after a tile change is the plain one.
def _design(kind, bm, fp8):
    mi = bm // 64
    # (FP8: the forward and data-gradient products, kinds 0 and 1; the FP8
    # weight gradient, kind 5, stays on the narrow ring)
    wide = bm == 256 and (kind in (0, 1, 2, 3, 4, 6) if not fp8 else kind in (0, 1))
    nst = 4 if bm == 256 else 3
    bkx = 64 if wide else 32
    nia, nib = bm * bkx * 2 // 4096, 256 * bkx * 2 // 4096
    epi = {0: 12 * mi, 1: 8 * mi, 2: 32 * mi, 3: 8 * mi, 4: 16 * mi, 5: None, 6: 16 * mi}[kind]
    scales = 0
    if fp8:
        nr = 4 * mi if kind == 0 else 8 * mi
        nc = 16 if kind == 0 else 8
        scales = nr + nc // 4
    # the bf16 M-grouped products and the router product compile the wide K loop
    # three times (all four 32-row blocks of a wave multiplied, the first two,
    # none: an expert's last row tile may end inside a wave's rows)
    forms = 3 if wide and not fp8 and kind in (0, 1, 2, 3, 6) else 1
    return {"nst": nst, "nd": nia + nib, "nia": nia, "epi": epi, "scales": scales, "sep": bm == 256,
            "wide": wide, "forms": forms}


GEMM_KERNELS = [(0, 256, False), (1, 256, False), (2, 256, False), (3, 256, False), (4, 256, False),
                (0, 256, True), (1, 256, True), (6, 256, False)]
GEMM_KERNELS_ALL = GEMM_KERNELS + [(5, 256, True)]


def _gemm_body(gemm_asm, kind, bm, fp8):
    wide = _design(kind, bm, fp8)["wide"]
    pat = r"gemm_kernelILi%dELi%dELb%dELb%dE" % (kind, bm, int(fp8), int(wide))
    f = _functions(gemm_asm, pat)
    assert len(f) == 1, (pat, list(f))
    return next(iter(f.values()))


@pytest.mark.parametrize("kind,bm,fp8", GEMM_KERNELS, ids=lambda v: str(v))
def test_gemm_epilogue_memory_ops_match_the_wait(gemm_asm, kind, bm, fp8):
    """The compiled epilogue issues exactly the vector memory instructions the
    first wait after a tile change is built from (plus, for FP8, the scale loads
    of the first tile, issued once before the loop)."""
    d = _design(kind, bm, fp8)
    body = _gemm_body(gemm_asm, kind, bm, fp8)
    # (the weight gradient's accumulating and folding epilogues, which take the
    # plain wait, use global loads and stores, not buffer instructions)
    got = _epilogue_ops(body)
    assert got == d["epi"] + 2 * d["scales"], (got, d)
    # no wait for every outstanding operation inside an unconditional
    # epilogue (it would drain the next tile's prefetched DMA): no more
    # vmcnt(0) waits than the down projection of the same precision, whose
    # epilogue only stores
    if d["sep"] and kind in (0, 2, 3):
        ref = _events(_gemm_body(gemm_asm, 1, 256, fp8)).count(0)
        assert _events(body).count(0) <= ref, (_events(body).count(0), ref)


@pytest.mark.parametrize("kind,bm,fp8", GEMM_KERNELS_ALL, ids=lambda v: str(v))
def test_gemm_ring_waits_are_correct_and_tight(gemm_asm, kind, bm, fp8):
    """Replays the ring: prologue, K steps, epilogue + next prologue, next K steps,
    with the DMA counts and wait values taken from the compiled kernel."""
    d = _design(kind, bm, fp8)
    ev = _events(_gemm_body(gemm_asm, kind, bm, fp8))
    if d["wide"]:
        _check_wide_ring(ev, d)
        return
    nst, nd = d["nst"], d["nd"]
    dmas = [e for e in ev if e == "D"]
    # prologue (steps 0 .. NST-2 and half of NST-1) twice, one K step's DMA in the loop
    assert len(dmas) == 2 * ((nst - 1) * nd + nd // 2) + nd, (len(dmas), d)
    waits = [e for e in ev if isinstance(e, int) and e > 0]
    k_first = (nst - 2) * nd + nd // 2
    k_loop = (nst - 2) * nd
    assert k_first in waits and k_loop in waits, (waits, k_first, k_loop)
    plain_after = d["epi"] is None
    k_epi = 0 if plain_after else d["epi"] + d["scales"]
    k_after = min(VMCNT_MAX, k_first + k_epi)
    if d["sep"]:
        assert k_after in waits, (waits, k_after)

    def prologue(f, tile):
        for st in range(nst):
            f.issue((tile, st), nd if st < nst - 1 else nd // 2)

    def k_loop_steps(f, tile, nk, first_wait):
        """The K loop of one tile: returns after the last step.  Checks that the
        step about to be read has landed at every wait, and that one more
        outstanding operation would have let it pass unlanded (tight)."""
        f.wait(first_wait)
        assert not f.pending((tile, 0))
        tight = Fifo()
        tight.q = list(f.q)
        for kt in range(nk):
            # sub-step 0: second half of step kt + NST - 1
            f.issue((tile, kt + nst - 1), nd - nd // 2)
            before = list(f.q)
            f.wait(k_loop)
            if kt + 1 < nk:
                assert not f.pending((tile, kt + 1)), (kt, f.q)
                if "epilogue" not in before:
                    # steady state (only DMA outstanding): one more would not do
                    probe = Fifo()
                    probe.q = before
                    probe.wait(k_loop + 1)
                    assert probe.pending((tile, kt + 1)), "wait not tight"
            # sub-step 1: first half of step kt + NST
            f.issue((tile, kt + nst), nd // 2)
        f.wait(0)                       # the ring drains before reuse

    f = Fifo()
    prologue(f, 0)
    before = list(f.q)
    k_loop_steps(f, 0, 24, k_first)
    probe = Fifo()
    probe.q = before
    probe.wait(k_first + 1)
    assert probe.pending((0, 0)), "first wait not tight"
    # tile change: next prologue, then this tile's epilogue (and FP8 scales)
    if d["sep"] and plain_after:
        # an uncounted epilogue of any size: the plain wait is still correct
        for n_epi in (0, 7, 40, 100):
            g = Fifo()
            prologue(g, 1)
            g.issue("epilogue", n_epi)
            k_loop_steps(g, 1, 24, k_first)
    elif d["sep"]:
        prologue(f, 1)
        f.issue("epilogue", k_epi)
        before = list(f.q)
        k_loop_steps(f, 1, 24, k_after)
        if k_first + k_epi <= VMCNT_MAX:
            probe = Fifo()
            probe.q = before
            probe.wait(k_after + 1)
            assert probe.pending((1, 0)), "wait after the epilogue not tight"
    else:
        f.issue("epilogue", k_epi)
        prologue(f, 1)
        k_loop_steps(f, 1, 24, k_first)


def _check_wide_ring(ev, d):
    """The wide ring: loads are labelled (tile, block, operand).  The prologue
    issues A and B of blocks 0 and 1 (NIA + NIB instructions each pair); in
    block j the kernel issues block j + 2's A (NIA), waits, and issues block
    j + 2's B (NIB).  The wait before block j + 1's fragments are read must
    leave block j + 1 landed and be tight; the first wait of a tile (plain, or
    after the previous epilogue's counted operations) must cover block 0."""
    nd, nia = d["nd"], d["nia"]
    nib = nd - nia
    dmas = [e for e in ev if e == "D"]
    # prologue twice (first tile, next tile), one block's two DMA groups in
    # each form of the loop
    assert len(dmas) == 2 * 2 * nd + d["forms"] * nd, (len(dmas), d)
    waits = [e for e in ev if isinstance(e, int) and e > 0]
    k_first, k_loop = nd, nia
    assert k_first in waits and k_loop in waits, (waits, k_first, k_loop)
    k_epi = d["epi"] + d["scales"]
    k_after = min(VMCNT_MAX, k_first + k_epi)
    assert k_after in waits, (waits, k_after)
    # inside each form of the loop exactly one wait, between the two DMA groups
    # (a K loop's header: one directly followed by a DMA; the tile loop's comes
    # first, epilogue loops come later); a body ends at the next loop header or
    # the drain after the loop
    hdrs = [i for i, e in enumerate(ev[:-1]) if e == "L" and ev[i + 1] == "D"]
    assert len(hdrs) == d["forms"], hdrs
    for hdr in hdrs:
        end = next(i for i in range(hdr + 1, len(ev)) if ev[i] == 0 or ev[i] == "L")
        body = ev[hdr + 1:end]
        assert body == ["D"] * nia + [k_loop] + ["D"] * nib, body

    def prologue(f, tile):
        for blk in range(2):
            f.issue((tile, blk, "A"), nia)
            f.issue((tile, blk, "B"), nib)

    def landed(f, tile, blk):
        return not f.pending((tile, blk, "A")) and not f.pending((tile, blk, "B"))

    def k_blocks(f, tile, nk, first_wait):
        f.wait(first_wait)
        assert landed(f, tile, 0)
        for j in range(nk):
            f.issue((tile, j + 2, "A"), nia)
            before = list(f.q)
            f.wait(k_loop)
            if j + 1 < nk:
                assert landed(f, tile, j + 1), (j, f.q)
                if "epilogue" not in before:
                    probe = Fifo()
                    probe.q = before
                    probe.wait(k_loop + 1)
                    assert not landed(probe, tile, j + 1), "wait not tight"
            f.issue((tile, j + 2, "B"), nib)
        f.wait(0)

    f = Fifo()
    prologue(f, 0)
    before = list(f.q)
    k_blocks(f, 0, 12, k_first)
    probe = Fifo()
    probe.q = before
    probe.wait(k_first + 1)
    assert not landed(probe, 0, 0), "first wait not tight"
    prologue(f, 1)
    f.issue("epilogue", k_epi)
    before = list(f.q)
    k_blocks(f, 1, 12, k_after)
    if k_first + k_epi <= VMCNT_MAX:
        probe = Fifo()
        probe.q = before
        probe.wait(k_after + 1)
        assert not landed(probe, 1, 0), "wait after the epilogue not tight"
    for nk in (1, 2, 3):  # short tiles: the killed loads past K still count
        g = Fifo()
        prologue(g, 2)
        k_blocks(g, 2, nk, k_first)


@pytest.mark.parametrize("kind,bm,fp8", [(2, 256, False), (3, 256, False), (4, 256, False),
                                         (5, 256, True)])
def test_tile_ticket_latency_stays_hidden(gemm_asm, kind, bm, fp8):
    """The products that take tiles from a device counter draw the ticket of the
    tile after next with one lane's atomic add and hand the previous ticket to
    the workgroup through LDS.  No wait for all memory operations may follow the
    atomic directly (its result is used one tile later), and the hand-off goes
    through LDS, not a flat store."""
    body = [l.strip() for l in _gemm_body(gemm_asm, kind, bm, fp8)]
    code = [l for l in body if l and not l.startswith(";") and not l.startswith(".")]
    at = [i for i, l in enumerate(code) if l.startswith("global_atomic_add")]
    assert at, "no ticket atomic"
    for i in at:
        nxt = code[i + 1:i + 6]
        assert not any(l.startswith("s_waitcnt") and "vmcnt(0)" in l for l in nxt), nxt
    assert not any(l.startswith("flat_store") for l in code)


@pytest.mark.parametrize("nb", [1, 2, 4])
def test_router_ring_waits_are_correct_and_tight(route_asm, nb):
    """route_fused_kernel<NB>: each wave's ring holds DW W_r stages of 16 rows
    (NB DMA instructions each) and DXQ x stages of 64 columns (4 each).  The
    prologue issues the steady state's refills of the steps before step 0; after
    step i the kernel refills W_r stage i + DW, and after the last step of x
    stage q also x stage q + DXQ.  Before reading step i + 1's fragments it waits;
    the wait values and the DMA counts between them are the compiled ones."""
    dw = 3 if nb == 4 else 4
    dxq = 2
    f = _functions(route_asm, r"route_fused_kernelILi%dE" % nb)
    assert len(f) == 1
    ev = _events(next(iter(f.values())))
    # prologue: DMAs up to the first wait; loop body: from the loop header up to
    # the first wait of the epilogue (vmcnt(0))
    first = next(i for i, e in enumerate(ev) if isinstance(e, int))
    pro = ev[:first].count("D")
    hdr = ev.index("L")
    end = next(i for i in range(hdr, len(ev)) if ev[i] == 0)
    body = [e for e in ev[hdr + 1:end]]
    # the body: four (wait, refill) pairs, one per step of an x stage
    waits = [e for e in body if isinstance(e, int)]
    assert len(waits) == 4, body
    per_step = []
    cnt = None
    for e in body:
        if isinstance(e, int):
            if cnt is not None:
                per_step.append(cnt)
            cnt = 0
        elif e == "D":
            cnt += 1
    per_step.append(cnt)
    assert per_step == [nb, nb, nb, nb + 4], per_step

    # the model's issue order
    fifo = Fifo()
    lo = -max(4 * dxq, dw)
    n_pro = 0
    for j in range(lo, 0):
        if j + dw >= 0:
            fifo.issue(("w", j + dw), nb)
            n_pro += nb
        if (j & 3) == 3 and (j >> 2) + dxq >= 0:
            fifo.issue(("x", (j >> 2) + dxq), 4)
            n_pro += 4
    assert n_pro == pro, (n_pro, pro)
    need = lambda i: [("w", i), ("x", i // 4)]

    def check(wait, i, before):
        fifo.wait(wait)
        for lab in need(i):
            assert not fifo.pending(lab), (i, wait, lab)
        probe = Fifo()
        probe.q = before
        probe.wait(wait + 1)
        assert any(probe.pending(lab) for lab in need(i)), f"wait before step {i} not tight"

    w0 = ev[first]
    check(w0, 0, list(fifo.q))
    for q in range(6):
        for s4 in range(4):
            i = 4 * q + s4
            check(waits[s4], i + 1, list(fifo.q))
            fifo.issue(("w", i + dw), nb)
            if s4 == 3:
                fifo.issue(("x", q + dxq), 4)
