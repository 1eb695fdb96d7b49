"""Host-side model of the GEMM's direct-to-LDS operand pipelines (no GPU).

The bf16 GEMM (csrc/gemm_bf16.hip, GemmCore::run) has two pipelines in which buffer loads
with the LDS flag write operands straight into LDS and are waited for by COUNT:
s_waitcnt vmcnt(N) returns once at most N of this thread's vector-memory operations are
still outstanding.

* ADIRECT (the 8-wave 256 x 192 tile): A goes straight into three LDS slots, two steps
  ahead; B goes through two register sets into two slots, its register loads three steps
  ahead.  Step k: direct loads of A(k+2) in sub-step 0; in sub-step 1 the store of B(k+1)
  from its registers (the compiler waits for those loads first) and the register loads of
  B(k+3) into the same set; then vmcnt(LA + 2 LB) lgkmcnt(0), barrier, and the first
  fragment read of step k+1.  Whole rounds of six steps (the slot pattern repeats every
  six), then a tail of 0..5 steps.
* KG2 (the 8-wave tiles in two K groups: 192 x 192 for the fp32 weight gradients,
  64 x 192 for plain 16-bit stores of K-contiguous operands): A and B both straight into
  three slots, two steps ahead; step k: loads of step k+2, vmcnt(NLD) lgkmcnt(0),
  barrier; the loop runs whole rounds of three steps.

The model replays one thread's program order (every thread of the workgroup runs the
same sequence; a barrier publishes what each of them has completed) for every step count
and every shape the pipelines serve or once served, and checks:

  RAW   every fragment read of step k finds step k's data in the slot, all of it written
        (direct loads complete, register stores issued before an lgkmcnt(0)) before the
        barrier that precedes the read;
  WAR   no write into a slot is issued before a barrier that follows the completion of
        every read of the slot's previous contents;
  regs  no register set is reloaded before its previous contents were stored.

Three completion models for the count-based waits:
  "in order"  vector-memory loads complete in issue order, direct-to-LDS and register
              loads alike (the model the compiler's own wait insertion uses: it counts
              direct-to-LDS loads in the same in-order counter as register loads);
  "per kind"  only loads of the same kind complete in order among themselves;
  "any order" no order at all (only vmcnt(0) proves anything).

Result (asserted below): under "in order" both pipelines are free of races for every
shape and every step count 1..24, including the tails.  KG2 stays race-free under
"per kind" (all its loads are of one kind) but not under "any order".  ADIRECT does not
stay race-free under "per kind": its wait for A(k+1) counts the younger register loads of
B, so it relies on the two kinds completing in issue order.  The slot layouts are also
checked: every slot is filled exactly once by the 16-byte pieces of all lanes, and the
slots are disjoint and fit the LDS a workgroup may hold at the tile's occupancy.
"""
from __future__ import annotations

import pytest

BK = 64  # K elements per step


def adirect_program(nk, LA, LB):
    """One thread's events for the ADIRECT pipeline over nk steps."""
    ev = []

    def dma(k):
        ev.append(("dma", ("A", k), ("a", k % 3), LA))

    def gld(k):
        ev.append(("gld", ("B", k), k % 2, LB))

    def st(k):
        ev.append(("st", ("B", k), ("b", k % 2), k % 2))

    def rd(k):
        ev.append(("rd", ("A", k), ("a", k % 3)))
        ev.append(("rd", ("B", k), ("b", k % 2)))

    # prologue: A0 direct, B0 to registers then LDS, B1, A1, B2, wait, barrier, read #0 of step 0
    dma(0)
    gld(0)
    st(0)
    gld(1)
    dma(1)
    gld(2)
    ev.append(("wait", LA + 2 * LB))
    ev.append(("bar",))
    rd(0)
    for k in range(nk):  # the unrolled rounds of six and the tail run the same per-step code
        rd(k)  # sub-step 0 (k16 #1)
        dma(k + 2)
        rd(k)  # sub-step 1 (k16 #2)
        st(k + 1)
        gld(k + 3)
        rd(k)  # sub-step 2 (k16 #3)
        ev.append(("wait", LA + 2 * LB))
        ev.append(("bar",))
        if k + 1 < nk:
            rd(k + 1)  # k16 #0 of the next step
        else:
            ev.append(("rd_unused", ("A", k + 1), ("a", (k + 1) % 3)))
    ev.append(("wait", 0))
    return ev


def kg2_program(nk, NLD):
    """One thread's events for the KG2 pipeline over nk steps (loop of whole rounds of three)."""
    ev = []

    def ld(k):
        ev.append(("dma", ("S", k), ("s", k % 3), NLD))

    ld(0)
    ld(1)
    ev.append(("wait", NLD))
    ev.append(("bar",))
    ev.append(("rd", ("S", 0), ("s", 0)))
    nrun = -(-nk // 3) * 3  # steps past the K range load zeros (out-of-range offsets)
    for k in range(nrun):
        ev.append(("rd", ("S", k), ("s", k % 3)))
        ld(k + 2)
        ev.append(("wait", NLD))
        ev.append(("bar",))
        ev.append(("rd", ("S", k + 1), ("s", (k + 1) % 3)))
    ev.append(("wait", 0))
    return ev


def check(ev, model):
    """Replay the events; return the list of violations."""
    ops = []            # vector-memory instructions: [kind, tag, complete]
    slot_tag = {}       # slot -> tag of its latest write
    pend_w = {}         # slot -> instruction indices of direct loads not yet complete
    st_pending = set()  # slots with register stores not yet past an lgkmcnt(0)
    published = {}      # slot -> tag fully visible to every wave (as of the last barrier)
    pend_r = set()      # slots read since the last lgkmcnt(0)
    done_r = set()      # slots whose reads completed, not yet past a barrier
    safe_w = {}         # slot -> True once a barrier followed the completion of all its reads
    regs = {}           # register set -> tag loaded and not yet stored
    viol = []

    def complete_older(n):
        tot = len(ops)
        for i, op in enumerate(ops):
            if op[2]:
                continue
            if model == "in order":
                ok = i < tot - n
            elif model == "per kind":
                ok = sum(1 for j in range(i + 1, tot) if ops[j][0] == op[0]) >= n
            else:
                ok = n == 0
            if ok:
                op[2] = True

    def write_check(slot, tag):
        if not safe_w.get(slot, True):
            viol.append(("WAR", tag, slot))
        safe_w[slot] = True
        slot_tag[slot] = tag

    for e in ev:
        kind = e[0]
        if kind == "dma":
            _, tag, slot, n = e
            write_check(slot, tag)
            pend_w[slot] = []
            published.pop(slot, None)
            for _ in range(n):
                pend_w[slot].append(len(ops))
                ops.append(["dma", tag, False])
        elif kind == "gld":
            _, tag, rset, n = e
            if regs.get(rset) is not None:
                viol.append(("regs", tag, rset, regs[rset]))
            regs[rset] = tag
            for _ in range(n):
                ops.append(["reg", tag, False])
        elif kind == "st":
            _, tag, slot, rset = e
            if regs.get(rset) != tag:
                viol.append(("store of the wrong registers", tag, rset, regs.get(rset)))
            # the compiler's own wait: the registers' loads complete before the store
            for op in ops:
                if op[0] == "reg" and op[1] == tag:
                    op[2] = True
            regs[rset] = None
            write_check(slot, tag)
            pend_w[slot] = []
            published.pop(slot, None)
            st_pending.add(slot)
        elif kind == "wait":
            complete_older(e[1])
            st_pending.clear()          # lgkmcnt(0): this thread's LDS stores and reads are done
            done_r |= pend_r
            pend_r.clear()
        elif kind == "bar":
            for slot, idx in pend_w.items():
                if slot not in st_pending and all(ops[i][2] for i in idx):
                    published[slot] = slot_tag[slot]
            for slot in done_r:
                safe_w[slot] = True
            done_r.clear()
        elif kind in ("rd", "rd_unused"):
            _, tag, slot = e
            if kind == "rd" and published.get(slot) != tag:
                viol.append(("RAW", tag, slot, published.get(slot)))
            pend_r.add(slot)
            safe_w[slot] = False
    return viol


# (name, BM, BN, waves, occupancy): LA = BM / (8 waves), LB = BN / (8 waves) instructions each
ADIRECT_TILES = [("256x192 w8 (ADIRECT)", 256, 192, 8, 1), ("256x192 w4", 256, 192, 4, 1),
                 ("128x192 w4", 128, 192, 4, 2), ("128x128 w4", 128, 128, 4, 2),
                 ("64x192 w4", 64, 192, 4, 2), ("64x64 w4", 64, 64, 4, 4)]
STEPS = list(range(1, 25))


def _nis(tile):
    _, bm, bn, w, _ = tile
    return bm // (8 * w), bn // (8 * w)


@pytest.mark.parametrize("tile", ADIRECT_TILES, ids=[t[0] for t in ADIRECT_TILES])
def test_adirect_race_free_in_issue_order(tile):
    la, lb = _nis(tile)
    for nk in STEPS:
        assert check(adirect_program(nk, la, lb), "in order") == [], nk


@pytest.mark.parametrize("tile", ADIRECT_TILES, ids=[t[0] for t in ADIRECT_TILES])
def test_adirect_relies_on_order_across_kinds(tile):
    la, lb = _nis(tile)
    v = check(adirect_program(6, la, lb), "per kind")
    # the only failures: fragment reads of A whose direct loads may still be in flight
    assert v and all(x[0] == "RAW" and x[1][0] == "A" for x in v)


@pytest.mark.parametrize("nld", [6, 4], ids=["192x192 (NLD 6)", "64x192 (NLD 4)"])
def test_kgroup_race_free_per_kind(nld):
    for nk in STEPS:
        for model in ("in order", "per kind"):
            assert check(kg2_program(nk, nld), model) == [], (nk, model)
    assert check(kg2_program(6, nld), "any order")  # the count-based wait needs some order


def test_model_catches_planted_mistakes():
    """The checker itself: a wait one too loose, a slot reused one step early and a
    register set reloaded before its store are all reported."""
    ev = adirect_program(6, 4, 3)
    loose = [("wait", 4 + 2 * 3 + 1) if e == ("wait", 4 + 2 * 3) else e for e in ev]
    assert any(x[0] == "RAW" for x in check(loose, "in order"))
    early = [("dma", e[1], ("a", (e[1][1] + 1) % 3), e[3]) if e[0] == "dma" and e[1][1] >= 2 else e for e in ev]
    assert check(early, "in order")
    bad = list(ev)
    i = next(j for j, e in enumerate(bad) if e[0] == "st" and e[1] == ("B", 2))
    bad.insert(i, ("gld", ("B", 9), 0, 3))
    assert any(x[0] == "regs" for x in check(bad, "in order"))
    kg = kg2_program(6, 6)
    assert check([("wait", 7) if e == ("wait", 6) else e for e in kg], "in order")


def _pieces(rows_or_cols, nwv):
    """(instruction q = wave + nwv*i, lane) -> LDS byte offset of its 16 bytes within the slot
    (both operand loaders: instruction base q*1024, lane l at +16 l)."""
    ni = rows_or_cols // (8 * nwv)
    return [(w + nwv * i) * 1024 + 16 * l for w in range(nwv) for i in range(ni) for l in range(64)]


KG2_TILES = [("192x192 w8 kg2", 192, 192, 8, 1), ("64x192 w8 kg2", 64, 192, 8, 1)]


@pytest.mark.parametrize("tile", ADIRECT_TILES + KG2_TILES, ids=[t[0] for t in ADIRECT_TILES + KG2_TILES])
def test_slot_layout(tile):
    _, bm, bn, w, occ = tile
    a_bytes, b_bytes = bm * BK * 2, bn * BK * 2
    for n, size in ((bm, a_bytes), (bn, b_bytes)):
        p = sorted(_pieces(n, w))
        assert p == list(range(0, size, 16))  # the slot, each 16 bytes written by exactly one lane
    if tile[0].endswith("kg2"):  # A then B in each of three slots
        slots = [(s * (a_bytes + b_bytes), (s + 1) * (a_bytes + b_bytes)) for s in range(3)]
    else:
        slots = [(s * a_bytes, (s + 1) * a_bytes) for s in range(3)]
        slots += [(3 * a_bytes + s * b_bytes, 3 * a_bytes + (s + 1) * b_bytes) for s in range(2)]
    for i, (lo, hi) in enumerate(slots):
        for lo2, hi2 in slots[i + 1:]:
            assert hi <= lo2 or hi2 <= lo
    assert slots[-1][1] <= 160 * 1024
