"""CPU models of the load schedules that the two LDS-pipelined kernels rely on.

Vector-memory operations of one wave complete in issue order, and `s_waitcnt vmcnt(N)`
waits until at most the N most recently issued are outstanding.  A kernel that waits with
a fixed N therefore depends on its exact issue order.  The models below replay each
kernel's issue order, waits and workgroup barriers as stated in the kernel sources
(`precompute.hip`: the LR precompute's X window and A_cat tile ring; `fla_bf16.hip`: the
prefill's two wave groups and three rotating tile buffers) for every tile count up to a
bound, and check:
  - every operand a step reads was issued, waited for by the wave(s) that loaded it, and
    published by a barrier before the read;
  - no load into a buffer or register slot is issued while the previous content can still
    be read (the read happened before a barrier that precedes the issue);
  - both wave groups of the prefill pass the same number of workgroup barriers (a mismatch
    would leave one group waiting for good);
  - every wait immediate fits the vmcnt field (0..63).
Changing a kernel's issue order, waits or rotation means changing the model with it."""

import pytest


class Wave:
    """One wave's in-order vector-memory queue.  Loads are (tag, ops) pairs."""

    def __init__(self):
        self.queue = []        # tags, one entry per operation, oldest first
        self.done = set()      # tags with every operation complete

    def issue(self, tag, ops):
        assert ops > 0
        self.queue.extend([tag] * ops)

    def wait(self, n):
        assert 0 <= n <= 63, f"vmcnt immediate {n}"
        while len(self.queue) > n:
            tag = self.queue.pop(0)
            if tag not in self.queue:
                self.done.add(tag)


# ---------------------------------------------------------------------------------------
# LR precompute (lr_precompute_bf16<NCB>): NT A_cat tiles in LDS, UNROLL X register slots
# ---------------------------------------------------------------------------------------

def precompute_schedule(nk, ncb, nt=4, unroll=8, nb=2):
    xn = nb * 2                  # X loads per wave per chunk (two k-steps)
    naw = ncb // 2               # 1 KB A_cat units per wave per chunk: 64 * ncb * 32 / 4096
    wait_n = 3 * xn + 2 * naw
    nk_pad = -(-nk // unroll) * unroll
    w = Wave()
    tile = {}                    # tile index -> chunk last loaded into it
    slot = {}                    # X slot -> chunk last loaded into it
    consumed = set()             # chunks whose step has passed its end-of-step barrier

    def load_a(c, step):
        t = c % nt
        prev = tile.get(t)
        # the previous chunk in this tile was read in a step that ended with a barrier
        assert prev is None or prev in consumed, (nk, step, c, prev)
        tile[t] = c
        w.issue(("A", c), naw)

    def load_x(c, step):
        s = c % unroll
        prev = slot.get(s)
        assert prev is None or prev in consumed, (nk, step, c, prev)
        slot[s] = c
        w.issue(("X", c), xn)

    # prologue: X(0) A(0) X(1) A(1) X(2) A(2) X(3)
    for i in range(nt - 1):
        load_x(i, -1)
        load_a(i, -1)
    load_x(nt - 1, -1)
    w.wait(wait_n)
    for kc in range(nk_pad):
        load_a(kc + nt - 1, kc)
        load_x(kc + nt, kc)
        # the step's MFMAs read tile kc % nt and X slot kc % unroll
        assert tile[kc % nt] == kc and ("A", kc) in w.done, (nk, kc)
        assert slot[kc % unroll] == kc and ("X", kc) in w.done, (nk, kc)
        w.wait(wait_n)
        consumed.add(kc)         # end-of-step barrier: every wave's reads of kc are over
    # what is still in flight at the end are loads of padded chunks (empty resources); the
    # epilogue's own argument loads wait with vmcnt(0), which retires them before any store
    assert all(tag[1] >= nk for tag in w.queue), (nk, w.queue)
    return wait_n


@pytest.mark.parametrize("ncb", [4, 8, 12, 16])
def test_precompute_schedule(ncb):
    for nk in range(1, 41):
        wait_n = precompute_schedule(nk, ncb)
    assert wait_n <= 63


def test_precompute_model_catches_a_short_wait():
    """The model rejects a schedule whose wait leaves one chunk too many in flight."""
    def bad(nk):
        w = Wave()
        for c in range(3):
            w.issue(("A", c), 6)
        w.wait(2 * 6)            # leaves A(1), A(2) in flight: A(0) done
        assert ("A", 0) in w.done
        w.issue(("A", 3), 6)
        w.wait(3 * 6)            # one tile's worth too lenient: A(1) not retired
        return ("A", 1) in w.done
    assert not bad(8)


# ---------------------------------------------------------------------------------------
# Prefill ping-pong (prefill_item<D, RB, EX>): groups A (K loads) and B (V_base + L loads)
# ---------------------------------------------------------------------------------------

N_K, N_V = 4, 6                  # direct loads per wave and tile (D = 128, RB > 0)


class Group:
    """One wave group's program: loads, waits and LDS accesses between barriers."""

    def __init__(self, name):
        self.name = name
        self.wave = Wave()
        self.seg = 0                       # index of the segment between barriers
        self.issues = []                   # (seg, buffer, region, tile)
        self.retired_at = {}               # (buffer, region, tile) -> segment of the wait
        self.reads = []                    # (seg, buffer, region, tile, checked)
        self.writes = []                   # (seg, buffer, region, tile): LDS stores

    def load(self, buf, regions, tile, ops):
        for r in regions:
            self.issues.append((self.seg, buf, r, tile))
        self.wave.issue((buf, tuple(regions), tile), ops)

    def wait(self, n):
        self.wave.wait(n)
        for (buf, regions, tile) in self.wave.done:
            for r in regions:
                self.retired_at.setdefault((buf, r, tile), self.seg)

    def read(self, buf, region, tile, checked=True):
        self.reads.append((self.seg, buf, region, tile, checked))

    def barrier(self):
        self.seg += 1


def prefill_programs(n, ex, lr=True, slack=0, nbuf=3):
    """Replay both groups for an item of n key tiles.  Regions: K, V (V_base), L.  slack
    loosens group A's K waits by that many operations and nbuf changes the number of
    rotating buffers (both for the model's own checks)."""
    a, b = Group("A"), Group("B")
    bufs = tuple(f"buf{i}" for i in range(nbuf))
    vl = ("V", "L") if lr else ("V",)
    nv = N_V if lr else N_K
    # every wave zeroes the V/L rows of buf2 ("tile -1") before the prologue
    for g in (a, b):
        for r in vl:
            g.writes.append((g.seg, bufs[-1], r, -1))
    # prologue
    if n > 0:
        a.load("buf0", ("K",), 0, N_K)
    if n > 1:
        a.load("buf1", ("K",), 1, N_K)
        a.wait(N_K)
    else:
        a.wait(0)
    if n > 0:
        b.load("buf0", vl, 0, nv)
    if ex and lr:
        b.load("btile", ("V",), "Bg", N_K)
    b.wait(0)
    a.barrier(), b.barrier()
    if n > 1:
        b.load("buf1", vl, 1, nv)
    b.barrier()                           # B starts one phase late

    def step(g, j):
        kbuf, vbuf = bufs[j % nbuf], bufs[(j - 1) % nbuf]
        dma = vbuf
        if ex and g is b and j < n:      # in-tile expansion of tile j (V += L·B_g)
            g.read(kbuf, "V", j), g.read(kbuf, "L", j), g.read("btile", "V", "Bg")
            g.writes.append((g.seg, kbuf, "V", j))
        # matrix phase: P·V (and P·L) of tile j - 1, then the scores of tile j
        g.read(vbuf, "V", j - 1)
        if lr and not ex:
            g.read(vbuf, "L", j - 1)
        g.read(kbuf, "K", j, checked=j < n)   # the last step's scores are never used
        if not ex and g is b:
            g.wait(nv if j + 1 < n else 0)
        g.barrier()
        if j + 2 < n:
            if g is b:
                g.load(dma, vl, j + 2, nv)
            else:
                g.load(dma, ("K",), j + 2, N_K)
        # softmax phase: no LDS access
        if g is a:
            g.wait(N_K + slack if j + 2 < n else 0)
        elif ex:
            g.wait(nv if j + 2 < n else 0)
        g.barrier()

    for j in range(n + 1):
        step(a, j)
        step(b, j)
    a.barrier()                          # matches B's extra barrier in the prologue
    # epilogue: B_g into buf0's V rows for the P·L term
    if lr and not ex:
        a.wait(0), b.wait(0)
        b.load("buf0", ("V",), "Bg", N_K)
        b.wait(0)
        a.barrier(), b.barrier()
        a.read("buf0", "V", "Bg"), b.read("buf0", "V", "Bg")
    return a, b


def check_prefill(n, ex, lr=True):
    a, b = prefill_programs(n, ex, lr)
    check_groups(a, b, n, ex)


def check_groups(a, b, n, ex):
    assert a.seg == b.seg, f"barrier counts differ: A {a.seg}, B {b.seg} (n={n}, ex={ex})"
    groups = (a, b)
    # content history of each (buffer, region): (segment it becomes readable, tile,
    # segment it was issued); LDS stores by the groups themselves become readable after
    # the next barrier
    events = {}
    for g in groups:
        for (seg, buf, r, tile) in g.issues:
            ready = g.retired_at.get((buf, r, tile))
            assert ready is not None, f"{g.name}: load of {buf}.{r} tile {tile} never waited for"
            events.setdefault((buf, r), []).append((seg, ready + 1, tile, "load"))
        for (seg, buf, r, tile) in g.writes:
            events.setdefault((buf, r), []).append((seg, seg + 1, tile, "store"))
    for key in events:
        events[key].sort(key=lambda e: (e[0], e[1]))
    reads = [(g.name,) + rd for g in groups for rd in g.reads]
    for (who, seg, buf, r, tile, checked) in reads:
        hist = events.get((buf, r), [])
        # what was issued into this region in earlier segments (a load issued in the read's
        # own segment cannot have landed; an in-place store there follows the read)
        before = [e for e in hist if e[0] < seg]
        if not checked:
            # a discarded read may see stale data, but no load may be landing meanwhile
            # in a way that matters; nothing to check beyond the region existing
            continue
        assert before, f"{who} reads {buf}.{r} tile {tile} at segment {seg}: nothing there"
        last = before[-1]
        # the latest content issued at or before the read must be the tile read ...
        assert last[2] == tile, (f"{who} reads {buf}.{r} at segment {seg} expecting tile "
                                 f"{tile}, but tile {last[2]} was issued there at segment "
                                 f"{last[0]} (n={n}, ex={ex})")
        # ... and complete and published before the read
        assert last[1] <= seg, (
            f"{who} reads {buf}.{r} tile {tile} at segment {seg}; issued {last[0]}, "
            f"readable from {last[1]} (n={n}, ex={ex})")
        # an in-place store (the expansion) must follow the load of the same tile, and
        # both must precede the read
        loads = [e for e in before if e[2] == tile and e[3] == "load"]
        if tile not in (-1, "Bg"):
            assert loads and loads[-1][1] <= seg, (who, seg, buf, r, tile)
    # write after read: a load into a region is issued only after every read of the
    # region's previous content is over (an earlier segment)
    for (buf, r), hist in events.items():
        for (seg, _, tile, kind) in hist:
            if kind != "load":
                # an in-place store: no other group may read the region meanwhile
                for (who, rseg, rbuf, rr, rtile, checked) in reads:
                    owner = [g.name for g in groups if (seg, buf, r, tile) in g.writes]
                    if (rbuf, rr) == (buf, r) and rseg == seg and who not in owner and checked:
                        raise AssertionError(f"{who} reads {buf}.{r} at segment {seg} while "
                                             f"it is being rewritten (n={n}, ex={ex})")
                continue
            for (who, rseg, rbuf, rr, rtile, checked) in reads:
                if (rbuf, rr) == (buf, r) and rtile != tile and checked:
                    # reads of older content must end before this issue; reads of newer
                    # content (a later tile) come after a later load, checked above
                    older = rtile == -1 or (isinstance(rtile, int) and isinstance(tile, int)
                                            and rtile < tile) or tile == "Bg"
                    if older:
                        assert rseg < seg, (f"load of {buf}.{r} tile {tile} at segment "
                                            f"{seg} while {who} still reads tile {rtile} "
                                            f"there at segment {rseg} (n={n}, ex={ex})")


@pytest.mark.parametrize("ex", [False, True])
@pytest.mark.parametrize("lr", [True, False])
def test_prefill_schedule(ex, lr):
    if ex and not lr:
        pytest.skip("the expansion comparator always has an LR tile")
    for n in range(0, 13):
        check_prefill(n, ex, lr)


def test_prefill_model_catches_a_missing_barrier():
    """Dropping group A's closing barrier is a barrier-count mismatch."""
    a, b = prefill_programs(5, False)
    a.seg -= 1
    assert a.seg != b.seg


def test_prefill_model_catches_a_premature_load():
    """A K load issued two phases early, into the buffer whose K tile the other group still
    reads, is a hazard."""
    a, b = prefill_programs(6, False)
    a.issues = [(s - 2, buf, r, t) if (r == "K" and t == 4) else (s, buf, r, t)
                for (s, buf, r, t) in a.issues]
    with pytest.raises(AssertionError):
        check_groups(a, b, 6, False)


def test_prefill_model_catches_a_lenient_wait():
    """Leaving one more K tile in flight at group A's wait means K(j + 1) is not complete
    when the matrix phase j + 1 reads it."""
    a, b = prefill_programs(6, False, slack=N_K)
    with pytest.raises(AssertionError):
        check_groups(a, b, 6, False)


def test_prefill_model_catches_two_buffers():
    """Tile j is read in phases 2j .. 2j + 3, so two rotating buffers are too few."""
    a, b = prefill_programs(6, False, nbuf=2)
    with pytest.raises(AssertionError):
        check_groups(a, b, 6, False)
