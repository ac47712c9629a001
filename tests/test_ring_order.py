"""CPU model of the claiming modes' tile-id ring: barrier intervals of ring writes and reads.

In the dynamic and cancel-and-reuse modes a claimed tile id reaches the other
waves of a workgroup through an LDS ring: thread 0 writes the entry, and a
workgroup barrier publishes it (KernelWiki "Persistent Kernels with Cluster
Launch Control", intro: the response to a work request arrives through shared
memory, ordered by a barrier). A wave may read an entry only in a barrier
interval after the one in which it was written; a read in the same interval
races with the write and may see whatever the slot held before.

This model lists, for one workgroup, every barrier and the interval of every
ring write and every tile-id read in the order the kernels execute them, for
the three tile bodies:

* lockstep, 16-bit types: two MFMA k-groups per step, one barrier in the
  middle of each step, the copy of step s + 2 begun after step s's barrier;
* lockstep, e4m3: one barrier at the top of each step, the copy of step s + 1
  begun after it;
* ping-pong: waves 0-3 (X) and 4-7 (Y) in opposite phases, two barriers per
  step, each group beginning its copy of step s + 1 in its memory phase of
  step s; claims finished at the end of X's compute phase;
* producer waves: copy waves (which also claim) and MFMA waves meet at one
  barrier per step; the copy waves begin step j + 2 after barrier j, and
  both roles must pass the same number of barriers.

It checks the shipped protocols for every k-loop length and tile count, and
it characterizes the variant dropped during development, which published the
first claimed tile later than the shipped code: a publication point is safe
exactly when its interval precedes the first read of the entry, so a variant
that publishes tile 1 in the interval of step 2 (after that step's barrier) is
safe from 6 k-steps per tile on and races at 4 -- M = N = K = 256 at 64-deep
steps, the only case where the variant gave a wrong C on the GPU.
"""
import itertools

import pytest


class Trace:
    """Sequence of barriers and events of one workgroup; interval i lies between barrier i-1 and barrier i."""

    def __init__(self):
        self.barriers = 0
        self.writes = {}   # tile sequence number -> interval of its ring write
        self.reads = []    # (tile sequence number, interval, who)

    def barrier(self):
        self.barriers += 1

    def write(self, q):
        self.writes[q] = self.barriers

    def read(self, q, who):
        self.reads.append((q, self.barriers, who))

    def races(self, ring_from=0):
        """Reads of ring entries (sequence numbers >= ring_from) not published before the read."""
        bad = []
        for q, iv, who in self.reads:
            if q < ring_from:
                continue
            w = self.writes.get(q)
            if w is None or w >= iv:
                bad.append((q, iv, w, who))
        return bad


def claims_plan(mode, nk, defer_publish):
    """(sequence number claimed, step of the issue, step of the publication) for tile 0 and
    later tiles, as the kernels make them: dynamic claims tile 1 in the prologue; cancel with
    >= 4 k-steps defers tile 1 into tile 0 (issued after step 0's barrier, published before
    step 1's); every tile q then claims tile q + 2 at its end (lockstep) or first step
    (ping-pong). `defer_publish` overrides the publication step of tile 1 (the dropped
    variant; None = shipped)."""
    defer = mode == "cancel" and nk >= 4
    if defer_publish is not None:
        defer = True
    return defer


def lockstep16(mode, nk, ntiles, defer_publish=None, publish_after_barrier=False):
    """16-bit lockstep body. `defer_publish`: step at which tile 1's entry is written (None:
    shipped behaviour). `publish_after_barrier`: the write follows that step's barrier instead of
    preceding it."""
    t = Trace()
    S = ntiles * nk
    defer = claims_plan(mode, nk, defer_publish)
    pub_step = (1 if defer_publish is None else defer_publish) if defer else None
    # prologue: claims, then the claims barrier
    if mode == "cancel":
        t.write(0)
    if not defer:
        t.write(1)
    t.barrier()
    if mode == "cancel":
        t.read(0, "exit check")
    t.read(0, "producer")          # copy of step 0 begins tile 0
    # copy of step 1 (same tile, nk >= 2); wait; prologue barrier
    t.barrier()
    t.read(0, "consumer")
    for cs in range(S):
        q, kt = divmod(cs, nk)
        # k-group 0 of step cs; mid-step barrier when a next step exists
        has_next = cs + 1 < S
        if has_next:
            if pub_step is not None and cs == pub_step and not publish_after_barrier:
                t.write(1)
            t.barrier()
            if pub_step is not None and cs == pub_step and publish_after_barrier:
                t.write(1)
            u = cs + 2   # copy of step cs + 2 begins
            if u < S + nk and u % nk == 0:
                t.read(u // nk, "producer")
        if kt == nk - 1:
            # tile q finished: epilogue claims tile q + 2 and writes its entry after the stores
            t.write(q + 2)
            if has_next:
                t.read(q + 1, "consumer")
    return t


def lockstep8(mode, nk, ntiles, defer_publish=None, publish_after_barrier=False):
    """e4m3 lockstep body: barrier at the top of every step."""
    t = Trace()
    S = ntiles * nk
    defer = claims_plan(mode, nk, defer_publish)
    pub_step = (1 if defer_publish is None else defer_publish) if defer else None
    if mode == "cancel":
        t.write(0)
    if not defer:
        t.write(1)
    t.barrier()
    if mode == "cancel":
        t.read(0, "exit check")
    t.read(0, "producer")
    t.read(0, "consumer")
    for cs in range(S):
        q, kt = divmod(cs, nk)
        if pub_step is not None and cs == pub_step and not publish_after_barrier:
            t.write(1)
        t.barrier()
        if pub_step is not None and cs == pub_step and publish_after_barrier:
            t.write(1)
        u = cs + 1   # copy of step cs + 1 begins after the barrier
        if u < S + nk and u % nk == 0:
            t.read(u // nk, "producer")
        if kt == nk - 1:
            t.write(q + 2)
            if cs + 1 < S:
                t.read(q + 1, "consumer")
    return t


def pingpong(mode, nk, ntiles):
    """Ping-pong body: barriers P1, P2, ... after the prologue; X's memory phase of step s lies
    between P(2s) and P(2s+1), its compute phase between P(2s+1) and P(2s+2); Y's phases lie one
    barrier later. Thread 0 (an X wave) issues a claim at the first step of a tile (steps 0 and 2
    of tile 0 for cancel with a deferred tile 1) and writes the entry at the end of that step's
    compute phase."""
    t = Trace()
    S = ntiles * nk
    defer = mode == "cancel" and nk >= 4
    t.write(0)          # both claiming modes keep their first tile in the ring
    if not defer:
        t.write(1)
    t.barrier()         # claims barrier
    if mode == "cancel":
        t.read(0, "exit check")
    t.read(0, "X producer")
    t.read(0, "Y producer")
    t.barrier()         # prologue barrier = P0
    # the phase intervals: P(j) is barrier number 2 + j (0-based: claims 0, prologue 1)
    events = []         # (interval, kind, q, who)
    base = 2            # barriers before P1
    for s in range(S):
        q, kt = divmod(s, nk)
        x_mem = base + 2 * s         # interval index after P(2s)
        y_mem = x_mem + 1
        x_comp = x_mem + 1
        u = s + 1
        if u % nk == 0:
            events.append((x_mem, "read", u // nk, "X producer"))
            events.append((y_mem, "read", u // nk, "Y producer"))
        limit = 4 if (defer and q == 0) else 2
        if kt % 2 == 0 and kt < limit:
            target = (1 + kt // 2) if (defer and q == 0) else q + 2
            events.append((x_comp, "write", target, "thread 0"))
        if kt == nk - 1:
            # termination checks after the tile's last compute phases
            events.append((base + 2 * s + 2, "read", q + 1, "X consumer"))
            events.append((base + 2 * s + 3, "read", q + 1, "Y consumer"))
    for iv, kind, q, who in sorted(events, key=lambda e: (e[0], e[1] == "read")):
        if kind == "write":
            t.writes.setdefault(q, iv)
        else:
            t.reads.append((q, iv, who))
    return t


def producer(mode, nk, ntiles):
    """Producer-wave body. Barrier numbering as in the other models: the claims barrier, then
    barrier 0 (step 0 has landed), then barrier j + 1 for every step j that has a successor.
    Copy waves: steps 0 and 1 are copied before barrier 0, step j + 2 after barrier j; a tile's
    first copy reads its ring entry; the claim for tile q + 1 is issued with the copy of tile q's
    step 1 (step 3 for cancel-and-reuse's tile 0 when nk >= 4) and written to the ring before the
    next barrier. MFMA waves: at the last step of tile q they read entry q + 1 to learn whether a
    step follows; the epilogue reads entry q. Returns the trace and the barrier counts of the two
    roles."""
    t = Trace()
    S = ntiles * nk
    defer = mode == "cancel" and nk >= 4

    def cstep(q):
        return 3 if (defer and q == 0) else 1

    # ---- copy waves
    t.write(0)          # both claiming modes keep their first tile in the ring
    t.barrier()         # claims barrier
    if mode == "cancel":
        t.read(0, "exit check")
    pending = []
    issued = [0]

    def issue(u):
        if u >= S:
            return False
        q, kt = divmod(u, nk)
        if kt == 0:
            t.read(q, "copy waves")
        if kt == cstep(q):
            pending.append(q + 1)   # the claim of tile q + 1 (tile ntiles: the failing one)
        issued[0] += 1
        return True

    def publish():
        while pending:
            t.write(pending.pop())

    issue(0)
    issue(1)
    publish()
    t.barrier()         # barrier 0
    j = 0
    while True:
        issue(j + 2)
        if j + 1 >= issued[0]:
            break
        publish()
        t.barrier()     # barrier j + 1
        j += 1
    copy_barriers = t.barriers
    # ---- MFMA waves (the same barriers, counted from the claims barrier)
    b = 1
    if mode == "cancel":
        t.reads.append((0, b, "exit check (MFMA waves)"))
    b += 1              # barrier 0
    for s in range(S):
        q, kt = divmod(s, nk)
        nxt = True
        if kt == nk - 1:
            t.reads.append((q + 1, b, "MFMA waves: next"))
            nxt = q + 1 < ntiles
        if nxt:
            b += 1
        if kt == nk - 1:
            t.reads.append((q, b, "MFMA waves: epilogue"))
    return t, copy_barriers, b


NKS = [2, 4, 6, 8, 16, 64]
BODIES = {"lockstep16": lockstep16, "lockstep8": lockstep8, "pingpong": pingpong}


@pytest.mark.parametrize("body", sorted(BODIES))
@pytest.mark.parametrize("mode", ["dynamic", "cancel"])
def test_shipped_protocols_publish_every_entry_before_it_is_read(body, mode):
    """Every tile-id read of the shipped kernels falls in a later barrier interval than the ring
    write it needs, for every k-loop length and tile count (the dynamic mode's tile 0 is the
    workgroup's own id, not a ring entry, in the lockstep bodies)."""
    for nk, ntiles in itertools.product(NKS, [1, 2, 3, 5, 9]):
        t = BODIES[body](mode, nk, ntiles)
        ring_from = 1 if (mode == "dynamic" and body != "pingpong") else 0
        assert t.races(ring_from) == [], (body, mode, nk, ntiles, t.races(ring_from))
        # every entry a reader needs is written (tiles 1..ntiles, the last one being the failed claim)
        needed = {q for q, _, _ in t.reads if q >= ring_from}
        assert needed <= set(t.writes), (body, mode, nk, ntiles)


def test_cancel_deferral_needs_four_steps_in_the_16bit_lockstep_body():
    """The shipped deferral of tile 1 (issued after step 0's barrier, published before step 1's)
    is safe at 4 k-steps; at 2 the producer reads tile 1's entry after step 0's barrier, before
    the publication -- which is why the kernels defer only when nk >= 4."""
    assert lockstep16("cancel", 4, 3).races() == []
    races = lockstep16("cancel", 2, 3, defer_publish=1).races()
    assert races and races[0][0] == 1 and races[0][3] == "producer"


@pytest.mark.parametrize("body", ["lockstep16", "lockstep8"])
def test_dropped_variant_races_exactly_at_short_k_loops(body):
    """The dropped variant published the dynamic mode's first claimed tile later than the
    prologue. Publication points are characterized by the smallest k-loop at which the first
    read of the entry follows them. Written after the barrier of step 2 -- one step after the
    shipped deferral's publication step, and after its barrier -- it races at 4 k-steps (the
    producer begins tile 1 in that same interval: M = N = K = 256 at 64-deep fp16 steps) and is
    safe from 6 on, which is the only failure the variant showed on the GPU. A stale entry
    there holds whatever the slot last held; before the unsigned range checks a negative one
    passed the producer's test and addressed memory outside the tile grid."""
    fn = BODIES[body]
    first_safe = {}
    for pub in range(0, 6):
        for after in (False, True):
            safe = [nk for nk in NKS if not fn("dynamic", nk, 3, defer_publish=pub, publish_after_barrier=after).races(1)]
            first_safe[(pub, after)] = min(safe) if safe else None
    if body == "lockstep16":
        assert first_safe[(1, False)] == 4       # the shipped deferral's publication point
        assert first_safe[(2, True)] == 6        # the dropped variant: races at nk = 4
        assert fn("dynamic", 4, 1, defer_publish=2, publish_after_barrier=True).races(1)
    else:
        assert first_safe[(1, False)] == 2
        assert first_safe[(2, True)] == 4
    # later publication never makes a shorter loop safe
    for after in (False, True):
        vals = [first_safe[(p, after)] for p in range(6)]
        vals = [v if v is not None else 10**9 for v in vals]
        assert vals == sorted(vals)


@pytest.mark.parametrize("mode", ["dynamic", "cancel"])
def test_producer_body_roles_pass_the_same_barriers_and_publish_before_reading(mode):
    """The copy waves and the MFMA waves of the producer-wave body must meet at exactly the same
    barriers (a mismatch would leave one role waiting forever), and every ring entry must be
    published before any wave reads it: for every even k-loop length and tile count."""
    for nk, ntiles in itertools.product([2, 4, 6, 8, 10, 16, 64], [1, 2, 3, 5, 9]):
        t, copy_b, mfma_b = producer(mode, nk, ntiles)
        assert copy_b == mfma_b == 1 + ntiles * nk, (mode, nk, ntiles, copy_b, mfma_b)
        assert t.races() == [], (mode, nk, ntiles, t.races())
        needed = {q for q, _, _ in t.reads}
        assert needed <= set(t.writes), (mode, nk, ntiles, needed - set(t.writes))
        # one claim per tile, the last of them the failing one (entry ntiles)
        assert sorted(t.writes) == list(range(ntiles + 1)), (mode, nk, ntiles)
