"""Stage-count, LDS-footprint and occupancy model, and a ring-schedule simulator.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Sources:
  * "Lesson 6: Shared Memory layout and async pipeline" (learn.payai.win,
    CUTLASS course), section 4 (performance trade-offs): the number of loads
    that must be in flight is the ceiling of T_copy / T_compute, plus one stage
    being computed on; the staging buffer grows linearly in the stage count,
    S * (tile_A + tile_B) * sizeof(T); the resident-block count is the buffer
    capacity divided by the per-block footprint, rounded down.  The exercise
    at the end of that page fixes three values of the stage formula and says
    both arguments must be positive integers.
  * "cute(9) multistage_gemm", sections 4-6 and 8: the ring state (next global
    K tile to load, slot being read, slot being written), the prologue that
    fills S-1 slots, the steady state that waits until at most S-2 batches are
    in flight, synchronises, prefetches and computes, and the worked trace for
    K=256, BK=32, S=3.
  * The same lesson, sections 2 and 3: the three-phase order (wait, barrier,
    issue load k+S-1 into the free slot, compute slot k; then drain) and the
    read-after-write / write-after-read hazards that it must avoid.
"""
from __future__ import annotations

from dataclasses import dataclass, field


# --------------------------------------------------------------------------
# Stage-count and footprint model

def minimum_stages(copy_cycles: int, compute_cycles: int) -> int:
    """Smallest stage count that hides a copy latency behind compute.

    In-flight loads >= ceil(copy / compute), plus the one stage being computed
    on.  Both arguments must be positive integers (anything else raises).
    Written with integer arithmetic only: ceil(c / t) = -((-c) // t)."""
    for v in (copy_cycles, compute_cycles):
        if isinstance(v, bool) or not isinstance(v, int) or v <= 0:
            raise ValueError("copy and compute cycle counts must be positive integers")
    in_flight = -((-copy_cycles) // compute_cycles)
    return in_flight + 1


def lds_bytes(tile_m: int, tile_n: int, tile_k: int, stages: int,
              elem_bytes: int = 2) -> int:
    """Staging-buffer footprint S * (tile_m*tile_k + tile_k*tile_n) * sizeof(T)."""
    if min(tile_m, tile_n, tile_k, stages, elem_bytes) <= 0:
        raise ValueError("all sizes must be positive")
    return stages * (tile_m * tile_k + tile_k * tile_n) * elem_bytes


def blocks_per_unit(footprint_bytes: int, capacity_bytes: int,
                    other_limit: int | None = None) -> int:
    """Resident blocks per compute unit: floor(capacity / footprint), further
    capped by any other per-unit limit (waves, registers, hardware slots)."""
    if footprint_bytes <= 0 or capacity_bytes <= 0:
        raise ValueError("footprint and capacity must be positive")
    n = capacity_bytes // footprint_bytes
    if other_limit is not None:
        n = min(n, other_limit)
    return n


# --------------------------------------------------------------------------
# Ring-schedule simulator
#
# A schedule is a list of operations executed identically by every thread of
# the block.  The simulator replays it against a worst-case memory system in
# which an outstanding load completes only when a wait forces it, and checks
# the invariants the pages state:
#   RAW   a slot is read only after the load that filled it was retired by a
#         wait that precedes a block-wide barrier that precedes the read;
#   WAR   a slot is refilled only after a barrier that follows every read of
#         its previous occupant;
#   every K tile is loaded exactly once and computed on in order, fragment by
#   fragment, from the slot it was loaded into;
#   never more than S-1 tiles are loaded but not yet retired.

@dataclass
class Op:
    kind: str            # "issue", "fence", "wait", "sync", "read", "compute"
    tile: int = -1
    slot: int = -1
    frag: int = -1
    n: int = -1          # wait: how many units may remain outstanding


@dataclass
class SimResult:
    ok: bool
    errors: list = field(default_factory=list)
    issued: list = field(default_factory=list)      # (tile, slot) in issue order
    reads: list = field(default_factory=list)       # (slot, tile, frag)
    computed: list = field(default_factory=list)    # (tile, frag)
    max_in_flight: int = 0


def simulate(ops: list[Op], ntile: int, stages: int, nfrag: int,
             units: str = "groups") -> SimResult:
    """Replay `ops`.  `units` says what a wait counts: "groups" (a fence
    closes a batch; waits count batches, empty batches included) or "loads"
    (every issue is one counted unit, no fences)."""
    res = SimResult(ok=True)
    slot_tile = [None] * stages         # tile currently held by each slot
    slot_ready = [False] * stages       # retired by a wait and published by a barrier
    slot_retired = [False] * stages     # retired by a wait, not yet published
    slot_last_read_epoch = [-1] * stages
    epoch = 0                           # barrier count
    outstanding = []                    # list of units; each unit = list of (tile, slot)
    open_group = []
    loaded = set()
    frag_regs = {}                      # frag -> (tile, slot) of the last read of that fragment

    def err(msg):
        res.ok = False
        res.errors.append(msg)

    def in_flight_tiles():
        tiles = {t for u in outstanding for (t, _) in u}
        tiles |= {t for (t, _) in open_group}
        return len(tiles)

    for op in ops:
        if op.kind == "issue":
            t, s = op.tile, op.slot
            if not (0 <= t < ntile):
                err(f"issue of tile {t} outside 0..{ntile - 1}")
            if t in loaded:
                err(f"tile {t} loaded twice")
            loaded.add(t)
            if slot_tile[s] is not None and slot_last_read_epoch[s] >= epoch:
                err(f"WAR: slot {s} refilled with tile {t} before a barrier after its last read")
            slot_tile[s] = t
            slot_ready[s] = False
            slot_retired[s] = False
            res.issued.append((t, s))
            if units == "groups":
                open_group.append((t, s))
            else:
                outstanding.append([(t, s)])
            res.max_in_flight = max(res.max_in_flight, in_flight_tiles())
        elif op.kind == "fence":
            outstanding.append(open_group)
            open_group = []
        elif op.kind == "wait":
            keep = max(op.n, 0)
            while len(outstanding) > keep:
                unit = outstanding.pop(0)
                for (t, s) in unit:
                    if slot_tile[s] == t:
                        slot_retired[s] = True
        elif op.kind == "sync":
            epoch += 1
            for s in range(stages):
                if slot_retired[s]:
                    slot_ready[s] = True
        elif op.kind == "read":
            s = op.slot
            t = slot_tile[s]
            res.reads.append((s, t, op.frag))
            frag_regs[op.frag] = (t, s, slot_ready[s])
            slot_last_read_epoch[s] = epoch
        elif op.kind == "compute":
            got = frag_regs.get(op.frag)
            if got is None:
                err(f"compute of tile {op.tile} fragment {op.frag} with no fragment read")
                continue
            t, s, ready = got
            if t != op.tile:
                err(f"compute of tile {op.tile} fragment {op.frag} used tile {t} from slot {s}")
            elif not ready:
                err(f"RAW: tile {t} read from slot {s} before it was retired and published")
            res.computed.append((op.tile, op.frag))
        else:
            raise ValueError(op.kind)

    expect = [(t, f) for t in range(ntile) for f in range(nfrag)]
    if res.computed != expect:
        err("tiles/fragments were not computed exactly once, in order")
    if sorted(loaded) != list(range(ntile)):
        err("not every tile was loaded")
    if res.max_in_flight > stages - 1:
        err(f"{res.max_in_flight} tiles in flight with {stages} stages")
    return res


def schedule_cute_multistage(ntile: int, stages: int, nfrag: int) -> list[Op]:
    """Ring schedule of the multistage kernel of "cute(9) multistage_gemm",
    sections 5, 6 and 8, rebuilt from the rules those sections state:

      * tile j always lives in slot j mod S;
      * each global load forms one commit group, closed by a fence; a group
        is committed even when no tile is left to load, so wait counts stay
        in step (section 8);
      * the prologue commits the groups of tiles 0 .. S-2 (section 5: S-1,
        not S, so the first refill has a free slot);
      * a tile becomes readable after a wait that leaves at most S-2 groups
        pending and a block-wide barrier; the same barrier ends every read of
        the slot that the next refill overwrites;
      * fragments are double-buffered in registers: while fragment f of tile
        t is multiplied, fragment f+1 is fetched -- at the last fragment that
        is fragment 0 of tile t+1, so the wait and barrier for tile t+1 come
        first (section 9: the read slot advances there);
      * the refill of tile t+S-1 is issued at the first fragment of tile t.

    The prologue only loads tiles that exist (the page assumes ntile >= S-1).
    With one fragment per tile the fetch would overwrite the fragment about to
    be used, so nfrag >= 2 is required (the page has two)."""
    if nfrag < 2:
        raise ValueError("the walked-through schedule needs at least two fragments per tile")
    ops: list[Op] = []

    def commit(tile: int) -> None:
        if tile < ntile:
            ops.append(Op("issue", tile=tile, slot=tile % stages))
        ops.append(Op("fence"))

    def publish() -> None:
        ops.append(Op("wait", n=stages - 2))
        ops.append(Op("sync"))

    for tile in range(stages - 1):
        commit(tile)
    publish()
    # Fragment registers are named by the fragment index; which tile's data a
    # fragment holds is what the compute check verifies.
    ops.append(Op("read", slot=0, frag=0))
    for t in range(ntile):
        for f in range(nfrag):
            last = f == nfrag - 1
            if last:
                publish()
            source = t + 1 if last else t      # at the very end: a read nobody uses
            ops.append(Op("read", slot=source % stages, frag=(f + 1) % nfrag))
            if f == 0:
                commit(t + stages - 1)
            ops.append(Op("compute", tile=t, frag=f))
    return ops


def schedule_three_phase(ntile: int, stages: int, nfrag: int,
                         wait_counts: list[int] | None = None,
                         loads_per_tile: int = 1) -> list[Op]:
    """The three-phase order of the CUTLASS lesson, section 2, counted in
    individual loads (no fences): prologue issues tiles 0..S-2; then for each
    tile k: wait, barrier, issue tile k+S-1 into slot (k+S-1) mod S if it
    exists, read and compute every fragment of slot k mod S.  `wait_counts[k]`
    is the number of loads allowed to remain outstanding at tile k; by default
    the loosest safe value is derived here."""
    ops: list[Op] = []
    for t in range(min(stages - 1, ntile)):
        for _ in range(loads_per_tile):
            ops.append(Op("issue_part", tile=t, slot=t % stages))
    for k in range(ntile):
        if wait_counts is None:
            # loads issued after tile k's loads, so far: tiles k+1 .. min(k+S-2, ntile-1)
            n = loads_per_tile * max(0, min(k + stages - 2, ntile - 1) - k)
        else:
            n = wait_counts[k]
        ops.append(Op("wait", n=n))
        ops.append(Op("sync"))
        nxt = k + stages - 1
        if nxt < ntile:
            for _ in range(loads_per_tile):
                ops.append(Op("issue_part", tile=nxt, slot=nxt % stages))
        for f in range(nfrag):
            ops.append(Op("read", slot=k % stages, frag=f))
            ops.append(Op("compute", tile=k, frag=f))
    return ops


def simulate_loads(ops: list[Op], ntile: int, stages: int, nfrag: int,
                   loads_per_tile: int) -> SimResult:
    """Replay a schedule whose issues are split into `loads_per_tile` counted
    loads per tile ("issue_part" ops); a tile is retired once all its parts
    are.  Waits count loads."""
    res = SimResult(ok=True)
    slot_tile = [None] * stages
    slot_parts_done = [0] * stages
    slot_published = [False] * stages
    slot_last_read_epoch = [-1] * stages
    epoch = 0
    outstanding = []            # (tile, slot) per load, in issue order
    issued_parts = {}
    frag_regs = {}

    def err(msg):
        res.ok = False
        res.errors.append(msg)

    for op in ops:
        if op.kind == "issue_part":
            t, s = op.tile, op.slot
            if not (0 <= t < ntile):
                err(f"issue of tile {t} outside 0..{ntile - 1}")
            parts = issued_parts.get(t, 0)
            if parts == 0:
                if slot_tile[s] is not None and slot_last_read_epoch[s] >= epoch:
                    err(f"WAR: slot {s} refilled with tile {t} before a barrier after its last read")
                slot_tile[s] = t
                slot_parts_done[s] = 0
                slot_published[s] = False
                res.issued.append((t, s))
            elif parts >= loads_per_tile:
                err(f"tile {t} loaded twice")
            issued_parts[t] = parts + 1
            outstanding.append((t, s))
            in_flight = len({tt for (tt, _) in outstanding if tt is not None})
            res.max_in_flight = max(res.max_in_flight, in_flight)
        elif op.kind in ("store", "dummy"):
            # a global store, or a load aimed out of range into scratch LDS:
            # counted by the same in-order counter, touches no ring slot
            outstanding.append((None, None))
        elif op.kind == "wait":
            keep = max(op.n, 0)
            while len(outstanding) > keep:
                t, s = outstanding.pop(0)
                if t is not None and slot_tile[s] == t:
                    slot_parts_done[s] += 1
        elif op.kind == "sync":
            epoch += 1
            for s in range(stages):
                if slot_tile[s] is not None and slot_parts_done[s] == loads_per_tile:
                    slot_published[s] = True
        elif op.kind == "read":
            s = op.slot
            frag_regs[op.frag] = (slot_tile[s], s, slot_published[s])
            res.reads.append((s, slot_tile[s], op.frag))
            slot_last_read_epoch[s] = epoch
        elif op.kind == "compute":
            t, s, ready = frag_regs[op.frag]
            if t != op.tile:
                err(f"compute of tile {op.tile} used tile {t} from slot {s}")
            elif not ready:
                err(f"RAW: tile {t} read from slot {s} before all its loads were retired and published")
            res.computed.append((op.tile, op.frag))
        else:
            raise ValueError(op.kind)
    expect = [(t, f) for t in range(ntile) for f in range(nfrag)]
    if res.computed != expect:
        err("tiles/fragments were not computed exactly once, in order")
    if sorted(issued_parts) != list(range(ntile)) or any(
            v != loads_per_tile for v in issued_parts.values()):
        err("not every tile was loaded completely")
    if res.max_in_flight > stages - 1:
        err(f"{res.max_in_flight} tiles in flight with {stages} stages")
    return res


def loosest_wait_counts(ntile: int, stages: int, loads_per_tile: int) -> list[int]:
    """For the three-phase order: the largest number of loads that may remain
    outstanding when tile k is about to be consumed, found by search against
    the simulator (largest n whose schedule still passes, tile by tile)."""
    counts: list[int] = []
    for k in range(ntile):
        best = 0
        for n in range(0, loads_per_tile * stages + 1):
            trial = counts + [n] + [0] * (ntile - k - 1)
            ops = schedule_three_phase(ntile, stages, 1, trial, loads_per_tile)
            r = simulate_loads(ops, ntile, stages, 1, loads_per_tile)
            # only the RAW check of tile k matters for this n
            raw_k = [e for e in r.errors if e.startswith(f"RAW: tile {k} ")]
            if not raw_k:
                best = n
            else:
                break
        counts.append(best)
    return counts


def schedule_cute_loads(ntile: int, stages: int, nfrag: int, loads_per_tile: int,
                        wait_counts: list[int] | None = None) -> list[Op]:
    """The order of "cute(9) multistage_gemm" sections 5-6 with each tile's
    copy split into `loads_per_tile` counted loads and no fences (waits count
    loads).  Prologue: tiles 0..S-2, wait for tile 0, barrier, read fragment 0
    of tile 0.  Then for tile k and fragment ik: at the last fragment (and
    only if tile k+1 exists) wait for tile k+1, barrier, read fragment 0 of
    tile k+1; otherwise read fragment ik+1 of tile k; at the first fragment
    issue tile k+S-1 if it exists; compute fragment ik of tile k.
    `wait_counts[t]` is the wait used before tile t is first read (default:
    the loads issued after tile t's, i.e. the loosest safe value)."""
    if nfrag < 2:
        raise ValueError("the walked-through schedule needs at least two fragments per tile")
    ops: list[Op] = []
    issued = []

    def issue(t):
        for _ in range(loads_per_tile):
            ops.append(Op("issue_part", tile=t, slot=t % stages))
        issued.append(t)

    def wait_for(t):
        if wait_counts is None:
            n = loads_per_tile * (max(issued) - t)
        else:
            n = wait_counts[t]
        ops.append(Op("wait", n=n))
        ops.append(Op("sync"))

    for t in range(min(stages - 1, ntile)):
        issue(t)
    if ntile == 0:
        return ops
    wait_for(0)
    ops.append(Op("read", slot=0, frag=0))
    for k in range(ntile):
        for ik in range(nfrag):
            if ik == nfrag - 1:
                if k + 1 < ntile:
                    wait_for(k + 1)
                    ops.append(Op("read", slot=(k + 1) % stages, frag=0))
            else:
                ops.append(Op("read", slot=k % stages, frag=ik + 1))
            if ik == 0 and k + stages - 1 < ntile:
                issue(k + stages - 1)
            ops.append(Op("compute", tile=k, frag=ik))
    return ops


def schedule_persistent_loads(ntile: int, ntiles_out: int, stages: int, nfrag: int,
                              loads_per_tile: int, stores_per_tile: int,
                              wait_counts: list[int]) -> list[Op]:
    """One workgroup that computes `ntiles_out` output tiles of `ntile` K
    tiles each as ONE stream of K tiles through the ring (stream tile
    g = u * ntile + k lives in slot g mod S).  The order of
    schedule_cute_loads over the whole stream ("cute(9) multistage_gemm"
    section 9: the wait for the next tile and its first fragment read sit at
    the last fragment of the current one; "Lesson 6": S - 1 tiles in flight),
    with two changes.  At each output-tile boundary, after the last compute
    of the output tile's last K tile g, the group of tile g + S is issued at
    once (if it exists), then the epilogue's `stores_per_tile` counted global
    stores.  And every K tile but the stream's last issues `loads_per_tile`
    counted operations at its first fragment: its group g + S - 1 if that
    exists and was not issued early, otherwise the same number of loads aimed
    out of range (they fill no slot).  Loads and stores share one in-order
    counter.  `wait_counts[g]` is the count used before stream tile g is
    first read."""
    if nfrag < 2:
        raise ValueError("the walked-through schedule needs at least two fragments per tile")
    total = ntile * ntiles_out
    ops: list[Op] = []
    issued: set[int] = set()

    def issue(t):
        for _ in range(loads_per_tile):
            ops.append(Op("issue_part", tile=t, slot=t % stages))
        issued.add(t)

    def wait_for(t):
        ops.append(Op("wait", n=wait_counts[t]))
        ops.append(Op("sync"))

    for t in range(min(stages - 1, total)):
        issue(t)
    if total == 0:
        return ops
    wait_for(0)
    ops.append(Op("read", slot=0, frag=0))
    for g in range(total):
        for f in range(nfrag):
            if f == nfrag - 1:
                if g + 1 < total:
                    wait_for(g + 1)
                    ops.append(Op("read", slot=(g + 1) % stages, frag=0))
            else:
                ops.append(Op("read", slot=g % stages, frag=f + 1))
            if f == 0 and g + 1 < total:
                nxt = g + stages - 1
                if nxt < total and nxt not in issued:
                    issue(nxt)
                else:
                    ops.extend(Op("dummy") for _ in range(loads_per_tile))
            ops.append(Op("compute", tile=g, frag=f))
        if (g + 1) % ntile == 0:
            if g + stages < total and g + stages not in issued:
                issue(g + stages)
            ops.extend(Op("store") for _ in range(stores_per_tile))
    return ops


def loosest_persistent_wait_counts(ntile: int, ntiles_out: int, stages: int,
                                   loads_per_tile: int, stores_per_tile: int,
                                   nfrag: int = 2) -> list[int]:
    """The largest count of outstanding counted operations (loads and
    stores) that still lets K tile g of the persistent stream be read safely,
    found tile by tile by search against the simulator."""
    total = ntile * ntiles_out
    counts: list[int] = []
    for g in range(total):
        best = 0
        for n in range(0, (loads_per_tile + stores_per_tile) * (stages + 1) + 1):
            trial = counts + [n] + [0] * (total - g - 1)
            ops = schedule_persistent_loads(ntile, ntiles_out, stages, nfrag, loads_per_tile,
                                            stores_per_tile, trial)
            r = simulate_loads(ops, total, stages, nfrag, loads_per_tile)
            if any(e.startswith(f"RAW: tile {g} ") for e in r.errors):
                break
            best = n
        counts.append(best)
    return counts


# --------------------------------------------------------------------------
# Two wave groups, one ring per operand
#
# The same RAW and WAR rules ("Lesson 6", sections 2-3), for a workgroup
# whose waves form groups that run different programs between common
# barriers, with the A and B tiles in rings of their own.  Each group is
# represented by one of its waves (every wave of a group runs the same
# program, and the load counter is per wave).  The simulator cuts every
# program at its barriers; the pieces with the same barrier count form one
# epoch, and ops of different groups within an epoch have no order.  So:
#   WAR   an issue into a slot conflicts with any read of that slot in the
#         same epoch, by any group (reads complete before the reader's next
#         barrier, so reads of earlier epochs are safe);
#   RAW   a read needs every counted load of that tile, from every group,
#         retired by a wait in an earlier epoch;
#   each group computes tiles 0..ntile-1 in order, from fragments of that
#   tile that it read; nothing is in flight at the end; every group passes
#   the same number of barriers.

@dataclass
class GroupOp:
    kind: str            # "issue", "wait", "sync", "read", "compute"
    operand: str = ""    # "A" or "B"
    tile: int = -1
    slot: int = -1
    n: int = 0           # issue: counted loads; wait: loads that may stay outstanding


def simulate_groups(programs: dict, ntile: int, slots: dict, parts) -> SimResult:
    """Replay the per-group programs `programs` ({name: [GroupOp]}).
    `slots[operand]` is the ring depth of that operand and `parts(operand,
    tile)` the number of counted loads (summed over the represented waves)
    that make the tile complete."""
    res = SimResult(ok=True)

    def err(msg):
        res.ok = False
        res.errors.append(msg)

    segs = {}
    for g, prog in programs.items():
        cur, lst = [], []
        for op in prog:
            if op.kind == "sync":
                lst.append(cur)
                cur = []
            else:
                cur.append(op)
        lst.append(cur)
        segs[g] = lst
    nseg = {len(v) for v in segs.values()}
    if len(nseg) != 1:
        err(f"groups pass different numbers of barriers: "
            f"{ {g: len(v) - 1 for g, v in segs.items()} }")
        return res
    nepoch = nseg.pop()

    ring = {o: [None] * slots[o] for o in slots}
    issued = {}                         # (operand, tile) -> counted loads issued
    retired = {}                        # (operand, tile) -> counted loads retired
    retire_epoch = {}                   # (operand, tile) -> epoch of the last retirement
    home = {}                           # (operand, tile) -> slot
    outstanding = {g: [] for g in programs}
    frags = {g: {} for g in programs}
    computed = {g: [] for g in programs}
    read_once = set()

    for e in range(nepoch):
        reads_now = []                  # (operand, slot, group)
        issues_now = []                 # (operand, slot, tile, group)
        for g in programs:
            for op in segs[g][e]:
                if op.kind == "issue":
                    key = (op.operand, op.tile)
                    if not (0 <= op.tile < ntile):
                        err(f"{g}: issue of {op.operand} tile {op.tile} outside 0..{ntile - 1}")
                        continue
                    if key in read_once or (key in home and home[key] != op.slot):
                        err(f"{g}: {op.operand} tile {op.tile} loaded twice")
                    if key not in home:
                        home[key] = op.slot
                        ring[op.operand][op.slot] = op.tile
                    issued[key] = issued.get(key, 0) + op.n
                    outstanding[g].extend([key] * op.n)
                    issues_now.append((op.operand, op.slot, op.tile, g))
                    res.issued.append((op.operand, op.tile, op.slot))
                elif op.kind == "wait":
                    while len(outstanding[g]) > max(op.n, 0):
                        key = outstanding[g].pop(0)
                        retired[key] = retired.get(key, 0) + 1
                        retire_epoch[key] = e
                elif op.kind == "read":
                    key = (op.operand, op.tile)
                    held = ring[op.operand][op.slot]
                    reads_now.append((op.operand, op.slot, g))
                    read_once.add(key)
                    res.reads.append((op.operand, op.slot, held, g))
                    if held != op.tile:
                        err(f"{g}: read of {op.operand} tile {op.tile} from slot {op.slot}, "
                            f"which holds tile {held}")
                    elif (issued.get(key, 0) != parts(op.operand, op.tile)
                          or retired.get(key, 0) != parts(op.operand, op.tile)
                          or retire_epoch.get(key, e) >= e):
                        err(f"RAW: {g} read {op.operand} tile {op.tile} from slot {op.slot} "
                            f"before all its loads were retired and published")
                    frags[g][op.operand] = held
                elif op.kind == "compute":
                    f = frags[g]
                    if f.get("A") != op.tile or f.get("B") != op.tile:
                        err(f"{g}: compute of tile {op.tile} with fragments of A tile "
                            f"{f.get('A')} and B tile {f.get('B')}")
                    computed[g].append(op.tile)
                else:
                    raise ValueError(op.kind)
        for (o, s, t, g) in issues_now:
            clash = sorted({rg for (ro, rs, rg) in reads_now if ro == o and rs == s})
            if clash:
                err(f"WAR: {g} refilled {o} slot {s} with tile {t} in the epoch in which "
                    f"{', '.join(clash)} read it")
        res.max_in_flight = max(res.max_in_flight,
                                max((len(set(v)) for v in outstanding.values()), default=0))
    for g in programs:
        if computed[g] != list(range(ntile)):
            err(f"{g}: computed tiles {computed[g]}, not 0..{ntile - 1} in order")
        if outstanding[g]:
            err(f"{g}: {len(outstanding[g])} loads still in flight at the end")
    for o in slots:
        for t in range(ntile):
            if issued.get((o, t), 0) != parts(o, t):
                err(f"{o} tile {t}: {issued.get((o, t), 0)} loads issued, {parts(o, t)} expected")
    return res


def schedule_pingpong(ntile: int, loads: int):
    """Ping-pong of two wave groups over one ring of two slots that holds A
    and B tile j in slot j mod 2.  Phase 2j: G0 issues all loads of tile j+1
    (`loads` per operand per wave), then reads tile j; G1 computes tile j-1.
    Phase 2j+1: G0 computes tile j and retires its loads; G1 reads tile j.
    Tile 0 is loaded by both groups (half of each operand each) before the
    first barrier.  Returns (programs, slots, parts)."""
    h = loads // 2
    g0, g1 = [], []
    if ntile > 0:
        for prog in (g0, g1):
            prog += [GroupOp("issue", "A", 0, 0, h), GroupOp("issue", "B", 0, 0, h)]
    for prog in (g0, g1):
        prog += [GroupOp("wait", n=0), GroupOp("sync")]
    g1.append(GroupOp("sync"))
    for j in range(ntile):
        if j + 1 < ntile:
            g0 += [GroupOp("issue", "A", j + 1, (j + 1) % 2, loads),
                   GroupOp("issue", "B", j + 1, (j + 1) % 2, loads)]
        for prog in (g0, g1):
            prog += [GroupOp("read", "A", j, j % 2), GroupOp("read", "B", j, j % 2)]
        g0 += [GroupOp("sync"), GroupOp("compute", tile=j), GroupOp("wait", n=0), GroupOp("sync")]
        g1 += [GroupOp("sync"), GroupOp("compute", tile=j), GroupOp("sync")]
    g0.append(GroupOp("sync"))
    return {"G0": g0, "G1": g1}, {"A": 2, "B": 2}, (lambda o, t: 2 * h if t == 0 else loads)


def schedule_split_pingpong(ntile: int, loads: int, a_slots: int = 2, b_slots: int = 3,
                            a_ahead: int = 1, b_ahead: int = 2, g0_keep: int = 0,
                            g1_keep: int | None = None):
    """The ping-pong with the loads split between the groups: G0 loads A
    tiles only, G1 B tiles only, `loads` per wave per tile, each in its
    fragment-read phase (the order of issues and reads within a phase does
    not matter here: no slot is read and refilled in the same phase).  A tile j lives in slot j mod a_slots, B tile j in slot
    j mod b_slots.  Phase 2j: G0 reads tile j, issues A(j + a_ahead); G1
    computes tile j-1.  Phase 2j+1: G0 computes tile j and waits until at
    most g0_keep loads remain; G1 reads tile j, issues B(j + b_ahead) and
    waits until at most g1_keep remain (default: the loads just issued).
    Before the first barrier G0 loads A tiles 0..a_ahead-1 and G1 B tiles
    0..b_ahead-1.  The defaults are the kernel's protocol; the parameters
    exist to plant mistakes.  Returns (programs, slots, parts)."""
    g0, g1 = [], []
    for t in range(min(a_ahead, ntile)):
        g0.append(GroupOp("issue", "A", t, t % a_slots, loads))
    for t in range(min(b_ahead, ntile)):
        g1.append(GroupOp("issue", "B", t, t % b_slots, loads))
    for prog in (g0, g1):
        prog += [GroupOp("wait", n=0), GroupOp("sync")]
    g1.append(GroupOp("sync"))
    for j in range(ntile):
        for prog in (g0, g1):
            prog += [GroupOp("read", "A", j, j % a_slots), GroupOp("read", "B", j, j % b_slots)]
        ta, tb = j + a_ahead, j + b_ahead
        if ta < ntile:
            g0.append(GroupOp("issue", "A", ta, ta % a_slots, loads))
        g0 += [GroupOp("sync"), GroupOp("compute", tile=j), GroupOp("wait", n=g0_keep),
               GroupOp("sync")]
        if tb < ntile:
            g1.append(GroupOp("issue", "B", tb, tb % b_slots, loads))
            g1.append(GroupOp("wait", n=loads if g1_keep is None else g1_keep))
        else:
            g1.append(GroupOp("wait", n=0))
        g1 += [GroupOp("sync"), GroupOp("compute", tile=j), GroupOp("sync")]
    g0.append(GroupOp("sync"))
    return {"G0": g0, "G1": g1}, {"A": a_slots, "B": b_slots}, (lambda o, t: loads)
