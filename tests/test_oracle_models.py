"""Pins of the stage-count / footprint / occupancy model and of the ring-schedule
simulator against the worked values the pages print, plus exhaustive invariant
sweeps and planted schedule mistakes that the simulator must catch."""
import json
import os

import pytest

import oracle
from oracle.models import (Op, schedule_cute_loads, schedule_cute_multistage, schedule_pingpong,
                           schedule_split_pingpong, schedule_three_phase, simulate,
                           simulate_groups, simulate_loads)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_minimum_stages_worked_values():
    for c in _golden("minimum_stages.json")["cases"]:
        assert oracle.minimum_stages(c["copy_cycles"], c["compute_cycles"]) == c["stages"]


@pytest.mark.parametrize("copy,compute,expect", [
    (119, 120, 2),      # copy shorter than compute: one load in flight
    (240, 120, 3),      # exact multiple: no extra stage
    (241, 120, 4),      # just above a multiple
    (1, 1, 2),
    (10**9, 1, 10**9 + 1),
])
def test_minimum_stages_boundaries(copy, compute, expect):
    assert oracle.minimum_stages(copy, compute) == expect


@pytest.mark.parametrize("bad", [(0, 120), (300, 0), (-1, 5), (2.5, 1), (True, 3)])
def test_minimum_stages_rejects_non_positive_or_non_integer(bad):
    with pytest.raises(ValueError):
        oracle.minimum_stages(*bad)


def test_lds_footprint_worked_value():
    f = _golden("lds_occupancy.json")["footprint"]
    assert oracle.lds_bytes(f["tile_m"], f["tile_n"], f["tile_k"], f["stages"],
                            f["elem_bytes"]) == f["bytes"]


def test_blocks_per_unit_worked_values():
    for c in _golden("lds_occupancy.json")["blocks_per_unit"]["cases"]:
        assert oracle.blocks_per_unit(c["footprint_kib"] * 1024, c["capacity_kib"] * 1024) == c["blocks"]


def test_footprint_linear_in_stages():
    # 2 -> 5 stages of a 20 KiB stage is 40 -> 100 KiB (the lesson's example)
    per = 20 * 1024
    assert [s * per for s in (2, 5)] == [40 * 1024, 100 * 1024]
    for s in range(1, 8):
        assert oracle.lds_bytes(256, 256, 32, s) == s * oracle.lds_bytes(256, 256, 32, 1)


def test_cute_trace_golden():
    g = _golden("cute_trace_k256_s3.json")
    ops = schedule_cute_multistage(g["ntile"], g["stages"], g["nfrag"])
    r = simulate(ops, g["ntile"], g["stages"], g["nfrag"])
    assert r.ok, r.errors
    assert [list(x) for x in r.issued] == g["issued_tile_slot"]
    # slot from which each tile's fragments were consumed
    used = {}
    for (slot, tile, frag) in r.reads:
        if tile is not None and tile < g["ntile"]:
            used.setdefault(tile, slot)
    assert [used[t] for t in range(g["ntile"])] == g["read_slot_per_tile"]
    assert r.max_in_flight == g["max_in_flight"]


@pytest.mark.parametrize("stages", [2, 3, 4, 5, 6])
def test_cute_schedule_invariants_exhaustive(stages):
    for ntile in range(1, 41):
        for nfrag in (2, 3, 4):
            ops = schedule_cute_multistage(ntile, stages, nfrag)
            r = simulate(ops, ntile, stages, nfrag)
            assert r.ok, (ntile, stages, nfrag, r.errors[:3])


@pytest.mark.parametrize("stages", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("L", [1, 2, 4, 8])
def test_three_phase_invariants_exhaustive(stages, L):
    for ntile in range(1, 41):
        ops = schedule_three_phase(ntile, stages, 2, None, L)
        r = simulate_loads(ops, ntile, stages, 2, L)
        assert r.ok, (ntile, stages, L, r.errors[:3])


def test_loosest_wait_counts_closed_form():
    # loads issued after tile k's and still allowed in flight: tiles
    # k+1 .. min(k+S-2, ntile-1), L loads each
    for stages in (2, 3, 4, 5):
        for L in (1, 4, 8):
            for ntile in (1, 2, 3, 7, 12):
                got = oracle.loosest_wait_counts(ntile, stages, L)
                want = [L * max(0, min(stages - 2, ntile - 1 - k)) for k in range(ntile)]
                assert got == want, (stages, L, ntile)


def test_planted_wait_too_loose_is_caught():
    # waiting for S-1 batches instead of S-2 reads a slot still in flight
    # ("cute(9) multistage_gemm", section 8.3)
    ntile, stages, nfrag = 8, 3, 2
    ops = schedule_cute_multistage(ntile, stages, nfrag)
    loose = [Op("wait", n=stages - 1) if o.kind == "wait" else o for o in ops]
    r = simulate(loose, ntile, stages, nfrag)
    assert not r.ok and any(e.startswith("RAW") for e in r.errors)


def test_planted_refill_before_barrier_is_caught():
    ntile, stages, L = 10, 3, 2
    ops = schedule_three_phase(ntile, stages, 2, None, L)
    # move every steady-state refill in front of its barrier
    out = []
    i = 0
    while i < len(ops):
        o = ops[i]
        if o.kind == "wait" and i + 2 < len(ops) and ops[i + 1].kind == "sync" and ops[i + 2].kind == "issue_part":
            j = i + 2
            issues = []
            while j < len(ops) and ops[j].kind == "issue_part":
                issues.append(ops[j])
                j += 1
            out += issues + [o, ops[i + 1]]
            i = j
        else:
            out.append(o)
            i += 1
    r = simulate_loads(out, ntile, stages, 2, L)
    assert not r.ok and any(e.startswith("WAR") for e in r.errors)


def test_planted_fill_of_all_slots_is_caught():
    # filling all S slots in the prologue leaves no free slot: the first
    # steady-state refill lands in the slot about to be consumed
    # ("cute(9) multistage_gemm", section 5.1)
    ntile, stages, L = 8, 3, 1
    ops = [Op("issue_part", tile=t, slot=t % stages) for t in range(stages)]
    for k in range(ntile):
        ops += [Op("wait", n=0), Op("sync")]
        if k + stages < ntile:
            ops.append(Op("issue_part", tile=k + stages, slot=(k + stages) % stages))
        ops += [Op("read", slot=k % stages, frag=0), Op("compute", tile=k, frag=0)]
    r = simulate_loads(ops, ntile, stages, 1, L)
    assert not r.ok


@pytest.mark.parametrize("stages", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("L", [1, 4, 8])
def test_cute_order_with_counted_loads_invariants(stages, L):
    for ntile in range(1, 41):
        for nfrag in (2, 4):
            ops = schedule_cute_loads(ntile, stages, nfrag, L)
            r = simulate_loads(ops, ntile, stages, nfrag, L)
            assert r.ok, (ntile, stages, nfrag, L, r.errors[:3])


def test_cute_order_with_counted_loads_catches_a_loose_wait():
    ntile, stages, L = 12, 4, 4
    base = [L * max(0, min(stages - 2, ntile - 1 - t)) for t in range(ntile)]
    for t in range(ntile):
        loose = list(base)
        loose[t] += 1
        r = simulate_loads(schedule_cute_loads(ntile, stages, 2, L, loose), ntile, stages, 2, L)
        assert not r.ok and any(e.startswith("RAW") for e in r.errors), t


# ---- two wave groups, one ring per operand

@pytest.mark.parametrize("ntile", range(0, 10))
def test_group_schedules_are_hazard_free(ntile):
    for make in (schedule_pingpong, schedule_split_pingpong):
        progs, slots, parts = make(ntile, 8)
        r = simulate_groups(progs, ntile, slots, parts)
        assert r.ok, (make.__name__, ntile, r.errors)


@pytest.mark.parametrize("plant,expect", [
    (dict(b_slots=2), "WAR"),        # B ring too shallow for loads two tiles ahead
    (dict(b_ahead=3), "WAR"),        # B loaded three tiles ahead into a three-slot ring
    (dict(a_ahead=2), "WAR"),        # A loaded two tiles ahead into a two-slot ring
    (dict(b_ahead=1), "RAW"),        # B loaded only one tile ahead: lands in the phase it is read
    (dict(g1_keep=16), "RAW"),       # G1 keeps two B tiles in flight
    (dict(g0_keep=1), "RAW"),        # G0 leaves one load of the next A tile unretired
])
def test_split_pingpong_planted_mistakes_are_caught(plant, expect):
    progs, slots, parts = schedule_split_pingpong(6, 8, **plant)
    r = simulate_groups(progs, 6, slots, parts)
    assert not r.ok
    assert any(e.startswith(expect) for e in r.errors), r.errors


def test_split_pingpong_group1_wait_is_the_loosest_safe():
    # G1 may keep exactly the B tile it just issued in flight, no load more
    results = []
    for keep in (8, 9):
        progs, slots, parts = schedule_split_pingpong(6, 8, g1_keep=keep)
        results.append(simulate_groups(progs, 6, slots, parts).ok)
    assert results == [True, False]


def test_group_simulator_catches_barrier_mismatch_and_missing_loads():
    progs, slots, parts = schedule_split_pingpong(4, 8)
    del progs["G0"][-1]                                   # G0 skips its last barrier
    assert any("barriers" in e for e in simulate_groups(progs, 4, slots, parts).errors)
    progs, slots, parts = schedule_pingpong(3, 8)
    progs["G0"] = [o for o in progs["G0"] if not (o.kind == "issue" and o.operand == "B" and o.tile == 2)]
    r = simulate_groups(progs, 3, slots, parts)
    assert not r.ok and any("B tile 2" in e for e in r.errors)
