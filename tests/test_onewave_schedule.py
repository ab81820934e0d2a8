"""CPU checks of the mainloop texts of schedules 10, 11, 12 and 14
(onewave_mainloop.inc, onewave_b3_mainloop.inc, onewave_b3h_mainloop.inc,
onewave128_mainloop.inc).

Each mainloop is one inline-assembly statement written by
gen_onewave_mainloop.py, so neither the compiler nor the GPU parity tests see
its hazards one by one.  This file executes the statement's text
symbolically, for one wave, for every K-tile count up to a few tiles past the
ring depth, and checks the ring protocol of "Lesson 6", section 4 (a slot is
refilled only after every wave's reads of it have completed and a barrier
has passed; a slot is read only after every load of its tile has retired
and a barrier has passed) together with the instruction-level rules the
text has to keep by itself:

  * every MFMA multiplies an A and a B fragment of the same K tile and K
    step, of the blocks its accumulator names, read from LDS after the tile
    was published and waited for with lgkmcnt; each accumulator sees the K
    steps in order, each once;
  * every LDS-DMA takes its source offsets from the offset block computed
    for the tile it loads, writes the slot and operand part its m0 names,
    and has one s_nop between the m0 write and itself;
  * SCC is not overwritten between a compare and its use;
  * no VOP2/VOPC reads more than one SGPR or VCC (the constant bus of gfx9);
  * nothing is in flight at the end, followed by the wait states the
    compiler's reads of the accumulators need.

All waves of the workgroup run the same text, so one wave's order of
barriers, waits and accesses stands for all of them.
"""
import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "stage_pipelined_mainloop_amd", "csrc")
PART = 32768          # one operand tile in LDS: 256 rows of 128 bytes


def slot_sched10(off):
    """Schedule 10: slot s holds A rows at s * 64 KiB, then B rows."""
    slot, within = divmod(off, 2 * PART)
    return ("A" if within < PART else "B"), slot


def slot_sched11(off):
    """Schedule 11: two A slots, then three B slots, 32 KiB each."""
    return ("A", off // PART) if off < 2 * PART else ("B", (off - 2 * PART) // PART)


def slot_sched14(off):
    """Schedule 14: four 32 KiB slots of 128 A rows, then 128 B rows."""
    slot, within = divmod(off, PART)
    return ("A" if within < PART // 2 else "B"), slot


# text file, its LDS layout, its mid-tile wait, its prologue wait, loads per
# lane per operand per tile, MFMA blocks per wave side, and the smallest
# number of MFMAs allowed between the last reader of a fragment register
# and the LDS read that overwrites it (an MFMA reads its A and B operands as
# it issues; the 16-MFMA halves of schedule 14 leave room for 7)
FORMS = {
    "sched10": ("onewave_mainloop.inc", slot_sched10, "s_waitcnt vmcnt(0) lgkmcnt(0)",
                "s_waitcnt vmcnt(16)", 8, 8, 28),
    "sched11": ("onewave_b3_mainloop.inc", slot_sched11, "s_waitcnt vmcnt(8) lgkmcnt(0)",
                "s_waitcnt vmcnt(24)", 8, 8, 28),
    "sched12": ("onewave_b3h_mainloop.inc", slot_sched11, "s_waitcnt vmcnt(8) lgkmcnt(0)",
                "s_waitcnt vmcnt(16)", 8, 8, 28),
    "sched14": ("onewave128_mainloop.inc", slot_sched14, "s_waitcnt vmcnt(12) lgkmcnt(0)",
                "s_waitcnt vmcnt(16)", 4, 4, 6),
}
SGPR_OPERANDS = {"wb", "rwa", "rwb", "nk", "kk", "sk", "st", "se"}


def _generator():
    spec = importlib.util.spec_from_file_location("gen_onewave_mainloop",
                                                  os.path.join(CSRC, "gen_onewave_mainloop.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def instructions(text: str) -> list[str]:
    """The statement's instructions, one string each, operands as written."""
    return [m.group(1) for m in re.finditer(r'^\s*"(.*)\\n"\s*$', text, re.M)]


class Hazard(AssertionError):
    pass


def run(code: list[str], nk: int, layout=slot_sched10, loads=8):
    """Execute `code` for nk K tiles.  Returns the per-accumulator sequences
    of (tile, K step) and the smallest number of MFMAs issued between an MFMA
    reading a fragment register and the next LDS read into it."""
    labels = {ins[:-1]: i for i, ins in enumerate(code) if ins.endswith(":")}
    reg = {"nk": nk, "kk": 64 * nk}        # scalar values (K a whole number of tiles)
    tag = {}                               # vector / symbolic values
    scc = None                             # (value, writer index)
    epoch = 0
    vm = []                                # outstanding LDS-DMA: [(operand, slot, tile)]
    lgkm = []                              # outstanding LDS reads: [register]
    dma_epochs = {}                        # (operand, slot, tile) -> [retire epoch | None]
    ring = {}                              # (operand, slot) -> tile last loaded there
    last_dma_epoch = {}                    # (operand, slot) -> epoch of its last DMA issue
    read_done = {}                         # (operand, slot) -> epochs of completed reads
    frag = {}                              # register -> (operand, tile, kstep, block, ready)
    pending = {}                           # register -> read still outstanding
    last_reader = {}                       # register -> MFMA count at its last MFMA read
    acc = {}
    mfmas = 0
    min_gap = None
    m0 = None
    m0_at = -10
    pc = 0
    steps = 0

    def fail(msg):
        raise Hazard(f"nk={nk}, instruction {pc} `{code[pc]}`: {msg}")

    def ops(ins):
        return [o.strip() for o in ins.split(None, 1)[1].split(",")] if " " in ins else []

    def name(o):
        m = re.fullmatch(r"%\[(\w+)\]", o)
        return m.group(1) if m else None

    def sval(o):
        n = name(o)
        if n is not None:
            if n not in reg:
                fail(f"{n} read before it is set")
            return reg[n]
        return int(o, 0)

    def retire_lgkm(keep):
        while len(lgkm) > keep:
            r, key = lgkm.pop(0)
            read_done.setdefault(key, []).append(epoch)
            pending.pop(r, None)

    while pc < len(code):
        steps += 1
        if steps > 200000:
            fail("does not terminate")
        ins = code[pc]
        if ins.endswith(":"):
            pc += 1
            continue
        op = ins.split()[0]
        a = ops(ins)
        # constant bus: one SGPR or VCC per VOP2 / VOPC
        if op.startswith("v_") and not op.startswith("v_mfma"):
            srcs = a[1:]
            bus = sum(1 for o in srcs if name(o) in SGPR_OPERANDS or o == "vcc")
            if bus > 1:
                fail("reads more than one SGPR or VCC")
        if op == "s_mov_b32":
            reg[name(a[0])] = sval(a[1])
        elif op == "s_add_u32" and a[0] == "m0":
            if name(a[1]) != "wb":
                fail("m0 not based on this wave's LDS address")
            m0, m0_at = int(a[2], 0), pc
            scc = None
        elif op in ("s_add_u32", "s_sub_i32", "s_lshl_b32"):
            x, y = sval(a[1]), sval(a[2])
            d = name(a[0])
            if op == "s_add_u32":
                reg[d] = x + y
            elif op == "s_sub_i32":
                reg[d] = x - y
            else:
                reg[d] = x << y
            # shifted tile index: remember which tile the value belongs to
            if op == "s_lshl_b32" and name(a[1]) == "st":
                tag[d] = ("kfirst" if y == 6 else "bytes", reg["st"])
            elif op == "s_sub_i32" and name(a[2]) == "se":
                tag[d] = ("kleft", tag.get("se", (None, None))[1])
            scc = None                                   # these write SCC
        elif op.startswith("s_cmp_"):
            x, y = sval(a[0]), sval(a[1])
            rel = op.split("_")[2]
            scc = ({"lt": x < y, "ge": x >= y, "eq": x == y}[rel], pc)
            if op.startswith("s_cmp_lt") and name(a[0]) == "st":
                tag["cmp"] = ("inrange", reg["st"])
        elif op == "s_cselect_b32":
            if scc is None:
                fail("SCC overwritten or unset before s_cselect")
            if tag.get("cmp", (None, None))[1] != tag.get("se", (None, None))[1]:
                fail("range test and K count belong to different tiles")
            reg[name(a[0])] = sval(a[1]) if scc[0] else sval(a[2])
        elif op in ("s_cbranch_scc1", "s_branch"):
            if op == "s_cbranch_scc1" and scc is None:
                fail("SCC overwritten or unset before the branch")
            taken = op == "s_branch" or scc[0]
            if taken:
                pc = labels[a[0]]
                continue
        elif op == "v_cmp_gt_i32":
            t = tag.get("se")
            if not t or t[0] != "kleft":
                fail("range compare not on the K count left")
            tag["vcc"] = ("range", t[1])
        elif op == "v_add_u32":
            d, x, y = name(a[0]), name(a[1]), name(a[2])
            if (x, y) == ("se", "lbase"):
                t = tag.get("se")
                if not t or t[0] != "bytes":
                    fail("first offset not from the tile's byte offset")
                tag[d] = ("off", t[1], 0, False)
            else:
                t, s = tag.get(x), tag.get(y)
                if not t or not s or t[0] != "off" or s[0] != "step" or t[1] != s[1] or not t[3]:
                    fail("offset chain mixes tiles or skips the range selection")
                tag[d] = ("off", t[1], t[2] + 1, True)
        elif op == "v_cndmask_b32":
            v = tag.get("vcc")
            d = name(a[0])
            if not v or v[0] != "range":
                fail("selection without the range compare")
            if d in ("vs", "ps"):
                tag[d] = ("step", v[1])
            else:
                t = tag.get(d)
                if not t or t[0] != "off" or t[1] != v[1]:
                    fail("range selection of another tile's offset")
                tag[d] = ("off", t[1], t[2], True)
        elif op == "s_nop":
            pass
        elif op == "buffer_load_dwordx4":
            if m0_at != pc - 2 or code[pc - 1] != "s_nop 0":
                fail("LDS-DMA not preceded by its m0 write and one s_nop")
            t = tag.get(name(a[0]))
            g = int(name(a[0])[1:])
            if not t or t[0] != "off" or not t[3] or t[2] != g:
                fail("source offset not from the offset block")
            tile = t[1]
            operand = {"rwa": "A", "rwb": "B"}[name(a[1])]
            named, slot = layout(m0)
            if named != operand or m0 % 4096:
                fail("m0 names another operand's part of the ring")
            key = (operand, slot)
            if any(e >= epoch for e in read_done.get(key, [])) or \
                    any(k == key for _, k in lgkm):
                fail(f"refills {operand} slot {slot} while reads of it may be in flight")
            if ring.get(key) != tile:
                ring[key] = tile
                dma_epochs[(operand, slot, tile)] = []
            last_dma_epoch[key] = epoch
            dma_epochs[(operand, slot, tile)].append(None)
            vm.append((operand, slot, tile))
        elif op == "s_waitcnt":
            m = re.search(r"vmcnt\((\d+)\)", ins)
            if m:
                while len(vm) > int(m.group(1)):
                    k = vm.pop(0)
                    lst = dma_epochs[k]
                    lst[lst.index(None)] = epoch
            m = re.search(r"lgkmcnt\((\d+)\)", ins)
            if m:
                retire_lgkm(int(m.group(1)))
        elif op == "s_barrier":
            if lgkm:
                fail("barrier with LDS reads in flight")
            epoch += 1
        elif op == "ds_read_b128":
            d = name(a[0])
            mo = re.fullmatch(r"%\[r([AB])(\d)(\d)\] offset:(\d+)", a[1])
            operand, slot, ks, off = mo.group(1), int(mo.group(2)), int(mo.group(3)), int(mo.group(4))
            if off % 2048:
                fail("fragment offset not a block boundary")
            if (d[1] == "a") != (operand == "A"):
                fail("A fragment register filled from B rows or the reverse")
            if d in last_reader:
                gap = mfmas - last_reader[d]
                min_gap = gap if min_gap is None else min(min_gap, gap)
            key = (operand, slot)
            tile = ring.get(key)
            done = dma_epochs.get((operand, slot, tile), [])
            ready = (tile is not None and tile < nk and len(done) == loads and
                     all(e is not None and e < epoch for e in done) and
                     last_dma_epoch[key] < epoch)
            frag[d] = (operand, tile, ks, off // 2048, ready)
            pending[d] = True
            lgkm.append((d, key))
        elif op == "v_mfma_f32_16x16x32_f16":
            c, b, x = name(a[0]), name(a[1]), name(a[2])
            if name(a[3]) != c:
                fail("accumulator in and out differ")
            i, j = int(c[1]), int(c[2])
            for r in (b, x):
                if pending.get(r):
                    fail(f"{r} used before its LDS read completed")
            fa, fb = frag.get(x), frag.get(b)
            if not fa or not fb or not fa[4] or not fb[4]:
                fail("fragment not published or past the last tile")
            if fa[0] != "A" or fb[0] != "B" or fa[1] != fb[1] or fa[2] != fb[2] or \
                    fa[3] != i or fb[3] != j or b[0] != x[0]:
                fail(f"multiplies {fa[:4]} by {fb[:4]} into c{i}{j}")
            acc.setdefault((i, j), []).append((fa[1], fa[2]))
            mfmas += 1
            last_reader[b] = last_reader[x] = mfmas
        else:
            fail("instruction the checker does not know")
        pc += 1
    if vm or lgkm:
        raise Hazard(f"nk={nk}: {len(vm)} loads and {len(lgkm)} reads in flight at the end")
    return acc, min_gap


def load(form):
    with open(os.path.join(CSRC, FORMS[form][0])) as f:
        return instructions(f.read())


def test_committed_texts_are_the_generator_output(tmp_path):
    paths = _generator().write(str(tmp_path))
    assert sorted(os.path.basename(p) for p in paths) == sorted(v[0] for v in FORMS.values())
    for path in paths:
        with open(path) as f, open(os.path.join(CSRC, os.path.basename(path))) as g:
            assert f.read() == g.read(), "regenerate " + os.path.basename(path)


@pytest.mark.parametrize("form", sorted(FORMS))
@pytest.mark.parametrize("nk", range(0, 10))
def test_ring_protocol_and_mfma_operands(form, nk):
    fname, layout, mid, pro, loads, blocks, gap = FORMS[form]
    acc, min_gap = run(load(form), nk, layout, loads)
    want = [(t, ks) for t in range(nk) for ks in (0, 1)]
    if nk == 0:
        assert acc == {}
    else:
        assert sorted(acc) == [(i, j) for i in range(blocks) for j in range(blocks)]
        for ij, seq in acc.items():
            assert seq == want, ij
        # a fragment register is rewritten only well after its last MFMA reader
        assert min_gap >= gap, min_gap


@pytest.mark.parametrize("form", sorted(FORMS))
def test_ends_drained_with_accumulator_wait_states(form):
    code = load(form)
    done = code.index(next(i for i in code if i.startswith("L_ow_done")))
    assert code[done + 1] == "s_waitcnt vmcnt(0) lgkmcnt(0)"
    assert code[done + 2:] == ["s_nop 7"] * 3


def _mutate(code, old, new, nth=0):
    idx = [i for i, ins in enumerate(code) if ins == old]
    out = list(code)
    out[idx[nth]] = new
    return out


@pytest.mark.parametrize("form", sorted(FORMS))
@pytest.mark.parametrize("case", ["mid wait", "prologue waits for all", "prologue keeps tile 0",
                                  "missing barrier", "missing lgkmcnt", "m0 nop", "mid wait one short"])
def test_checker_catches_planted_mistakes(form, case):
    fname, layout, mid, pro, loads = FORMS[form][:5]
    code = load(form)
    keep = int(re.search(r"vmcnt\((\d+)\)", mid).group(1))
    mutation, expect = {
        # the wait before the mid-tile barrier no longer retires the next tile
        "mid wait": ((mid, "s_waitcnt lgkmcnt(0)"), "not published"),
        # the prologue barrier waits for every prologue load: still correct
        "prologue waits for all": ((pro, "s_waitcnt vmcnt(0)"), None),
        # the prologue keeps part of tile 0 in flight
        "prologue keeps tile 0": ((pro, "s_waitcnt vmcnt(40)"), "not published"),
        # the mid-tile barrier of the first tile gone: a refill in the phase
        # that reads the slot, or reads of a tile not yet published
        "missing barrier": (("s_barrier", "s_nop 0", 1),
                            "while reads of it may be in flight|not published"),
        # x fragments used before their reads complete
        "missing lgkmcnt": (("s_waitcnt lgkmcnt(0)", "s_nop 0"), "before its LDS read completed"),
        # m0 hazard: no s_nop between the m0 write and the DMA
        "m0 nop": (("s_nop 0", "s_nop 1"), "not preceded by its m0 write"),
        # one more load left in flight at the mid-tile barrier
        "mid wait one short": ((mid, f"s_waitcnt vmcnt({keep + 1}) lgkmcnt(0)"), "not published"),
    }[case]
    old, new = mutation[0], mutation[1]
    nth = mutation[2] if len(mutation) > 2 else 0
    bad = _mutate(code, old, new, nth)
    if expect is None:
        run(bad, 4, layout, loads)
        return
    with pytest.raises(Hazard, match=expect):
        for nk in range(1, 6):
            run(bad, nk, layout, loads)
