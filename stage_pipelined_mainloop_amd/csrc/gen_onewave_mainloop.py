"""Write onewave_mainloop.inc, onewave_b3_mainloop.inc and
onewave_b3h_mainloop.inc, the mainloops of schedules 10, 11 and 12, each as
one inline-assembly statement (included by gemm_kernel.hpp; `python
gen_onewave_mainloop.py` in this directory regenerates them, and a CPU test
checks that the committed files are this script's output).

Schedule 10: a 256x256 output tile, 4 waves (one per SIMD), 128x128 per wave
as 8x8 blocks of v_mfma_f32_16x16x32_f16 with the 64 accumulator quads in
the 256 AGPRs; 64-deep K tiles in a ring of two LDS slots (64 KiB each: A
rows then B rows, 128 bytes per row, chunks swizzled as in the other
schedules).  Each K tile k is two 32-deep halves with one workgroup barrier
between them:

  first half   MFMAs of (k, K step 0) from fragment buffer x; read the
               fragments of (k, K step 1) into y from slot k % 2; compute the
               load offsets of tile k + 2.
  wait         this wave's loads of tile k + 1 (vmcnt 0) and its reads of
               slot k % 2 (lgkmcnt 0); barrier.  After it, tile k + 1 is in
               LDS for every wave and nobody reads slot k % 2 any more.
  second half  MFMAs of (k, K step 1) from y; read (k + 1, K step 0) into x
               from slot (k + 1) % 2; LDS-DMA tile k + 2 into slot k % 2.

Schedules 11 and 12 keep A in two slots of 32 KiB and B in three (160 KiB).
Schedule 11 loads B(k + 3) with A(k + 2) in the second half of tile k, into
the slot B(k) leaves.  Schedule 12 moves the B loads to the first half of
tile k: B(k + 2), into the slot B(k - 1) left at the barrier in the middle of
tile k - 1, so each half tile issues 8 loads per wave instead of 16.  Both
wait with vmcnt(8) at the mid-tile barrier: the 8 B loads issued last may
stay in flight.

One barrier per 2048 MFMA cycles.  Tile k + 2's loads are issued over the
second half of tile k and first needed at the barrier in the middle of tile
k + 1: between half a tile and a whole tile of MFMA time to land (the
measured global-to-LDS copy of a 64-deep tile under load is about 1600
shader cycles against 2048 for a tile's MFMAs).  The statement holds the
whole loop, so no compiler code runs between MFMAs: the compiler does not
know these are MFMAs and would not insert the wait states an MFMA result
needs before its own instructions read or copy the accumulators.

Hazards handled in the text: s_nop 0 between each write of m0 and the
LDS-DMA that uses it; s_waitcnt before every fragment use and before the
barrier; three s_nop 7 after the last MFMA so the compiler's epilogue can
read the accumulators; fragment registers are rewritten only after at least
28 MFMAs have issued since their last reader; no SCC-writing instruction
(an m0 update is an s_add_u32, which writes SCC) between a compare and the
select that reads its SCC; every VOP2/VOPC reads at most one SGPR or VCC.

Operands (named in the text): acc[8][8] ("+a"), fragment buffers xa, xb,
ya, yb[8] and load offsets o0..o7, vs (and, for schedules 11 and 12, the
B tile's p0..p7, ps) ("=&v"), scalar temporaries sk, st, se ("=&s"); inputs rA<slot><kstep>, rB<slot><kstep> (LDS byte address of
this lane's first A / B fragment for that slot and K step), lbase / lch8 /
lstep (this lane's LDS-DMA source offset of tile 0, 8 x its chunk index,
and the offset step of one load), oor (an offset past every buffer range),
wb (LDS address of this wave's first 1 KiB), rwa / rwb (buffer resources of
the workgroup's A and B rows), ow_nk (K tiles), ow_kk (K), all wave-uniform."""
import math
import os

A_PART = 32768        # bytes of one operand tile: 256 rows of 128 bytes
FRAG = 2048           # 16 rows of 128 bytes: one MFMA block of fragments


class Form:
    """One mainloop form: B ring depth and how far ahead B is loaded (A
    always has two slots and is loaded two tiles ahead), and the LDS byte
    offset of each slot."""

    def __init__(self, b_slots, b_first_half=False):
        self.b_slots = b_slots
        # B loads in the first half of tile k (B(k + 2), into the slot B(k - 1)
        # left) or with the A loads in the second half (B(k + b_slots), into
        # the slot B(k) leaves)
        self.b_first = b_first_half
        self.b_ahead = 2 if b_first_half else b_slots
        self.unroll = math.lcm(2, b_slots)
        self.split = b_slots != 2       # A and B use separate offset registers

    def a_off(self, slot):
        # schedule 10: slot s = A rows then B rows at s * 64 KiB;
        # schedule 11: two A slots, then three B slots, 32 KiB each
        return slot * 2 * A_PART if not self.split else slot * A_PART

    def b_off(self, slot):
        return slot * 2 * A_PART + A_PART if not self.split else 2 * A_PART + slot * A_PART


def q(x):
    return '"' + x + '\\n"'


def mfma(m, buf):
    """MFMA m (0..63) of a 32-deep step: block (i, j) = divmod(m, 8), operands
    swapped (B fragment first) so each lane's accumulators are 4 consecutive
    columns of one row of D."""
    i, j = divmod(m, 8)
    return q(f'v_mfma_f32_16x16x32_f16 %[c{i}{j}], %[{buf}b{j}], %[{buf}a{i}], %[c{i}{j}]')


def offsets(first, reg="o", step="vs"):
    """LDS-DMA source offsets of the tile whose index `first` puts in st:
    reg0 = this lane's offset of load 0 (or oor when the tile is past the
    last one or this lane's 16-byte chunk lies past K), reg1..reg7 = reg0 +
    i * step (step 0 for an out-of-range lane).  A list of chunks: the
    compare and the select that reads its SCC stay together, so nothing that
    writes SCC (an m0 update) can be placed between them."""
    return [[x] for x in first] + [
        [q('s_lshl_b32 %[se], %[st], 6')],               # first K index of the tile
        [q('s_sub_i32 %[se], %[kk], %[se]')],            # K left from there
        [q('s_cmp_lt_u32 %[st], %[nk]'),
         q('s_cselect_b32 %[se], %[se], 0x80000000')],   # none left past the last tile
        [q('v_cmp_gt_i32 vcc, %[se], %[lch8]')],         # this lane's chunk in range
        [q('s_lshl_b32 %[se], %[st], 7')],               # byte offset of the tile
        [q(f'v_add_u32 %[{reg}0], %[se], %[lbase]')],
        [q(f'v_cndmask_b32 %[{reg}0], %[oor], %[{reg}0], vcc')],
        [q(f'v_cndmask_b32 %[{step}], 0, %[lstep], vcc')],
    ] + [[q(f'v_add_u32 %[{reg}{i}], %[{reg}{i - 1}], %[{step}]')] for i in range(1, 8)]


def flat(chunks):
    return [x for c in chunks for x in c]


def spread(chunks, g, n=14):
    """The instructions of `chunks` that go after MFMA group g (2..15):
    the chunks dealt in order, ceil(len / n) to a group.  In a half without
    LDS-DMA loads nothing between the chunks writes SCC, so there the
    instructions are dealt one by one (single-instruction chunks)."""
    per = -(-len(chunks) // n)
    return flat(chunks[(g - 2) * per:(g - 1) * per]) if g >= 2 else []


def dma(f, g, a_slot, b_slot, b_reg="o"):
    """LDS-DMA load g (0..15) of a tile: loads 0..7 fill A rows
    32 i + (8 wave .. 8 wave + 7) of slot a_slot, loads 8..15 the same B rows
    of slot b_slot."""
    if g < 8:
        off, rsrc, reg = f.a_off(a_slot) + g * 4096, "rwa", "o"
    else:
        off, rsrc, reg = f.b_off(b_slot) + (g - 8) * 4096, "rwb", b_reg
    return [q(f's_add_u32 m0, %[wb], {off}'), q('s_nop 0'),
            q(f'buffer_load_dwordx4 %[{reg}{g % 8}], %[{rsrc}], 0 offen lds')]


def reads(buf, a_slot, b_slot, ks):
    """The 16 fragment reads of one 32-deep step: 8 A blocks then 8 B blocks."""
    return ([q(f'ds_read_b128 %[{buf}a{g}], %[rA{a_slot}{ks}] offset:{g * FRAG}') for g in range(8)] +
            [q(f'ds_read_b128 %[{buf}b{g}], %[rB{b_slot}{ks}] offset:{g * FRAG}') for g in range(8)])


def mainloop(f):
    body = []
    breg = "p" if f.split else "o"
    # prologue: A and B tiles 0 and 1, and B tiles up to b_ahead - 1 (or the
    # offsets of B tile 2 when the first half of tile 0 loads it); tile 0
    # landed; its first step
    for t in range(2):
        body += flat(offsets([q(f's_mov_b32 %[st], {t}')]))
        for g in range(16):
            body += dma(f, g, t, t)
    for t in range(2, 3 if f.b_first else f.b_ahead):
        if f.b_first:
            body += flat(offsets([q(f's_mov_b32 %[st], {t}')], "p", "ps"))
        else:
            body += flat(offsets([q(f's_mov_b32 %[st], {t}')]))
            for g in range(8, 16):
                body += dma(f, g, None, t)
    pro_keep = 0 if f.b_first else 8 * (f.b_ahead - 2)
    body += [q(f's_waitcnt vmcnt({16 + pro_keep})'), q('s_barrier')]
    body += reads('x', 0, 0, 0)
    body += [q('s_mov_b32 %[sk], 0'), q('s_cmp_eq_u32 %[nk], 0'), q('s_cbranch_scc1 L_ow_done_%=')]
    body += [q('L_ow_top_%=:')]
    for p in range(f.unroll):                           # tile k with k % unroll == p
        sa, sb = p % 2, p % f.b_slots
        na, nb = (p + 1) % 2, (p + 1) % f.b_slots
        # offsets of A(k + 2), loaded in this tile's second half, and of the
        # B tile loaded with it or, when B loads in first halves, of B(k + 3)
        # for the next tile's first half
        a_off = offsets([q('s_add_u32 %[st], %[sk], 2')])
        b_tile = 3 if f.b_first else f.b_ahead
        b_off = offsets([q(f's_add_u32 %[st], %[sk], {b_tile}')], "p", "ps") if f.split else []
        first_off = a_off if f.b_first else [[x] for x in flat(a_off + b_off)]
        body += [q('s_waitcnt lgkmcnt(0)')]
        rd = reads('y', sa, sb, 1)
        for g in range(16):
            body += [mfma(4 * g, 'x'), mfma(4 * g + 1, 'x'), rd[g], mfma(4 * g + 2, 'x')]
            if f.b_first and g % 2 == 1:                # B(k + 2) into the slot B(k - 1) left
                body += dma(f, 8 + g // 2, None, (p + 2) % f.b_slots, breg)
            # from two groups in (the previous half's last loads have issued)
            body += spread(first_off, g)
            body.append(mfma(4 * g + 3, 'x'))
        # tile k + 1 landed for this wave (the B tile loaded last may stay
        # in flight), and this wave's reads of slot (sa, sb) are done
        keep = 8 if f.split else 0
        body += [q(f's_waitcnt vmcnt({keep}) lgkmcnt(0)'), q('s_barrier')]
        rd = reads('x', na, nb, 0)
        for g in range(16):
            body += [mfma(4 * g, 'y'), mfma(4 * g + 1, 'y'), rd[g], mfma(4 * g + 2, 'y')]
            if not f.b_first:
                body += dma(f, g, sa, sb, breg)
            elif g % 2 == 0:                            # A(k + 2) into the slot A(k) leaves
                body += dma(f, g // 2, sa, None)
            if f.b_first:
                body += spread(b_off, g)
            body.append(mfma(4 * g + 3, 'y'))
        body += [q('s_add_u32 %[sk], %[sk], 1'), q('s_cmp_ge_u32 %[sk], %[nk]'),
                 q('s_cbranch_scc1 L_ow_done_%=')]
    body += [q('s_branch L_ow_top_%=')]
    body += [q('L_ow_done_%=:'), q('s_waitcnt vmcnt(0) lgkmcnt(0)'),
             q('s_nop 7'), q('s_nop 7'), q('s_nop 7')]
    return body


def mainloop128():
    """Schedule 14: a 128x128 tile, 4 waves of 64x64 (4x4 blocks), 64-deep K
    tiles in a ring of four 32 KiB slots (A rows then B rows), one barrier
    per tile between its halves.  Tile k + 3 goes into the slot tile k - 1
    left, its 4 A loads per wave in the first half of tile k and its 4 B
    loads early in the second; its offsets are computed late in the second
    half of tile k - 1.  The mid-tile wait keeps the
    loads of tile k + 2 and the first half's loads of tile k + 3 in flight."""
    SL, AP = 32768, 16384

    def dma4(g, slot):
        off = slot * SL + (g * 4096 if g < 4 else AP + (g - 4) * 4096)
        rsrc = 'rwa' if g < 4 else 'rwb'
        return [q(f's_add_u32 m0, %[wb], {off}'), q('s_nop 0'),
                q(f'buffer_load_dwordx4 %[o{g % 4}], %[{rsrc}], 0 offen lds')]

    def offs4(first):
        return [[x] for x in first] + [
            [q('s_lshl_b32 %[se], %[st], 6')],
            [q('s_sub_i32 %[se], %[kk], %[se]')],
            [q('s_cmp_lt_u32 %[st], %[nk]'), q('s_cselect_b32 %[se], %[se], 0x80000000')],
            [q('v_cmp_gt_i32 vcc, %[se], %[lch8]')],
            [q('s_lshl_b32 %[se], %[st], 7')],
            [q('v_add_u32 %[o0], %[se], %[lbase]')],
            [q('v_cndmask_b32 %[o0], %[oor], %[o0], vcc')],
            [q('v_cndmask_b32 %[vs], 0, %[lstep], vcc')],
        ] + [[q(f'v_add_u32 %[o{i}], %[o{i - 1}], %[vs]')] for i in range(1, 4)]

    def rd4(buf, slot, ks):
        return ([q(f'ds_read_b128 %[{buf}a{g}], %[rA{slot}{ks}] offset:{g * FRAG}') for g in range(4)] +
                [q(f'ds_read_b128 %[{buf}b{g}], %[rB{slot}{ks}] offset:{g * FRAG}') for g in range(4)])

    def mf(m, buf):
        i, j = divmod(m, 4)
        return q(f'v_mfma_f32_16x16x32_f16 %[c{i}{j}], %[{buf}b{j}], %[{buf}a{i}], %[c{i}{j}]')

    body = []
    for t in range(3):                                  # prologue: tiles 0..2 into slots 0..2
        body += flat(offs4([q(f's_mov_b32 %[st], {t}')]))
        for g in range(8):
            body += dma4(g, t)
    body += flat(offs4([q('s_mov_b32 %[st], 3')]))     # offsets of tile 3
    body += [q('s_waitcnt vmcnt(16)'), q('s_barrier')]
    body += rd4('x', 0, 0)
    body += [q('s_mov_b32 %[sk], 0'), q('s_cmp_eq_u32 %[nk], 0'), q('s_cbranch_scc1 L_ow_done_%=')]
    body += [q('L_ow_top_%=:')]
    for p in range(4):                                  # tile k with k % 4 == p
        s, nx, w = p, (p + 1) % 4, (p + 3) % 4          # read slot, next slot, refill slot
        body += [q('s_waitcnt lgkmcnt(0)')]
        rd = rd4('y', s, 1)
        for g in range(8):                              # 16 MFMAs: 8 groups of 2
            body += [mf(2 * g, 'x'), rd[g]]
            if g % 2 == 1:                              # A loads 0..3 of tile k + 3
                body += dma4(g // 2, w)
            body.append(mf(2 * g + 1, 'x'))
        body += [q('s_waitcnt vmcnt(12) lgkmcnt(0)'), q('s_barrier')]
        rd = rd4('x', nx, 0)
        # B loads of tile k + 3 in the first four groups, then the offsets of
        # tile k + 4 (loaded in tile k + 1), which overwrite the registers
        nxt = offs4([q('s_add_u32 %[st], %[sk], 4')])
        for g in range(8):
            body += [mf(2 * g, 'y'), rd[g]]
            if g < 4:
                body += dma4(4 + g, w)
            else:
                body += flat(nxt[(g - 4) * 4:(g - 3) * 4])
            body.append(mf(2 * g + 1, 'y'))
        body += flat(nxt[16:])
        body += [q('s_add_u32 %[sk], %[sk], 1'), q('s_cmp_ge_u32 %[sk], %[nk]'),
                 q('s_cbranch_scc1 L_ow_done_%=')]
    body += [q('s_branch L_ow_top_%=')]
    body += [q('L_ow_done_%=:'), q('s_waitcnt vmcnt(0) lgkmcnt(0)'),
             q('s_nop 7'), q('s_nop 7'), q('s_nop 7')]
    return body


def statement128(name):
    outs = [f'[c{i}{j}] "+a"(acc[{i}][{j}])' for i in range(4) for j in range(4)]
    outs += [f'[{b}{o}{i}] "=&v"({b}{o}[{i}])' for b in 'xy' for o in 'ab' for i in range(4)]
    outs += [f'[o{i}] "=&v"(o{i})' for i in range(4)] + ['[vs] "=&v"(vs)']
    outs += [f'[{n}] "=&s"({n})' for n in ('sk', 'st', 'se')]
    ins = [f'[r{o}{s}{k}] "v"(r{o}{s}{k})' for o in 'AB' for s in range(4) for k in range(2)]
    ins += [f'[{n}] "v"({n})' for n in ('lbase', 'lch8', 'lstep', 'oor')]
    ins += [f'[{n}] "s"({n})' for n in ('wb', 'rwa', 'rwb')] + ['[nk] "s"(ow_nk)', '[kk] "s"(ow_kk)']
    lines = [f"// Generated by gen_onewave_mainloop.py (same directory); do not edit.  {name}",
             "asm volatile("]
    lines += ["    " + ln for ln in mainloop128()]
    lines.append("    : " + ",\n      ".join(outs))
    lines.append("    : " + ",\n      ".join(ins))
    lines.append('    : "memory", "m0", "scc", "vcc");')
    return "\n".join(lines) + "\n"


def statement(f, name):
    outs = [f'[c{i}{j}] "+a"(acc[{i}][{j}])' for i in range(8) for j in range(8)]
    outs += [f'[{b}{o}{i}] "=&v"({b}{o}[{i}])' for b in 'xy' for o in 'ab' for i in range(8)]
    outs += [f'[o{i}] "=&v"(o{i})' for i in range(8)] + ['[vs] "=&v"(vs)']
    if f.split:
        outs += [f'[p{i}] "=&v"(p{i})' for i in range(8)] + ['[ps] "=&v"(ps)']
    outs += [f'[{n}] "=&s"({n})' for n in ('sk', 'st', 'se')]
    ins = [f'[rA{s}{k}] "v"(rA{s}{k})' for s in range(2) for k in range(2)]
    ins += [f'[rB{s}{k}] "v"(rB{s}{k})' for s in range(f.b_slots) for k in range(2)]
    ins += [f'[{n}] "v"({n})' for n in ('lbase', 'lch8', 'lstep', 'oor')]
    ins += [f'[{n}] "s"({n})' for n in ('wb', 'rwa', 'rwb')] + ['[nk] "s"(ow_nk)', '[kk] "s"(ow_kk)']
    lines = [f"// Generated by gen_onewave_mainloop.py (same directory); do not edit.  {name}",
             "asm volatile("]
    lines += ["    " + ln for ln in mainloop(f)]
    lines.append("    : " + ",\n      ".join(outs))
    lines.append("    : " + ",\n      ".join(ins))
    lines.append('    : "memory", "m0", "scc", "vcc");')
    return "\n".join(lines) + "\n"


FORMS = {"onewave_mainloop.inc": (Form(2), "Schedule 10: A and B in two slots."),
         "onewave_b3_mainloop.inc": (Form(3), "Schedule 11: A in two slots, B in three."),
         "onewave_b3h_mainloop.inc": (Form(3, True),
                                      "Schedule 12: A in two slots, B in three, B loaded in first halves.")}


def write(directory=None):
    directory = directory or os.path.dirname(os.path.abspath(__file__))
    paths = []
    texts = {fname: statement(f, name) for fname, (f, name) in FORMS.items()}
    texts["onewave128_mainloop.inc"] = statement128(
        "Schedule 14: a 128x128 tile, four slots, tile k + 3 loaded over both halves of tile k.")
    for fname, text in texts.items():
        path = os.path.join(directory, fname)
        with open(path, "w") as fh:
            fh.write(text)
        paths.append(path)
    return paths


if __name__ == "__main__":
    print("\n".join(write()))
