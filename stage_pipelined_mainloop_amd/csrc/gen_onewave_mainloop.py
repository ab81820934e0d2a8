"""Write onewave_mainloop.inc, the mainloop of schedule 10 as one inline-assembly
statement (included by gemm_kernel.hpp; `python gen_onewave_mainloop.py` in
this directory regenerates it, and a CPU test checks that the committed file
is this script's output).

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
28 MFMAs have issued since their last reader; SCC-using pairs (s_cmp,
s_cselect) have no SCC-writing instruction between them; every VOP2/VOPC
reads at most one SGPR or VCC.

Operands (named in the text): acc[8][8] ("+a"), fragment buffers xa, xb,
ya, yb[8] and load offsets o0..o7, vs ("=&v"), scalar temporaries sk, st,
se ("=&s"); inputs rA<slot><kstep>, rB<slot><kstep> (LDS byte address of
this lane's first A / B fragment for that slot and K step), lbase / lch8 /
lstep (this lane's LDS-DMA source offset of tile 0, 8 x its chunk index,
and the offset step of one load), oor (an offset past every buffer range),
wb (LDS address of this wave's first 1 KiB), rwa / rwb (buffer resources of
the workgroup's A and B rows), ow_nk (K tiles), ow_kk (K), all wave-uniform."""
import os

SLOT = 65536          # bytes of one ring slot: 256 A rows + 256 B rows of 128 bytes
B_OFF = 32768         # B rows within a slot
FRAG = 2048           # 16 rows of 128 bytes: one MFMA block of fragments


def q(x):
    return '"' + x + '\\n"'


def mfma(m, buf):
    """MFMA m (0..63) of a 32-deep step: block (i, j) = divmod(m, 8), operands
    swapped (B fragment first) so each lane's accumulators are 4 consecutive
    columns of one row of D."""
    i, j = divmod(m, 8)
    return q(f'v_mfma_f32_16x16x32_f16 %[c{i}{j}], %[{buf}b{j}], %[{buf}a{i}], %[c{i}{j}]')


def offsets(first):
    """LDS-DMA source offsets of the tile whose index `first` puts in st:
    o0 = this lane's offset of load 0 (or oor when the tile is past the last
    one or this lane's 16-byte chunk lies past K), o1..o7 = o0 + i * step
    (step 0 for an out-of-range lane)."""
    return first + [
        q('s_lshl_b32 %[se], %[st], 6'),                 # first K index of the tile
        q('s_sub_i32 %[se], %[kk], %[se]'),              # K left from there
        q('s_cmp_lt_u32 %[st], %[nk]'),
        q('s_cselect_b32 %[se], %[se], 0x80000000'),     # none left past the last tile
        q('v_cmp_gt_i32 vcc, %[se], %[lch8]'),           # this lane's chunk in range
        q('s_lshl_b32 %[se], %[st], 7'),                 # byte offset of the tile
        q('v_add_u32 %[o0], %[se], %[lbase]'),
        q('v_cndmask_b32 %[o0], %[oor], %[o0], vcc'),
        q('v_cndmask_b32 %[vs], 0, %[lstep], vcc'),
    ] + [q(f'v_add_u32 %[o{i}], %[o{i - 1}], %[vs]') for i in range(1, 8)]


def dma(g, slot):
    """LDS-DMA load g (0..15) of a tile into `slot`: loads 0..7 fill A rows
    32 i + (8 wave .. 8 wave + 7), loads 8..15 the same B rows."""
    off = slot * SLOT + (g * 4096 if g < 8 else B_OFF + (g - 8) * 4096)
    rsrc = 'rwa' if g < 8 else 'rwb'
    return [q(f's_add_u32 m0, %[wb], {off}'), q('s_nop 0'),
            q(f'buffer_load_dwordx4 %[o{g % 8}], %[{rsrc}], 0 offen lds')]


def reads(buf, slot, ks):
    """The 16 fragment reads of one 32-deep step: 8 A blocks then 8 B blocks."""
    return ([q(f'ds_read_b128 %[{buf}a{g}], %[rA{slot}{ks}] offset:{g * FRAG}') for g in range(8)] +
            [q(f'ds_read_b128 %[{buf}b{g}], %[rB{slot}{ks}] offset:{g * FRAG}') for g in range(8)])


def mainloop():
    body = []
    # prologue: tiles 0 and 1 into slots 0 and 1; tile 0 landed; its first step
    for t in range(2):
        body += offsets([q(f's_mov_b32 %[st], {t}')])
        for g in range(16):
            body += dma(g, t)
    body += [q('s_waitcnt vmcnt(16)'), q('s_barrier')]
    body += reads('x', 0, 0)
    body += [q('s_mov_b32 %[sk], 0'), q('s_cmp_eq_u32 %[nk], 0'), q('s_cbranch_scc1 L_ow_done_%=')]
    body += [q('L_ow_top_%=:')]
    for s in range(2):                                  # tile k with k % 2 == s
        load_off = offsets([q('s_add_u32 %[st], %[sk], 2')])   # tile k + 2, loaded this tile
        body += [q('s_waitcnt lgkmcnt(0)')]
        rd = reads('y', s, 1)
        for g in range(16):
            body += [mfma(4 * g, 'x'), mfma(4 * g + 1, 'x'), rd[g], mfma(4 * g + 2, 'x')]
            h = g - 2                                   # two groups in: the last loads have issued
            if 0 <= h < 8:
                body += load_off[2 * h:2 * h + 2]
            elif h == 8:
                body += load_off[16:]
            body.append(mfma(4 * g + 3, 'x'))
        body += [q('s_waitcnt vmcnt(0) lgkmcnt(0)'), q('s_barrier')]
        rd = reads('x', 1 - s, 0)
        for g in range(16):
            body += [mfma(4 * g, 'y'), mfma(4 * g + 1, 'y'), rd[g], mfma(4 * g + 2, 'y')]
            body += dma(g, s)
            body.append(mfma(4 * g + 3, 'y'))
        body += [q('s_add_u32 %[sk], %[sk], 1'), q('s_cmp_ge_u32 %[sk], %[nk]'),
                 q('s_cbranch_scc1 L_ow_done_%=')]
    body += [q('s_branch L_ow_top_%=')]
    body += [q('L_ow_done_%=:'), q('s_waitcnt vmcnt(0) lgkmcnt(0)'),
             q('s_nop 7'), q('s_nop 7'), q('s_nop 7')]
    return body


def statement():
    outs = [f'[c{i}{j}] "+a"(acc[{i}][{j}])' for i in range(8) for j in range(8)]
    outs += [f'[{b}{o}{i}] "=&v"({b}{o}[{i}])' for b in 'xy' for o in 'ab' for i in range(8)]
    outs += [f'[o{i}] "=&v"(o{i})' for i in range(8)] + ['[vs] "=&v"(vs)']
    outs += [f'[{n}] "=&s"({n})' for n in ('sk', 'st', 'se')]
    ins = [f'[r{o}{s}{k}] "v"(r{o}{s}{k})' for o in 'AB' for s in range(2) for k in range(2)]
    ins += [f'[{n}] "v"({n})' for n in ('lbase', 'lch8', 'lstep', 'oor')]
    ins += [f'[{n}] "s"({n})' for n in ('wb', 'rwa', 'rwb')] + ['[nk] "s"(ow_nk)', '[kk] "s"(ow_kk)']
    lines = ["// Generated by gen_onewave_mainloop.py (same directory); do not edit.",
             "asm volatile("]
    lines += ["    " + ln for ln in mainloop()]
    lines.append("    : " + ",\n      ".join(outs))
    lines.append("    : " + ",\n      ".join(ins))
    lines.append('    : "memory", "m0", "scc", "vcc");')
    return "\n".join(lines) + "\n"


def write(path=None):
    path = path or os.path.join(os.path.dirname(os.path.abspath(__file__)), "onewave_mainloop.inc")
    with open(path, "w") as f:
        f.write(statement())
    return path


if __name__ == "__main__":
    print(write())
