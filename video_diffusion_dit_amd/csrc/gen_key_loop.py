#!/usr/bin/env python3
"""Writes key_loop_gfx950.inc and key_loop_idx_gfx950.inc: the key loop of the attention
forward kernel for gfx950, as one inline-asm block with fixed registers, over a contiguous
range of key tiles or over a list of key tiles. attn_fwd_gfx950.hip includes the files inside
attn_rows(); build.py runs this script before every compile, and a CPU test checks that the
committed files are what this script writes.

Method (online softmax with BF16 probabilities and FP32 accumulation): page "[sglang]
SANA-Video 2.0 anchor attention ... FP32 upcast" (blog on sglang PR #49219), "lessons" list
(QK^T, softmax and PV accumulate in FP32 from BF16 inputs) and documentation item (the
probabilities are rounded to BF16 before the PV product); page "PR #33702 report",
motivation (online softmax over KV blocks).

One wave per SIMD owns 64 query rows (row blocks rb = 0, 1 of 32 rows) and walks all 64-key
tiles t of its key range. Per tile:
    QK(t+1): 32 MFMAs  S^T = K.Q^T into the other S buffer, beside the second softmax half of
                       tile t (keys 32..63), then the rescale check of tile t; the first
                       V fragments of tile t are read after its 25th MFMA
    PV(t):   32 MFMAs  O^T += V^T.P^T, beside the first softmax half of tile t+1 (keys 0..31);
                       in its middle the one barrier of the tile, then the loads of tile t+3,
                       and after its 25th MFMA the first K fragments of tile t+2 (visible
                       since the barrier)
so that about 3.5 VALU instructions issue in the shadow of every MFMA. K and V tiles sit in
four LDS stages (K at 16 KiB * stage, V at 64 KiB + 16 KiB * stage) and arrive by
buffer->LDS loads three tiles ahead. Tile t uses stage t%4 and S buffer t%2, so the loop body
holds four tiles.

Softmax bookkeeping (per row block): m (the reference the probabilities are taken against,
log2 units of the scaled logit), l (the lane's partial row sum of the FP32 probabilities) and C
(the lane's normaliser correction). The first tile of a range of two or more tiles takes m =
(row maximum of S*c) + 48 from its own scores before its softmax. The common path computes
p = exp2(S*c - m) and checks that no lane's tile sum exceeds its limit min(l, 2^24); when one
does (always on the first tile, where l = 0) the wave calls the slow path. If a tile sum exceeds 2^24 (or is not a
number) the reference moves: the rebase path shifts it by a whole power of two using the
packed BF16 probabilities, or, when one of them is inf or NaN, the full path recomputes S of
the tile from LDS, moves m to the running row maximum plus a headroom of 48, rescales O and
l, and recomputes P. Every slow path ends in the correction, C += (sum of the tile's BF16
probabilities) - (its FP32 tile sum), so O / (l + C) normalises the tiles that hold a lane's
dominant keys by the BF16 values O used for them.

Register map (per lane):
    v[0:63], v[64:127]   S buffers: block (rb, kb) at 16*(2*kb + rb); P packed to BF16 in
                         place (pair j of a block at 8*(j/4) + j%4)
    v[128:143]           K fragment ring (4 x 4)       v[144:159]   V fragment ring (4 x 4)
    v160..v175           m, l, partial sums, C, check limits, mask limit, -inf, tile sums
    v176..v199           temporaries (check, exact path)
    s[40:61]             resource cursors, counters, masks, return address, BF16 ones; s61 keeps the
                         caller's M0 (the loads move it), which is restored at the end
    a[0:127]             O^T: block (db, rb) at 16*(2*db + rb)
    a[128:191]           Q fragments: (rb, s) at 128 + 4*(8*rb + s)
The block hands O^T back in v[0:127] (same numbering), m, l and C in operands.

Tile-list variant (block-skip attention, page "PR #33702 report", motivation: KV blocks
routed by a threshold are skipped): the tiles walked are the entries of an int32 list in
global memory (ascending tile indices; the list is readable at least 8 entries past its
count). The cursors move by (next - current) tiles instead of one; each index is clamped to
[current, ntk] first, so whatever the list holds, loads stay inside the sequence (an index of
ntk reads zeros, as loads past the end do). Entries 1..3 come by one scalar load in the
set-up; entry t+5 is fetched by a vector load in tile t, which the next tile's vmcnt(0) before
its barrier completes, and moved to an SGPR with v_readfirstlane when the cursors advance.
Extra registers: v200 (the fetched index), v201 (zero offset), s[62:63] list cursor,
s[64:67] set-up entries, s68 current tile, s69 next tile, s70 byte step, s71 ntk.

The script tracks the LDS reads in flight (inserting s_waitcnt lgkmcnt) and inserts s_nop
for the gfx950 wait states that hand-written code must provide itself:
    VALU write -> MFMA read of the register                            2
    MFMA (8 passes) write -> non-MFMA access of the register           12
    MFMA write -> MFMA read as A/B, or as a C that is not its own chain 12
    MFMA read as C -> VALU write of the register                        12
    transcendental write -> VALU read                                   1
    DOT write -> read by another instruction (except a DOT of the same
                 opcode that takes it as its accumulator)               3
    SALU write of M0 -> buffer load to LDS                              1
"""
import os
import struct
import sys

# ---------------------------------------------------------------- register map
S_BASE = (0, 64)
KR, VR = 128, 144
M = (160, 161)
L = (162, 163)
H1 = ((164, 165), (166, 167))      # the tile's partial sums [rb][2]: the first key half starts
H2 = H1                            # them, the second half adds to the same registers
C = (168, 169)                     # normaliser correction: sum of BF16 minus FP32 probabilities
LIM = (170, 171)                   # the next tile's check limit: min(l, 2^24)
KLIM_R = 172                       # key limit the exact path masks with (1000: no mask)
NEG_INF = 173
TS = (174, 175)                    # tile sums
TMP0 = 176
NV = 200
O_BASE, Q_BASE, NA = 0, 128, 192
SK, SV = 40, 44                    # buffer-resource cursors s[40:43] (K), s[44:47] (V)
S_T, S_TLAST, S_LIM = 49, 50, 52   # tile counter, last loop tile, rescale limit
S_RA = 54                          # exact-path return address s[54:55]
S_C1, S_C2 = 56, 58                # check masks
S_STG = 60                         # K stage offset handed to the exact path
S_M0 = 61                          # M0 of the caller, restored at the end
S_ONES = 53                        # 0x3f803f80: BF16 1.0 in both halves (sums packed pairs)
NS_LO, NS_HI = 40, 61
# tile-list variant
V_IDX, V_ZERO = 200, 201
S_LP, S_I, S_PREV, S_NEXT, S_D, S_NTK = 62, 64, 68, 69, 70, 71
INDEXED = False                    # set by render()

K_STAGE = 16384
V_BASE = 65536
V_STAGE = 16384
# The largest tile sum accepted without moving the reference: 2^24 as an FP32 bit pattern.
# Accepted probabilities stay below 2^24, so O sums at most N * 2^24 * max|v| (FP32 holds it
# for max|v| < 2^86 at N = 2^17); a larger limit sends fewer tiles to the exact path when the
# running maximum keeps climbing (outlier channels).
RESCALE_LIMIT_BITS = 0x4B800000

# Headroom: the exact path sets the reference m to the row's running maximum + 48 instead of
# the maximum itself, so a later key must exceed that maximum by more than 24 + 48 log2 units
# before the wave moves the reference again (rows whose maximum keeps climbing, as with
# outlier channels, move it far less often). Probabilities right after a move are <= 2^-48;
# a key more than 78 log2 units below the maximum (relative weight < 2^-78) can fall below
# the FP32 normal range, and sum(p v) stays normal while max|v| >= 2^-78.

# Schedule knobs (the values the kernel is built with).
OPTS = {
    "k_ahead": 2,        # K fragments read this many fragment pairs ahead of their MFMAs
    "v_ahead": 2,        # V fragments likewise
    "qk_valu_slots": 30, # QK phase: the exp work and the check spread over this many MFMAs
    "pv_valu_slots": 31, # PV phase: the exp work spread over this many MFMAs
    "barrier_after": 15, # PV phase: barrier and tile loads after this MFMA
    "kpre_after": 24,    # PV phase: the next QK phase's first K fragments read after this MFMA
    "vpre_after": 24,    # QK phase: the next PV phase's first V fragments read after this MFMA
    "limit_bits": RESCALE_LIMIT_BITS,
    "stagger": 1,        # softmax groups: fma, exp and sum/pack of a group this many groups apart
    "headroom": 48,      # the exact path moves m to the running maximum plus this (log2 units)
}


def sblk(buf, rb, kb):
    return S_BASE[buf] + 16 * (2 * kb + rb)


def oblk(db, rb):
    return O_BASE + 16 * (2 * db + rb)


def qfrag(rb, s):
    return Q_BASE + 4 * (8 * rb + s)


def vr(lo, n=1):
    return "v%d" % lo if n == 1 else "v[%d:%d]" % (lo, lo + n - 1)


def ar(lo, n=1):
    return "a%d" % lo if n == 1 else "a[%d:%d]" % (lo, lo + n - 1)


def vset(lo, n=1):
    return {("v", i) for i in range(lo, lo + n)}


def aset(lo, n=1):
    return {("a", i) for i in range(lo, lo + n)}


VCC = {("vcc",)}


class Ins:
    __slots__ = ("text", "kind", "rd", "wr", "rdc", "lds", "m0w", "m0r", "ws")

    def __init__(self, text, kind, rd=(), wr=(), rdc=(), lds=False, m0w=False, m0r=False, ws=1):
        self.text, self.kind = text, kind
        self.rd, self.wr, self.rdc = set(rd), set(wr), set(rdc)
        self.lds, self.m0w, self.m0r, self.ws = lds, m0w, m0r, ws


def need(prev, cur):
    """Wait states required between an earlier instruction prev and cur."""
    r = 0
    if prev.kind in ("valu", "trans") and cur.kind == "mfma" and prev.wr & (cur.rd | cur.rdc):
        r = max(r, 2)
    if prev.kind == "mfma":
        if cur.kind == "mfma":
            if prev.wr & cur.rd:
                r = max(r, 12)
            if prev.wr & cur.rdc and not (prev.wr == cur.rdc == cur.wr):
                r = max(r, 12)
        elif prev.wr & (cur.rd | cur.wr | cur.rdc):
            r = max(r, 12)
        if cur.kind in ("valu", "trans", "lds") and prev.rdc & cur.wr:
            r = max(r, 12)
    if prev.kind == "trans" and cur.kind in ("valu", "trans") and prev.wr & cur.rd:
        r = max(r, 1)
    if prev.kind == "dot" and prev.wr & cur.rd:
        r = max(r, 3)
    if prev.kind == "dot" and prev.wr & cur.rdc and (cur.kind != "dot" or cur.text.split()[0] != prev.text.split()[0]):
        r = max(r, 3)   # only a DOT of the same opcode reading it as its accumulator needs none
    if prev.m0w and cur.m0r:
        r = max(r, 1)
    return r


class Emitter:
    """Appends instructions, inserting s_waitcnt lgkmcnt and s_nop where required. Wait
    states are counted per incoming path (hists): a label reached from several places
    carries the history of each."""

    def __init__(self):
        self.out = []
        self.hists = [[]]
        self.pending = []      # register sets written by LDS ops in flight, oldest first
        self.calls = {0: [], 1: []}   # histories at the calls of each S buffer's slow path

    def fresh(self):
        self.hists = [[]]

    def state(self):
        return [list(h) for h in self.hists], list(self.pending)

    def set_state(self, st):
        self.hists, self.pending = [list(h) for h in st[0]], list(st[1])

    def label(self, name):
        self.out.append(name + ":")

    def raw(self, text):
        """An instruction outside the hazard model (branches, barriers, waits)."""
        self.out.append("\t" + text)

    def _push(self, ins):
        self.out.append("\t" + ins.text)
        for h in self.hists:
            h.append(ins)
            tot = 0
            for i in range(len(h) - 1, -1, -1):
                tot += h[i].ws
                if tot > 14:
                    del h[:i]
                    break

    def nop(self, n):
        while n > 0:
            k = min(n, 8)
            self._push(Ins("s_nop %d" % (k - 1), "nop", ws=k))
            n -= k

    def wait_lgkm(self, regs):
        idx = -1
        for i, p in enumerate(self.pending):
            if p & regs:
                idx = i
        if idx < 0:
            return
        after = min(len(self.pending) - 1 - idx, 15)
        self._push(Ins("s_waitcnt lgkmcnt(%d)" % after, "waitcnt"))
        self.pending = self.pending[len(self.pending) - after:] if after else []

    def emit(self, ins):
        self.wait_lgkm(ins.rd | ins.rdc | ins.wr)
        req = 0
        for hist in self.hists:
            dist = 0
            for p in reversed(hist):
                r = need(p, ins)
                if r > dist:
                    req = max(req, r - dist)
                dist += p.ws
                if dist >= 12:
                    break
        if req:
            self.nop(req)
        self._push(ins)
        if ins.lds:
            self.pending.append(set(ins.wr))

    def valu(self, text, rd=(), wr=()):
        self.emit(Ins(text, "valu", rd, wr))

    def trans(self, text, rd=(), wr=()):
        self.emit(Ins(text, "trans", rd, wr))

    def salu(self, text, m0w=False):
        self.emit(Ins(text, "salu", m0w=m0w))


# ---------------------------------------------------------------- building blocks
def mfma_qk(E, buf, rb, kb, s, kslot):
    """S^T block (rb, kb) += K fragment (kb, s) . Q fragment (rb, s)."""
    d = sblk(buf, rb, kb)
    src_c = "0" if s == 0 else vr(d, 16)
    E.emit(Ins("v_mfma_f32_32x32x16_bf16 %s, %s, %s, %s" % (vr(d, 16), vr(KR + 4 * kslot, 4), ar(qfrag(rb, s), 4), src_c),
               "mfma", rd=vset(KR + 4 * kslot, 4) | aset(qfrag(rb, s), 4), wr=vset(d, 16),
               rdc=(vset(d, 16) if s else ())))


def mfma_pv(E, buf, db, rb, h, vslot):
    """O^T block (db, rb) += V^T fragment (db, key step h) . P fragment (rb, h)."""
    o = oblk(db, rb)
    p = sblk(buf, rb, h >> 1) + 8 * (h & 1)
    E.emit(Ins("v_mfma_f32_32x32x16_bf16 %s, %s, %s, %s" % (ar(o, 16), vr(VR + 4 * vslot, 4), vr(p, 4), ar(o, 16)),
               "mfma", rd=vset(VR + 4 * vslot, 4) | vset(p, 4), wr=aset(o, 16), rdc=aset(o, 16)))


def read_k(E, slot, s, kb, stage, base_reg=None):
    """K fragment (kb, d-step s) of a stage into ring slot. Addresses: the ka operands (stage
    0) plus an immediate, or per-call registers base_reg+s (exact path)."""
    if base_reg is None:
        addr, off, rd = "%%[ka%d]" % s, K_STAGE * stage + 8192 * kb, ()
    else:
        addr, off, rd = vr(base_reg + s), 8192 * kb, vset(base_reg + s)
    E.emit(Ins("ds_read_b128 %s, %s offset:%d" % (vr(KR + 4 * slot, 4), addr, off), "lds",
               rd=rd, wr=vset(KR + 4 * slot, 4), lds=True))


def read_v(E, slot, db, h, stage):
    """V^T fragment (dim block db, key step h): two transposing reads."""
    off = V_STAGE * stage + 4096 * h
    for t in range(2):
        E.emit(Ins("ds_read_b64_tr_b16 %s, %%[va%d] offset:%d" % (vr(VR + 4 * slot + 2 * t, 2), 2 * db + t, off), "lds",
                   wr=vset(VR + 4 * slot + 2 * t, 2), lds=True))


def key_const(kb, r):
    """Key (within the tile) of S register r of block kb, less the lane's 8*g."""
    return 32 * kb + 16 * (r >> 3) + (r & 7)


def softmax_half(buf, kb, masked, klim, hs):
    """VALU stream for p = exp2(S*c - m) over blocks (0, kb) and (1, kb) of S buffer buf,
    accumulating the partial sums hs[rb] and packing P to BF16 in place. masked: keys at or
    past the limit klim = (operand text, registers read) give p = 0."""
    def group(rb, j):
        base = sblk(buf, rb, kb)
        a, b = base + 2 * j, base + 2 * j + 1
        m = M[rb]
        st1 = [lambda E, x=x: E.valu("v_fma_f32 %s, %s, %%[c], -%s" % (vr(x), vr(x), vr(m)), rd=vset(x) | vset(m), wr=vset(x))
               for x in (a, b)]
        st2 = [lambda E, x=x: E.trans("v_exp_f32 %s, %s" % (vr(x), vr(x)), rd=vset(x), wr=vset(x)) for x in (a, b)]
        if masked:
            for x, r in ((a, 2 * j), (b, 2 * j + 1)):
                st2.append(lambda E, x=x, kc=key_const(kb, r): (
                    E.valu("v_cmp_lt_i32 vcc, %d, %s" % (kc, klim[0]), rd=klim[1], wr=VCC),
                    E.valu("v_cndmask_b32 %s, 0, %s, vcc" % (vr(x), vr(x)), rd=vset(x) | VCC, wr=vset(x))))
        h0, h1 = hs[rb]
        if j == 0 and kb == 0:   # the first pair of a tile starts its two partial sums
            st3 = [lambda E: E.valu("v_mov_b32 %s, %s" % (vr(h0), vr(a)), rd=vset(a), wr=vset(h0)),
                   lambda E: E.valu("v_mov_b32 %s, %s" % (vr(h1), vr(b)), rd=vset(b), wr=vset(h1))]
        else:
            st3 = [lambda E: E.valu("v_add_f32 %s, %s, %s" % (vr(h0), vr(h0), vr(a)), rd=vset(h0) | vset(a), wr=vset(h0)),
                   lambda E: E.valu("v_add_f32 %s, %s, %s" % (vr(h1), vr(h1), vr(b)), rd=vset(h1) | vset(b), wr=vset(h1))]
        dst = base + 8 * (j // 4) + (j % 4)
        st3.append(lambda E: E.valu("v_cvt_pk_bf16_f32 %s, %s, %s" % (vr(dst), vr(a), vr(b)), rd=vset(a) | vset(b), wr=vset(dst)))
        return [st1, st2, st3]

    staged = [group(rb, j) for j in range(8) for rb in range(2)]
    stream = []   # stage s of group g issues at step g + s * stagger
    k = OPTS["stagger"]
    for step in range(len(staged) + 2 * k):
        for s in range(3):
            g = step - s * k
            if 0 <= g < len(staged):
                stream.extend(staged[g][s])
    return stream


N_TILE_SUM_OPS = 2    # the VALU instructions of check_ops() that form the tile sums


def check_ops():
    """Tile sums per row block (into TS, from the two partial sums both key halves added to)
    and the slow-path condition (into S_C1/S_C2): a lane's tile sum above its limit
    min(l, 2^24), or not a number."""
    def add(d, x, y):
        return lambda E: E.valu("v_add_f32 %s, %s, %s" % (vr(d), vr(x), vr(y)), rd=vset(x) | vset(y), wr=vset(d))
    ops = [add(TS[0], *H1[0]), add(TS[1], *H1[1])]
    for rb, sc in ((0, S_C1), (1, S_C2)):
        ops.append(lambda E, rb=rb, sc=sc: E.valu("v_cmp_nge_f32_e64 s[%d:%d], %s, %s" % (sc, sc + 1, vr(LIM[rb]), vr(TS[rb])),
                                                  rd=vset(LIM[rb]) | vset(TS[rb])))
    return ops


def distribute(E, mfmas, valu, extra=None, valu_slots=None):
    """Issue the MFMAs in order; after MFMA i, whatever extra[i] holds, then an even share of
    the VALU stream (spread over the first valu_slots MFMAs)."""
    n = len(mfmas)
    vs = n if valu_slots is None else valu_slots
    pos = 0
    for i in range(n):
        mfmas[i](E)
        for f in (extra or {}).get(i, []):
            f(E)
        if i < vs:
            k = (len(valu) - pos + (vs - i) - 1) // (vs - i)
            for f in valu[pos:pos + k]:
                f(E)
            pos += k
    for f in valu[pos:]:
        f(E)


def qk_phase(E, buf, stage, valu, valu_slots=None, extra=None):
    """S^T of a tile (K from stage) into S buffer buf; K fragments 0 and 1 are read before."""
    mf = []
    ex = {i: list(v) for i, v in (extra or {}).items()}
    for f in range(16):
        kb, s = f >> 3, f & 7
        for rb in range(2):
            mf.append(lambda E, rb=rb, kb=kb, s=s, f=f: mfma_qk(E, buf, rb, kb, s, f & 3))
        g = f + OPTS["k_ahead"]
        if g < 16:
            ex.setdefault(2 * f + 1, []).insert(0, lambda E, g=g: read_k(E, g & 3, g & 7, g >> 3, stage))
    distribute(E, mf, valu, ex, valu_slots)


def pv_phase(E, buf, stage, valu, valu_slots=None, extra=None):
    """O^T += V^T P^T for the tile whose P is in S buffer buf (V from stage); V fragments 0
    and 1 are read before."""
    mf = []
    ex = {i: list(v) for i, v in (extra or {}).items()}
    for v in range(16):
        h, db = v >> 2, v & 3
        for rb in range(2):
            mf.append(lambda E, db=db, rb=rb, h=h, v=v: mfma_pv(E, buf, db, rb, h, v & 3))
        g = v + OPTS["v_ahead"]
        if g < 16:
            ex.setdefault(2 * v + 1, []).insert(0, lambda E, g=g: read_v(E, g & 3, g & 3, g >> 2, stage))
    distribute(E, mf, valu, ex, valu_slots)


def prefetch_k(E, stage):
    for g in range(OPTS["k_ahead"]):
        read_k(E, g, g, 0, stage)


def prefetch_v(E, stage):
    for g in range(OPTS["v_ahead"]):
        read_v(E, g, g, 0, stage)


def tile_loads(stage, src=None):
    """Buffer->LDS loads of one tile (this wave's quarter of K and of V) into a stage; then
    both resource cursors move one tile on (records clamped at zero, so loads past the
    sequence end read zeros). Tile-list variant: the cursors move to the tile whose index is
    in SGPR src (set-up), or in v200 (loop: fetched one tile earlier, complete after the
    tile's vmcnt(0)), which then fetches the index after it."""
    ops = []
    if INDEXED and src is None:
        ops.append(lambda E: (E.emit(Ins("v_readfirstlane_b32 s%d, %s" % (S_NEXT, vr(V_IDX)), "valu", rd=vset(V_IDX))),
                              E.nop(4)))
    for i in range(4):
        for base, cur, name in ((K_STAGE * stage, SK, "ko"), (V_BASE + V_STAGE * stage, SV, "vo")):
            ops.append(lambda E, i=i, base=base, cur=cur, name=name: (
                E.salu("s_add_u32 m0, %%[ldsw], %d" % (base + 1024 * i), m0w=True),
                E.emit(Ins("buffer_load_dwordx4 %%[%s%d], s[%d:%d], 0 offen lds" % (name, i, cur, cur + 3), "vmem", m0r=True))))

    def advance(E):
        step = "%[tb]"
        if INDEXED:
            nxt = S_NEXT if src is None else src
            E.salu("s_max_i32 s%d, s%d, s%d" % (nxt, nxt, S_PREV))
            E.salu("s_min_i32 s%d, s%d, s%d" % (nxt, nxt, S_NTK))
            E.salu("s_sub_i32 s%d, s%d, s%d" % (S_D, nxt, S_PREV))
            E.salu("s_mul_i32 s%d, s%d, %%[tb]" % (S_D, S_D))
            E.salu("s_mov_b32 s%d, s%d" % (S_PREV, nxt))
            step = "s%d" % S_D
        for cur in (SK, SV):
            E.salu("s_add_u32 s%d, s%d, %s" % (cur, cur, step))
            E.salu("s_addc_u32 s%d, s%d, 0" % (cur + 1, cur + 1))
            E.salu("s_sub_i32 s%d, s%d, %s" % (cur + 2, cur + 2, step))
            E.salu("s_max_i32 s%d, s%d, 0" % (cur + 2, cur + 2))
        if INDEXED and src is None:
            fetch_index(E)
    ops.append(advance)
    return ops


def fetch_index(E):
    """v200 = the list entry at s[62:63], which then moves on one entry."""
    E.salu("s_add_u32 s%d, s%d, 4" % (S_LP, S_LP))
    E.salu("s_addc_u32 s%d, s%d, 0" % (S_LP + 1, S_LP + 1))
    E.emit(Ins("global_load_dword %s, %s, s[%d:%d] offset:-4" % (vr(V_IDX), vr(V_ZERO), S_LP, S_LP + 1), "vmem",
               rd=vset(V_ZERO), wr=vset(V_IDX)))


def rare_call(E, X, stage, uid):
    """If the check failed (either mask set), call the exact path of S buffer X with the K
    stage of the tile; it returns to the instruction after the call."""
    E.salu("s_or_b64 s[%d:%d], s[%d:%d], s[%d:%d]" % (S_C1, S_C1 + 1, S_C1, S_C1 + 1, S_C2, S_C2 + 1))
    E.raw("s_cbranch_scc0 .Lok%s_%%=" % uid)
    E.raw("s_mov_b32 s%d, %d" % (S_STG, K_STAGE * stage))
    E.raw("s_getpc_b64 s[%d:%d]" % (S_RA, S_RA + 1))
    E.label(".Lpc%s_%%=" % uid)
    E.raw("s_add_u32 s%d, s%d, .Lok%s_%%=-.Lpc%s_%%=" % (S_RA, S_RA, uid, uid))
    E.raw("s_addc_u32 s%d, s%d, 0" % (S_RA + 1, S_RA + 1))
    E.calls[X].extend(list(h) for h in E.hists)
    E.raw("s_branch .Lrare%d_%%=" % X)
    E.label(".Lok%s_%%=" % uid)


def add_l(E):
    """l += tile sum; the next tile's limit min(l, 2^24)."""
    for rb in range(2):
        E.valu("v_add_f32 %s, %s, %s" % (vr(L[rb]), vr(L[rb]), vr(TS[rb])), rd=vset(L[rb]) | vset(TS[rb]), wr=vset(L[rb]))
    for rb in range(2):
        E.valu("v_min_f32 %s, s%d, %s" % (vr(LIM[rb]), S_LIM, vr(L[rb])), rd=vset(L[rb]), wr=vset(LIM[rb]))


KLIM_IN = ("%[klim]", set())
KLIM_EXACT = (vr(KLIM_R), vset(KLIM_R))


def packed_p(X, rb):
    """The 16 registers that hold row block rb's 64 probabilities of S buffer X as BF16 pairs."""
    return [sblk(X, rb, kb) + off for kb in range(2) for off in (0, 1, 2, 3, 8, 9, 10, 11)]


def rescale_o(E, factor, op="v_mul_f32"):
    """O^T rows of row block rb scaled by factor[rb] (AGPR read, op, write back): op v_mul_f32
    with an FP32 factor, or v_ldexp_f32 with an integer exponent."""
    tmps = [TMP0 + 17 + i for i in range(7)]
    k = 0
    for rb in range(2):
        for db in range(4):
            for r in range(16):
                a, t = oblk(db, rb) + r, tmps[k % 7]
                k += 1
                E.valu("v_accvgpr_read_b32 %s, %s" % (vr(t), ar(a)), rd=aset(a), wr=vset(t))
                E.valu("%s %s, %s, %s" % (op, vr(t), vr(t), vr(factor[rb])), rd=vset(t) | vset(factor[rb]), wr=vset(t))
                E.valu("v_accvgpr_write_b32 %s, %s" % (ar(a), vr(t)), rd=vset(t), wr=aset(a))


def rebase_path(E, X):
    """Fast exact path for the tile in S buffer X: move the reference without recomputing S.

    The probabilities of the tile are already BF16 in registers, taken against the old
    reference m. Any reference keeps the softmax exact; it only has to bound them. Their
    largest value across the row (u16 maximum of the packed BF16 patterns, which order like
    the non-negative values; the partner lane l^32 holds the row's other keys) has binary
    exponent e, so with k = max(e + 1 + headroom, 0) the new reference m + k puts every
    probability below 2^-headroom. Scaling by 2^-k is exact: P in place by subtracting k
    from each BF16 exponent field (u16 max then subtract, so values that would drop below the
    normal range, weights under 2^-126 of the new reference, become 0), l, the tile sums and
    O by v_ldexp_f32 with -k. (Not by a multiplication with 2^-k: k reaches 177 when a key
    lies up to 128 log2 units above the old reference, and 2^-k then is no FP32 number, while
    the tile's own sum times 2^-k is about 2^-49.) A probability that is inf or NaN (the tile of
    a one-tile range, where m = -inf, or a key beyond the FP32 range of the old reference) carries
    no usable maximum:
    then the full path below recomputes S. Entered from the slow-path entry (no LDS read in
    flight); goes on to the correction with all wait states satisfied."""
    E.label(".Lmove%d_%%=" % X)
    mx, px, kk, negk = (TMP0 + 2, TMP0 + 3), (TMP0 + 4, TMP0 + 5), (TMP0 + 6, TMP0 + 7), (TMP0 + 8, TMP0 + 9)
    ki, t = TMP0 + 10, TMP0 + 11
    for rb in range(2):
        regs = packed_p(X, rb)
        E.valu("v_pk_max_u16 %s, %s, %s" % (vr(mx[rb]), vr(regs[0]), vr(regs[1])), rd=vset(regs[0]) | vset(regs[1]),
               wr=vset(mx[rb]))
        for r in regs[2:]:
            E.valu("v_pk_max_u16 %s, %s, %s" % (vr(mx[rb]), vr(mx[rb]), vr(r)), rd=vset(mx[rb]) | vset(r), wr=vset(mx[rb]))
        E.valu("v_lshrrev_b32 %s, 16, %s" % (vr(t), vr(mx[rb])), rd=vset(mx[rb]), wr=vset(t))
        E.valu("v_and_b32 %s, 0xffff, %s" % (vr(mx[rb]), vr(mx[rb])), rd=vset(mx[rb]), wr=vset(mx[rb]))
        E.valu("v_max_u32 %s, %s, %s" % (vr(mx[rb]), vr(mx[rb]), vr(t)), rd=vset(mx[rb]) | vset(t), wr=vset(mx[rb]))
    for rb in range(2):
        E.emit(Ins("ds_bpermute_b32 %s, %%[bperm], %s" % (vr(px[rb]), vr(mx[rb])), "lds", rd=vset(mx[rb]), wr=vset(px[rb]),
                   lds=True))
    for rb in range(2):   # any lane whose maximum is an inf/NaN pattern (>= 0x7f80)?
        E.valu("v_max_u32 %s, %s, %s" % (vr(mx[rb]), vr(mx[rb]), vr(px[rb])), rd=vset(mx[rb]) | vset(px[rb]), wr=vset(mx[rb]))
        E.valu("v_cmp_le_u32 vcc, 0x7f80, %s" % vr(mx[rb]), rd=vset(mx[rb]), wr=VCC)
        if rb == 0:
            E.salu("s_mov_b64 s[%d:%d], vcc" % (S_C1, S_C1 + 1))
    E.salu("s_or_b64 s[%d:%d], s[%d:%d], vcc" % (S_C1, S_C1 + 1, S_C1, S_C1 + 1))
    E.raw("s_cbranch_scc1 .Lfull%d_%%=" % X)
    bias = 126 - OPTS["headroom"]    # k = (biased exponent - 127) + 1 + headroom
    for rb in range(2):
        E.valu("v_lshrrev_b32 %s, 7, %s" % (vr(ki), vr(mx[rb])), rd=vset(mx[rb]), wr=vset(ki))
        E.valu("v_subrev_u32 %s, %d, %s" % (vr(ki), bias, vr(ki)), rd=vset(ki), wr=vset(ki))
        E.valu("v_max_i32 %s, 0, %s" % (vr(ki), vr(ki)), rd=vset(ki), wr=vset(ki))
        E.valu("v_cvt_f32_i32 %s, %s" % (vr(t), vr(ki)), rd=vset(ki), wr=vset(t))
        E.valu("v_add_f32 %s, %s, %s" % (vr(M[rb]), vr(M[rb]), vr(t)), rd=vset(M[rb]) | vset(t), wr=vset(M[rb]))
        E.valu("v_sub_u32 %s, 0, %s" % (vr(negk[rb]), vr(ki)), rd=vset(ki), wr=vset(negk[rb]))
        E.valu("v_lshlrev_b32 %s, 7, %s" % (vr(kk[rb]), vr(ki)), rd=vset(ki), wr=vset(kk[rb]))
        E.valu("v_lshl_or_b32 %s, %s, 16, %s" % (vr(kk[rb]), vr(kk[rb]), vr(kk[rb])), rd=vset(kk[rb]), wr=vset(kk[rb]))
        for r in packed_p(X, rb):
            E.valu("v_pk_max_u16 %s, %s, %s" % (vr(r), vr(r), vr(kk[rb])), rd=vset(r) | vset(kk[rb]), wr=vset(r))
            E.valu("v_pk_sub_u16 %s, %s, %s" % (vr(r), vr(r), vr(kk[rb])), rd=vset(r) | vset(kk[rb]), wr=vset(r))
        for x in (L[rb], TS[rb], C[rb]):
            E.valu("v_ldexp_f32 %s, %s, %s" % (vr(x), vr(x), vr(negk[rb])), rd=vset(x) | vset(negk[rb]), wr=vset(x))
    rescale_o(E, negk, "v_ldexp_f32")
    E.fresh()
    E.nop(12)
    E.raw("s_branch .Lfix%d_%%=" % X)


def rare_path(E, X):
    """Full exact path for the tile in S buffer X whose K sits at LDS offset s[S_STG] (+ the ka
    operands): recompute S, take the row maximum (masked keys excluded), rescale O and l,
    recompute P and the tile sums. Entered and left with all wait states satisfied."""
    E.label(".Lfull%d_%%=" % X)
    E.fresh()
    E.nop(12)
    E.raw("s_waitcnt lgkmcnt(0)")
    E.pending = []
    ka = TMP0 + 2
    for s in range(8):
        E.valu("v_add_u32 %s, s%d, %%[ka%d]" % (vr(ka + s), S_STG, s), wr=vset(ka + s))
    for g in range(2):
        read_k(E, g, g, 0, 0, base_reg=ka)
    for f in range(16):
        kb, s = f >> 3, f & 7
        for rb in range(2):
            mfma_qk(E, X, rb, kb, s, f & 3)
        if f + 2 < 16:
            g = f + 2
            read_k(E, g & 3, g & 7, g >> 3, 0, base_reg=ka)
    tm, tm2 = (TMP0 + 10, TMP0 + 11), (TMP0 + 12, TMP0 + 13)
    tt = TMP0 + 14
    for rb in range(2):
        first = [True, True]
        for kb in range(2):
            for r in range(16):
                x = sblk(X, rb, kb) + r
                acc = (tm, tm2)[r & 1][rb]
                E.valu("v_mul_f32 %s, %%[c], %s" % (vr(tt), vr(x)), rd=vset(x), wr=vset(tt))
                E.valu("v_cmp_lt_i32 vcc, %d, %s" % (key_const(kb, r), vr(KLIM_R)), rd=vset(KLIM_R), wr=VCC)
                E.valu("v_cndmask_b32 %s, %s, %s, vcc" % (vr(tt), vr(NEG_INF), vr(tt)), rd=vset(tt) | vset(NEG_INF) | VCC, wr=vset(tt))
                if first[r & 1]:
                    E.valu("v_mov_b32 %s, %s" % (vr(acc), vr(tt)), rd=vset(tt), wr=vset(acc))
                    first[r & 1] = False
                else:
                    E.valu("v_max_f32 %s, %s, %s" % (vr(acc), vr(acc), vr(tt)), rd=vset(acc) | vset(tt), wr=vset(acc))
        E.valu("v_max_f32 %s, %s, %s" % (vr(tm[rb]), vr(tm[rb]), vr(tm2[rb])), rd=vset(tm[rb]) | vset(tm2[rb]), wr=vset(tm[rb]))
    for rb in range(2):   # the partner lane (l ^ 32) holds the other keys of each row
        E.emit(Ins("ds_bpermute_b32 %s, %%[bperm], %s" % (vr(tm2[rb]), vr(tm[rb])), "lds", rd=vset(tm[rb]), wr=vset(tm2[rb]), lds=True))
    alpha = (TMP0 + 15, TMP0 + 16)
    for rb in range(2):
        E.valu("v_max_f32 %s, %s, %s" % (vr(tm[rb]), vr(tm[rb]), vr(tm2[rb])), rd=vset(tm[rb]) | vset(tm2[rb]), wr=vset(tm[rb]))
        if OPTS["headroom"]:
            E.valu("v_add_f32 %s, 0x%08x, %s" % (vr(tm[rb]), struct.unpack("<I", struct.pack("<f", float(OPTS["headroom"])))[0],
                                                 vr(tm[rb])), rd=vset(tm[rb]), wr=vset(tm[rb]))
        E.valu("v_max_f32 %s, %s, %s" % (vr(tm[rb]), vr(tm[rb]), vr(M[rb])), rd=vset(tm[rb]) | vset(M[rb]), wr=vset(tm[rb]))
        E.valu("v_sub_f32 %s, %s, %s" % (vr(alpha[rb]), vr(M[rb]), vr(tm[rb])), rd=vset(M[rb]) | vset(tm[rb]), wr=vset(alpha[rb]))
        E.trans("v_exp_f32 %s, %s" % (vr(alpha[rb]), vr(alpha[rb])), rd=vset(alpha[rb]), wr=vset(alpha[rb]))
        E.valu("v_mov_b32 %s, %s" % (vr(M[rb]), vr(tm[rb])), rd=vset(tm[rb]), wr=vset(M[rb]))
    for rb in range(2):
        for x in (L[rb], C[rb]):
            E.valu("v_mul_f32 %s, %s, %s" % (vr(x), vr(x), vr(alpha[rb])), rd=vset(x) | vset(alpha[rb]), wr=vset(x))
    rescale_o(E, alpha)
    for f in softmax_half(X, 0, True, KLIM_EXACT, H1) + softmax_half(X, 1, True, KLIM_EXACT, H2) + \
            check_ops()[:N_TILE_SUM_OPS]:
        f(E)
    E.fresh()
    E.nop(12)
    E.raw("s_branch .Lfix%d_%%=" % X)


def slow_path(E, X):
    """The wave's slow path for the tile in S buffer X, entered when some lane's tile sum
    exceeds its limit min(l, 2^24) (or is not a number).

    A tile sum above 2^24 or not a number needs a new reference: the rebase path, or the full
    path when a probability is inf or NaN. Either way (and when the limit was l, which a tile
    holding more than half of the lane's running sum exceeds) the tile's correction follows:
    C += (sum of the tile's BF16 probabilities) - (their FP32 tile sum). O is later divided by
    l + C, the sum of the BF16 probabilities that O's products used, for the keys of these
    tiles: a key that ends with half or more of its lane's weight sits in such a tile, so the
    weights of the keys that dominate a row add up to one exactly, whatever the BF16 rounding
    of their probabilities. The LSE keeps the FP32 sum l."""
    E.label(".Lrare%d_%%=" % X)
    E.hists = [list(h) for h in E.calls[X]] or [[]]   # wait states as seen from every call
    E.raw("s_waitcnt lgkmcnt(0)")
    E.pending = []
    for rb in range(2):   # does any lane need a new reference (tile sum above 2^24, or NaN)?
        E.valu("v_cmp_nge_f32 vcc, s%d, %s" % (S_LIM, vr(TS[rb])), rd=vset(TS[rb]), wr=VCC)
        if rb == 0:
            E.salu("s_mov_b64 s[%d:%d], vcc" % (S_C1, S_C1 + 1))
    E.salu("s_or_b64 s[%d:%d], s[%d:%d], vcc" % (S_C1, S_C1 + 1, S_C1, S_C1 + 1))
    E.raw("s_cbranch_scc1 .Lmove%d_%%=" % X)
    at_move = E.state()
    E.label(".Lfix%d_%%=" % X)
    # four chains of v_dot2c_f32_bf16 (row block rb, odd/even packed register): a DOT result
    # goes straight to the next DOT of the same opcode as its accumulator, but any other
    # reader waits 3 wait states
    acc = [[TMP0 + 2, TMP0 + 4], [TMP0 + 3, TMP0 + 5]]
    for i in range(8):
        for rb in range(2):
            for half in range(2):
                a, r = acc[rb][half], packed_p(X, rb)[2 * i + half]
                if i == 0:   # the chain starts with the three-operand form and a zero accumulator
                    E.emit(Ins("v_dot2_f32_bf16 %s, %s, s%d, 0" % (vr(a), vr(r), S_ONES), "dot", rd=vset(r), wr=vset(a)))
                else:
                    E.emit(Ins("v_dot2c_f32_bf16 %s, s%d, %s" % (vr(a), S_ONES, vr(r)), "dot", rd=vset(r),
                               wr=vset(a), rdc=vset(a)))
    for rb in range(2):
        a, b = acc[rb]
        E.valu("v_add_f32 %s, %s, %s" % (vr(a), vr(a), vr(b)), rd=vset(a) | vset(b), wr=vset(a))
        E.valu("v_sub_f32 %s, %s, %s" % (vr(a), vr(a), vr(TS[rb])), rd=vset(a) | vset(TS[rb]), wr=vset(a))
        E.valu("v_add_f32 %s, %s, %s" % (vr(C[rb]), vr(C[rb]), vr(a)), rd=vset(C[rb]) | vset(a), wr=vset(C[rb]))
    # no wait owed on return: the path writes only C and its temporaries, which no MFMA reads,
    # and its DOT results are read inside it
    E.raw("s_setpc_b64 s[%d:%d]" % (S_RA, S_RA + 1))
    E.set_state(at_move)


def first_reference(E, X):
    """Reference of a range's first tile (S buffer X) taken from its scores, for ranges of two or
    more tiles, whose first tile holds no key past the sequence end: m = (row maximum of S*c) +
    headroom. The row maximum's probability is then 2^-headroom (rounding aside) and the tile
    needs no reference move, only the slow path's correction, instead of the full path that
    m = -inf would send it to. The row maximum of S*c is c * max S for c >= 0 and c * min S
    otherwise; both chains run over the lane's 32 scores per row block and the partner lane's
    (l ^ 32), and the larger product wins."""
    mx, mn = (TMP0 + 2, TMP0 + 3), (TMP0 + 4, TMP0 + 5)
    px, pn = (TMP0 + 6, TMP0 + 7), (TMP0 + 8, TMP0 + 9)
    for rb in range(2):
        regs = [sblk(X, rb, kb) + r for kb in range(2) for r in range(16)]
        for acc, op3, op2 in ((mx[rb], "v_max3_f32", "v_max_f32"), (mn[rb], "v_min3_f32", "v_min_f32")):
            E.valu("%s %s, %s, %s, %s" % (op3, vr(acc), vr(regs[0]), vr(regs[1]), vr(regs[2])),
                   rd=vset(regs[0]) | vset(regs[1]) | vset(regs[2]), wr=vset(acc))
            i = 3
            while i + 1 < len(regs):
                E.valu("%s %s, %s, %s, %s" % (op3, vr(acc), vr(acc), vr(regs[i]), vr(regs[i + 1])),
                       rd=vset(acc) | vset(regs[i]) | vset(regs[i + 1]), wr=vset(acc))
                i += 2
            if i < len(regs):
                E.valu("%s %s, %s, %s" % (op2, vr(acc), vr(acc), vr(regs[i])), rd=vset(acc) | vset(regs[i]), wr=vset(acc))
    for rb in range(2):
        for src, dst in ((mx[rb], px[rb]), (mn[rb], pn[rb])):
            E.emit(Ins("ds_bpermute_b32 %s, %%[bperm], %s" % (vr(dst), vr(src)), "lds", rd=vset(src), wr=vset(dst), lds=True))
    hr = struct.unpack("<I", struct.pack("<f", float(OPTS["headroom"])))[0]
    for rb in range(2):
        E.valu("v_max_f32 %s, %s, %s" % (vr(mx[rb]), vr(mx[rb]), vr(px[rb])), rd=vset(mx[rb]) | vset(px[rb]), wr=vset(mx[rb]))
        E.valu("v_min_f32 %s, %s, %s" % (vr(mn[rb]), vr(mn[rb]), vr(pn[rb])), rd=vset(mn[rb]) | vset(pn[rb]), wr=vset(mn[rb]))
        E.valu("v_mul_f32 %s, %%[c], %s" % (vr(mx[rb]), vr(mx[rb])), rd=vset(mx[rb]), wr=vset(mx[rb]))
        E.valu("v_mul_f32 %s, %%[c], %s" % (vr(mn[rb]), vr(mn[rb])), rd=vset(mn[rb]), wr=vset(mn[rb]))
        E.valu("v_max_f32 %s, %s, %s" % (vr(M[rb]), vr(mx[rb]), vr(mn[rb])), rd=vset(mx[rb]) | vset(mn[rb]), wr=vset(M[rb]))
        E.valu("v_add_f32 %s, 0x%08x, %s" % (vr(M[rb]), hr, vr(M[rb])), rd=vset(M[rb]), wr=vset(M[rb]))


def final_phase(E, Y, stage, uid):
    """The last tile (S buffer Y, LDS stage): masked second softmax half, check, PV."""
    for f in softmax_half(Y, 1, True, KLIM_IN, H2):
        f(E)
    prefetch_v(E, stage)
    for f in check_ops():
        f(E)
    rare_call(E, Y, stage, uid)
    add_l(E)
    pv_phase(E, Y, stage, [])
    E.raw("s_branch .Ldone_%=")


def generate(backedge=None):
    E = Emitter()
    # ---- set-up: cursors, statistics, Q (to AGPRs), O = 0, tiles 0..2
    E.raw("s_mov_b32 s%d, m0" % S_M0)
    for i in range(4):
        E.salu("s_mov_b32 s%d, %%[rk%d]" % (SK + i, i))
        E.salu("s_mov_b32 s%d, %%[rv%d]" % (SV + i, i))
    if INDEXED:
        # list cursor at entry 1; entries 1..3 (and 4) by one scalar load; entry 4 to v200
        E.salu("s_mov_b32 s%d, %%[lp0]" % S_LP)
        E.salu("s_mov_b32 s%d, %%[lp1]" % (S_LP + 1))
        E.raw("s_load_dwordx4 s[%d:%d], s[%d:%d], 0x4" % (S_I, S_I + 3, S_LP, S_LP + 1))
        E.salu("s_mov_b32 s%d, %%[i0]" % S_PREV)
        E.salu("s_mov_b32 s%d, %%[ntk]" % S_NTK)
        E.raw("s_waitcnt lgkmcnt(0)")
        E.valu("v_mov_b32 %s, 0" % vr(V_ZERO), wr=vset(V_ZERO))
        E.salu("s_add_u32 s%d, s%d, 16" % (S_LP, S_LP))
        E.salu("s_addc_u32 s%d, s%d, 0" % (S_LP + 1, S_LP + 1))
        fetch_index(E)
    E.salu("s_mov_b32 s%d, 0" % S_T)
    E.salu("s_sub_u32 s%d, %%[T], 2" % S_TLAST)
    E.salu("s_mov_b32 s%d, 0x%08x" % (S_LIM, OPTS["limit_bits"]))
    E.salu("s_mov_b32 s%d, 0x3f803f80" % S_ONES)
    for rb in range(2):
        E.valu("v_mov_b32 %s, 0xff800000" % vr(M[rb]), wr=vset(M[rb]))
        E.valu("v_mov_b32 %s, 0" % vr(L[rb]), wr=vset(L[rb]))
        E.valu("v_mov_b32 %s, 0" % vr(C[rb]), wr=vset(C[rb]))
        E.valu("v_mov_b32 %s, 0" % vr(LIM[rb]), wr=vset(LIM[rb]))
    E.valu("v_mov_b32 %s, 1000" % vr(KLIM_R), wr=vset(KLIM_R))
    E.valu("v_mov_b32 %s, 0xff800000" % vr(NEG_INF), wr=vset(NEG_INF))
    for rb in range(2):
        for s in range(8):
            E.emit(Ins("global_load_dwordx4 %s, %%[qa%d], off offset:%d" % (ar(qfrag(rb, s), 4), rb, 32 * s), "vmem",
                       wr=aset(qfrag(rb, s), 4)))
    for i in range(128):
        E.valu("v_accvgpr_write_b32 %s, 0" % ar(O_BASE + i), wr=aset(O_BASE + i))
    for u in range(3):
        for f in tile_loads(u, S_I + u if INDEXED else None):
            f(E)
    E.raw("s_waitcnt vmcnt(0)")
    E.raw("s_barrier")
    prefetch_k(E, 0)
    qk_phase(E, 0, 0, [])
    E.raw("s_cmp_eq_u32 %[T], 1")
    E.raw("s_cbranch_scc1 .LT1_%=")
    first_reference(E, 0)
    for f in softmax_half(0, 0, False, None, H1):
        f(E)
    prefetch_k(E, 1)

    # ---- loop: four tiles per trip; leaves after the QK phase of tile T-2
    if backedge is not None:
        E.hists = E.hists + [list(h) for h in backedge]
    E.label(".Lloop_%=")
    tail_state = {}
    for k in range(4):
        X, Y = k % 2, (k + 1) % 2
        qk_phase(E, Y, (k + 1) % 4, softmax_half(X, 1, False, None, H2) + check_ops(), valu_slots=OPTS["qk_valu_slots"],
                 extra={OPTS["vpre_after"]: [lambda E, st=k: prefetch_v(E, st)]})
        rare_call(E, X, k, "A%d" % k)
        add_l(E)
        E.salu("s_cmp_eq_u32 s%d, s%d" % (S_T, S_TLAST))
        E.raw("s_cbranch_scc1 .Ltail%d_%%=" % k)
        tail_state[k] = E.state()
        bar = OPTS["barrier_after"]
        extra = {bar: [lambda E: E.raw("s_waitcnt vmcnt(0)"), lambda E: E.raw("s_barrier")]}
        for i, f in enumerate(tile_loads((k + 3) % 4)):
            extra.setdefault(bar + 1 + i, []).append(f)
        assert OPTS["kpre_after"] > bar, "K of the next tile is visible only after the barrier"
        extra.setdefault(OPTS["kpre_after"], []).append(lambda E, st=(k + 2) % 4: prefetch_k(E, st))
        pv_phase(E, X, k, softmax_half(Y, 0, False, None, H1), valu_slots=OPTS["pv_valu_slots"], extra=extra)
        E.salu("s_add_u32 s%d, s%d, 1" % (S_T, S_T))
    loop_end = [list(h) for h in E.hists]
    E.raw("s_branch .Lloop_%=")

    # ---- tails: PV of tile T-2 beside the masked first half of tile T-1, then tile T-1
    for k in range(4):
        X, Y = k % 2, (k + 1) % 2
        E.label(".Ltail%d_%%=" % k)
        E.set_state(tail_state[k])
        E.valu("v_mov_b32 %s, %%[klim]" % vr(KLIM_R), wr=vset(KLIM_R))
        pv_phase(E, X, k, softmax_half(Y, 0, True, KLIM_IN, H1))
        final_phase(E, Y, (k + 1) % 4, "F%d" % k)

    # ---- a range of one tile
    E.label(".LT1_%=")
    E.fresh()
    E.nop(12)
    E.valu("v_mov_b32 %s, %%[klim]" % vr(KLIM_R), wr=vset(KLIM_R))
    for f in softmax_half(0, 0, True, KLIM_IN, H1):
        f(E)
    final_phase(E, 0, 0, "S")

    for X in range(2):
        slow_path(E, X)
        rebase_path(E, X)
        rare_path(E, X)

    E.label(".Ldone_%=")
    E.fresh()
    E.nop(12)
    E.raw("s_waitcnt vmcnt(0) lgkmcnt(0)")
    E.raw("s_mov_b32 m0, s%d" % S_M0)
    for i in range(128):
        E.raw("v_accvgpr_read_b32 v%d, a%d" % (i, O_BASE + i))
    for rb in range(2):
        E.raw("v_mov_b32 %%[m%d], %s" % (rb, vr(M[rb])))
        E.raw("v_mov_b32 %%[l%d], %s" % (rb, vr(L[rb])))
        E.raw("v_mov_b32 %%[c%d], %s" % (rb, vr(C[rb])))
    return E.out, loop_end


def render(indexed=False):
    global INDEXED
    INDEXED = indexed
    try:
        return _render()
    finally:
        INDEXED = False


def _render():
    nv, ns_hi = (V_ZERO + 1, S_NTK) if INDEXED else (NV, NS_HI)
    lines, back = generate()
    for _ in range(4):   # the loop head is reached from the set-up and from the loop end
        lines2, back2 = generate(back)
        if lines2 == lines:
            break
        lines, back = lines2, back2
    else:
        raise SystemExit("wait-state pass did not converge")
    clob = ['"v%d"' % i for i in range(128, nv)] + ['"a%d"' % i for i in range(NA)] + \
           ['"s%d"' % i for i in range(NS_LO, ns_hi + 1)] + ['"vcc"', '"scc"', '"memory"']
    outs = ['[o%d%d] "=&{v[%d:%d]}"(o[%d][%d])' % (db, rb, oblk(db, rb), oblk(db, rb) + 15, db, rb)
            for db in range(4) for rb in range(2)]
    outs += ['[m0] "=v"(mref[0])', '[m1] "=v"(mref[1])', '[l0] "=v"(lsum[0])', '[l1] "=v"(lsum[1])',
             '[c0] "=v"(lcor[0])', '[c1] "=v"(lcor[1])']
    ins = ['[rk%d] "s"(rk[%d])' % (i, i) for i in range(4)] + ['[rv%d] "s"(rv[%d])' % (i, i) for i in range(4)]
    ins += ['[ka%d] "v"(ka[%d])' % (i, i) for i in range(8)] + ['[va%d] "v"(va[%d])' % (i, i) for i in range(8)]
    ins += ['[ko%d] "v"(ko[%d])' % (i, i) for i in range(4)] + ['[vo%d] "v"(vo[%d])' % (i, i) for i in range(4)]
    ins += ['[qa0] "v"(qa[0])', '[qa1] "v"(qa[1])', '[ldsw] "s"(ldsw)', '[tb] "s"(tb)', '[T] "s"(ntile)',
            '[c] "s"(c)', '[klim] "v"(klim)', '[bperm] "v"(bperm)']
    if INDEXED:
        ins += ['[lp0] "s"(lp[0])', '[lp1] "s"(lp[1])', '[i0] "s"(idx0)', '[ntk] "s"(ntk)']
    n_ins = sum(1 for l in lines if l.startswith("\t"))
    n_nop = sum(1 for l in lines if l.strip().startswith("s_nop"))
    what = ", over a list of key tiles" if INDEXED else ""
    text = ["// Written by gen_key_loop.py (do not edit): the key loop of attn_rows() for gfx950%s." % what,
            "// %d instructions, %d of them s_nop." % (n_ins, n_nop),
            "asm volatile("]
    text += ['        "%s\\n"' % l.replace("\\", "\\\\").replace('"', '\\"') for l in lines]
    text.append("        : " + ",\n          ".join(outs))
    text.append("        : " + ",\n          ".join(ins))
    text.append("        : " + ", ".join(clob) + ");")
    return "\n".join(text) + "\n"


OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "key_loop_gfx950.inc")
OUT_IDX = os.path.join(os.path.dirname(os.path.abspath(__file__)), "key_loop_idx_gfx950.inc")

if __name__ == "__main__":
    # gen_key_loop.py: both files; gen_key_loop.py out.inc [knob=value ...]: the range
    # variant with schedule knobs changed (indexed=1 for the list variant)
    if len(sys.argv) == 1:
        for path, idx in ((OUT, False), (OUT_IDX, True)):
            with open(path, "w") as f:
                f.write(render(idx))
        sys.exit(0)
    indexed = False
    for kv in sys.argv[2:]:
        k, v = kv.split("=")
        if k == "indexed":
            indexed = bool(int(v))
            continue
        assert k in OPTS, k
        OPTS[k] = int(v, 0)
    with open(sys.argv[1], "w") as f:
        f.write(render(indexed))
