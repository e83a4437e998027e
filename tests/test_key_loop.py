"""CPU checks of the hand-scheduled key loop (csrc/key_loop_gfx950.inc, and its tile-list
variant csrc/key_loop_idx_gfx950.inc for block-skip attention).

The loop is written by csrc/gen_key_loop.py, which inserts the s_waitcnt and s_nop the
hardware needs. These tests re-derive those requirements with a separate, simpler scan of the
emitted text, so a mistake in the generator's bookkeeping shows up here:
  * the committed file is exactly what the generator writes;
  * every LDS read has landed (lgkmcnt) before an instruction touches its registers;
  * the MFMA wait states (result read by non-MFMA code, VALU write before an MFMA read) hold
    along the straight-line code;
  * only the registers the asm declares are written, and the control flow (labels, branches,
    barriers) is consistent.
"""
import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "video_diffusion_dit_amd", "csrc")


def load_gen():
    spec = importlib.util.spec_from_file_location("gen_key_loop", os.path.join(CSRC, "gen_key_loop.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    return gen


@pytest.fixture(scope="module")
def gen():
    return load_gen()


FILES = {"range": "key_loop_gfx950.inc", "list": "key_loop_idx_gfx950.inc"}


def read_asm(name):
    text = open(os.path.join(CSRC, name)).read()
    out = []
    for line in text.splitlines():
        m = re.match(r'\s*"(.*)\\n"\s*$', line)
        if m:
            out.append(m.group(1).replace("\\t", "\t").strip())
    return out


@pytest.fixture(scope="module", params=sorted(FILES))
def asm_lines(request):
    return read_asm(FILES[request.param])


def test_committed_files_are_generated(gen):
    assert open(gen.OUT).read() == gen.render()
    assert open(gen.OUT_IDX).read() == gen.render(True)


def regs(tok):
    tok = tok.strip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def parse(line):
    op, _, rest = line.partition(" ")
    ops = [t.strip() for t in rest.split(",")] if rest else []
    return op, ops


def ws_of(op, ops):
    return int(ops[0]) + 1 if op == "s_nop" else 1


def is_block_end(op):
    """An instruction after which straight-line code does not continue (a conditional branch
    falls through, so the scans go on past it)."""
    return op.startswith("s_branch") or op == "s_setpc_b64"


def lds_violations(asm_lines):
    """Simulate lgkmcnt in program order (a path that reaches a label with more reads in
    flight only waits longer, since LDS ops complete in order)."""
    pending = []   # register sets of LDS ops in flight, oldest first
    bad = []
    for line in asm_lines:
        if line.endswith(":"):
            continue
        op, ops = parse(line)
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", line)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if n else []
            continue
        touched = set()
        for t in ops:
            touched |= regs(t)
        if any(p & touched for p in pending):
            bad.append(line)
        if op.startswith("ds_read") or op.startswith("ds_bpermute"):
            pending.append(regs(ops[0]))
    return bad


def mfma_violations(asm_lines):
    """Straight-line check of the wait-state rules that protect MFMA data."""
    ins = []
    for line in asm_lines:
        if line.endswith(":"):
            ins.append(("<label>", []))
            continue
        ins.append(parse(line))
    bad = []
    for k, (op, ops) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        dst = regs(ops[0])
        srcs = regs(ops[1]) | regs(ops[2]) | regs(ops[3])
        # (1) a VALU write of any source fewer than 2 wait states before
        ws = 0
        for j in range(k - 1, max(k - 6, -1), -1):
            qop, qops = ins[j]
            if qop == "<label>" or is_block_end(qop):
                break
            if qop.startswith("v_") and not qop.startswith("v_mfma") and qops and regs(qops[0]) & srcs and ws < 2:
                bad.append(("valu->mfma", k, op))
            ws += ws_of(qop, qops)
            if ws >= 2:
                break
        # (2) a non-MFMA access of the result fewer than 12 wait states after
        ws = 0
        for j in range(k + 1, min(k + 30, len(ins))):
            qop, qops = ins[j]
            if qop == "<label>" or is_block_end(qop):
                break
            if qop.startswith("v_mfma"):
                if (regs(qops[1]) | regs(qops[2])) & dst and ws < 12:
                    bad.append(("mfma->mfma A/B", k, qop))
                ws += 1
                continue
            touched = set()
            for t in qops:
                touched |= regs(t)
            if touched & dst and ws < 12:
                bad.append(("mfma->access", k, qop))
            ws += ws_of(qop, qops)
            if ws >= 12:
                break
    return bad


def dot_violations(asm_lines):
    """A DOT result (v_dot2_f32_bf16, v_dot2c_f32_bf16) read fewer than 3 wait states later by
    anything but a DOT of the same opcode that takes it as its accumulator, along the
    straight-line code."""
    ins = [("<label>", []) if l.endswith(":") else parse(l) for l in asm_lines]
    bad = []
    for k, (op, ops) in enumerate(ins):
        if not op.startswith("v_dot2"):
            continue
        dst = regs(ops[0])
        ws = 0
        for j in range(k + 1, min(k + 8, len(ins))):
            qop, qops = ins[j]
            if qop == "<label>" or is_block_end(qop):
                break
            if qop.startswith("v_dot2c"):
                srcs = regs(qops[1]) | regs(qops[2])      # multiplicands; the accumulator is the dst
                if qop != op:                             # another DOT opcode: its accumulator read counts
                    srcs |= regs(qops[0])
            else:
                srcs = set()
                for t in qops[1:]:
                    srcs |= regs(t)
            if srcs & dst and ws < 3:
                bad.append(("dot->read", k, qop))
            ws += ws_of(qop, qops)
            if ws >= 3:
                break
    return bad


def test_dot_wait_states(asm_lines):
    assert dot_violations(asm_lines) == []
    # not vacuous: a read right after a DOT is reported
    k = next(i for i, l in enumerate(asm_lines) if l.startswith("v_dot2c_f32_bf16"))
    dst = parse(asm_lines[k])[1][0]
    assert dot_violations(asm_lines[:k + 1] + ["v_add_f32 v199, %s, %s" % (dst, dst)] + asm_lines[k + 1:])
    # and a chain that switches DOT opcode on its accumulator right away
    k = next(i for i, l in enumerate(asm_lines) if l.startswith("v_dot2_f32_bf16"))
    dst = parse(asm_lines[k])[1][0]
    assert dot_violations(asm_lines[:k + 1] + ["v_dot2c_f32_bf16 %s, s53, v0" % dst] + asm_lines[k + 1:])


def test_lds_results_waited(asm_lines):
    assert lds_violations(asm_lines) == []


def test_mfma_wait_states(asm_lines):
    assert mfma_violations(asm_lines) == []


def test_scans_catch_a_missing_wait(asm_lines):
    """The scans are not vacuous: a dropped LDS wait, an MFMA result read at once and a
    VALU write just before an MFMA reads it are all reported."""
    i = next(k for k, l in enumerate(asm_lines) if l.startswith("s_waitcnt lgkmcnt(1)"))
    assert lds_violations(asm_lines[:i] + asm_lines[i + 1:])
    j = next(k for k, l in enumerate(asm_lines) if l.startswith("v_mfma_f32_32x32x16_bf16 v[0:15]"))
    assert mfma_violations(asm_lines[:j + 1] + ["v_add_f32 v0, v0, v0"] + asm_lines[j + 1:])
    assert mfma_violations(asm_lines[:j] + ["v_mov_b32 v130, 0"] + asm_lines[j:])


def test_control_flow_and_registers(gen, asm_lines):
    labels = {l[:-1] for l in asm_lines if l.endswith(":")}
    for line in asm_lines:
        m = re.match(r"s_(c)?branch\w*\s+(\S+)", line)
        if m:
            assert m.group(2) in labels, line
    # one barrier in the set-up and one per tile of the four-tile loop body; none elsewhere
    assert sum(1 for l in asm_lines if l == "s_barrier") == 5
    # registers named stay inside what the asm statement declares (v0..v199, a0..a191; the
    # tile-list variant also v200, v201)
    nv = gen.V_ZERO + 1 if any(l.startswith("global_load_dword v200") for l in asm_lines) else gen.NV
    for line in asm_lines:
        _, ops = parse(line)
        for t in ops:
            for kind, i in regs(t):
                assert (kind == "v" and i < nv) or (kind == "a" and i < gen.NA), line
    # every return address points at a label that follows its call
    calls = [l for l in asm_lines if l.startswith("s_add_u32 s54")]
    assert len(calls) == 9 and all(re.search(r"\.Lok\w+_%=-\.Lpc\w+_%=", c) for c in calls)


def test_loop_schedule_shape(gen):
    """Per tile of the loop: 64 MFMAs, 64 exps per lane, one barrier, eight buffer->LDS loads."""
    lines, _ = gen.generate()
    start = lines.index(".Lloop_%=:")
    end = next(i for i in range(start, len(lines)) if lines[i].strip() == "s_branch .Lloop_%=")
    body = [l.strip() for l in lines[start:end]]
    assert sum(l.startswith("v_mfma") for l in body) == 4 * 64
    assert sum(l.startswith("v_exp_f32") for l in body) == 4 * 64
    assert sum(l == "s_barrier" for l in body) == 4
    assert sum(l.startswith("buffer_load_dwordx4") for l in body) == 4 * 8
    nops = sum(int(l.split()[1]) + 1 for l in body if l.startswith("s_nop"))
    assert nops < 64, nops   # the schedule keeps hazards apart by itself


def test_tile_list_index_flow(gen):
    """Tile-list variant: every index read (v_readfirstlane of v200) follows an s_waitcnt
    vmcnt(0) issued after the load that wrote v200; the set-up's scalar list load is waited
    for before its registers are read; every index is clamped to [current, ntk] before the
    cursors move by it; per loop tile exactly one index read and one index load."""
    lines = read_asm(FILES["list"])
    loaded = False
    smem = False
    for line in lines:
        if line.startswith("global_load_dword v200"):
            loaded = True
        if line.startswith("s_waitcnt") and "vmcnt(0)" in line:
            loaded = False
        if line.startswith("v_readfirstlane_b32 s69, v200"):
            assert not loaded, "index read before its load completed"
        if line.startswith("s_load_dwordx4 s[64:67]"):
            smem = True
        if line.startswith("s_waitcnt") and "lgkmcnt(0)" in line:
            smem = False
        if smem:
            _, ops = parse(line)
            assert not any(re.fullmatch(r"s6[4-7]", o) for o in ops), line
    # the byte step is computed from a clamped index: s_max, s_min, s_sub, s_mul in a row
    for i, line in enumerate(lines):
        if line.startswith("s_sub_i32 s70"):
            nxt = parse(line)[1][1]
            assert lines[i - 2] == "s_max_i32 %s, %s, s68" % (nxt, nxt), lines[i - 2]
            assert lines[i - 1] == "s_min_i32 %s, %s, s71" % (nxt, nxt), lines[i - 1]
            assert lines[i + 1] == "s_mul_i32 s70, s70, %[tb]" and lines[i + 2] == "s_mov_b32 s68, %s" % nxt
    start = lines.index(".Lloop_%=:")
    end = lines.index("s_branch .Lloop_%=")
    body = lines[start:end]
    assert sum(l.startswith("v_readfirstlane_b32 s69, v200") for l in body) == 4
    assert sum(l.startswith("global_load_dword v200") for l in body) == 4
    assert sum(l.startswith("s_sub_i32 s70") for l in lines) == 3 + 4   # set-up tiles 1..3, loop tiles
    # cursor moves use the clamped step only
    assert not any("%[tb]" in l and l.startswith(("s_add_u32 s40", "s_add_u32 s44")) for l in lines)


def test_tile_list_variant_differs_only_in_tile_movement():
    """Apart from the index bookkeeping, the two loops hold the same instructions (the extra
    index read shifts where the loads fall between MFMAs) with the MFMAs in the same order."""
    rng, lst = read_asm(FILES["range"]), read_asm(FILES["list"])
    book = re.compile(r"^(s_max_i32 s6[4-9]|s_min_i32 s6[4-9]|s_sub_i32 s70|s_mul_i32 s70|s_mov_b32 s6[2389]|"
                      r"s_mov_b32 s71|s_load_dwordx4|s_add_u32 s62|s_addc_u32 s63|global_load_dword v200|"
                      r"v_readfirstlane_b32 s69|v_mov_b32 v201|s_waitcnt lgkmcnt\(0\)$|s_nop)")
    norm = lambda xs: [re.sub(r"s70|%\[tb\]", "STEP", l) for l in xs if not book.match(l)]
    a = [l for l in norm(rng) if not l.startswith("s_waitcnt lgkmcnt(0)")]
    b = [l for l in norm(lst) if not l.startswith("s_waitcnt lgkmcnt(0)")]
    assert sorted(a) == sorted(b)
    assert [l for l in a if l.startswith("v_mfma")] == [l for l in b if l.startswith("v_mfma")]
    labels = lambda xs: [l for l in xs if l.endswith(":") or l.startswith(("s_branch", "s_cbranch", "s_barrier"))]
    assert labels(a) == labels(b)


# ---- the fast exact path (rebase): new reference from the packed BF16 probabilities

def bf16_value(bits):
    import numpy as np
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_rebase_arithmetic_is_an_exact_power_of_two_shift(gen):
    """The rebase path's integer steps, emulated exactly: k = max(e + 1 + headroom, 0) from the
    u16 maximum of the BF16 patterns, then each BF16 p becomes max(p, k<<7) - (k<<7) (u16).
    For every finite non-negative BF16 value and every k the kernel can form, that is exactly
    p * 2^-k when the result is a normal number, and below 2^-126 otherwise (weights under
    2^-126 of the new reference); the largest probability ends in [2^-(h+1), 2^-h)."""
    import numpy as np
    p = np.arange(0, 0x7F80, dtype=np.uint32)              # every finite non-negative BF16 pattern
    exact = bf16_value(p)
    for k in range(0, 127 + 1 + gen.OPTS["headroom"] + 1):
        kk = k << 7
        got = bf16_value(np.maximum(p, kk) - kk)
        want = exact * 2.0 ** -k
        normal = want >= 2.0 ** -126
        assert np.array_equal(got[normal], want[normal]), k
        assert np.all(got[~normal] < 2.0 ** -126) and np.all(got >= 0), k
    h = gen.OPTS["headroom"]
    bias = 126 - h
    for mx in range(0, 0x7F80):
        k = max((mx >> 7) - bias, 0)
        top = bf16_value(mx) * 2.0 ** -k
        if k > 0:
            assert 2.0 ** -(h + 1) <= top < 2.0 ** -h, mx
        else:   # the row already sits below 2^-h: its reference stays
            assert top < 2.0 ** -h, mx


def test_rebase_path_leaves_the_state_alone_until_it_commits(gen, asm_lines):
    """Each rebase path reads the packed probabilities and may still hand the tile to the full
    path (an inf/NaN maximum): up to that branch it writes only its temporaries, never m, l,
    the correction, the tile sums, P or O, so the full path starts from the state the check
    saw."""
    owned = {("v", r) for r in range(gen.TMP0, gen.TMP0 + 24)}
    for X in range(2):
        start = asm_lines.index(".Lmove%d_%%=:" % X)
        branch = next(i for i in range(start, len(asm_lines))
                      if asm_lines[i].startswith("s_cbranch_scc1 .Lfull%d_" % X))
        assert asm_lines[branch + 1:].index(".Lfull%d_%%=:" % X) > 0
        for line in asm_lines[start + 1:branch]:
            op, ops = parse(line)
            if op.startswith("s_") or not ops:
                continue
            dst = regs(ops[0])
            assert dst <= owned or op.startswith("v_cmp"), line
        # after the branch the path moves m, l, the correction, the tile sums, every packed P
        # register and O, then goes on to the tile's correction
        tail = asm_lines[branch:asm_lines.index(".Lfull%d_%%=:" % X)]
        written = set()
        for line in tail:
            op, ops = parse(line)
            if ops and not op.startswith("s_"):
                written |= regs(ops[0])
        for rb in range(2):
            assert {("v", gen.M[rb]), ("v", gen.L[rb]), ("v", gen.TS[rb]), ("v", gen.C[rb])} <= written
            assert {("v", r) for r in gen.packed_p(X, rb)} <= written
        assert {("a", i) for i in range(128)} <= written
        assert tail[-1] == "s_branch .Lfix%d_%%=" % X


def test_slow_path_entry_and_correction(gen, asm_lines):
    """The slow-path entry only tests whether a new reference is needed (a tile sum above 2^24
    or not a number) before it branches to the rebase; the correction that every slow path
    ends in reads the packed probabilities of its own S buffer and the tile sums, writes only
    its four temporaries and C, and returns; the rebase and the full path both end in it."""
    owned = {("v", gen.TMP0 + i) for i in range(2, 6)} | {("v", c) for c in gen.C}
    for X in range(2):
        start = asm_lines.index(".Lrare%d_%%=:" % X)
        fix = asm_lines.index(".Lfix%d_%%=:" % X)
        entry = asm_lines[start + 1:fix]
        assert entry[-1] == "s_cbranch_scc1 .Lmove%d_%%=" % X
        assert [l for l in entry if l.startswith("v_")] == ["v_cmp_nge_f32 vcc, s%d, v%d" % (gen.S_LIM, t)
                                                            for t in gen.TS]
        end = next(i for i in range(fix, len(asm_lines)) if asm_lines[i].startswith("s_setpc_b64"))
        body = asm_lines[fix + 1:end]
        read, written = set(), set()
        for line in body:
            op, ops = parse(line)
            if op.startswith("s_") or not ops:
                continue
            written |= regs(ops[0])
            for t in ops[1:]:
                read |= regs(t)
        assert written <= owned, written - owned
        packed = {("v", r) for rb in range(2) for r in gen.packed_p(X, rb)}
        assert packed <= read and read <= packed | owned | {("v", t) for t in gen.TS}
        assert sum(l.startswith(("v_dot2_f32_bf16", "v_dot2c_f32_bf16")) for l in body) == 32
        assert all("s%d" % gen.S_ONES in l for l in body if l.startswith("v_dot2"))
        assert sum(l == "s_branch .Lfix%d_%%=" % X for l in asm_lines) == 2
    assert any(l == "s_mov_b32 s%d, 0x3f803f80" % gen.S_ONES for l in asm_lines)


def test_check_limit_follows_l(gen, asm_lines):
    """The check compares each tile sum with the lane's own limit, which is set to
    min(l, 2^24) right after every update of l."""
    for i, line in enumerate(asm_lines):
        if line.startswith("v_add_f32 v%d, v%d, v%d" % (gen.L[0], gen.L[0], gen.TS[0])):
            nxt = asm_lines[i + 1:i + 4]
            for rb in range(2):
                assert "v_min_f32 v%d, s%d, v%d" % (gen.LIM[rb], gen.S_LIM, gen.L[rb]) in nxt, nxt
    cmps = [l for l in asm_lines if l.startswith("v_cmp_nge_f32_e64")]
    assert cmps and all(re.match(r"v_cmp_nge_f32_e64 s\[\d+:\d+\], v(170|171), v(174|175)$", l) for l in cmps), cmps[:2]


def test_slow_path_wait_states_from_every_call(asm_lines):
    """The slow path starts without s_nop of its own: the generator counts the wait states owed
    by the code before each of its calls. Re-check that here: the straight-line code before every
    call, followed by the entry and the correction (and by the entry and the rebase's opening),
    passes the MFMA and DOT scans."""
    def body(start_label, stop):
        i = asm_lines.index(start_label) + 1
        out = []
        while not stop(asm_lines[i]):
            if not asm_lines[i].endswith(":"):
                out.append(asm_lines[i])
            i += 1
        return out
    checked = 0
    for X in range(2):
        entry = body(".Lrare%d_%%=:" % X, lambda l: l.startswith("s_cbranch_scc1 .Lmove"))
        fix = body(".Lfix%d_%%=:" % X, lambda l: l.startswith("s_setpc_b64"))
        move = body(".Lmove%d_%%=:" % X, lambda l: l.startswith("s_cbranch"))
        calls = [i for i, l in enumerate(asm_lines) if l == "s_branch .Lrare%d_%%=" % X]
        assert calls
        for i in calls:
            pre = [l for l in asm_lines[max(0, i - 80):i] if not l.endswith(":") and not is_block_end(l.split()[0])]
            for tail in (fix, move):
                seq = pre + entry + tail
                assert mfma_violations(seq) == [] and dot_violations(seq) == [], (X, i)
            # not vacuous: reading the result of the call site's last MFMA at the entry is flagged
            recent = [l for l in pre[-8:] if l.startswith("v_mfma")]
            if recent:   # calls right after a QK phase (not those after the last tile's check)
                res = parse(recent[-1])[1][0].split(":")[0].replace("[", "")
                assert mfma_violations(pre + ["v_add_f32 v199, %s, %s" % (res, res)] + entry + fix)
                checked += 1
    assert checked >= 4   # the four calls of the loop body
