"""Host check of the fp8-activation 256-row kernel's LDS pipelines (no GPU).

`mx_tile` in gemm_mx.hip copies each stage of a tile straight from global memory
into a ring of LDS slots several stages ahead, with `global_load_lds` copies whose
completion the loop counts itself (`s_waitcnt vmcnt(n)` before each barrier,
copies completing in issue order per wave), and with K a multiple of 512 it copies
the block scales in 16-byte groups into a separate two-buffer ring. The copy
placement (which rows and chunks land where), the copy counts per body, the wait
counts and the slot and buffer reuse are restated here in plain Python and run
over tile heights (JV = 1..4 32-row blocks per row-wave) and stage counts: every
fragment and scale read must see exactly the row, stage and chunk it expects, both
when copies land only at the waits and when they land as soon as they are issued.
The GPU tests check the kernel itself (bit-exact FC2 on exact operands for every
tile height, with and without scale groups).
"""
import pytest

LDS_BYTES = 160 * 1024


def _run_mxfp4(JV, ktiles, SG, eager):
    XROWS = 64 * JV
    XC = XROWS // 32
    NC = XC + (4 if SG else 6)
    NC2 = NC // 2
    NSLOT = 4 if JV <= 2 else 3
    XT_B, WT_B = XROWS * 128, 256 * 64
    STAGE_B = XT_B + WT_B + (0 if SG else 2048)
    SG_B = NSLOT * STAGE_B
    assert SG_B + (16384 if SG else 0) <= LDS_BYTES
    NWAIT = (NSLOT - 2) * NC
    lds, inflight, errs = {}, [[] for _ in range(4)], []

    def issue(w, ops):
        if eager:
            lds.update(ops)
        else:
            inflight[w].append(ops)

    def cp(w, c, q, d):
        ops = {}
        for lane in range(64):
            if c < XC:
                row = 32 * c + 8 * w + lane // 8
                ops[d + c * 4096 + 1024 * w + 16 * lane] = ("x", row, q, (lane & 7) ^ ((4 * w + (lane >> 4)) & 7))
            elif c < XC + 4:
                row = 64 * (c - XC) + 16 * w + lane // 4
                ops[d + XT_B + (c - XC) * 4096 + 1024 * w + 16 * lane] = ("w", row, q, (lane & 3) ^ ((lane >> 4) & 3))
            elif c == XC + 4:
                ops[d + XT_B + WT_B + 256 * w + 4 * lane] = ("xs", (64 * w + lane) % XROWS, q)
            else:
                ops[d + XT_B + WT_B + 1024 + 256 * w + 4 * lane] = ("ws", 64 * w + lane, q)
        issue(w, ops)

    def cp_group(w, q):
        gb = SG_B + ((q >> 2) & 1) * 8192 + w * 1024
        issue(w, {gb + 16 * lane + 4 * ph: ("xs", (64 * w + lane) % XROWS, q + ph)
                  for lane in range(64) for ph in range(4)})
        issue(w, {gb + 4096 + 16 * lane + 4 * ph: ("ws", 64 * w + lane, q + ph)
                  for lane in range(64) for ph in range(4)})

    def wait(w, n):
        while len(inflight[w]) > n:
            lds.update(inflight[w].pop(0))

    def check(addr, exp):
        if lds.get(addr) != exp:
            errs.append((addr, lds.get(addr), exp))

    def reads(w, slot, st):
        wn, wm, base = w & 1, w >> 1, slot * STAGE_B
        for lane in range(64):
            rsel, g = lane & 31, lane >> 5
            for i in range(4):
                r = wn * 128 + i * 32 + rsel
                if SG:
                    check(SG_B + ((st >> 2) & 1) * 8192 + 4096 + 4 * (r * 4 + (st & 3)), ("ws", r, st))
                else:
                    check(base + XT_B + WT_B + 1024 + 4 * r, ("ws", r, st))
            for j in range(JV):
                r = (2 * j + wm) * 32 + rsel
                if SG:
                    check(SG_B + ((st >> 2) & 1) * 8192 + 4 * (r * 4 + (st & 3)), ("xs", r, st))
                else:
                    check(base + XT_B + WT_B + 4 * r, ("xs", r, st))
            for kk in (0, 1):
                for i in range(4):
                    r = wn * 128 + i * 32 + rsel
                    ch = 2 * kk + g
                    check(base + XT_B + 16 * (r * 4 + (ch ^ ((r >> 2) & 3))), ("w", r, st, ch))
                for j in range(JV):
                    r = (2 * j + wm) * 32 + rsel
                    for ch in (4 * kk + g, 4 * kk + 2 + g):
                        check(base + 16 * (r * 8 + (ch ^ ((r >> 1) & 7))), ("x", r, st, ch))

    def copies(w, q, d, qraw):
        n0 = len(inflight[w])
        if SG and (qraw & 3) == 0 and qraw < ktiles:
            cp_group(w, q)
        for c0 in (0, NC2):   # the two steps' reads each carry NC2 copies
            for i in range(4):
                if i < NC2:
                    cp(w, c0 + i, q, d)
            for j in range(JV):
                if j < NC2 - 4:
                    cp(w, c0 + 4 + j, q, d)
        if not eager:
            assert len(inflight[w]) - n0 in (NC, NC + 2)

    for w in range(4):
        for q in range(NSLOT - 1):
            if SG and (q & 3) == 0 and q < ktiles:
                cp_group(w, q)
            for c in range(NC):
                cp(w, c, min(q, ktiles - 1), q * STAGE_B)
    for w in range(4):
        wait(w, NWAIT)
    for st in range(ktiles):
        slot, qraw = st % NSLOT, st + NSLOT - 1
        q, d = min(qraw, ktiles - 1), (qraw % NSLOT) * STAGE_B
        for w in range(4):   # a body's reads precede later bodies' copies (barrier)
            reads(w, slot, st)
            if eager:
                copies(w, q, d, qraw)
        if not eager:
            for w in range(4):
                copies(w, q, d, qraw)
        for w in range(4):
            wait(w, NWAIT)
    return errs


def _run_mx8(JV, nsub, BS, SG, eager):
    XROWS, XC8 = 64 * JV, JV
    XCODE_B, WCODE_B = XROWS * 64, 16384
    SLOT_B = (JV * 256 + 1024 + (128 if (BS and not SG) else 0)) * 16
    SG_B = 4 * SLOT_B
    assert SG_B + (16384 if SG else 0) <= LDS_BYTES
    NWAIT = 2 * (XC8 + 4) + (2 if (BS and not SG) else 0)
    lds, inflight, errs = {}, [[] for _ in range(4)], []

    def issue(w, ops):
        if eager:
            lds.update(ops)
        else:
            inflight[w].append(ops)

    def cp(w, c, q, d):
        ops = {}
        for lane in range(64):
            ch = (lane & 3) ^ ((lane >> 4) & 3)
            if c < XC8:
                ops[d + c * 4096 + 1024 * w + 16 * lane] = ("x", 64 * c + 16 * w + lane // 4, q, ch)
            elif c < XC8 + 4:
                ops[d + XCODE_B + (c - XC8) * 4096 + 1024 * w + 16 * lane] = ("w", 64 * (c - XC8) + 16 * w + lane // 4, q, ch)
            elif c == XC8 + 4:
                ops[d + XCODE_B + WCODE_B + 256 * w + 4 * lane] = ("xs", (64 * w + lane) % XROWS, q >> 1)
            else:
                ops[d + XCODE_B + WCODE_B + 1024 + 256 * w + 4 * lane] = ("ws", 64 * w + lane, q >> 1)
        issue(w, ops)

    def cp_group(w, q):
        gb = SG_B + ((q >> 3) & 1) * 8192 + w * 1024
        issue(w, {gb + 16 * lane + 4 * ph: ("xs", (64 * w + lane) % XROWS, (q >> 1) + ph)
                  for lane in range(64) for ph in range(4)})
        issue(w, {gb + 4096 + 16 * lane + 4 * ph: ("ws", 64 * w + lane, (q >> 1) + ph)
                  for lane in range(64) for ph in range(4)})

    def wait(w, n):
        while len(inflight[w]) > n:
            lds.update(inflight[w].pop(0))

    def check(addr, exp):
        if lds.get(addr) != exp:
            errs.append((addr, lds.get(addr), exp))

    def reads(w, slot, st):
        wn, wm = w & 1, w >> 1
        X = slot * SLOT_B
        W = X + XROWS * 64
        for lane in range(64):
            rsel, g = lane & 31, lane >> 5
            if BS and (st & 1) == 0:   # the odd stage reuses the even one's words
                for i in range(4):
                    r = wn * 128 + i * 32 + rsel
                    if SG:
                        check(SG_B + ((st >> 3) & 1) * 8192 + 4096 + 4 * (r * 4 + ((st >> 1) & 3)), ("ws", r, st >> 1))
                    else:
                        check(W + 16384 + 1024 + 4 * r, ("ws", r, st >> 1))
                for j in range(JV):
                    r = (2 * j + wm) * 32 + rsel
                    if SG:
                        check(SG_B + ((st >> 3) & 1) * 8192 + 4 * (r * 4 + ((st >> 1) & 3)), ("xs", r, st >> 1))
                    else:
                        check(W + 16384 + 4 * r, ("xs", r, st >> 1))
            for i in range(4):
                r = wn * 128 + i * 32 + rsel
                for ch in (g, 2 + g):
                    check(W + 16 * (r * 4 + (ch ^ ((r >> 2) & 3))), ("w", r, st, ch))
            for j in range(JV):
                r = (2 * j + wm) * 32 + rsel
                for ch in (g, 2 + g):
                    check(X + 16 * (r * 4 + (ch ^ ((r >> 2) & 3))), ("x", r, st, ch))

    def copies(w, st, q, d):
        if SG and ((st + 3) & 7) == 0 and st + 3 < nsub:
            cp_group(w, q)
        for i in range(4):
            cp(w, i, q, d)
        for j in range(JV):
            cp(w, 4 + j, q, d)
        if BS and not SG and (st & 1) == 1:
            cp(w, XC8 + 4, q, d)
            cp(w, XC8 + 5, q, d)

    for w in range(4):
        for q in range(3):
            if SG and q == 0:
                cp_group(w, 0)
            for c in range((XC8 + 6) if (BS and not SG and (q & 1) == 0) else (XC8 + 4)):
                cp(w, c, min(q, nsub - 1), q * SLOT_B)
    for w in range(4):
        wait(w, NWAIT)
    for st in range(nsub):
        slot, q, d = st & 3, min(st + 3, nsub - 1), ((st + 3) & 3) * SLOT_B
        for w in range(4):
            reads(w, slot, st)
            if eager:
                copies(w, st, q, d)
        if not eager:
            for w in range(4):
                copies(w, st, q, d)
        for w in range(4):
            wait(w, NWAIT)
    return errs


@pytest.mark.parametrize("eager", [False, True])
@pytest.mark.parametrize("JV", [1, 2, 3, 4])
def test_mxfp4_stage_ring(JV, eager):
    for kt in (1, 2, 3, 5, 9):
        assert _run_mxfp4(JV, kt, False, eager) == [], (JV, kt)
    for kt in (4, 8, 16):   # scale groups: K a multiple of 512
        assert _run_mxfp4(JV, kt, True, eager) == [], (JV, kt)


@pytest.mark.parametrize("eager", [False, True])
@pytest.mark.parametrize("JV", [1, 2, 3, 4])
def test_8bit_stage_ring(JV, eager):
    for ns in (2, 4, 6, 10):
        assert _run_mx8(JV, ns, False, False, eager) == [], ("fp8", JV, ns)
        assert _run_mx8(JV, ns, True, False, eager) == [], ("mxfp8", JV, ns)
    for ns in (8, 16, 24):   # MXFP8 scale groups
        assert _run_mx8(JV, ns, True, True, eager) == [], ("mxfp8 groups", JV, ns)


def test_model_catches_a_short_wait():
    """The model is not vacuous: one wait count too permissive lets a read see a
    stage that has not landed."""
    JV, kt = 3, 6   # a 3-slot ring
    errs_ok = _run_mxfp4(JV, kt, False, False)
    assert errs_ok == []
    bad = _short_wait_mxfp4(JV, kt)
    assert bad != []


def _short_wait_mxfp4(JV, ktiles):
    """_run_mxfp4 with NWAIT one stage too large (copies of the stage to be read may
    still be in flight at the barrier)."""
    XROWS = 64 * JV
    XC, NC = XROWS // 32, XROWS // 32 + 6
    NSLOT = 3
    XT_B, WT_B = XROWS * 128, 256 * 64
    STAGE_B = XT_B + WT_B + 2048
    NWAIT = (NSLOT - 1) * NC   # wrong: should be (NSLOT - 2) * NC
    lds, inflight, errs = {}, [[] for _ in range(4)], []

    def cp(w, c, q, d):
        ops = {}
        for lane in range(64):
            if c < XC:
                ops[d + c * 4096 + 1024 * w + 16 * lane] = ("x", 32 * c + 8 * w + lane // 8, q)
            elif c < XC + 4:
                ops[d + XT_B + (c - XC) * 4096 + 1024 * w + 16 * lane] = ("w", 64 * (c - XC) + 16 * w + lane // 4, q)
        inflight[w].append(ops)

    def wait(w, n):
        while len(inflight[w]) > n:
            lds.update(inflight[w].pop(0))

    for w in range(4):
        for q in range(NSLOT - 1):
            for c in range(NC):
                cp(w, c, min(q, ktiles - 1), q * STAGE_B)
    for w in range(4):
        wait(w, NWAIT)
    for st in range(ktiles):
        slot = st % NSLOT
        got = lds.get(slot * STAGE_B + 16 * 0)   # row 0's first chunk
        if got is None or got[2] != st:
            errs.append((st, got))
        qraw = st + NSLOT - 1
        for w in range(4):
            for c in range(NC):
                cp(w, c, min(qraw, ktiles - 1), (qraw % NSLOT) * STAGE_B)
        for w in range(4):
            wait(w, NWAIT)
    return errs
