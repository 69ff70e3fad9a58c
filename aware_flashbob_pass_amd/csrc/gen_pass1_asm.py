"""Generate pass1_asm_loop.inc: the step loop of pass 1's non-causal d = 64 bf16 sweep
(tau folded into the resident rows) as one inline-assembly block with a fixed schedule.

    python gen_pass1_asm.py            # rewrites pass1_asm_loop.inc beside this file

The step computes what bob_pass1_kernel's pipelined two-pass step computes (FlashBoB
review page, Summary; Strengths on Prop. 4.1): the next step's score tiles S, G, dP, H
on the matrix cores, the element-wise work (p, the bf16 weights W_a, W_b, P, P G and the
row sums alpha, e0) and the four alpha-free accumulations. The order of the work is
fixed here instead of by the compiler. LDS operands are read one k-step (score
products) or one product group (accumulating products) ahead, and every wait is
computed from the order of issue. The element-wise work is spread over all 44 products
of a step (the constants below), including the accumulating products of k-step 1,
which run the first element pairs of the NEXT step: their score tiles were formed
earlier in the step, so the vector ALU has work while the last 12 products run.

Measured on the MI355X with s_memtime timers in the loop (32-key steps, one wave per
SIMD; the shader clock holds ~1.95 GHz under this load): ~2240 cycles per step, against
~2380 for a first version of this schedule (element work only beside the products of
the same step) and ~2600 for the compiler's schedule of the same source; the 44
products alone take 1408. Vector instructions issued beside the score products (whose
C and D tiles are VGPRs) overlap them less than those beside the accumulating products
(AGPR tiles), hence the split.

Register map (per lane). VGPRs: v[0:63] and v[64:127] the two score-tile buffers
(S, G, dP, H at +0, +16, +32, +48; step j reads buffer j % 2 and writes the other);
v[128:159] the weight tiles (wa, wb, pp, pg at 128, 136, 144, 152; + 4 t for k-step t);
v[160:175] -D in every slot (the C operand of the dP products of k-step 0);
v[224:239] element temporaries; v240, v241 the next step's share of alpha and e0;
v243 the lane's byte offset for the direct copies; v[244:247] the row-read addresses
of k-steps 0..3; v[248:251] the transposing-read addresses (head-dim block 0 rows +0 /
+8, block 1 rows +0 / +8); v252 L log2(e), v253 D, v254 alpha, v255 e0. AGPRs:
a[0:127] the accumulators (A, B, C, X at 0, 32, 64, 96; + 16 mb), a[128:175] the
resident tau Q, tau UQ, dO operands (k-step t at 128 + 12 t, + 4, + 8), a[176:207] two
buffers of score operands (K, V, UK, UV rows), a[208:239] two buffers of transposed
operands (K^T, UK^T, V^T, UV^T). SGPRs: s[40:47] the copy sources of K, V, UK, UV (row
block of step j + AHEAD), s48 the wave's LDS base, s49 the steps of the whole sweep (the
copies run ahead to its end, also past the block's last step), s50 the step index, s51
the block's step count, s52 scratch, s53 log2(e), s54 the caller's m0, s55 packed bf16
(1, 1) for the row sums (DOT_SUMS).

Options kept for measurement (all produce the same results): the LDS operands in VGPRs
(OPERANDS = "v"; no faster), more LDS stages and a longer copy distance (NBUF, AHEAD;
no faster: the copies land in time), no -D seed, other work splits.
"""

import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "pass1_asm_loop.inc")

NBUF = 4                 # LDS slots (32 keys of K, V, UK, UV each; 16 KiB a slot)
TILE_BYTES = 32 * 64 * 2  # one 32-key tile of one tensor
AHEAD = 3                # copies run three steps ahead (at most NBUF - 1)
HIGH_BASE = 184          # with more than 4 slots: v[184:187] row and v[188:191] transposing
                         # addresses of slots 4.. (64 KiB further on: beyond a 16-bit offset)
LOG2E_BITS = 0x3FB8AA3B

# How the element-wise work (10 vector instructions per element with DBIAS, 8 pairs of
# elements)
# rides along the matrix-core products: pairs PAIRS_A of the step during its 20 score
# products (VALU_FIRST before the first, VALU_PER_SCORE after each, the rest after the
# last), pairs PAIRS_B during the 12 accumulating products of k-step 0 (VALU_PER_ACC
# after each; all of it before the products of k-step 1, which read its weights), and
# pairs PAIRS_C of the NEXT step during the 12 accumulating products of k-step 1
# (VALU_PER_ACC_C after each), their share of alpha and e0 kept apart until that step
# starts (the last step's is never added). PAIRS_C lie in k-step 0 (pairs 0..3), whose
# weight registers the products of k-step 0 have read by then; PAIRS_B in k-step 1.
PAIRS_A = (3, 4)
PAIRS_B = (5, 6, 7)
PAIRS_C = (0, 1, 2)
VALU_FIRST = 4
VALU_PER_SCORE = 2
VALU_PER_ACC = 5
VALU_PER_ACC_C = 5
PARTIAL = (240, 241)  # the next step's share of alpha and e0 (PAIRS_C)
# Register file of the LDS operands: "v" (v[160:191] rows, v[192:223] transposed) or "a"
# (a[176:207], a[208:239]), where their return data stays out of the VGPR file that the
# vector ALU works in.
OPERANDS = "a"
# With the operands in AGPRs: v[160:175] holds -D in every slot and seeds the dP products
# of k-step 0 (their C operand), so the tile holds dP - D exactly as float32 and each step
# saves its 16 subtractions.
DBIAS = True
DBIAS_TILE = 160
# True: the row sums alpha and e0 of a pair of elements as one v_dot2_f32_bf16 of the
# pair's packed bf16 weights (P G and w_b, the values the accumulating products use)
# against packed (1, 1) in s55, instead of two float32 additions each: 16 fewer vector
# instructions per step and the same errors against the oracle, but pass 1 ran 2.5%
# slower (315 vs 307 us at N = 16384). False: the float32 additions.
DOT_SUMS = False
ONES_BF16X2 = 0x3F803F80
# Steps per workgroup barrier in the loop's full groups: 1, or 2 (a barrier after every
# second step; it then has to publish the stages of the next two steps, so copies run at
# least four steps ahead, and a copy issued while a slower wave is still one step behind
# must not overwrite what that wave reads: NBUF >= AHEAD + 2). Tail steps keep one
# barrier each, so the block always ends with its stages published.
BARRIER_EVERY = 1


def operand_bases():
    return ("v", 160, 192) if OPERANDS == "v" else ("a", 176, 208)


class Step:
    """One step's instruction list with LDS-wait and hazard bookkeeping."""

    def __init__(self):
        self.ins = []
        self.lds_q = []          # ids of LDS reads in flight, in issue order
        self.valu_write = {}     # register -> index of the VALU instruction that wrote it
        self.trans_write = {}    # register -> index of the v_exp that wrote it

    def emit(self, text):
        self.ins.append(text)

    def lds(self, text, ident):
        self.ins.append(text)
        self.lds_q.append(ident)

    def wait_lds(self, idents):
        idents = [i for i in idents if i in self.lds_q]
        if not idents:
            return
        last = max(self.lds_q.index(i) for i in idents)
        after = len(self.lds_q) - 1 - last
        self.ins.append(f"s_waitcnt lgkmcnt({min(after, 15)})")
        del self.lds_q[:last + 1]

    def valu(self, text, dst, srcs, trans=False):
        # a vector instruction reading a transcendental result needs one wait state
        for r in srcs:
            if r in self.trans_write and len(self.ins) - self.trans_write[r] < 2:
                self.ins.append("s_nop 0")
        self.ins.append(text)
        self.valu_write[dst] = len(self.ins) - 1
        if trans:
            self.trans_write[dst] = len(self.ins) - 1
        elif dst in self.trans_write:
            del self.trans_write[dst]

    def mfma(self, text, srcs):
        # an MFMA reading a VGPR a vector instruction just wrote needs two wait states
        need = 0
        for r in srcs:
            if r in self.valu_write:
                need = max(need, 3 - (len(self.ins) - self.valu_write[r]))
        if need > 0:
            self.ins.append(f"s_nop {need - 1}")
        self.ins.append(text)


def vrange(base, n):
    return list(range(base, base + n))


def element_pair(p, cur, tmp, sums=(254, 255), init=False):
    """The element-wise work of elements 2p and 2p + 1 of the tiles at `cur` (20 vector
    instructions; 18 with DOT_SUMS, 22 without DBIAS):
    p = exp2(S log2(e) - L log2(e)), t = dP - D, alpha += p G, w_b = p (G t + H),
    e0 += w_b, and the bf16 weights W_a = p t, W_b = w_b, P = p, P G.
    tmp: 8 temporaries (P0, P1, T0, T1, PG0, PG1, WB0, WB1); sums: the registers
    alpha and e0 accumulate into (init: element 2p starts them)."""
    P, T, PG, WB = tmp[0:2], tmp[2:4], tmp[4:6], tmp[6:8]
    al, e0 = sums
    out = []
    es = (2 * p, 2 * p + 1)
    S = [cur + e for e in es]
    G = [cur + 16 + e for e in es]
    DP = [cur + 32 + e for e in es]
    H = [cur + 48 + e for e in es]
    for i in range(2):
        out.append((f"v_fma_f32 v{P[i]}, v{S[i]}, s53, -v252", P[i], [S[i], 252], False))
    for i in range(2):
        out.append((f"v_exp_f32 v{P[i]}, v{P[i]}", P[i], [P[i]], True))
    if DBIAS:  # the dP tile holds dP - D already
        TD = DP
    else:
        TD = T
        for i in range(2):
            out.append((f"v_sub_f32 v{T[i]}, v{DP[i]}, v253", T[i], [DP[i], 253], False))
    for i in range(2):
        out.append((f"v_mul_f32 v{PG[i]}, v{P[i]}, v{G[i]}", PG[i], [P[i], G[i]], False))
    if not DOT_SUMS:
        for i in range(2):
            src = "0" if init and i == 0 else f"v{al}"
            out.append((f"v_add_f32 v{al}, {src}, v{PG[i]}", al, [PG[i], al], False))
    for i in range(2):
        out.append((f"v_fma_f32 v{WB[i]}, v{G[i]}, v{TD[i]}, v{H[i]}", WB[i], [G[i], TD[i], H[i]], False))
    for i in range(2):
        out.append((f"v_mul_f32 v{WB[i]}, v{P[i]}, v{WB[i]}", WB[i], [P[i], WB[i]], False))
    if not DOT_SUMS:
        for i in range(2):
            src = "0" if init and i == 0 else f"v{e0}"
            out.append((f"v_add_f32 v{e0}, {src}, v{WB[i]}", e0, [WB[i], e0], False))
    for i in range(2):
        out.append((f"v_mul_f32 v{T[i]}, v{P[i]}, v{TD[i]}", T[i], [P[i], TD[i]], False))
    t, reg = (2 * p) >> 3, ((2 * p) & 7) >> 1
    packed = {}
    for base, src in ((128, T), (136, WB), (144, P), (152, PG)):
        d = base + 4 * t + reg
        packed[base] = d
        out.append((f"v_cvt_pk_bf16_f32 v{d}, v{src[0]}, v{src[1]}", d, [src[0], src[1]], False))
    if DOT_SUMS:  # alpha += (P G)_2p + (P G)_2p+1, e0 += w_b,2p + w_b,2p+1 from the packed weights
        for acc, base in ((al, 152), (e0, 136)):
            src = "0" if init else f"v{acc}"
            out.append((f"v_dot2_f32_bf16 v{acc}, v{packed[base]}, s55, {src}", acc,
                        [packed[base]] + ([] if init else [acc]), False))
    return out


def interleave(a, b):
    """Two pairs' instruction lists merged two at a time (the pair lists hold each
    operation for both elements back to back), so the row sums still add the
    elements in ascending order."""
    out = []
    for i in range(0, max(len(a), len(b)), 2):
        out += a[i:i + 2] + b[i:i + 2]
    return out


def valu_rows(pairs, cur, sums=(254, 255)):
    """Element-wise work of the given element pairs, two pairs interleaved at a time on
    the two temporary sets. Sums other than alpha and e0 themselves start at the first
    element."""
    t0, t1 = vrange(224, 8), vrange(232, 8)
    init = sums != (254, 255)
    out = []
    pairs = list(pairs)
    for k in range(0, len(pairs), 2):
        first = element_pair(pairs[k], cur, t0, sums, init and k == 0)
        if k + 1 < len(pairs):
            out += interleave(first, element_pair(pairs[k + 1], cur, t1, sums))
        else:
            out += first
    return out


def step_body(S):
    """Instruction list of one step in LDS slot S (compile-time), with the copies and
    the end-of-step wait and barrier left to the caller."""
    st = Step()
    cur = 0 if S % 2 == 0 else 64
    nxt = 64 - cur
    sn = (S + 1) % NBUF  # slot of the next step: its score tiles are formed now
    valu_a = valu_rows(PAIRS_A, cur)  # during the score products
    valu_b = valu_rows(PAIRS_B, cur)  # during the accumulations of k-step 0
    valu_c = valu_rows(PAIRS_C, nxt, PARTIAL)  # the next step's, during those of k-step 1

    rf, row_base, tr_base = operand_bases()

    def row_reads(t):
        buf = row_base + 16 * (t % 2)
        for k in range(4):  # K, V, UK, UV
            base, off = (244 + t, (sn * 4 + k) * TILE_BYTES) if sn < 4 else \
                (HIGH_BASE + t, ((sn - 4) * 4 + k) * TILE_BYTES)
            st.lds(f"ds_read_b128 {rf}[{buf + 4 * k}:{buf + 4 * k + 3}], v{base} offset:{off}",
                   ("r", t, k))

    def tr_reads(q):
        t, mb = q // 2, q % 2
        buf = tr_base + 16 * (q % 2)
        for k, tensor in enumerate((0, 2, 1, 3)):  # K^T, UK^T, V^T, UV^T from slots K, UK, V, UV
            base = 248 if S < 4 else HIGH_BASE + 4
            off = ((S % 4) * 4 + tensor) * TILE_BYTES + t * 16 * 128
            d = buf + 4 * k
            st.lds(f"ds_read_b64_tr_b16 {rf}[{d}:{d + 1}], v{base + 2 * mb} offset:{off}", ("t", q, k, 0))
            st.lds(f"ds_read_b64_tr_b16 {rf}[{d + 2}:{d + 3}], v{base + 1 + 2 * mb} offset:{off}", ("t", q, k, 1))

    def opnd(r):  # VGPRs of an LDS operand (tracked for vector-write hazards)
        return vrange(r, 4) if rf == "v" else []

    def pop_valu(queue, n):
        for _ in range(min(n, len(queue))):
            text, dst, srcs, trans = queue.pop(0)
            st.valu(text, dst, srcs, trans)

    # ---- phase A: the next step's score tiles with rows 0..7 of this step ----------------
    # k-step t's operands are read one k-step ahead (two buffers): k-steps 0 and 1 at the
    # start, k-step t + 1 once k-step t's have landed (its buffer was last read by the
    # products of k-step t - 1); the transposed operands of groups 0 and 1 from k-step 2 on.
    if PAIRS_C:  # this step's PAIRS_C share of the row sums, formed during the previous step
        st.valu(f"v_add_f32 v254, v254, v{PARTIAL[0]}", 254, [254, PARTIAL[0]])
        st.valu(f"v_add_f32 v255, v255, v{PARTIAL[1]}", 255, [255, PARTIAL[1]])
    row_reads(0)
    row_reads(1)
    pop_valu(valu_a, VALU_FIRST)
    for t in range(4):
        st.wait_lds([("r", t, k) for k in range(4)])
        if 1 <= t and t + 1 < 4:
            row_reads(t + 1)
        if t >= 2:
            tr_reads(t - 2)
        buf = row_base + 16 * (t % 2)
        ak, av, auk, auv = buf, buf + 4, buf + 8, buf + 12
        res = 128 + 12 * t
        z = (lambda r: "0") if t == 0 else (lambda r: f"v[{r}:{r + 15}]")
        zd = (lambda r: f"v[{DBIAS_TILE}:{DBIAS_TILE + 15}]") if t == 0 and DBIAS else z
        prods = [
            (f"v_mfma_f32_32x32x16_bf16 v[{nxt}:{nxt + 15}], {rf}[{ak}:{ak + 3}], a[{res}:{res + 3}], {z(nxt)}", ak),
            (f"v_mfma_f32_32x32x16_bf16 v[{nxt + 16}:{nxt + 31}], {rf}[{ak}:{ak + 3}], a[{res + 4}:{res + 7}], "
             f"{z(nxt + 16)}", ak),
            (f"v_mfma_f32_32x32x16_bf16 v[{nxt + 32}:{nxt + 47}], {rf}[{av}:{av + 3}], a[{res + 8}:{res + 11}], "
             f"{zd(nxt + 32)}", av),
            (f"v_mfma_f32_32x32x16_bf16 v[{nxt + 16}:{nxt + 31}], {rf}[{auk}:{auk + 3}], a[{res}:{res + 3}], "
             f"v[{nxt + 16}:{nxt + 31}]", auk),
            (f"v_mfma_f32_32x32x16_bf16 v[{nxt + 48}:{nxt + 63}], {rf}[{auv}:{auv + 3}], a[{res + 8}:{res + 11}], "
             f"{z(nxt + 48)}", auv),
        ]
        for text, src in prods:
            st.mfma(text, vrange(src, 4) if rf == "v" else [])
            pop_valu(valu_a, VALU_PER_SCORE)
    pop_valu(valu_a, len(valu_a))

    # ---- phases B and C: the accumulations; PAIRS_B of this step during B, PAIRS_C of the
    # next step during C (its score tiles were formed in phase A; the weight registers of
    # k-step 0 it writes were last read by the products of B, all issued) -------------------
    for q in range(4):
        t, mb = q // 2, q % 2
        st.wait_lds([("t", q, k, h) for k in range(4) for h in range(2)])
        buf = tr_base + 16 * (q % 2)
        kT, ukT, vT, uvT = buf, buf + 4, buf + 8, buf + 12
        wa, wb, pp, pg = 128 + 4 * t, 136 + 4 * t, 144 + 4 * t, 152 + 4 * t
        A, B, C, X = 16 * mb, 32 + 16 * mb, 64 + 16 * mb, 96 + 16 * mb
        prods = [
            (f"v_mfma_f32_32x32x16_bf16 a[{A}:{A + 15}], {rf}[{ukT}:{ukT + 3}], v[{wa}:{wa + 3}], a[{A}:{A + 15}]",
             opnd(ukT) + vrange(wa, 4)),
            (f"v_mfma_f32_32x32x16_bf16 a[{B}:{B + 15}], {rf}[{kT}:{kT + 3}], v[{wa}:{wa + 3}], a[{B}:{B + 15}]",
             opnd(kT) + vrange(wa, 4)),
            (f"v_mfma_f32_32x32x16_bf16 a[{X}:{X + 15}], {rf}[{uvT}:{uvT + 3}], v[{pp}:{pp + 3}], a[{X}:{X + 15}]",
             opnd(uvT) + vrange(pp, 4)),
            (f"v_mfma_f32_32x32x16_bf16 a[{A}:{A + 15}], {rf}[{kT}:{kT + 3}], v[{wb}:{wb + 3}], a[{A}:{A + 15}]",
             opnd(kT) + vrange(wb, 4)),
            (f"v_mfma_f32_32x32x16_bf16 a[{C}:{C + 15}], {rf}[{kT}:{kT + 3}], v[{pp}:{pp + 3}], a[{C}:{C + 15}]",
             opnd(kT) + vrange(pp, 4)),
            (f"v_mfma_f32_32x32x16_bf16 a[{X}:{X + 15}], {rf}[{vT}:{vT + 3}], v[{pg}:{pg + 3}], a[{X}:{X + 15}]",
             opnd(vT) + vrange(pg, 4)),
        ]
        if q == 2:
            pop_valu(valu_b, len(valu_b))  # k-step 1's weights complete before its products
        for text, srcs in prods:
            st.mfma(text, srcs)
            if q < 2:
                pop_valu(valu_b, VALU_PER_ACC)
            else:
                pop_valu(valu_c, VALU_PER_ACC_C)
        if q + 2 < 4:
            tr_reads(q + 2)  # after all six products of group q have been issued
    assert not valu_b
    pop_valu(valu_c, len(valu_c))
    return st.ins


def step_text(S, label, tail=False):
    """One complete step: guarded copies, the body, the copy wait and the barrier (with
    BARRIER_EVERY = 2, only after odd steps of a full group)."""
    ins = []
    ins.append("s_add_u32 s52, s50, %d" % AHEAD)
    ins.append("s_cmp_lt_u32 s52, s49")
    ins.append(f"s_cbranch_scc0 L_nocopy_{label}_%=")
    sc = (S + AHEAD) % NBUF
    for k in range(4):
        ins.append(f"s_add_u32 m0, s48, {(sc * 4 + k) * TILE_BYTES}")
        ins.append("s_nop 0")
        ins.append(f"global_load_lds_dwordx4 v243, s[{40 + 2 * k}:{41 + 2 * k}] offset:0")
    ins.append(f"L_nocopy_{label}_%=:")
    ins += step_body(S)
    for k in range(4):  # the copy sources advance by one 32-row block every step
        ins.append(f"s_add_u32 s{40 + 2 * k}, s{40 + 2 * k}, {TILE_BYTES}")
        ins.append(f"s_addc_u32 s{41 + 2 * k}, s{41 + 2 * k}, 0")
    per_step = BARRIER_EVERY == 1 or tail
    if per_step or S % 2 == 1:
        # per step: the copies of step j + 2 (read from step j + 1 on) have landed, those of
        # the AHEAD - 2 latest steps may stay in flight; every second step: those of steps
        # j + 2 and j + 3 (read by the next two steps), AHEAD - 3 in flight
        keep = AHEAD - 2 if per_step else AHEAD - 3
        ins.append("s_add_u32 s52, s50, %d" % AHEAD)
        ins.append("s_cmp_lt_u32 s52, s49")
        ins.append(f"s_cbranch_scc0 L_wait0_{label}_%=")
        ins.append(f"s_waitcnt vmcnt({4 * keep})")
        ins.append(f"s_branch L_waited_{label}_%=")
        ins.append(f"L_wait0_{label}_%=:")
        ins.append("s_waitcnt vmcnt(0)")
        ins.append(f"L_waited_{label}_%=:")
        ins.append("s_barrier")
    ins.append("s_add_u32 s50, s50, 1")
    return ins


def loop_text():
    ins = ["s_nop 7", "s_nop 7", "s_nop 7",  # the prologue's score products complete before use
           "s_waitcnt vmcnt(0) lgkmcnt(0)",  # the counts below assume nothing else in flight
           "s_mov_b32 s54, m0",  # m0 is the compiler's: restored at the end
           f"s_mov_b32 s53, 0x{LOG2E_BITS:08x}", "s_mov_b32 s50, 0"]
    if DOT_SUMS:
        ins.append(f"s_mov_b32 s55, 0x{ONES_BF16X2:08x}")
    assert sorted(PAIRS_A + PAIRS_B + PAIRS_C) == list(range(8))
    assert not DBIAS or OPERANDS == "a"
    assert 3 <= AHEAD < NBUF and NBUF % 2 == 0 and 4 * (AHEAD - 2) <= 63 and (NBUF <= 4 or OPERANDS == "a")
    assert BARRIER_EVERY in (1, 2) and (BARRIER_EVERY == 1 or (AHEAD >= 4 and NBUF >= AHEAD + 2))
    if NBUF > 4:  # addresses of the upper slots
        ins += [f"v_add_u32 v{HIGH_BASE + i}, 0x10000, v{244 + i}" for i in range(8)]
    if DBIAS:  # the -D tile, and step 0's dP tile (formed by the caller) less D
        ins += [f"v_sub_f32 v{DBIAS_TILE + i}, 0, v253" for i in range(16)]
        ins += [f"v_sub_f32 v{32 + i}, v{32 + i}, v253" for i in range(16)]
        ins += ["s_nop 1"]
    assert all(p >= 4 for p in PAIRS_B) and all(p < 4 for p in PAIRS_C)
    if PAIRS_C:  # step 0's PAIRS_C share (its score tiles came in with the entry state)
        st = Step()
        for text, dst, srcs, trans in valu_rows(PAIRS_C, 0, PARTIAL):
            st.valu(text, dst, srcs, trans)
        ins += st.ins
    ins.append("L_loop_%=:")
    ins.append("s_add_u32 s52, s50, %d" % NBUF)
    ins.append("s_cmp_gt_u32 s52, s51")
    ins.append("s_cbranch_scc1 L_tail_%=")
    for S in range(NBUF):
        ins += step_text(S, f"m{S}")
    ins.append("s_branch L_loop_%=")
    ins.append("L_tail_%=:")
    for S in range(NBUF - 1):
        ins.append("s_cmp_ge_u32 s50, s51")
        ins.append("s_cbranch_scc1 L_end_%=")
        ins += step_text(S, f"t{S}", tail=True)
    ins.append("L_end_%=:")
    ins += ["s_mov_b32 m0, s54", "s_nop 7", "s_nop 7", "s_nop 7"]  # the last accumulating products complete
    return ins


def written_registers(ins):
    """The VGPRs and AGPRs the instructions write (their first operand), as sorted lists."""
    out = {"v": set(), "a": set()}
    for x in ins:
        op = x.split()[0]
        if not (op.startswith("v_") or op.startswith("ds_read")):
            continue
        dst = x.split(None, 1)[1].split(",")[0].strip()
        m = re.fullmatch(r"([va])(\d+)", dst) or re.fullmatch(r"([va])\[(\d+):(\d+)\]", dst)
        if m:
            lo = int(m.group(2))
            hi = int(m.group(3)) if m.lastindex == 3 else lo
            out[m.group(1)].update(range(lo, hi + 1))
    return sorted(out["v"]), sorted(out["a"])


# Registers bound to the block's outputs (the compiler knows they change): the score tiles,
# the row sums and the accumulators. Every other register the block writes is a clobber.
BOUND_V = set(range(0, 64)) | {254, 255}
BOUND_A = set(range(0, 128))


def render():
    ins = loop_text()
    wv, wa = written_registers(ins)
    assert not set(wv) & set(range(243, 254)) and not set(wa) & set(range(128, 176)), "block writes an input"
    clob = ", ".join([f'"v{r}"' for r in wv if r not in BOUND_V] + [f'"a{r}"' for r in wa if r not in BOUND_A])
    clob += ', "s50", "s52", "s53", "s54"' + (', "s55"' if DOT_SUMS else "") + ', "scc", "memory"'
    return ("// Generated by gen_pass1_asm.py (same directory); do not edit by hand.\n"
            "// The step loop of pass 1's non-causal d = 64 bf16 sweep with tau folded: the\n"
            "// generator's docstring gives the schedule and the register map.\n"
            f"// {len(ins)} instructions and labels.\n"
            "#define FB_PASS1_ASM_LOOP \\\n" + " \\\n".join(f'  "{x}\\n\\t"' for x in ins) + "\n"
            "#define FB_PASS1_ASM_CLOBBERS " + clob + "\n"
            f"#define FB_PASS1_ASM_SLOTS {NBUF}\n"
            f"#define FB_PASS1_ASM_DBIAS {int(DBIAS)}\n"
            f"#define FB_PASS1_ASM_AHEAD {AHEAD}\n")


def main():
    text = render()
    with open(OUT, "w") as fh:
        fh.write(text)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
