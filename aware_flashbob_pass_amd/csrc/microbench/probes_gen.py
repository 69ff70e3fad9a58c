"""Write microbench_probes.hip: the microbenchmarks and skeleton kernels that the
bound analysis of the kernels rests on, as one HIP program (one compile). Run it with
`python bench.py --microbench [OUT.md]`, which builds it with hipcc and runs it.

Every probe keeps its LDS addresses inside its allocation and its registers inside its
clobber list; the skeletons' data are meaningless (only the instruction stream and its
dependencies matter) and nothing but a per-wave cycle count leaves the GPU.

Probes (each prints one line "name: value unit"):
- mfma_rate: independent v_mfma_f32_32x32x16_bf16 chains from registers on every SIMD
  (two waves per SIMD), for about a third of a second: sustained TFLOP/s and the
  shader clock (s_memtime cycles over s_memrealtime's 100 MHz ticks).
- lds_rate_*: back-to-back LDS reads (ds_read_b128, ds_read_b64, ds_read_b64_tr_b16;
  8 per block, waited in the block) at 4, 8 and 16 waves per CU: bytes per clock per CU.
- p1mix_*: pass 1's per-step instruction mix (44 MFMAs, 229 vector instructions of the
  kernel's kinds with 16 v_exp_f32, 16 ds_read_b128 + 32 ds_read_b64_tr_b16 at
  conflict-free addresses, one barrier) with no data dependencies, one wave per SIMD,
  restricted to a subset of the kinds: cycles per step.
- p1dep_*: one pass-1 step with its data dependencies (score tiles double-buffered,
  weights written by vector instructions and read by the accumulating products),
  in two orders: element work beside the score products ("interleaved") or after
  them ("phased").
- p2dep_*: one pass-2 step at one wave per SIMD (next step's score tiles beside this
  step's element work, 7 vector instructions per element with the row scalars seeded
  into the products, 12 row + 24 transposing + 16 row-scalar reads), with 0, 2 or 4
  element pairs beside the score products.
- gchain_*: 20 score products per step with the G tile as one chain of dependent
  products two issue slots apart, or split over two tiles.
- rate_*: 64 independent vector instructions of one kind per step (v_fma_f32,
  v_exp_f32), one wave per SIMD: cycles per instruction.
- rate_fma_banks, rate_add_chain, rate_exp_dep: the same with the FMA's three sources
  in three register banks, a chain of dependent adds, and exponential/add pairs whose add
  reads the exponential.
- fwddep_*: one step of the statistics kernel (32 queries x 32 keys per wave, d = 64:
  4 score products chained over the head dimension, 4 P V products into two
  accumulator tiles, 16 weights p = 2^(fma(s, c, -m)) with their sum and 8 bf16 packs,
  4 ds_read_b128 + 8 ds_read_b64_tr_b16, one barrier) at one wave per SIMD, in two
  orders: "phased" (this step's score products, then its weights, then its P V
  products: the order of the compiled kernel) and "skewed" (the score products of step
  j + 2 and the P V products of step j beside the weights of step j + 1, so nothing in a
  step waits for anything else in it); "skewed_noexp" replaces the exponentials by
  moves, "skewed_mfma" keeps only the products and "skewed_valu" only the vector work;
  "skewed_banks" is "skewed" with no two VGPR sources of an instruction in one register
  bank and the step's sum split over two partial sums.
"""

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "microbench_probes.hip")


def _esc(lines):
    return "\\n\\t".join(lines)


# ---- pass-1 instruction mix, no dependencies --------------------------------------------
def p1_mix(mode):
    use_m = mode in ("full", "mfma", "mfma_lds", "mfma_valu")
    use_v = mode in ("full", "mfma_valu", "valu")
    use_l = mode in ("full", "mfma_lds", "lds")
    cnt = {"v": 0, "l": 0}

    def score(i):
        t = i % 4
        return f"v_mfma_f32_32x32x16_bf16 v[{16 * t}:{16 * t + 15}], v[64:67], v[68:71], v[{16 * t}:{16 * t + 15}]"

    def acc(i):
        t = i % 8
        return f"v_mfma_f32_32x32x16_bf16 a[{16 * t}:{16 * t + 15}], v[72:75], v[76:79], a[{16 * t}:{16 * t + 15}]"

    def valu():
        k = cnt["v"]
        cnt["v"] += 1
        r = 100 + (k % 90)
        if k % 15 == 7:
            return f"v_exp_f32 v{r}, v{r}"
        if k % 15 == 3:
            return f"v_cvt_pk_bf16_f32 v{r}, v{r}, v{r + 1}"
        return f"v_fma_f32 v{r}, v{r}, v{r + 1}, v{r + 2}" if k % 2 else f"v_mul_f32 v{r}, v{r}, v{r + 1}"

    def row():
        k = cnt["l"]
        cnt["l"] += 1
        r = 200 + 4 * (k % 8)
        return f"ds_read_b128 v[{r}:{r + 3}], v80 offset:{(k % 16) * 1024}"

    def tr():
        k = cnt["l"]
        cnt["l"] += 1
        r = 232 + 2 * (k % 8)
        return f"ds_read_b64_tr_b16 v[{r}:{r + 1}], v81 offset:{(k % 32) * 512}"

    step, rows = [], 0
    for i in range(20):  # score products, 5 vector instructions each, a row read each
        if use_m:
            step.append(score(i))
        if use_v:
            step += [valu() for _ in range(5)]
        if use_l:
            if rows < 16:
                step.append(row())
                rows += 1
            else:
                step.append(tr())
            if i % 4 == 3:
                step.append("s_waitcnt lgkmcnt(4)")
    for i in range(12):  # accumulating products with rows 8..15's work
        if use_m:
            step.append(acc(i))
        if use_v:
            step += [valu() for _ in range(8)]
        if use_l:
            step += [tr(), tr()]
            if i % 2 == 1:
                step.append("s_waitcnt lgkmcnt(6)")
    for i in range(12):
        if use_m:
            step.append(acc(12 + i))
        if use_v:
            step += [valu() for _ in range(3 if i < 9 else 2)]
        if use_l and i % 3 == 0:
            step += [tr(), "s_waitcnt lgkmcnt(2)"]
    if use_l:
        step.append("s_waitcnt lgkmcnt(0)")
    step += ["s_nop 7", "s_nop 7", "s_nop 7", "s_barrier"]
    return step, ["v80", "v81"]


# ---- pass-1 step with dependencies -------------------------------------------------------
def p1_dep(order):
    def one(cur, nxt):
        score = []
        for t in range(4):
            ob, res = 160 + 16 * (t % 2), 128 + 12 * t
            score += [f"v_mfma_f32_32x32x16_bf16 v[{nxt}:{nxt + 15}], v[{ob}:{ob + 3}], a[{res}:{res + 3}], v[{nxt}:{nxt + 15}]",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 16}:{nxt + 31}], v[{ob}:{ob + 3}], a[{res + 4}:{res + 7}], v[{nxt + 16}:{nxt + 31}]",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 32}:{nxt + 47}], v[{ob + 4}:{ob + 7}], a[{res + 8}:{res + 11}], v[{nxt + 32}:{nxt + 47}]",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 16}:{nxt + 31}], v[{ob + 8}:{ob + 11}], a[{res}:{res + 3}], v[{nxt + 16}:{nxt + 31}]",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 48}:{nxt + 63}], v[{ob + 12}:{ob + 15}], a[{res + 8}:{res + 11}], v[{nxt + 48}:{nxt + 63}]"]

        def rows(t):
            ob = 160 + 16 * (t % 2)
            return [f"ds_read_b128 v[{ob + 4 * i}:{ob + 4 * i + 3}], v244 offset:{(t * 4 + i) * 1024 % 16384}" for i in range(4)]

        def elem(r):
            s, g, dp, h = cur + r, cur + 16 + r, cur + 32 + r, cur + 48 + r
            t0 = 224 + (r % 4) * 5
            w = 128 + r // 2
            return [f"v_fma_f32 v{t0}, v{s}, v245, -v246", f"v_exp_f32 v{t0}, v{t0}", f"v_mul_f32 v{t0 + 1}, v{g}, v247",
                    f"v_sub_f32 v{t0 + 2}, v{dp}, v246", f"v_mul_f32 v{t0 + 3}, v{t0}, v{t0 + 1}",
                    f"v_fmac_f32 v248, v{t0}, v{t0 + 1}", f"v_fma_f32 v{t0 + 4}, v{t0 + 1}, v{t0 + 2}, v{h}",
                    f"v_mul_f32 v{t0 + 4}, v{t0}, v{t0 + 4}", f"v_fmac_f32 v249, v{t0}, v{t0 + 4}",
                    f"v_mul_f32 v{t0 + 2}, v{t0}, v{t0 + 2}", f"v_cvt_pk_bf16_f32 v{w}, v{t0 + 2}, v{t0 + 3}",
                    f"v_cvt_pk_bf16_f32 v{w + 8}, v{t0 + 4}, v{t0}"]

        def trs(q):
            ob = 192 + 16 * (q % 2)
            return [f"ds_read_b64_tr_b16 v[{ob + 2 * i}:{ob + 2 * i + 1}], v250 offset:{(q * 8 + i) * 512 % 16384}" for i in range(8)]

        def acc(q):
            ob, t, mb = 192 + 16 * (q % 2), q // 2, q % 2
            wa, wb, pp, pg = 128 + 4 * t, 136 + 4 * t, 144 + 4 * t, 152 + 4 * t
            A, B, C, X = 16 * mb, 32 + 16 * mb, 64 + 16 * mb, 96 + 16 * mb
            return ["s_nop 1",
                    f"v_mfma_f32_32x32x16_bf16 a[{A}:{A + 15}], v[{ob + 4}:{ob + 7}], v[{wa}:{wa + 3}], a[{A}:{A + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{B}:{B + 15}], v[{ob}:{ob + 3}], v[{wa}:{wa + 3}], a[{B}:{B + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{X}:{X + 15}], v[{ob + 12}:{ob + 15}], v[{pp}:{pp + 3}], a[{X}:{X + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{A}:{A + 15}], v[{ob}:{ob + 3}], v[{wb}:{wb + 3}], a[{A}:{A + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{C}:{C + 15}], v[{ob}:{ob + 3}], v[{pp}:{pp + 3}], a[{C}:{C + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{X}:{X + 15}], v[{ob + 8}:{ob + 11}], v[{pg}:{pg + 3}], a[{X}:{X + 15}]"]

        ins = rows(0) + ["s_waitcnt lgkmcnt(0)"]
        if order == "interleaved":
            vq = [x for r in range(8) for x in elem(r)]
            for i, m in enumerate(score):
                t = i // 5
                if i % 5 == 0 and t + 1 < 4:
                    ins += rows(t + 1)
                if i % 5 == 0 and t == 3:
                    ins += trs(0)
                ins.append(m)
                ins += vq[:5]
                vq = vq[5:]
                if i % 5 == 4:
                    ins.append("s_waitcnt lgkmcnt(4)")
            ins += vq
            vq = [x for r in range(8, 16) for x in elem(r)]
            for q in range(4):
                ins.append("s_waitcnt lgkmcnt(0)")
                if q + 1 < 4:
                    ins += trs(q + 1)
                for m in acc(q):
                    ins.append(m)
                    if not m.startswith("s_nop"):
                        n = 8 if q < 2 else 4
                        ins += vq[:n]
                        vq = vq[n:]
            ins += vq
        else:
            for i, m in enumerate(score):
                t = i // 5
                if i % 5 == 0 and t + 1 < 4:
                    ins += rows(t + 1)
                ins.append(m)
                if i % 5 == 4:
                    ins.append("s_waitcnt lgkmcnt(0)")
            ins += [x for r in range(16) for x in elem(r)]
            for q in range(4):
                ins += trs(q) + ["s_waitcnt lgkmcnt(0)"] + acc(q)
        ins.append("s_waitcnt lgkmcnt(0)")
        return ins

    return one(0, 64) + ["s_barrier"] + one(64, 0) + ["s_barrier"], ["v244", "v250"]


# ---- pass-2 step at one wave per SIMD, with dependencies -------------------------------------
def p2_dep(split):
    def one(cur, nxt):
        def rows(t):
            ob = 128 + 12 * (t % 2)
            return [f"ds_read_b128 a[{ob + 4 * i}:{ob + 4 * i + 3}], v244 offset:{(t * 3 + i) * 1024 % 16384}" for i in range(3)]

        def scal():  # 16-byte aligned, two addresses per wave (lane groups), as the kernel's row scalars
            return [f"ds_read_b128 v[{152 + 4 * i}:{152 + 4 * i + 3}], v245 offset:{i * 128}" for i in range(16)]

        def trs(q):
            ob = 152 + 12 * (q % 2)
            return [f"ds_read_b64_tr_b16 a[{ob + 2 * i}:{ob + 2 * i + 1}], v246 offset:{(q * 6 + i) * 512 % 16384}" for i in range(6)]

        score = []
        for t in range(4):
            ob, res = 128 + 12 * (t % 2), 64 + 16 * t

            def c(r, seed):
                return f"v[{seed}:{seed + 15}]" if t == 0 else f"v[{r}:{r + 15}]"

            score += [f"v_mfma_f32_32x32x16_bf16 v[{nxt}:{nxt + 15}], a[{ob}:{ob + 3}], a[{res}:{res + 3}], {c(nxt, 152)}",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 16}:{nxt + 31}], a[{ob + 8}:{ob + 11}], a[{res}:{res + 3}], {c(nxt + 16, 184)}",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 32}:{nxt + 47}], a[{ob + 4}:{ob + 7}], a[{res + 4}:{res + 7}], {c(nxt + 32, 168)}",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 16}:{nxt + 31}], a[{ob}:{ob + 3}], a[{res + 8}:{res + 11}], v[{nxt + 16}:{nxt + 31}]",
                      f"v_mfma_f32_32x32x16_bf16 v[{nxt + 48}:{nxt + 63}], a[{ob + 4}:{ob + 7}], a[{res + 12}:{res + 15}], {c(nxt + 48, 200)}"]

        def elem(r):
            s, g, dp, h = cur + r, cur + 16 + r, cur + 32 + r, cur + 48 + r
            t0 = 216 + (r % 4) * 6
            w = 128 + (r // 2) % 4 + 4 * (r // 8)
            last = (f"v_cvt_pk_bf16_f32 v{w}, v{t0 + 2}, v{t0 + 2}" if r % 2 else
                    f"v_cvt_pk_bf16_f32 v{w + 8}, v{t0 + 3}, v{t0 + 3}")
            return [f"v_fma_f32 v{t0}, v{s}, v247, -v{152 + r}", f"v_exp_f32 v{t0}, v{t0}",
                    f"v_mul_f32 v{t0 + 1}, v{t0}, v{g}", f"v_mul_f32 v{t0 + 2}, v{t0}, v{dp}",
                    f"v_mul_f32 v{t0 + 3}, v{t0}, v{h}", f"v_fma_f32 v{t0 + 3}, v{t0 + 1}, v{dp}, v{t0 + 3}", last]

        def acc(q):
            ob, t, mb = 152 + 12 * (q % 2), q // 2, q % 2
            wds, wsb, wdp = 128 + 4 * t, 136 + 4 * t, 144 + 4 * t
            K, V = 16 * mb, 32 + 16 * mb
            return ["s_nop 1",
                    f"v_mfma_f32_32x32x16_bf16 a[{K}:{K + 15}], a[{ob}:{ob + 3}], v[{wds}:{wds + 3}], a[{K}:{K + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{K}:{K + 15}], a[{ob + 4}:{ob + 7}], v[{wsb}:{wsb + 3}], a[{K}:{K + 15}]",
                    f"v_mfma_f32_32x32x16_bf16 a[{V}:{V + 15}], a[{ob + 8}:{ob + 11}], v[{wdp}:{wdp + 3}], a[{V}:{V + 15}]"]

        va = [x for r in range(2 * split) for x in elem(r)]
        vb = [x for r in range(2 * split, 16) for x in elem(r)]
        ins = scal() + rows(0) + rows(1) + ["s_waitcnt lgkmcnt(3)"]
        per = -(-len(va) // 20) if va else 0
        for i, m in enumerate(score):
            t = i // 5
            if i % 5 == 0 and t >= 1:
                ins.append("s_waitcnt lgkmcnt(0)")
                if t + 1 < 4:
                    ins += rows(t + 1)
                if t == 2:
                    ins += trs(0)
                if t == 3:
                    ins += trs(1)
            ins.append(m)
            ins += va[:per]
            va = va[per:]
        ins += va
        per_b = -(-len(vb) // 6) if vb else 0
        for q in range(4):
            ins.append("s_waitcnt lgkmcnt(6)" if q < 3 else "s_waitcnt lgkmcnt(0)")
            for m in acc(q):
                ins.append(m)
                if q < 2 and not m.startswith("s_nop"):
                    ins += vb[:per_b]
                    vb = vb[per_b:]
            if q + 2 < 4:
                ins += trs(q + 2)
        ins += vb
        ins.append("s_waitcnt lgkmcnt(0)")
        return ins

    return one(0, 64) + ["s_barrier"] + one(64, 0) + ["s_barrier"], ["v244", "v245", "v246"]


def gchain(split):
    ins = []
    for _ in range(4):
        g2 = "v[64:79]" if split else "v[16:31]"
        ins += ["v_mfma_f32_32x32x16_bf16 v[0:15], v[80:83], v[84:87], v[0:15]",
                "v_mfma_f32_32x32x16_bf16 v[16:31], v[80:83], v[88:91], v[16:31]",
                "v_mfma_f32_32x32x16_bf16 v[32:47], v[80:83], v[84:87], v[32:47]",
                f"v_mfma_f32_32x32x16_bf16 {g2}, v[80:83], v[84:87], {g2}",
                "v_mfma_f32_32x32x16_bf16 v[48:63], v[80:83], v[88:91], v[48:63]"]
    return ins, []


def rate(kind):
    ins = []
    for k in range(64):
        r = 100 + (k % 64)
        if kind == "exp":
            ins.append(f"v_exp_f32 v{r}, v{r}")
        elif kind == "fma_banks":  # sources in three different banks
            ins.append(f"v_fma_f32 v{r}, v{r}, v{r + 65}, v{r + 66}")
        elif kind == "add_chain":  # every add reads the previous one's result
            ins.append(f"v_add_f32 v99, v99, v{r}")
        elif kind == "exp_dep":  # exponential, then an add that reads it
            ins.append(f"v_exp_f32 v{r}, v{r}" if k % 2 == 0 else f"v_add_f32 v{r}, v{r - 1}, v{r + 64}")
        else:
            ins.append(f"v_fma_f32 v{r}, v{r}, v{r + 64}, v{r + 65}")
    return ins, []


def fwd_dep(order):
    """One statistics-kernel step per list entry pair (two steps per body, buffers swapped).
    Registers: score tiles v[0:15] / v[16:31]; weights (packed) v[64:71] / v[72:79]; Q
    operands v[80:95]; K row operands v[96:111] / v[212:227]; V^T operands v[112:127] /
    v[228:243]; element temporaries v[128:159]; step sum v200, row sum v201, -m v202,
    scale v247; accumulators a[0:31]."""
    use_m = order != "skewed_valu"
    use_v = order != "skewed_mfma"

    def elem_pair(sbuf, pbuf, p):
        a, b = 2 * p, 2 * p + 1
        ta, tb = 128 + a, 128 + b
        ex = "v_mov_b32" if order == "skewed_noexp" else "v_exp_f32"
        if order == "skewed_banks":
            # no two VGPR sources of one instruction in the same bank (bank = register
            # number mod 4): the scale as an inline constant, -m in v202 (bank 2) for
            # elements in banks 0/1 and in v205 (bank 1) for banks 2/3, and two partial
            # sums, v203 (bank 3) for the even elements and v206 (bank 2) for the odd ones
            nm = "v202" if a % 4 < 2 else "v205"
            out = [f"v_fma_f32 v{ta}, v{sbuf + a}, 0.5, {nm}", f"v_fma_f32 v{tb}, v{sbuf + b}, 0.5, {nm}",
                   f"{ex} v{ta}, v{ta}", f"{ex} v{tb}, v{tb}",
                   f"v_add_f32 v203, v203, v{ta}", f"v_add_f32 v206, v206, v{tb}",
                   f"v_cvt_pk_bf16_f32 v{pbuf + p}, v{ta}, v{tb}"]
            return out
        out = [f"v_fma_f32 v{ta}, v{sbuf + a}, v247, v202", f"v_fma_f32 v{tb}, v{sbuf + b}, v247, v202",
               f"{ex} v{ta}, v{ta}", f"{ex} v{tb}, v{tb}",
               (f"v_add_f32 v200, v{ta}, v{tb}" if p == 0 else f"v_add_f32 v200, v200, v{ta}"),
               f"v_cvt_pk_bf16_f32 v{pbuf + p}, v{ta}, v{tb}"]
        if p > 0:
            out.insert(5, f"v_add_f32 v200, v200, v{tb}")
        return out

    def step(s_next, s_cur, p_cur, p_prev, ob):
        """s_next: tile the score products write; s_cur: tile the weights read; p_cur: weights
        written; p_prev: weights the P V products read; ob: operand buffer (0/1)."""
        krow, vtr = (96, 112) if ob == 0 else (212, 228)
        nk, nv = (212, 228) if ob == 0 else (96, 112)
        score = [f"v_mfma_f32_32x32x16_bf16 v[{s_next}:{s_next + 15}], v[{krow + 4 * t}:{krow + 4 * t + 3}], "
                 f"v[{80 + 4 * t}:{80 + 4 * t + 3}], " + ("0" if t == 0 else f"v[{s_next}:{s_next + 15}]")
                 for t in range(4)]
        pv = [f"v_mfma_f32_32x32x16_bf16 a[{16 * (i % 2)}:{16 * (i % 2) + 15}], v[{vtr + 4 * i}:{vtr + 4 * i + 3}], "
              f"v[{p_prev + 4 * (i // 2)}:{p_prev + 4 * (i // 2) + 3}], a[{16 * (i % 2)}:{16 * (i % 2) + 15}]"
              for i in range(4)]
        valu = [x for p in range(8) for x in elem_pair(s_cur, p_cur, p)]
        if order == "skewed_banks":
            valu += ["v_add_f32 v200, v203, v206", "v_add_f32 v201, v201, v200", "v_cmp_ge_u32 vcc, v200, v247"]
        else:
            valu += ["v_add_f32 v201, v201, v200", "v_cmp_ge_u32 vcc, v200, v247"]
        reads = [f"ds_read_b128 v[{nk + 4 * t}:{nk + 4 * t + 3}], v244 offset:{t * 1024}" for t in range(4)]
        reads += [f"ds_read_b64_tr_b16 v[{nv + 2 * i}:{nv + 2 * i + 1}], v246 offset:{4096 + i * 512}"
                  for i in range(8)]
        if not use_m:
            score, pv = [], []
        if not use_v:
            valu = []
        ins = []
        if order == "phased":
            # this step's tile: score products, then (after the chain completes) the weights,
            # then the P V products; the operand reads of the next step go out with the products
            ins += score
            ins += reads[:4]
            ins += valu
            ins += ["s_nop 1"]
            ins += pv
            ins += reads[4:]
        else:
            mf = [x for pair in zip(score, pv) for x in pair] if use_m else []
            per = -(-len(valu) // max(1, len(mf))) if mf else len(valu)
            rd = list(reads)
            for k in range(max(len(mf), 1)):
                if k < len(mf):
                    ins.append(mf[k])
                ins += valu[:per]
                valu = valu[per:]
                if k >= 1:
                    ins += rd[:2]
                    rd = rd[2:]
            ins += valu + rd
        ins += ["s_waitcnt lgkmcnt(0)", "s_barrier"]
        return ins

    if order == "phased":
        a = step(0, 0, 64, 64, 0)
        b = step(16, 16, 72, 72, 1)
    else:
        # step j: products write tile (j+2)%2, weights read tile (j+1)%2 and write pack (j+1)%2,
        # P V reads pack j%2
        a = step(0, 16, 72, 64, 0)
        b = step(16, 0, 64, 72, 1)
    return _mfma_read_waits(a + b), []


def _regs(op):
    """VGPR numbers an operand names (v5, v[0:15]); none for AGPRs, constants, vcc."""
    import re
    m = re.fullmatch(r"v(\d+)", op) or re.fullmatch(r"v\[(\d+):(\d+)\]", op)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def _mfma_read_waits(ins, need=19):
    """Insert s_nop before any vector instruction that reads a VGPR an MFMA wrote fewer than
    `need` wait states earlier (the loop body repeats, so the scan runs over it twice)."""
    def ops(x):
        parts = x.replace(",", " ").split()
        return parts[0], parts[1:]

    out, last = [], {}
    for rep in range(2):
        pos = 0
        res = []
        for x in ins:
            op, args = ops(x)
            if op.startswith("v_") and not op.startswith("v_mfma") and args:
                reads = set().union(*[_regs(a) for a in args[1:]]) if len(args) > 1 else set()
                gap = min([pos - last[r] for r in reads if r in last] or [need])
                if gap < need:
                    res.append(f"s_nop {need - gap - 1}")
                    pos += need - gap
            if op.startswith("v_mfma") and args[0].startswith("v"):
                for r in _regs(args[0]):
                    last[r] = pos
            pos += int(op == "s_nop" and args[0]) + 1 if op == "s_nop" else 1
            res.append(x)
        out = res
        last = {r: v - pos for r, v in last.items()}
    return out


SKELETONS = ([(f"p1mix_{m}", p1_mix(m), 1) for m in ("mfma", "valu", "lds", "mfma_valu", "mfma_lds", "full")] +
             [(f"p1dep_{o}", p1_dep(o), 2) for o in ("interleaved", "phased")] +
             [(f"p2dep_split{s}", p2_dep(s), 2) for s in (0, 2, 4)] +
             [(f"gchain_{n}", gchain(s), 1) for n, s in (("one_chain", False), ("split", True))] +
             [(f"rate_{k}", rate(k), 64) for k in ("fma", "exp")] +
             [(f"fwddep_{o}", fwd_dep(o), 2) for o in ("phased", "skewed", "skewed_noexp", "skewed_mfma",
                                                          "skewed_valu", "skewed_banks")] +
             [(f"rate_{k}", rate(k), 64) for k in ("fma_banks", "add_chain", "exp_dep")])


def _skeleton_kernel(name, ins, addr_regs):
    """A kernel issuing `ins` (steps_per_body steps) per loop trip. addr_regs: the VGPRs
    the body reads LDS addresses (or constants) from, set at the start of each trip."""
    clob = ", ".join([f'"v{i}"' for i in range(0, 252)] + [f'"a{i}"' for i in range(0, 256)])
    return f'''
__global__ __launch_bounds__(256, 1) void {name}(unsigned long long* out, int trips) {{
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384; i += 256) reinterpret_cast<float*>(lds)[i] = 0.25f;
  __syncthreads();
  const unsigned a_row = lane * 16, a_tr = lane * 8, a_sc = (lane >> 5) * 16;
  unsigned long long t0, t1;
  asm volatile("s_memtime %0\\n\\ts_waitcnt lgkmcnt(0)" : "=s"(t0));
  for (int s = 0; s < trips; ++s) {{
    asm volatile(
      "v_mov_b32 v80, %0\\n\\tv_mov_b32 v81, %1\\n\\tv_mov_b32 v244, %0\\n\\tv_mov_b32 v245, %2\\n\\t"
      "v_mov_b32 v246, %1\\n\\tv_mov_b32 v250, %1\\n\\tv_mov_b32 v247, 0.125\\n\\ts_nop 1\\n\\t"
      "{_esc(ins)}"
      :: "v"(a_row), "v"(a_tr), "v"(a_sc)
      : "memory", {clob});
  }}
  asm volatile("s_nop 7\\n\\ts_nop 7\\n\\ts_nop 7\\n\\ts_memtime %0\\n\\ts_waitcnt lgkmcnt(0)" : "=s"(t1));
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = t1 - t0;
}}
'''


STATIC = r'''
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- matrix-core rate: independent chains, two waves per SIMD --------------------------
__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(float* out, unsigned long long* clk, int iters) {
  const int t = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * ((t + i) & 7));
    b[i] = (__bf16)(0.002f * ((t * 3 + i) & 7));
  }
  f32x16 acc[6];
  for (int c = 0; c < 6; ++c)
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 6; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int c = 0; c < 6; ++c)
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[blockIdx.x * 256 + t] = s;
  if (t == 0) {
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// ---- LDS read rates (8 reads per asm block, waited in the block; addresses < 32 KiB) ------
template <int MODE>
__global__ __launch_bounds__(256) void lds_rate_kernel(unsigned long long* cyc, unsigned* out, int iters) {
  __shared__ __align__(16) unsigned char buf[32768];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 32768 / 4; i += 256) reinterpret_cast<unsigned*>(buf)[i] = i * 2654435761u;
  __syncthreads();
  unsigned acc = 0;
  int addr;
  if (MODE == 0) addr = wave * 8192 + lane * 16;
  else if (MODE == 1) addr = wave * 8192 + lane * 8;
  else {
    const int r = (lane >> 2) & 15, c = lane & 3;
    addr = wave * 8192 + r * 128 + ((((c >> 1) ^ ((r >> 1) & 7)) << 4) | ((c & 1) << 3));
  }
  const unsigned a = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)(buf + addr);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) {
      uint4 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\tds_read_b128 %2, %8 offset:2048\n\t"
                   "ds_read_b128 %3, %8 offset:3072\n\tds_read_b128 %4, %8 offset:4096\n\t"
                   "ds_read_b128 %5, %8 offset:5120\n\tds_read_b128 %6, %8 offset:6144\n\t"
                   "ds_read_b128 %7, %8 offset:7168\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
                   : "v"(a) : "memory");
      acc ^= v0.x ^ v1.x ^ v2.x ^ v3.x ^ v4.x ^ v5.x ^ v6.x ^ v7.w;
    } else if constexpr (MODE == 1) {
      uint2 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile("ds_read_b64 %0, %8\n\tds_read_b64 %1, %8 offset:1024\n\tds_read_b64 %2, %8 offset:2048\n\t"
                   "ds_read_b64 %3, %8 offset:3072\n\tds_read_b64 %4, %8 offset:4096\n\t"
                   "ds_read_b64 %5, %8 offset:5120\n\tds_read_b64 %6, %8 offset:6144\n\t"
                   "ds_read_b64 %7, %8 offset:7168\n\ts_waitcnt lgkmcnt(0)"
                   : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
                   : "v"(a) : "memory");
      acc ^= v0.x ^ v1.x ^ v2.x ^ v3.x ^ v4.x ^ v5.x ^ v6.x ^ v7.y;
    } else {
      uint2 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile("ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:512\n\t"
                   "ds_read_b64_tr_b16 %2, %8 offset:1024\n\tds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
                   "ds_read_b64_tr_b16 %4, %8 offset:2048\n\tds_read_b64_tr_b16 %5, %8 offset:2560\n\t"
                   "ds_read_b64_tr_b16 %6, %8 offset:3072\n\tds_read_b64_tr_b16 %7, %8 offset:3584\n\t"
                   "s_waitcnt lgkmcnt(0)"
                   : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
                   : "v"(a) : "memory");
      acc ^= v0.x ^ v1.x ^ v2.x ^ v3.x ^ v4.x ^ v5.x ^ v6.x ^ v7.y;
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * 256 + tid] = acc;
  if (lane == 0) cyc[blockIdx.x * 4 + wave] = t1 - t0;
}

static bool ok(hipError_t e) { return e == hipSuccess; }

static int run_mfma_rate(float* fbuf, unsigned long long* clk) {
  std::vector<unsigned long long> h(2 * 512);
  const int blocks = 512, iters = 200000;  // two waves per SIMD, about a third of a second
  double best = 0, ghz = 0;
  for (int rep = 0; rep < 3; ++rep) {
    hipEvent_t e0, e1;
    if (!ok(hipEventCreate(&e0)) || !ok(hipEventCreate(&e1))) return 1;
    if (!ok(hipEventRecord(e0, 0))) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, 0, fbuf, clk, iters);
    if (!ok(hipEventRecord(e1, 0)) || !ok(hipEventSynchronize(e1))) return 1;
    float ms = 0;
    if (!ok(hipEventElapsedTime(&ms, e0, e1))) return 1;
    if (!ok(hipMemcpy(h.data(), clk, h.size() * 8, hipMemcpyDeviceToHost))) return 1;
    double g = 0;
    for (int b = 0; b < blocks; ++b) g += (double)h[2 * b] / (double)h[2 * b + 1] * 0.1;
    const double tf = (double)blocks * 4 * iters * 6 * 32768.0 / (ms * 1e-3) / 1e12;
    if (tf > best) { best = tf; ghz = g / blocks; }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  printf("mfma_rate: %.1f TFLOP/s\nmfma_rate_clock: %.3f GHz\n", best, ghz);
  return 0;
}

template <int MODE>
static int run_lds(const char* name, double bytes, unsigned long long* cyc, unsigned* ubuf) {
  std::vector<unsigned long long> h(1024 * 4);
  const int iters = 4096;
  for (int blocks : {256, 512, 1024}) {
    for (int rep = 0; rep < 2; ++rep) hipLaunchKernelGGL(lds_rate_kernel<MODE>, dim3(blocks), dim3(256), 0, 0, cyc, ubuf, iters);
    if (!ok(hipDeviceSynchronize())) return 1;
    if (!ok(hipMemcpy(h.data(), cyc, blocks * 4 * 8, hipMemcpyDeviceToHost))) return 1;
    double s = 0;
    for (int i = 0; i < blocks * 4; ++i) s += h[i];
    const double avg = s / (blocks * 4);
    const int wpc = blocks * 4 / 256;
    printf("lds_rate_%s_%dwaves: %.1f B/clk/CU\n", name, wpc, wpc * bytes * 8.0 * iters / avg);
  }
  return 0;
}

static int run_skeleton(const char* name, void (*k)(unsigned long long*, int), int steps_per_trip,
                        unsigned long long* out) {
  const int blocks = 256, trips = 1000;  // one wave per SIMD
  if (!ok(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, 65536))) return 1;
  std::vector<unsigned long long> h(blocks * 4);
  for (int rep = 0; rep < 3; ++rep) hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 65536, 0, out, trips);
  if (!ok(hipDeviceSynchronize())) return 1;
  if (!ok(hipMemcpy(h.data(), out, h.size() * 8, hipMemcpyDeviceToHost))) return 1;
  double s = 0;
  for (auto v : h) s += v;
  printf("%s: %.1f cycles/step\n", name, s / h.size() / ((double)trips * steps_per_trip));
  return 0;
}
'''


def render():
    parts = ["// Generated by probes_gen.py (same directory); do not edit by hand.",
             "// Microbenchmarks and skeleton kernels behind the bound analysis of the kernels.",
             "#include <hip/hip_runtime.h>", "#include <cstdio>", "#include <vector>", STATIC]
    for name, (ins, _), _steps in SKELETONS:
        parts.append(_skeleton_kernel(name, ins, None))
    main = ["int main() {", "  float* fbuf; unsigned long long* clk; unsigned long long* cyc; unsigned* ubuf;",
            "  if (!ok(hipMalloc(&fbuf, 1024 * 256 * 4)) || !ok(hipMalloc(&clk, 2048 * 8)) ||",
            "      !ok(hipMalloc(&cyc, 4096 * 8)) || !ok(hipMalloc(&ubuf, 1024 * 256 * 4))) return 1;",
            "  if (run_mfma_rate(fbuf, clk)) return 1;",
            '  if (run_lds<0>("b128", 1024.0, cyc, ubuf) || run_lds<1>("b64", 512.0, cyc, ubuf) ||',
            '      run_lds<2>("tr_b64", 512.0, cyc, ubuf)) return 1;']
    for name, _, steps in SKELETONS:
        main.append(f'  if (run_skeleton("{name}", {name}, {steps}, cyc)) return 1;')
    main += ['  printf("status: %s\\n", hipGetErrorString(hipGetLastError()));', "  return 0;", "}"]
    parts.append("\n".join(main))
    return "\n".join(parts) + "\n"


def main():
    with open(OUT, "w") as fh:
        fh.write(render())
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
