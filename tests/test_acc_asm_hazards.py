"""Matrix-core hazard waits around inline assembly, checked on the built gfx950 code.

The two-pass sweeps compiled in matrix-core VGPR form (bob_pass1_vgpr.hip,
bob_pass2_vgpr.hip) issue matrix-core products the compiler cannot see: the
accumulating products of mfma_acc (AGPR tiles) and the scheduled pass-1 step loop.
The compiler therefore inserts no waits for them, and the code supplies its own: an
s_nop 1 in front of each accumulating product, the settle waits after a sweep, the
generator's schedule inside the loop. A change of toolchain could still place a copy
of an accumulator, or some other access, inside one of those windows.

This test compiles both files to assembly with the library's own flags and walks
every kernel's control-flow graph (branches, loops, the loop's own labels included),
tracking per register how many wait states have passed since the last product that
wrote it and since the last vector instruction that wrote it. Wherever at least one
side is inline assembly it requires
  - 19 wait states between a product writing a register and any non-product
    instruction reading or writing it (a 16-pass product's result needs 18), and
    between such a product and another product reading it as source A or B (a
    product reading its own destination as source C, the accumulation chain, is
    exempt);
  - 2 wait states between a vector instruction writing a register and a product
    reading it as source A or B.
Pairs the compiler sees on both sides are its own to order. Wait states are counted
as the library's generator counts them: s_nop N gives N + 1, every other instruction 1.
"""

import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

FILES = ["bob_pass1_vgpr.hip", "bob_pass2_vgpr.hip", "pass1_q16.hip"]
PRODUCT_TO_ACCESS = 19
VALU_TO_PRODUCT = 2
CAP = 32  # gaps at or above this no longer matter

REG = re.compile(r"^-?([va])(?:(\d+)|\[(\d+):(\d+)\])$")
LABEL = re.compile(r"^([.\w$]+):\s*(?:;.*)?$")
BRANCH = re.compile(r"^s_(?:c?branch\w*)\s+([.\w$]+)")


def _regs(op):
    m = REG.match(op.strip())
    if not m:
        return []
    kind = m.group(1)
    if m.group(2) is not None:
        return [f"{kind}{m.group(2)}"]
    return [f"{kind}{n}" for n in range(int(m.group(3)), int(m.group(4)) + 1)]


def _split_ops(rest):
    return [o.strip() for o in re.split(r",(?![^\[]*\])", rest) if o.strip()]


class Ins:
    __slots__ = ("op", "ops", "asm", "ws", "text")

    def __init__(self, text, asm):
        parts = text.split(None, 1)
        self.op = parts[0]
        # comma-separated operands; modifiers after the last one (offset:, glc, ...) stay
        # attached to it and are dropped where registers are read
        self.ops = _split_ops(parts[1]) if len(parts) > 1 else []
        self.asm = asm
        self.text = text
        m = re.match(r"s_nop\s+(\d+)", text)
        self.ws = int(m.group(1)) + 1 if m else 1

    @property
    def is_product(self):
        return self.op.startswith("v_mfma")

    def access(self):
        """(destination registers, source registers) of a vector-register instruction."""
        op, ops = self.op, [o.split()[0] if o else o for o in self.ops]
        regs = [_regs(o) for o in ops]
        if op.startswith(("ds_write", "ds_store", "global_store", "buffer_store", "flat_store", "scratch_store",
                          "global_load_lds", "buffer_load_lds")):
            return [], [r for rs in regs for r in rs]
        if op.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
            if not regs:
                return [], []
            return regs[0], [r for rs in regs[1:] for r in rs]
        return [], []


def _body(text):
    """Instructions and labels of one function's body, in layout order."""
    items, in_asm = [], False
    for raw in text.splitlines():
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line or line.startswith((";", "//")):
            continue
        m = LABEL.match(line)
        if m:
            items.append(("label", m.group(1)))
            continue
        if line.startswith("."):
            continue
        items.append(Ins(line.split(";")[0].split("//")[0].strip(), in_asm))
    return items


def _parse(text):
    """{kernel symbol: body items} for every function the assembly defines."""
    funcs = {}
    for name in set(re.findall(r"\.type\s+(_Z\w+),@function", text)):
        i = text.index(f"\n{name}:") + len(name) + 2
        j = text.index(".Lfunc_end", i)
        funcs[name] = _body(text[i:j])
    return funcs


def _blocks(items):
    """Basic blocks: list of (instructions, successor indices)."""
    blocks, labels, cur = [], {}, []
    ends = []  # per block: ('fall' | 'jump' | 'cond' | 'stop', target label)

    def close(kind, target=None):
        nonlocal cur
        blocks.append(cur)
        ends.append((kind, target))
        cur = []

    for it in items:
        if isinstance(it, tuple):
            if cur:
                close("fall")
            labels[it[1]] = len(blocks)
            continue
        cur.append(it)
        m = BRANCH.match(it.text)
        if it.op == "s_branch" and m:
            close("jump", m.group(1))
        elif it.op.startswith("s_cbranch") and m:
            close("cond", m.group(1))
        elif it.op in ("s_endpgm", "s_setpc_b64"):
            close("stop")
    if cur:
        close("stop")
    succ = []
    for b, (kind, target) in enumerate(ends):
        s = []
        if kind in ("jump", "cond"):
            assert target in labels, f"branch to unknown label {target}"
            s.append(labels[target])
        if kind in ("fall", "cond") and b + 1 < len(blocks):
            s.append(b + 1)
        succ.append(s)
    return blocks, succ


def _run_block(ins, state, errors=None):
    """Simulate one block from its entry gaps; return the exit gaps.
    state: dict kind -> {reg: gap} for kinds 'pa' (product in inline asm), 'pc' (compiled
    product), 'va', 'vc' (vector writes, asm / compiled)."""
    last = {k: {r: -g for r, g in d.items()} for k, d in state.items()}
    pos = 0
    for x in ins:
        dst, src = x.access()
        if dst or src:
            exempt = set()
            if x.is_product and len(x.ops) >= 4 and x.ops[3].split()[0] == x.ops[0].split()[0]:
                exempt = set(dst)  # accumulation chain: source C is the destination
            # sources A and B of a product; every other access of a non-product
            ab = set(r for o in x.ops[1:3] for r in _regs(o.split()[0])) if x.is_product else set()
            touched = (ab | (set(dst) - exempt) | (set(src) - ab - exempt)) if x.is_product else set(dst) | set(src)
            kinds = ("pa", "pc") if x.asm else ("pa",)
            for k in kinds:
                for r in touched:
                    if r in last[k] and pos - last[k][r] < PRODUCT_TO_ACCESS and errors is not None:
                        errors.append(f"{x.text}: {r} {pos - last[k][r]} wait states after a product")
            if x.is_product:
                kinds = ("va", "vc") if x.asm else ("va",)
                for k in kinds:
                    for r in ab:
                        if r in last[k] and pos - last[k][r] < VALU_TO_PRODUCT and errors is not None:
                            errors.append(f"{x.text}: {r} {pos - last[k][r]} wait states after a vector write")
            # the instruction's own writes
            for r in dst:
                for k in ("pa", "pc", "va", "vc"):
                    last[k].pop(r, None)
                if x.is_product:
                    last["pa" if x.asm else "pc"][r] = pos + x.ws
                elif x.op.startswith("v_"):
                    last["va" if x.asm else "vc"][r] = pos + x.ws
        pos += x.ws
    return {k: {r: pos - p for r, p in d.items() if pos - p < CAP} for k, d in last.items()}


def _merge(states):
    out = {k: {} for k in ("pa", "pc", "va", "vc")}
    for st in states:
        for k, d in st.items():
            o = out[k]
            for r, g in d.items():
                if r not in o or g < o[r]:
                    o[r] = g
    return out


def check_function(items):
    blocks, succ = _blocks(items)
    preds = [[] for _ in blocks]
    for b, s in enumerate(succ):
        for t in s:
            preds[t].append(b)
    empty = {k: {} for k in ("pa", "pc", "va", "vc")}
    out = [None] * len(blocks)
    for _ in range(50):
        changed = False
        for b in range(len(blocks)):
            ins_state = _merge([out[p] for p in preds[b] if out[p] is not None]) if preds[b] else empty
            new = _run_block(blocks[b], ins_state)
            if new != out[b]:
                out[b], changed = new, True
        if not changed:
            break
    else:
        raise AssertionError("gap propagation did not settle")
    errors = []
    for b in range(len(blocks)):
        ins_state = _merge([out[p] for p in preds[b] if out[p] is not None]) if preds[b] else empty
        _run_block(blocks[b], ins_state, errors)
    return errors


def _compile_asm(src, out):
    import aware_flashbob_pass_amd.build as B

    flags = [f for f in B.COMMON_FLAGS if f != "-fPIC"]
    cmd = [B.hipcc(), *flags, *B.EXTRA_FLAGS.get(src, []), "-S", "--cuda-device-only", "-o", out,
           os.path.join(B.CSRC, src)]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


@pytest.fixture(scope="module")
def assembly():
    try:
        import aware_flashbob_pass_amd.build as B

        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="fb_hazards_")
    procs = {src: (_compile_asm(src, os.path.join(tmp, src + ".s")), os.path.join(tmp, src + ".s")) for src in FILES}
    out = {}
    for src, (p, path) in procs.items():
        log = p.communicate()[0]
        assert p.returncode == 0, log[-2000:]
        out[src] = open(path).read()
    return out


@pytest.mark.parametrize("src", FILES)
def test_inline_products_have_their_waits(assembly, src):
    funcs = _parse(assembly[src])
    checked = 0
    for name, items in funcs.items():
        if not any(isinstance(x, Ins) and x.asm and x.is_product for x in items):
            continue
        checked += 1
        errors = check_function(items)
        assert not errors, f"{name}: {errors[:5]}"
    assert checked > 0, "no kernel with inline-assembly products found"


def test_checker_catches_a_missing_settle_wait():
    """A product in inline assembly, then a compiled read of its destination after too
    few wait states (directly, and across a branch), is reported; enough waits pass."""
    def prog(nops, branch):
        items = [Ins("v_mov_b32 v0, 0", False), Ins("s_nop 1", True),
                 Ins("v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]", True)]
        items += [Ins("s_nop 7", True)] * nops
        if branch:
            items += [Ins("s_cbranch_scc1 .LBB0_2", False), ("label", ".LBB0_1"), Ins("s_nop 0", False),
                      ("label", ".LBB0_2")]
        items += [Ins("v_accvgpr_read_b32 v8, a3", False), Ins("s_endpgm", False)]
        return items

    for branch in (False, True):
        assert check_function(prog(0, branch)), "missing settle not reported"
        assert check_function(prog(2, branch)), "16 wait states reported as enough"
        assert not check_function(prog(3, branch)), "24 wait states reported as too few"


def test_checker_catches_a_loop_carried_hazard():
    """A loop whose last instruction is a product and whose first reads its result."""
    items = [("label", ".LBB0_1"), Ins("v_add_f32 v20, v0, v1", True), Ins("s_nop 1", True),
             Ins("v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0", True),
             Ins("s_cbranch_scc1 .LBB0_1", False), Ins("s_endpgm", False)]
    errs = check_function(items)
    assert any("after a product" in e for e in errs)
    # the vector write two wait states before the product is fine; one is not
    items2 = [Ins("v_add_f32 v20, v0, v1", True), Ins("v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]",
                                                     True), Ins("s_endpgm", False)]
    assert any("after a vector write" in e for e in check_function(items2))
