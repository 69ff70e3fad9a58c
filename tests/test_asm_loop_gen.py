"""The generated inline-assembly step loop of pass 1 (non-causal d = 64 bf16 sweep):
the committed include matches its generator, and an independent replay of every
generated step checks the waits and register use the schedule relies on."""

import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "aware_flashbob_pass_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_pass1_asm", os.path.join(CSRC, "gen_pass1_asm.py"))
    g = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(g)
    return g


def _regs(op):
    """Register numbers of one operand: ('v' | 'a', [n, ...]) or None."""
    m = re.fullmatch(r"([va])(\d+)", op)
    if m:
        return m.group(1), [int(m.group(2))]
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", op)
    if m:
        return m.group(1), list(range(int(m.group(2)), int(m.group(3)) + 1))
    return None


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    ops = [o.strip() for o in re.split(r",(?![^\[]*\])", parts[1])]
    return parts[0], ops


def test_include_is_generated():
    g = _gen()
    with open(os.path.join(CSRC, "pass1_asm_loop.inc")) as fh:
        assert fh.read() == g.render(), "pass1_asm_loop.inc is stale: run gen_pass1_asm.py"


def _replay(ins):
    """Walk one instruction list with an in-order LDS return queue (the LDS returns in
    issue order, so lgkmcnt(N) retires all but the newest N reads). Checks: no matrix
    product or vector instruction reads a register an LDS read still has in flight; a
    matrix product does not read a VGPR written by a vector instruction in the two
    instructions before it; nothing reads a transcendental result in the next
    instruction; a vector instruction reads a matrix product's result only 19 or more
    wait states after the product (a 16-pass product needs 19; these are 8-pass).
    Returns the set of registers written."""
    inflight = []  # list of sets of ('v'|'a', n)
    last_mfma = {}
    last_valu = {}  # ('v', n) -> index of the vector instruction that wrote it
    last_trans = {}
    written = set()
    for i, line in enumerate(ins):
        op, ops = _operands(line)
        if op.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", line)
            if m:
                keep = int(m.group(1))
                inflight = inflight[len(inflight) - keep:] if keep < len(inflight) else inflight
            continue
        if op.startswith("ds_read"):
            kind, regs = _regs(ops[0])
            dst = {(kind, r) for r in regs}
            inflight.append(dst)
            written |= dst
            continue
        if op.startswith("v_"):
            srcs = set()
            dst = set()
            for k, o in enumerate(ops):
                r = _regs(o.lstrip("-"))
                if r:
                    (dst if k == 0 else srcs).update((r[0], n) for n in r[1])
            pending = set().union(*inflight) if inflight else set()
            assert not (srcs & pending), f"{line}: reads an LDS result still in flight"

            def gap_since(j):
                return sum(int(x.split()[1]) + 1 if x.startswith("s_nop") else 1 for x in ins[j + 1:i])

            if op.startswith("v_mfma"):
                for reg in dst:
                    last_mfma[reg] = i
                for reg in srcs:
                    if reg in last_valu:
                        gap = gap_since(last_valu[reg])
                        assert gap >= 2, f"{line}: {reg} written by a vector instruction {gap} wait states before"
            else:
                for reg in srcs:
                    if reg in last_mfma:
                        assert gap_since(last_mfma[reg]) >= 19, f"{line}: reads {reg} too soon after a product"
                    if reg in last_trans:
                        assert i - last_trans[reg] >= 2, f"{line}: reads a transcendental result too early"
                for reg in dst:
                    last_valu[reg] = i
                    last_trans.pop(reg, None)
                    if op == "v_exp_f32":
                        last_trans[reg] = i
            written |= dst
    assert not inflight, "LDS reads left in flight at the end of the step"
    return written


def test_generated_steps_respect_waits_and_hazards():
    g = _gen()
    declared = {("v", n) for n in range(64, 243)} | {("v", n) for n in (254, 255)} | {("v", n) for n in range(64)}
    if g.OPERANDS == "a":
        declared |= {("a", n) for n in range(176, 240)}
    declared |= {("a", n) for n in range(128)}  # accumulators: in/out operands
    for S in range(g.NBUF):
        written = _replay(g.step_body(S))
        assert written <= declared, sorted(written - declared)[:5]
        # the resident operands (inputs) and the addresses are never written
        assert not written & {("a", n) for n in range(128, 176)}
        assert not written & {("v", n) for n in range(243, 254)}


def test_clobbers_cover_every_written_register():
    """Every VGPR or AGPR the block writes (its prologue included) is either bound to an
    output (score tiles v[0:63], row sums v254 and v255, accumulators a[0:127]) or in
    its clobber list; no input register (v[243:253], a[128:175]) is written."""
    g = _gen()
    text = g.render()
    line = next(l for l in text.splitlines() if l.startswith("#define FB_PASS1_ASM_CLOBBERS"))
    clob = set(re.findall(r'"([va]\d+)"', line))
    written = set()
    for x in g.loop_text():
        op, ops = _operands(x)
        if (op.startswith("v_") or op.startswith("ds_read")) and ops:
            r = _regs(ops[0])
            if r:
                written |= {f"{r[0]}{n}" for n in r[1]}
    bound = {f"v{n}" for n in list(range(64)) + [254, 255]} | {f"a{n}" for n in range(128)}
    inputs = {f"v{n}" for n in range(243, 254)} | {f"a{n}" for n in range(128, 176)}
    assert not written & inputs
    assert written - bound <= clob, sorted(written - bound - clob)[:5]


SCALAR_OK = {"s_nop", "s_waitcnt", "s_mov_b32", "s_add_u32", "s_addc_u32", "s_cmp_lt_u32", "s_cmp_gt_u32",
             "s_cmp_ge_u32", "s_cbranch_scc0", "s_cbranch_scc1", "s_branch", "s_barrier"}


def test_generated_loop_uses_only_listed_scalar_instructions():
    """Scalar work in the loop is control and address arithmetic only: no scalar memory
    instructions of any kind (every store goes through vector memory)."""
    g = _gen()
    ins = g.loop_text()
    used = {x.split()[0] for x in ins if x.startswith("s_")}
    assert used <= SCALAR_OK, sorted(used - SCALAR_OK)
    vector_mem = {x.split()[0] for x in ins if x.startswith(("global_", "buffer_", "flat_"))}
    assert vector_mem == {"global_load_lds_dwordx4"}


@pytest.mark.parametrize("over", [dict(OPERANDS="v", DBIAS=False, PAIRS_A=(0, 1, 2, 3), PAIRS_B=(4, 5, 6, 7),
                                       PAIRS_C=(), VALU_FIRST=12, VALU_PER_SCORE=4, VALU_PER_ACC=8),
                                  dict(NBUF=8, AHEAD=6), dict(DOT_SUMS=True),
                                  dict(NBUF=6, AHEAD=4, BARRIER_EVERY=2)])
def test_generator_options_replay(over):
    """The options kept for measurement generate schedules that pass the same replay."""
    g = _gen()
    for k, v in over.items():
        setattr(g, k, v)
    g.render()
    for S in range(g.NBUF):
        _replay(g.step_body(S))


def test_replay_catches_a_missing_wait():
    """The replay is not vacuous: a step with its first LDS wait removed fails it."""
    g = _gen()
    ins = g.step_body(0)
    k = next(i for i, x in enumerate(ins) if x.startswith("s_waitcnt lgkmcnt"))
    with pytest.raises(AssertionError, match="in flight"):
        _replay(ins[:k] + ins[k + 1:])
