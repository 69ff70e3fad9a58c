"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one: a dropped term, a wrong sign, a wrong or transposed
operand, a missing scale, a wrong reduction axis."""

import os
import types

import pytest

from oracle_pins import PINS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "bob.py")

# (label, text in oracle/bob.py, replacement)
MUTANTS = [
    ("drop H (dV node into bar_P)", "bar_p = do_r @ uv.T", "bar_p = 0.0 * (do_r @ uv.T)"),
    ("transposed H operands", "bar_p = do_r @ uv.T", "bar_p = uv[r0:r1] @ do.T"),
    ("drop P UV in gdO", "bar_do = p @ uv", "bar_do = 0.0 * (p @ uv)"),
    ("wrong operand UQ for UK in gQ", "bar_q = tau * (ds @ uk)", "bar_q = tau * (ds @ uq)"),
    ("swap roles in dK cotangent", "bar_ds = tau * (q_r @ uk.T)", "bar_ds = tau * (uk[r0:r1] @ q.T)"),
    ("drop tau in dQ cotangent", "bar_ds = bar_ds + tau * (uq_r @ k.T)", "bar_ds = bar_ds + (uq_r @ k.T)"),
    ("drop D in dS node", "bar_p = bar_p + bar_ds * (dp - dd[:, None])", "bar_p = bar_p + bar_ds * dp"),
    ("sign of alpha", "bar_dd = -np.sum(bar_ds * p, axis=1)", "bar_dd = np.sum(bar_ds * p, axis=1)"),
    ("drop D node into bar_P", "bar_p = bar_p + bar_dd[:, None] * dp", "bar_p = bar_p"),
    ("drop D node into bar_dP", "bar_dp = bar_dp + bar_dd[:, None] * p", "bar_dp = bar_dp"),
    ("wrong operand in gdO", "bar_do = bar_do + bar_dp @ v", "bar_do = bar_do + bar_dp @ k"),
    ("drop E in softmax node", "bar_s = p * (bar_p - e_row[:, None])", "bar_s = p * bar_p"),
    ("column sum for E", "e_row = np.sum(p * bar_p, axis=1)", "e_row = np.sum(p * bar_p, axis=0)"),
    ("drop tau in S node", "bar_q = bar_q + tau * (bar_s @ k)", "bar_q = bar_q + (bar_s @ k)"),
    ("drop dS^T UQ in gK", "g_k += tau * (t[\"_ds\"].T @ t[\"_uq\"]) + ", "g_k += "),
    ("wrong operand in gV", "g_v += t[\"_bar_dp\"].T @ t[\"_do\"]", "g_v += t[\"_bar_dp\"].T @ t[\"_q\"]"),
    ("column routine drops dS^T UQ", "g_k += tau * (t[\"_ds\"][:, cols].T @ t[\"_uq\"]) + ", "g_k += "),
    ("column routine uses Q for dO", "g_v += t[\"_bar_dp\"][:, cols].T @ t[\"_do\"]",
     "g_v += t[\"_bar_dp\"][:, cols].T @ t[\"_q\"]"),
    ("D without P", "dd = np.sum(p * dp, axis=1)\n    ds = p * (dp - dd[:, None])\n\n    # node dV",
     "dd = np.sum(dp, axis=1) / dp.shape[1]\n    ds = p * (dp - dd[:, None])\n\n    # node dV"),
    ("causal mask off by one", "s[cols[None, :] > row_idx[:, None]] = -np.inf", "s[cols[None, :] >= row_idx[:, None] + 2] = -np.inf"),
    ("first backward: dK untransposed", "return tau * (ds @ k), tau * (ds.T @ q)", "return tau * (ds @ k), tau * (ds @ q)"),
    ("LSE without the max shift", "lse = (m + np.log(z))[:, 0]", "lse = np.log(z)[:, 0]"),
]

# the sympy pin is slow; every mutant must be caught by the others
FAST_PINS = {k: v for k, v in PINS.items() if k != "sympy_exact"}


def _load_mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant.py", "exec"), mod.__dict__)
    return mod


def _caught(mod):
    failed = []
    for name, (pin, bound) in FAST_PINS.items():
        try:
            err = pin(mod)
        except Exception as exc:  # a crash also counts as caught
            failed.append(f"{name} (raised {type(exc).__name__})")
            continue
        if not (err <= bound):
            failed.append(name)
    return failed


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(label, old, new):
    failed = _caught(_load_mutant(old, new))
    assert failed, f"no pin caught the planted mistake: {label}"


def test_unmutated_copy_passes():
    src = open(ORACLE_SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy.py", "exec"), mod.__dict__)
    assert _caught(mod) == []
