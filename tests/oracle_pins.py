"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each pin takes the oracle module (so that the mutation test can hand it a copy
with a planted mistake) and returns the worst relative error it saw; the caller
compares it with the pin's bound. The facts used:

* the definition of softmax attention, evaluated with scalar Python loops;
* central finite differences (the first backward is the gradient of
  <dO, O(Q,K,V)>, and BoB is the gradient of <U, g>);
* symmetry of second derivatives (g is a gradient, so its Jacobian in
  (Q, K, V) is a Hessian) and linearity of g in dO;
* the closed-form reduction of the review page (Strengths, Lemma E.2): with
  V = dO = UQ = UK = 0 and UV = W, the dO-cotangent is softmax(tau Q K^T) W and
  the other three are zero;
* invariances of attention (shifting every key or every value row by the same
  vector), which force the key and value cotangents to sum to zero over keys;
* torch's autograd double backward in float64 on the CPU (an independent
  implementation of reverse mode), and sympy's symbolic differentiation.
"""

import math

import numpy as np

RNG_SEED = 20240917


def _rand_case(n, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    names = ("q", "k", "v", "do", "uq", "uk", "uv")
    return {nm: scale * rng.standard_normal((n, d)) for nm in names}


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


def _g(mod, c, tau, causal):
    dq, dk, dv, _ = mod.first_backward_head(c["q"], c["k"], c["v"], c["do"], tau, causal)
    return dq, dk, dv


def _bob(mod, c, tau, causal, **kw):
    return mod.bob_head(c["q"], c["k"], c["v"], c["do"], c["uq"], c["uk"], c["uv"], tau, causal, **kw)


# ---------------------------------------------------------------- forward ----
def pin_forward_loops(mod):
    """O and L against the definition written with scalar loops (math.exp)."""
    worst = 0.0
    for causal in (False, True):
        c = _rand_case(5, 3, RNG_SEED + 1)
        tau = 0.7
        o, lse = mod.attention_forward_head(c["q"], c["k"], c["v"], tau, causal)
        n, d = c["q"].shape
        o_ref = np.zeros((n, d))
        l_ref = np.zeros(n)
        for i in range(n):
            keys = range(i + 1) if causal else range(n)
            s = {j: tau * sum(c["q"][i][t] * c["k"][j][t] for t in range(d)) for j in keys}
            z = math.fsum(math.exp(s[j]) for j in keys)
            l_ref[i] = math.log(z)
            for t in range(d):
                o_ref[i][t] = math.fsum(math.exp(s[j]) / z * c["v"][j][t] for j in keys)
        worst = max(worst, _rel(o, o_ref), _rel(lse, l_ref))
    return worst


# ----------------------------------------------------------- first backward --
def pin_first_backward_fd(mod):
    """Every element of (dQ, dK, dV) against the central difference of <dO, O>."""
    worst = 0.0
    eps = 1e-6
    for causal in (False, True):
        c = _rand_case(4, 3, RNG_SEED + 2)
        tau = 0.9

        def f(q, k, v):
            o, _ = mod.attention_forward_head(q, k, v, tau, causal)
            return float(np.sum(c["do"] * o))

        grads = _g(mod, c, tau, causal)
        for which, g_an in zip(("q", "k", "v"), grads):
            fd = np.zeros_like(g_an)
            for idx in np.ndindex(*g_an.shape):
                args = {nm: c[nm].copy() for nm in ("q", "k", "v")}
                args[which][idx] += eps
                fp = f(args["q"], args["k"], args["v"])
                args[which][idx] -= 2 * eps
                fm = f(args["q"], args["k"], args["v"])
                fd[idx] = (fp - fm) / (2 * eps)
            worst = max(worst, _rel(g_an, fd))
        # D has two forms: rowsum(P * dP) and the row dot product dO . O
        _, _, _, dd = mod.first_backward_head(c["q"], c["k"], c["v"], c["do"], tau, causal)
        o, _ = mod.attention_forward_head(c["q"], c["k"], c["v"], tau, causal)
        worst = max(worst, _rel(dd, np.sum(c["do"] * o, axis=1)))
    return worst


# --------------------------------------------------------------------- BoB ---
def pin_bob_fd_elementwise(mod):
    """Every element of the four BoB outputs against the central difference of
    <U, g(Q, K, V, dO)> with respect to that input element (tiny N)."""
    worst = 0.0
    eps = 1e-6
    for causal in (False, True):
        c = _rand_case(5, 3, RNG_SEED + 3)
        tau = 0.8

        def lu(cc):
            dq, dk, dv = _g(mod, cc, tau, causal)
            return float(np.sum(cc["uq"] * dq) + np.sum(cc["uk"] * dk) + np.sum(cc["uv"] * dv))

        out = _bob(mod, c, tau, causal)
        for which, key in (("q", "gQ"), ("k", "gK"), ("v", "gV"), ("do", "gdO")):
            fd = np.zeros_like(c[which])
            for idx in np.ndindex(*fd.shape):
                cc = dict(c)
                cc[which] = c[which].copy()
                cc[which][idx] += eps
                fp = lu(cc)
                cc[which][idx] -= 2 * eps
                fm = lu(cc)
                fd[idx] = (fp - fm) / (2 * eps)
            worst = max(worst, _rel(out[key], fd))
    return worst


def pin_bob_fd_directional(mod):
    """<U, g(x + eps v) - g(x - eps v)> / (2 eps) = <BoB(U), v> for random directions
    v over all of (Q, K, V, dO), at a size with several rows and columns."""
    worst = 0.0
    eps = 1e-5
    rng = np.random.default_rng(RNG_SEED + 4)
    for causal in (False, True):
        c = _rand_case(24, 8, RNG_SEED + 5)
        tau = 1.0 / math.sqrt(8)
        out = _bob(mod, c, tau, causal)
        for _ in range(3):
            dirs = {nm: rng.standard_normal(c[nm].shape) for nm in ("q", "k", "v", "do")}
            cp = dict(c)
            cm = dict(c)
            for nm in dirs:
                cp[nm] = c[nm] + eps * dirs[nm]
                cm[nm] = c[nm] - eps * dirs[nm]
            gp, gm = _g(mod, cp, tau, causal), _g(mod, cm, tau, causal)
            lhs = sum(float(np.sum(u * (a - b))) for u, a, b in zip((c["uq"], c["uk"], c["uv"]), gp, gm)) / (2 * eps)
            rhs = (np.sum(out["gQ"] * dirs["q"]) + np.sum(out["gK"] * dirs["k"])
                   + np.sum(out["gV"] * dirs["v"]) + np.sum(out["gdO"] * dirs["do"]))
            worst = max(worst, abs(lhs - rhs) / max(abs(rhs), 1e-300))
    return worst


def pin_hessian_symmetry(mod):
    """(gQ, gK, gV) = [g(x + eps U) - g(x - eps U)] / (2 eps): the Jacobian of g in
    (Q, K, V) is the Hessian of <dO, O>, which is symmetric. Checked per element."""
    worst = 0.0
    eps = 1e-5
    for causal in (False, True):
        c = _rand_case(16, 8, RNG_SEED + 6)
        tau = 0.35
        out = _bob(mod, c, tau, causal)
        cp, cm = dict(c), dict(c)
        for nm, un in (("q", "uq"), ("k", "uk"), ("v", "uv")):
            cp[nm] = c[nm] + eps * c[un]
            cm[nm] = c[nm] - eps * c[un]
        gp, gm = _g(mod, cp, tau, causal), _g(mod, cm, tau, causal)
        for key, a, b in zip(("gQ", "gK", "gV"), gp, gm):
            worst = max(worst, _rel(out[key], (a - b) / (2 * eps)))
    return worst


def pin_gdo_is_forward_jvp(mod):
    """gdO = d/de O(Q + e UQ, K + e UK, V + e UV) at e = 0 (g is linear in dO, and
    <U, g> = the directional derivative of <dO, O> along U); checked per element
    by central differences of the forward; gdO does not depend on dO."""
    worst = 0.0
    eps = 1e-5
    for causal in (False, True):
        c = _rand_case(16, 8, RNG_SEED + 7)
        tau = 0.35
        out = _bob(mod, c, tau, causal)
        op, _ = mod.attention_forward_head(c["q"] + eps * c["uq"], c["k"] + eps * c["uk"], c["v"] + eps * c["uv"], tau, causal)
        om, _ = mod.attention_forward_head(c["q"] - eps * c["uq"], c["k"] - eps * c["uk"], c["v"] - eps * c["uv"], tau, causal)
        worst = max(worst, _rel(out["gdO"], (op - om) / (2 * eps)))
        c3 = dict(c)
        c3["do"] = 3.0 * c["do"]
        worst = max(worst, _rel(_bob(mod, c3, tau, causal)["gdO"], out["gdO"]))
    return worst


def pin_lemma_e2(mod):
    """Review page, Strengths (Lemma E.2): V = dO = UQ = UK = 0 and UV = W give
    gdO = softmax(tau Q K^T) W and gQ = gK = gV = 0."""
    from scipy.special import softmax

    worst = 0.0
    for causal in (False, True):
        c = _rand_case(20, 6, RNG_SEED + 8)
        for nm in ("v", "do", "uq", "uk"):
            c[nm] = np.zeros_like(c[nm])
        tau = 0.5
        out = _bob(mod, c, tau, causal)
        s = tau * c["q"] @ c["k"].T
        if causal:
            s = np.where(np.tril(np.ones_like(s)) > 0, s, -np.inf)
        worst = max(worst, _rel(out["gdO"], softmax(s, axis=1) @ c["uv"]))
        for key in ("gQ", "gK", "gV"):
            worst = max(worst, float(np.max(np.abs(out[key]))))
    return worst


def pin_linearity(mod):
    """BoB is linear in U; (gQ, gK, gV) are linear in dO (g is linear in dO)."""
    worst = 0.0
    for causal in (False, True):
        c1 = _rand_case(12, 5, RNG_SEED + 9)
        c2 = _rand_case(12, 5, RNG_SEED + 10)
        tau = 0.6
        a, b = 1.7, -0.4
        cm = dict(c1)
        cb = dict(c1)
        for nm in ("uq", "uk", "uv"):
            cm[nm] = a * c1[nm] + b * c2[nm]
            cb[nm] = c2[nm]
        o1, o2, om = _bob(mod, c1, tau, causal), _bob(mod, cb, tau, causal), _bob(mod, cm, tau, causal)
        for key in ("gQ", "gK", "gV", "gdO"):
            worst = max(worst, _rel(om[key], a * o1[key] + b * o2[key]))
        cs = dict(c1)
        cs["do"] = -2.5 * c1["do"]
        os_ = _bob(mod, cs, tau, causal)
        for key in ("gQ", "gK", "gV"):
            worst = max(worst, _rel(os_[key], -2.5 * o1[key]))
    return worst


def pin_shift_invariance(mod):
    """Adding the same vector c to every key row shifts each score row by a
    constant, and adding it to every value row shifts dP by a per-row constant;
    neither changes g = (dQ, dK, dV) (the rows of dS sum to zero). So <U, g> is
    invariant under both shifts and, for any inputs, sum_j gK_j = 0 and
    sum_j gV_j = 0. With UK = 1 c^T and UQ = UV = 0, <U, g> = c . sum_j dK_j is
    identically zero, so all four outputs vanish."""
    worst = 0.0
    for causal in (False, True):
        c = _rand_case(18, 7, RNG_SEED + 11)
        tau = 0.45
        out = _bob(mod, c, tau, causal)
        worst = max(worst, float(np.linalg.norm(out["gK"].sum(0))) / np.linalg.norm(out["gK"]))
        worst = max(worst, float(np.linalg.norm(out["gV"].sum(0))) / np.linalg.norm(out["gV"]))
        c0 = dict(c)
        c0["uq"] = np.zeros_like(c["uq"])
        c0["uv"] = np.zeros_like(c["uv"])
        c0["uk"] = np.ones((18, 1)) * np.arange(1, 8)[None, :]
        out0 = _bob(mod, c0, tau, causal)
        for key in ("gQ", "gK", "gV", "gdO"):
            worst = max(worst, float(np.max(np.abs(out0[key]))))
    return worst


def pin_special_cases(mod):
    """N = 1: the softmax is identically 1, so g = (0, 0, dO) and BoB = (0, 0, 0, UV).
    Causal: row 0 sees only key 0, so gQ_0 = 0 and gdO_0 = UV_0; and the causal
    row outputs of row i equal the non-causal ones of the prefix [0..i]."""
    worst = 0.0
    c = _rand_case(1, 4, RNG_SEED + 12)
    out = _bob(mod, c, 0.5, False)
    worst = max(worst, float(np.max(np.abs(out["gQ"]))), float(np.max(np.abs(out["gK"]))),
                float(np.max(np.abs(out["gV"]))), _rel(out["gdO"], c["uv"]))
    c = _rand_case(10, 4, RNG_SEED + 13)
    tau = 0.5
    out = _bob(mod, c, tau, True)
    worst = max(worst, float(np.max(np.abs(out["gQ"][0]))), _rel(out["gdO"][0], c["uv"][0]))
    for i in (3, 6, 9):
        pre = {nm: c[nm][: i + 1] for nm in c}
        op = _bob(mod, pre, tau, False)
        worst = max(worst, _rel(out["gQ"][i], op["gQ"][i]), _rel(out["gdO"][i], op["gdO"][i]))
    return worst


def pin_torch_double_backward(mod, n=33, d=8):
    """Against torch autograd double backward (float64, CPU) through plain attention."""
    import torch

    worst = 0.0
    for causal in (False, True):
        c = _rand_case(n, d, RNG_SEED + 14)
        tau = 1.0 / math.sqrt(d)
        t = {nm: torch.tensor(c[nm], dtype=torch.float64, requires_grad=nm in ("q", "k", "v", "do")) for nm in c}
        s = tau * (t["q"] @ t["k"].T)
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ t["v"]
        dq, dk, dv = torch.autograd.grad(o, (t["q"], t["k"], t["v"]), grad_outputs=t["do"], create_graph=True)
        lu = (t["uq"] * dq).sum() + (t["uk"] * dk).sum() + (t["uv"] * dv).sum()
        gq, gk, gv, gdo = torch.autograd.grad(lu, (t["q"], t["k"], t["v"], t["do"]))
        out = _bob(mod, c, tau, causal)
        for key, ref in (("gQ", gq), ("gK", gk), ("gV", gv), ("gdO", gdo)):
            worst = max(worst, _rel(out[key], ref.numpy()))
    return worst


def pin_sympy_exact(mod):
    """Against sympy's symbolic derivative (N = 3, d = 2, causal and not), evaluated
    at 30 digits: an independent derivation of the whole second-order map.
    <U, g> is formed as the derivative of <dO, O(Q + e UQ, K + e UK, V + e UV)> in
    e at e = 0 (the directional derivative of the function g is the gradient
    of), then differentiated symbolically with respect to every input element."""
    import sympy as sp

    worst = 0.0
    n, d = 3, 2
    rng = np.random.default_rng(RNG_SEED + 15)
    vals = {nm: np.round(rng.standard_normal((n, d)) * 4) / 4 for nm in ("q", "k", "v", "do", "uq", "uk", "uv")}

    def rat(x):
        return sp.Rational(x).limit_denominator(16)

    tau = sp.Rational(3, 5)
    e = sp.Symbol("e")
    sym = {nm: sp.Matrix(n, d, lambda i, j, nm=nm: sp.Symbol(f"{nm}_{i}_{j}")) for nm in ("q", "k", "v", "do")}
    shifted = {nm: sym[nm] + e * sp.Matrix(n, d, lambda i, j, un=un: rat(vals[un][i, j]))
               for nm, un in (("q", "uq"), ("k", "uk"), ("v", "uv"))}
    subs = {sym[nm][i, t]: rat(vals[nm][i, t]) for nm in sym for i in range(n) for t in range(d)}
    c = {nm: np.array(vals[nm], dtype=np.float64) for nm in vals}
    for causal in (False, True):
        s = tau * shifted["q"] * shifted["k"].T
        f = 0
        for i in range(n):
            keys = range(i + 1) if causal else range(n)
            z = sum(sp.exp(s[i, j]) for j in keys)
            for t in range(d):
                f += sym["do"][i, t] * sum(sp.exp(s[i, j]) / z * shifted["v"][j, t] for j in keys)
        lu = sp.diff(f, e).subs(e, 0)
        out = _bob(mod, c, float(tau), causal)
        for nm, key in (("q", "gQ"), ("k", "gK"), ("v", "gV"), ("do", "gdO")):
            ref = np.array([[float(sp.diff(lu, sym[nm][i, t]).evalf(30, subs=subs)) for t in range(d)]
                            for i in range(n)])
            worst = max(worst, _rel(out[key], ref))
    return worst


def pin_blocked_and_sampled(mod):
    """Row-blocked evaluation, the single-row routine and the column routine give
    the one-block result (the only difference is summation order)."""
    worst = 0.0
    for causal in (False, True):
        c = _rand_case(37, 6, RNG_SEED + 16)
        tau = 0.4
        full = _bob(mod, c, tau, causal)
        blk = _bob(mod, c, tau, causal, row_block=8)
        for key in ("gQ", "gK", "gV", "gdO", "L", "D", "alpha", "E"):
            worst = max(worst, _rel(blk[key], full[key]))
        rows = [0, 5, 17, 36]
        r = mod.bob_rows_head(c["q"], c["k"], c["v"], c["do"], c["uq"], c["uk"], c["uv"], tau, causal, rows)
        for key in ("gQ", "gdO", "L", "D", "alpha", "E"):
            worst = max(worst, _rel(r[key], full[key][rows]))
        # two row ranges add up to the whole computation
        pa = _bob(mod, c, tau, causal, row_block=4, row_range=(0, 19))
        pb = _bob(mod, c, tau, causal, row_block=7, row_range=(19, 37))
        for key in ("gQ", "gK", "gV", "gdO", "alpha", "E"):
            worst = max(worst, _rel(pa[key] + pb[key], full[key]))
        cols = [1, 2, 30, 36]
        args = (c["q"], c["k"], c["v"], c["do"], c["uq"], c["uk"], c["uv"], tau, causal, cols)
        cc = mod.bob_cols_head(*args, row_block=5)
        # the column routine over two row ranges adds up to the one-range sweep
        ca = mod.bob_cols_head(*args, row_block=3, row_range=(0, 11))
        cb = mod.bob_cols_head(*args, row_block=6, row_range=(11, 37))
        for key in ("gK", "gV"):
            worst = max(worst, _rel(cc[key], full[key][cols]))
            worst = max(worst, _rel(ca[key] + cb[key], full[key][cols]))
    return worst


# name -> (pin, bound on the worst relative error)
PINS = {
    "forward_loops": (pin_forward_loops, 1e-13),
    "first_backward_fd": (pin_first_backward_fd, 1e-7),
    "bob_fd_elementwise": (pin_bob_fd_elementwise, 1e-6),
    "bob_fd_directional": (pin_bob_fd_directional, 1e-6),
    "hessian_symmetry": (pin_hessian_symmetry, 1e-7),
    "gdo_is_forward_jvp": (pin_gdo_is_forward_jvp, 1e-7),
    "lemma_e2": (pin_lemma_e2, 1e-12),
    "linearity": (pin_linearity, 1e-12),
    "shift_invariance": (pin_shift_invariance, 1e-12),
    "special_cases": (pin_special_cases, 1e-12),
    "torch_double_backward": (pin_torch_double_backward, 1e-12),
    "sympy_exact": (pin_sympy_exact, 1e-12),
    "blocked_and_sampled": (pin_blocked_and_sampled, 1e-12),
}
