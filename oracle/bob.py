"""Plain fp64 CPU oracle for exact backward-over-backward (BoB) through softmax attention.

TEST INFRASTRUCTURE ONLY. This module is the reference that the HIP path is
checked against. Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the library itself never calls it, and it
shares no code with the HIP kernels or their host code.

What it computes (FlashBoB pages: arXiv abstract page, and the evolve.pub review
page, sections "Key claims under review" and "Report preview / Scope & Claims"):
for attention O = softmax(tau Q K^T) V and its first backward
g(Q, K, V, dO) = (dQ, dK, dV), BoB applies the transposed Jacobian of g to
upstream cotangents (UQ, UK, UV) placed on (dQ, dK, dV), and returns the
cotangents of the four inputs (gQ, gK, gV, gdO). The review (Strengths, on
Appendix C; FAQ "Is FlashBoB an approximation?") states that the method's
identities follow from the reverse-mode chain rule applied graph node by graph
node and that its result is exact, so the oracle is that plain definition: the
reverse-mode derivative of  <UQ, dQ> + <UK, dK> + <UV, dV>  with respect to
(Q, K, V, dO), written out one graph node at a time, with every N x N matrix
materialised, in float64. Matrix products use numpy's matmul as a library step.

Shapes: one head is handled at a time, q, k, v, do, uq, uk, uv are (N, d)
float64 arrays. The batched wrappers take (B, H, N, d).

Rows are independent in this definition (each query row has its own softmax),
so the whole computation can be evaluated on any subset of query rows: the row
outputs of those rows are exact, and their contributions to the column outputs
(gK, gV) are exact partial sums. `bob_head` uses that to evaluate the same
formulas on blocks of rows when N x N does not fit in memory; the sum over row
blocks is the only reordering and it is pinned against the one-block evaluation.

Causal masking: row i attends to keys j <= i (square, top-left aligned). Masked
scores are -inf, so their probabilities are exactly 0 and they carry no
gradient.
"""

import numpy as np

__all__ = [
    "attention_forward_head",
    "first_backward_head",
    "bob_head",
    "bob_rows_head",
    "bob_cols_head",
    "attention_forward",
    "first_backward",
    "bob",
]


def _scores(q_rows, row_idx, k, tau, causal):
    """S = tau * Q_R K^T for the query rows R, with causal entries j > i set to -inf."""
    s = tau * (q_rows @ k.T)
    if causal:
        cols = np.arange(k.shape[0])
        s[cols[None, :] > row_idx[:, None]] = -np.inf
    return s


def _softmax_rows(s):
    """Row-wise softmax and its log-sum-exp, with the usual max shift."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    return e / z, lse


def attention_forward_head(q, k, v, tau, causal=False):
    """Forward attention of one head: O = softmax(tau Q K^T) V and the row LSE L.

    L_i is the natural-log log-sum-exp of row i of tau Q K^T (the statistic the
    score-recomputation model keeps, review page, Strengths: Theorem 4.5).
    """
    rows = np.arange(q.shape[0])
    p, lse = _softmax_rows(_scores(q, rows, k, tau, causal))
    return p @ v, lse


def first_backward_head(q, k, v, do, tau, causal=False):
    """First backward g of one head: (dQ, dK, dV) and the row scalar D.

    Reverse mode through S = tau Q K^T, P = softmax(S), O = P V with upstream dO:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D),  dQ = tau dS K,  dK = tau dS^T Q.
    """
    rows = np.arange(q.shape[0])
    p, _ = _softmax_rows(_scores(q, rows, k, tau, causal))
    dp = do @ v.T
    dd = np.sum(p * dp, axis=1)
    ds = p * (dp - dd[:, None])
    return tau * (ds @ k), tau * (ds.T @ q), p.T @ do, dd


def _bob_nodes(q, k, v, do, uq, uk, uv, tau, causal, r0, r1, row_outputs=True):
    """All BoB quantities for query rows [r0, r1) of one head.

    Forward of the first backward (the graph being differentiated), rows R:
      S = tau Q_R K^T, P = softmax_rows(S), dP = dO_R V^T,
      D = rowsum(P * dP), dS = P * (dP - D),
      dQ_R = tau dS K, dK += tau dS^T Q_R, dV += P^T dO_R.
    Reverse sweep with cotangents UQ_R on dQ_R, UK on dK, UV on dV, visiting the
    nodes in reverse order. "bar_X" is the cotangent of X.
    Returns the row outputs (gQ_R, gdO_R), the row scalars, and the terms whose
    transposed products give this block's contribution to gK and gV. With
    row_outputs=False the four products that only feed gQ_R and gdO_R are not
    formed (those entries are None); every other value is the same.
    """
    rows = np.arange(r0, r1)
    q_r, do_r, uq_r = q[r0:r1], do[r0:r1], uq[r0:r1]

    # forward of g on these rows
    s = _scores(q_r, rows, k, tau, causal)
    p, lse = _softmax_rows(s)
    dp = do_r @ v.T
    dd = np.sum(p * dp, axis=1)
    ds = p * (dp - dd[:, None])

    # node dV = P^T dO  (cotangent UV): feeds bar_P and bar_dO
    bar_p = do_r @ uv.T
    bar_do = p @ uv if row_outputs else None

    # node dK = tau dS^T Q  (cotangent UK): feeds bar_dS and bar_Q
    bar_ds = tau * (q_r @ uk.T)
    bar_q = tau * (ds @ uk) if row_outputs else None

    # node dQ = tau dS K  (cotangent UQ_R): feeds bar_dS and bar_K
    bar_ds = bar_ds + tau * (uq_r @ k.T)
    # bar_K contribution tau dS^T UQ_R is formed by the caller from ds and uq_r

    # node dS = P * (dP - D): feeds bar_P, bar_dP, bar_D
    bar_p = bar_p + bar_ds * (dp - dd[:, None])
    bar_dp = bar_ds * p
    bar_dd = -np.sum(bar_ds * p, axis=1)

    # node D = rowsum(P * dP): feeds bar_P and bar_dP
    bar_p = bar_p + bar_dd[:, None] * dp
    bar_dp = bar_dp + bar_dd[:, None] * p

    # node dP = dO V^T: feeds bar_dO and bar_V (bar_V formed by the caller)
    if row_outputs:
        bar_do = bar_do + bar_dp @ v

    # node P = softmax(S), row-wise: bar_S = P * (bar_P - rowsum(P * bar_P))
    e_row = np.sum(p * bar_p, axis=1)
    bar_s = p * (bar_p - e_row[:, None])

    # node S = tau Q K^T: feeds bar_Q and bar_K (bar_K formed by the caller)
    if row_outputs:
        bar_q = bar_q + tau * (bar_s @ k)

    return {
        "gQ": bar_q,
        "gdO": bar_do,
        "L": lse,
        "D": dd,
        "alpha": -bar_dd,
        "E": e_row,
        # terms for the column outputs of this block
        "_ds": ds,
        "_bar_s": bar_s,
        "_bar_dp": bar_dp,
        "_q": q_r,
        "_uq": uq_r,
        "_do": do_r,
    }


def bob_head(q, k, v, do, uq, uk, uv, tau, causal=False, row_block=None, row_range=None):
    """BoB of one head: returns dict with gQ, gK, gV, gdO (N, d) and the row
    scalars L, D, alpha, E (N,).

    alpha_i = -(cotangent of D_i) = sum_j P_ij * bar_dS_ij and
    E_i = sum_j P_ij * bar_P_ij are the two row scalars of the softmax double
    backward (review page, Summary and Strengths, Prop. 4.1).
    row_block=None evaluates all N rows at once (full N x N materialisation);
    an integer evaluates the same formulas on row blocks of that height.
    row_range=(r0, r1) evaluates only the query rows r0..r1-1: their row outputs
    and scalars are exact, gK and gV hold only those rows' contributions, and
    the other rows stay zero (a bounded sample of the whole computation).
    """
    n, d = q.shape
    rb = n if row_block is None else max(1, int(row_block))
    lo, hi = (0, n) if row_range is None else (max(0, int(row_range[0])), min(n, int(row_range[1])))
    g_q = np.zeros((n, d))
    g_do = np.zeros((n, d))
    g_k = np.zeros((n, d))
    g_v = np.zeros((n, d))
    scal = {name: np.zeros(n) for name in ("L", "D", "alpha", "E")}
    for r0 in range(lo, hi, rb):
        r1 = min(hi, r0 + rb)
        t = _bob_nodes(q, k, v, do, uq, uk, uv, tau, causal, r0, r1)
        g_q[r0:r1] = t["gQ"]
        g_do[r0:r1] = t["gdO"]
        # node dQ = tau dS K gives bar_K += tau dS^T UQ; node S gives tau bar_S^T Q
        g_k += tau * (t["_ds"].T @ t["_uq"]) + tau * (t["_bar_s"].T @ t["_q"])
        # node dP = dO V^T gives bar_V += bar_dP^T dO
        g_v += t["_bar_dp"].T @ t["_do"]
        for name in scal:
            scal[name][r0:r1] = t[name]
    out = {"gQ": g_q, "gK": g_k, "gV": g_v, "gdO": g_do}
    out.update(scal)
    return out


def bob_rows_head(q, k, v, do, uq, uk, uv, tau, causal, rows):
    """Row outputs gQ[rows], gdO[rows] and the row scalars for the listed rows only.

    Each row's outputs depend on that row's sweep over all keys alone, so they
    are computed one row at a time with the same node formulas.
    """
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[1]
    out = {"gQ": np.zeros((len(rows), d)), "gdO": np.zeros((len(rows), d))}
    for name in ("L", "D", "alpha", "E"):
        out[name] = np.zeros(len(rows))
    for t_i, r in enumerate(rows):
        t = _bob_nodes(q, k, v, do, uq, uk, uv, tau, causal, int(r), int(r) + 1)
        for name in ("gQ", "gdO"):
            out[name][t_i] = t[name][0]
        for name in ("L", "D", "alpha", "E"):
            out[name][t_i] = t[name][0]
    return out


def bob_cols_head(q, k, v, do, uq, uk, uv, tau, causal, cols, row_block=256, row_range=None):
    """Column outputs gK[cols], gV[cols] (a full sweep over all query rows, since
    every row contributes to every column), evaluated on row blocks. Each block
    still forms its rows' scalars D, alpha, E from all keys; the products that
    only feed the row outputs are skipped. row_range=(r0, r1) restricts the sweep
    to those query rows: the result is then their exact contribution, and the
    contributions of disjoint ranges add up to the whole."""
    cols = np.asarray(cols, dtype=np.int64)
    n, d = q.shape
    lo, hi = (0, n) if row_range is None else (max(0, int(row_range[0])), min(n, int(row_range[1])))
    g_k = np.zeros((len(cols), d))
    g_v = np.zeros((len(cols), d))
    for r0 in range(lo, hi, row_block):
        r1 = min(hi, r0 + row_block)
        t = _bob_nodes(q, k, v, do, uq, uk, uv, tau, causal, r0, r1, row_outputs=False)
        g_k += tau * (t["_ds"][:, cols].T @ t["_uq"]) + tau * (t["_bar_s"][:, cols].T @ t["_q"])
        g_v += t["_bar_dp"][:, cols].T @ t["_do"]
    return {"gK": g_k, "gV": g_v}


def _per_head(fn, arrays, *args, **kw):
    b, h = arrays[0].shape[:2]
    res = None
    for bi in range(b):
        for hi in range(h):
            r = fn(*[np.asarray(a[bi, hi], dtype=np.float64) for a in arrays], *args, **kw)
            if not isinstance(r, dict):
                r = dict(enumerate(r))
            if res is None:
                res = {key: np.zeros((b, h) + np.shape(val)) for key, val in r.items()}
            for key, val in r.items():
                res[key][bi, hi] = val
    return res


def attention_forward(Q, K, V, tau, causal=False):
    """Batched forward over (B, H, N, d): returns (O, L)."""
    r = _per_head(attention_forward_head, [Q, K, V], tau, causal)
    return r[0], r[1]


def first_backward(Q, K, V, dO, tau, causal=False):
    """Batched first backward over (B, H, N, d): returns (dQ, dK, dV, D)."""
    r = _per_head(first_backward_head, [Q, K, V, dO], tau, causal)
    return r[0], r[1], r[2], r[3]


def bob(Q, K, V, dO, UQ, UK, UV, tau, causal=False, row_block=None):
    """Batched BoB over (B, H, N, d): dict of gQ, gK, gV, gdO, L, D, alpha, E."""
    return _per_head(bob_head, [Q, K, V, dO, UQ, UK, UV], tau, causal, row_block=row_block)
