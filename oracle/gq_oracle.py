"""fp64 CPU oracle for the GuidedQuant Fisher and the LNQ alternating optimisation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and this module imports
nothing from the product package.

Every function is the plain definition (or, for the iterative LNQ, the steps in
the pages' order), in float64 with NumPy.  Sources:

  [GQ-obj]   "GuidedQuant" blog page (jinukkim.me/blog/guidedquant), the
             GuidedQuant objective equation and the sentence after it (block-
             diagonal Fisher, grouped and averaged within each group).
  [GQ-lw]    same page, item 1: layer-wise output reconstruction equation.
  [LNQ-prob] same page, section "LNQ": the per-row problem over a one-hot
             assignment P^(j) with P 1_m = 1 and a codebook c^(j).
  [LNQ-alg]  same page, section "LNQ": the repeat-loop with the "(codebook)"
             closed form and the "(assignment)" coordinate loop i = 1..d_in.
  [GQ-abs]   aitopics.org "squeezellm" page, GuidedQuant abstract: the
             non-uniform scalar algorithm decreases the objective monotonically.
  [GANQ]     atlas.scime.ai GANQ summary page, "Approach": alternating updates, an
             assignment of the codebook indices by Cholesky / back-substitution
             and a closed-form least-squares codebook update.

Readings where the pages are silent (the same readings the GPU library uses):
  * F_j = X^T diag(G[:, j]^2) X without the 1/n factor (the objective equation
    carries a leading n and leaves F_j undefined; LNQ is invariant to scaling F).
  * Groups are contiguous equal blocks of output channels; averaging F_j over a
    group equals using s_g[t] = mean_{j in g} G[t, j]^2 (linearity).
  * Damping: F' = F_g + lambda_g I with lambda_g = rho * mean(diag F_g) (plus an
    optional fixed term); F' is used everywhere (objective, codebook, sweep).
  * Initial codebook: m quantiles of w_j at levels (q + 1/2)/m with linear
    interpolation between order statistics, stored as float32; initial codes
    are the nearest entry (lowest index on ties).  Parity unpinned by the pages
    (they do not state an initialisation); pinned only to the textbook
    quantile definition.
  * Empty code q (no coordinate assigned): c_q is kept unchanged.
  * Assignment: coordinates in ascending order; a coordinate moves only on a
    strict decrease of the objective, to the lowest-index minimiser.
  * GANQ-style assignment ([GANQ] below): back-substitution over F' = L L^T,
    coordinates from the last to the first, each taking the entry nearest to
    w_j - s_j / L_jj; the codebook step is LNQ's.
  * LUT dequantisation GEMV: y = W_hat x with W_hat[j][i] = c^(j)[p_ji]; the
    packed index layout is this library's own (the pages fix none).  For
    bfloat16 activations the lookup table holds the codebook rounded to
    bfloat16 (the inference kernel the pages refer to keeps a 16-bit table).
  * Fixed-grid backend (the blog page's remark that the objective plugs into
    any layer-wise quantizer): a uniform min-max grid per row, kept fixed, and
    the assignment pass only.  The grid is the plain definition of an equally
    spaced grid from the row's minimum to its maximum.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "group_scale", "fisher", "fisher_entry", "fisher_per_channel", "ridge_lambda",
    "damped", "init_quantile", "one_hot", "codebook_system", "codebook_update",
    "assign_deltas", "assign_sweep", "objective", "lnq_row", "guided_loss",
    "replay_sweep", "init_uniform_grid", "grid_row", "lut_codes_per_word", "lut_row_words",
    "lut_pack", "lut_unpack", "bf16_round", "lut_gemv", "ganq_assign", "ganq_row",
    "ganq_replay",
]


# ----------------------------------------------------------------------------
# Fisher [GQ-obj]
# ----------------------------------------------------------------------------

def group_scale(G: np.ndarray, groups: int) -> np.ndarray:
    """s_g[t] = mean over the output channels j of group g of G[t, j]^2  -> [groups][n].

    [GQ-obj]: the per-channel blocks F_j are averaged within each group; with
    F_j = X^T diag(G[:, j]^2) X the average is X^T diag(s_g) X.
    """
    G = np.asarray(G, dtype=np.float64)
    n, d_out = G.shape
    if d_out % groups:
        raise ValueError("d_out must be a multiple of groups")
    size = d_out // groups
    S = np.empty((groups, n))
    for g in range(groups):
        S[g] = np.mean(G[:, g * size:(g + 1) * size] ** 2, axis=1)
    return S


def fisher(X: np.ndarray, G: np.ndarray, groups: int) -> np.ndarray:
    """Grouped Fisher blocks F_g = X^T diag(s_g) X -> [groups][d_in][d_in]  [GQ-obj]."""
    X = np.asarray(X, dtype=np.float64)
    S = group_scale(G, groups)
    return np.stack([X.T @ (S[g][:, None] * X) for g in range(groups)])


def fisher_entry(x_a: np.ndarray, x_b: np.ndarray, s_g: np.ndarray) -> float:
    """One entry F_g[a, b] = sum_t s_g[t] X[t, a] X[t, b]  [GQ-obj]."""
    return float(np.dot(np.asarray(s_g, np.float64) * np.asarray(x_a, np.float64),
                        np.asarray(x_b, np.float64)))


def fisher_per_channel(X: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Per-output-channel blocks F_j = X^T diag(G[:, j]^2) X -> [d_out][d_in][d_in]  [GQ-obj]."""
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    return np.stack([X.T @ ((G[:, j] ** 2)[:, None] * X) for j in range(G.shape[1])])


def guided_loss(X: np.ndarray, G: np.ndarray, W: np.ndarray, W_hat: np.ndarray) -> float:
    """|| G (.) (X W^T - X W_hat^T) ||_F^2 with W stored [d_out][d_in]  [GQ-obj] left side."""
    X = np.asarray(X, np.float64)
    Z = X @ np.asarray(W, np.float64).T
    Z_hat = X @ np.asarray(W_hat, np.float64).T
    return float(np.sum((np.asarray(G, np.float64) * (Z - Z_hat)) ** 2))


# ----------------------------------------------------------------------------
# Damping (reading: GPTQ-style relative ridge on F itself)
# ----------------------------------------------------------------------------

def ridge_lambda(F_g: np.ndarray, rho: float, lam_abs: float = 0.0) -> float:
    """lambda_g = rho * mean(diag F_g) + lam_abs.

    The relative term is the ridge the tiny 128 -> 64 workload states (1e-6 times
    the mean of diag F), which scales with the Fisher ("adaptive"); lam_abs is a
    fixed ridge independent of F, the alternative the GANQ summary page's ablation
    table sets against adaptive preconditioning.  Only the diagonal enters.
    """
    F_g = np.asarray(F_g, np.float64)
    return float(rho * np.trace(F_g) / F_g.shape[0]) + float(lam_abs)


def damped(F_g: np.ndarray, rho: float, lam_abs: float = 0.0) -> np.ndarray:
    """F' = F_g + lambda_g I."""
    F_g = np.asarray(F_g, np.float64)
    return F_g + ridge_lambda(F_g, rho, lam_abs) * np.eye(F_g.shape[0])


# ----------------------------------------------------------------------------
# LNQ [LNQ-prob], [LNQ-alg]
# ----------------------------------------------------------------------------

def init_quantile(w: np.ndarray, m: int):
    """Initial codebook (m quantiles of w at levels (q+1/2)/m, float32-stored) and codes.

    Quantile at level t of N sorted values: position h = (N-1) t, value
    x[floor h] + frac(h) * (x[floor h + 1] - x[floor h]).  The position is
    formed as (N-1)(2q+1) / (2m).  Codes: index of the nearest entry, the
    lowest index on ties, compared in float64 on the stored float32 values.
    """
    w = np.asarray(w, np.float64)
    xs = np.sort(w)
    N = xs.shape[0]
    c = np.empty(m)
    for q in range(m):
        h = float((N - 1) * (2 * q + 1)) / float(2 * m)
        lo = int(np.floor(h))
        frac = h - lo
        hi = min(lo + 1, N - 1)
        c[q] = xs[lo] + frac * (xs[hi] - xs[lo])
    c = c.astype(np.float32).astype(np.float64)
    p = np.argmin(np.abs(w[:, None] - c[None, :]), axis=1).astype(np.int64)
    return c, p


def one_hot(p: np.ndarray, m: int) -> np.ndarray:
    """P^(j) in {0,1}^{d_in x m} with P 1_m = 1  [LNQ-prob]."""
    p = np.asarray(p, np.int64)
    Q = np.zeros((p.shape[0], m))
    Q[np.arange(p.shape[0]), p] = 1.0
    return Q


def codebook_system(Fp: np.ndarray, w: np.ndarray, p: np.ndarray, m: int):
    """A = P^T F' P and b = P^T F' w of the "(codebook)" step  [LNQ-alg]."""
    Q = one_hot(p, m)
    A = Q.T @ Fp @ Q
    b = Q.T @ (Fp @ np.asarray(w, np.float64))
    return A, b


def codebook_update(Fp: np.ndarray, w: np.ndarray, p: np.ndarray, c: np.ndarray) -> np.ndarray:
    """c <- (P^T F' P)^{-1} P^T F' w on the non-empty codes; empty codes keep c  [LNQ-alg].

    When P^T F' P on the non-empty codes is not positive definite (F' = 0, the
    damped Fisher of a group whose gradients all vanish) the closed form does not
    exist and the codebook is kept unchanged.
    """
    m = c.shape[0]
    A, b = codebook_system(Fp, w, p, m)
    counts = np.bincount(np.asarray(p, np.int64), minlength=m)
    S = np.nonzero(counts > 0)[0]
    try:
        L = np.linalg.cholesky(A[np.ix_(S, S)])
    except np.linalg.LinAlgError:
        return np.array(c, dtype=np.float64, copy=True)
    y = np.linalg.solve(L, b[S])
    x = np.linalg.solve(L.T, y)
    c_new = np.array(c, dtype=np.float64, copy=True)
    c_new[S] = x
    return c_new


def objective(Fp: np.ndarray, w: np.ndarray, c: np.ndarray, p: np.ndarray) -> float:
    """(w_hat - w)^T F' (w_hat - w) with w_hat = P c  [LNQ-prob], [GQ-obj]."""
    e = np.asarray(c, np.float64)[np.asarray(p, np.int64)] - np.asarray(w, np.float64)
    return float(e @ (Fp @ e))


def assign_deltas(Fp_ii: float, r_i: float, c: np.ndarray, cur: float) -> np.ndarray:
    """Exact objective change when coordinate i moves from value `cur` to each c_q.

    With r = F'(w_hat - w) and delta = c_q - cur:
      (e + delta u_i)^T F' (e + delta u_i) - e^T F' e = delta (F'_ii delta + 2 r_i).
    """
    delta = np.asarray(c, np.float64) - cur
    return delta * (Fp_ii * delta + 2.0 * r_i)


def assign_sweep(Fp: np.ndarray, w: np.ndarray, c: np.ndarray, p: np.ndarray,
                 return_steps: bool = False):
    """One "(assignment)" pass over i = 1..d_in in order  [LNQ-alg].

    For each coordinate, pick the codebook entry minimising the row objective
    with every other coordinate fixed; keep the current entry unless some entry
    strictly decreases it, then take the lowest-index minimiser.  F' is
    symmetric (a damped Fisher X^T diag(s) X + lambda I), so the residual update
    r += delta F'[:, i] reads row i, the same numbers as column i.
    """
    c = np.asarray(c, np.float64)
    p = np.array(p, dtype=np.int64, copy=True)
    w = np.asarray(w, np.float64)
    r = Fp @ (c[p] - w)
    steps = []
    for i in range(w.shape[0]):
        D = assign_deltas(Fp[i, i], r[i], c, c[p[i]])
        q = int(np.argmin(D))          # first occurrence = lowest index
        if return_steps:
            steps.append(D.copy())
        if D[q] < 0.0:
            r += (c[q] - c[p[i]]) * Fp[i]
            p[i] = q
    if return_steps:
        return p, steps
    return p


def lnq_row(Fp: np.ndarray, w: np.ndarray, m: int, iters: int, c0=None, p0=None,
            trace: bool = True):
    """LNQ for one row: init, then `iters` x (codebook, assignment)  [LNQ-alg].

    Returns (c, p, trace) with trace[0] the objective at the start and
    trace[2t-1], trace[2t] after the codebook and assignment steps of pass t.
    With trace=False the steps are the same and only the final objective is
    evaluated (trace = [objective at the end]).
    """
    if c0 is None:
        c, p = init_quantile(w, m)
    else:
        c = np.asarray(c0, np.float64).copy()
        p = np.asarray(p0, np.int64).copy()
    tr = [objective(Fp, w, c, p)] if trace else []
    for _ in range(iters):
        c = codebook_update(Fp, w, p, c)
        if trace:
            tr.append(objective(Fp, w, c, p))
        p = assign_sweep(Fp, w, c, p)
        if trace:
            tr.append(objective(Fp, w, c, p))
    if not trace:
        tr = [objective(Fp, w, c, p)]
    return c, p, np.array(tr)


def replay_sweep(Fp: np.ndarray, w: np.ndarray, c: np.ndarray, p_start: np.ndarray,
                 p_dev: np.ndarray, tol_rel: float):
    """Walk one assignment pass in order but follow the device's decisions.

    At each coordinate the exact fp64 changes D_q are formed from the current
    state; the device's choice q_dev must satisfy
        D[q_dev] <= min(min_q D_q, 0) + tol_rel * |objective of the row so far|.
    Returns (worst excess over the allowance (<= 0 means every decision is
    valid), number of decisions that differ from the fp64 choice).
    """
    c = np.asarray(c, np.float64)
    p = np.array(p_start, dtype=np.int64, copy=True)
    p_dev = np.asarray(p_dev, np.int64)
    w = np.asarray(w, np.float64)
    e = c[p] - w
    r = Fp @ e
    obj = float(e @ r)
    worst = -np.inf
    differ = 0
    for i in range(w.shape[0]):
        D = assign_deltas(Fp[i, i], r[i], c, c[p[i]])
        q_ref = int(np.argmin(D))
        best = min(float(D[q_ref]), 0.0)
        if not D[q_ref] < 0.0:
            q_ref = int(p[i])
        q = int(p_dev[i])
        worst = max(worst, float(D[q]) - best - tol_rel * abs(obj))
        if q != q_ref:
            differ += 1
        if q != p[i]:
            r += (c[q] - c[p[i]]) * Fp[i]          # row i = column i (F' symmetric)
            obj += float(D[q])
            p[i] = q
    return worst, differ


# ----------------------------------------------------------------------------
# Fixed-grid scalar backend [GQ-obj], [LNQ-alg]
# ----------------------------------------------------------------------------
# The blog page says the GuidedQuant objective can serve any layer-wise
# quantizer.  The plainest scalar one keeps a uniform grid per row and runs only
# the "(assignment)" pass of the LNQ algorithm box on that objective.

def init_uniform_grid(w: np.ndarray, m: int):
    """Uniform grid of a row and its nearest codes.

    m >= 2 equally spaced values from lo = min(w) to hi = max(w):
    c_q = lo + q * ((hi - lo) / (m - 1)), each product and sum rounded in
    float64, then stored as float32.  Codes: index of the nearest entry, the
    lowest index on ties, compared in float64 on the stored values.  The pages
    name no grid; this is the min-max grid's definition.
    """
    w = np.asarray(w, np.float64)
    lo, hi = float(np.min(w)), float(np.max(w))
    step = (hi - lo) / float(m - 1)
    c = np.array([lo + float(q) * step for q in range(m)])
    c = c.astype(np.float32).astype(np.float64)
    p = np.argmin(np.abs(w[:, None] - c[None, :]), axis=1).astype(np.int64)
    return c, p


def grid_row(Fp: np.ndarray, w: np.ndarray, m: int, iters: int, c0=None, p0=None):
    """Fixed-grid backend for one row: the grid stays, `iters` assignment passes.

    Returns (c, p, trace) with trace[t] the objective before pass t + 1 and
    trace[iters] the objective after the last pass.
    """
    if c0 is None:
        c, p = init_uniform_grid(w, m)
    else:
        c = np.asarray(c0, np.float64).copy()
        p = np.asarray(p0, np.int64).copy()
    trace = [objective(Fp, w, c, p)]
    for _ in range(iters):
        p = assign_sweep(Fp, w, c, p)
        trace.append(objective(Fp, w, c, p))
    return c, p, np.array(trace)


# ----------------------------------------------------------------------------
# LUT dequantisation GEMV for the (C, P) format [LNQ-prob]
# ----------------------------------------------------------------------------
# The blog page notes that LNQ's output runs on the same lookup-table kernel as
# SqueezeLLM: each row keeps its codebook c^(j) and b-bit indices P^(j), and a
# product with activations reads w_hat_ji = c^(j)[p_ji].  The packed layout is
# this library's own (the pages fix none):
#   * codes are taken in pairs (i, i + 1); a pair forms the 2b-bit index
#     code_i | code_{i+1} << b;
#   * a 32-bit word holds floor(16 / b) pairs, the first pair in the low bits;
#     codes per word cpw = 2 floor(16 / b): 32, 16, 10, 8 for b = 1, 2, 3, 4;
#   * a row is ceil(d_in / cpw) words, padded with zero words to a multiple of
#     4 words; code slots past d_in hold 0.

def lut_codes_per_word(bits: int) -> int:
    return 2 * (16 // bits)


def lut_row_words(d_in: int, bits: int) -> int:
    cpw = lut_codes_per_word(bits)
    return -(-(-(-d_in // cpw)) // 4) * 4


def lut_pack(P: np.ndarray, bits: int) -> np.ndarray:
    """Packed codes [d_out][row words] (uint32) of P [d_out][d_in], per the layout above."""
    P = np.asarray(P, np.int64)
    d_out, d_in = P.shape
    cpw = lut_codes_per_word(bits)
    rw = lut_row_words(d_in, bits)
    Q = np.zeros((d_out, rw), dtype=np.uint64)
    for i in range(d_in):
        word, slot = divmod(i, cpw)
        shift = bits * slot            # pair slot // 2 at 2b (slot // 2), half at b (slot % 2)
        Q[:, word] |= (P[:, i] & ((1 << bits) - 1)).astype(np.uint64) << np.uint64(shift)
    return Q.astype(np.uint32)


def lut_unpack(Q: np.ndarray, d_in: int, bits: int) -> np.ndarray:
    """Codes [d_out][d_in] back from the packed words."""
    Q = np.asarray(Q, np.uint64)
    cpw = lut_codes_per_word(bits)
    i = np.arange(d_in)
    words = Q[:, i // cpw]
    return ((words >> (np.uint64(bits) * (i % cpw).astype(np.uint64))) &
            np.uint64((1 << bits) - 1)).astype(np.int64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float64.

    The high 16 bits of the float32 pattern after adding 0x7FFF plus the lowest
    kept bit; finite inputs only.
    """
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def lut_gemv(C: np.ndarray, P: np.ndarray, x: np.ndarray, lut_bf16: bool) -> np.ndarray:
    """y[b][j] = sum_i v(C[j][P[j][i]]) x[b][i] in float64.

    v rounds the codebook entry to bfloat16 when the lookup table is held in
    bfloat16 (the path taken for bfloat16 activations), else keeps float32.
    """
    C = np.asarray(C, np.float32)
    Cv = bf16_round(C) if lut_bf16 else C.astype(np.float64)
    W_hat = np.take_along_axis(Cv, np.asarray(P, np.int64), axis=1)
    x = np.atleast_2d(np.asarray(x, np.float64))
    return x @ W_hat.T


# ----------------------------------------------------------------------------
# GANQ-style assignment [GANQ]
# ----------------------------------------------------------------------------
# The GANQ summary page describes the per-row problem solved by alternating a
# closed-form least-squares codebook update with an assignment of the indices by
# Cholesky / back-substitution.  Reading: with F' = L L^T (L lower triangular) the
# row objective is ||L^T e||^2, e = w_hat - w, whose j-th term
# (L^T e)_j = L_jj e_j + sum_{k>j} L_kj e_k involves only coordinates j..d-1; the
# assignment visits j = d-1 down to 0 and gives coordinate j the codebook entry
# that minimises that term with the later coordinates already fixed, i.e. the
# entry nearest to w_j - s_j / L_jj with s_j = sum_{k>j} L_kj e_k (lowest index on
# ties).  The codebook step is the LNQ closed form above.

def ganq_assign(Fp: np.ndarray, w: np.ndarray, c: np.ndarray, L: np.ndarray | None = None,
                return_targets: bool = False):
    """Back-substitution assignment of one row against F' = L L^T  [GANQ]."""
    if L is None:
        L = np.linalg.cholesky(np.asarray(Fp, np.float64))
    w = np.asarray(w, np.float64)
    c = np.asarray(c, np.float64)
    d = w.shape[0]
    e = np.zeros(d)
    p = np.empty(d, dtype=np.int64)
    targets = np.empty(d)
    for j in range(d - 1, -1, -1):
        s = float(L[j + 1:, j] @ e[j + 1:])
        t = w[j] - s / L[j, j]
        q = int(np.argmin(np.abs(t - c)))       # first occurrence = lowest index
        p[j] = q
        e[j] = c[q] - w[j]
        targets[j] = t
    if return_targets:
        return p, targets
    return p


def ganq_row(Fp: np.ndarray, w: np.ndarray, m: int, iters: int, c0=None, p0=None):
    """GANQ-style alternation for one row: init, then `iters` x (codebook, assignment).

    Returns (c, p, trace) laid out as lnq_row's: trace[2t-1] after the codebook step
    and trace[2t] after the assignment of pass t.  The assignment solves the
    back-substitution problem, so the trace need not decrease.
    """
    L = np.linalg.cholesky(np.asarray(Fp, np.float64))
    if c0 is None:
        c, p = init_quantile(w, m)
    else:
        c = np.asarray(c0, np.float64).copy()
        p = np.asarray(p0, np.int64).copy()
    trace = [objective(Fp, w, c, p)]
    for _ in range(iters):
        c = codebook_update(Fp, w, p, c)
        trace.append(objective(Fp, w, c, p))
        p = ganq_assign(Fp, w, c, L)
        trace.append(objective(Fp, w, c, p))
    return c, p, np.array(trace)


def ganq_replay(Fp: np.ndarray, w: np.ndarray, c: np.ndarray, p_dev: np.ndarray, tol: float,
                L: np.ndarray | None = None):
    """Follow the device's decisions of one assignment pass (from the last coordinate
    down) and check each: with the device's later decisions fixed, its entry must be
    within `tol` * L_jj * (largest codebook gap) of the nearest one to the target,
    measured on the term |L_jj (c_q - w_j) + s_j|.  Returns (worst excess over the
    allowance, number of decisions that differ from the fp64 choice)."""
    if L is None:
        L = np.linalg.cholesky(np.asarray(Fp, np.float64))
    w = np.asarray(w, np.float64)
    c = np.asarray(c, np.float64)
    p_dev = np.asarray(p_dev, np.int64)
    d = w.shape[0]
    gap = float(np.max(np.diff(np.sort(c)))) if c.shape[0] > 1 else 0.0
    e = np.zeros(d)
    worst = -np.inf
    differ = 0
    for j in range(d - 1, -1, -1):
        s = float(L[j + 1:, j] @ e[j + 1:])
        term = np.abs(L[j, j] * (c - w[j]) + s)
        q_ref = int(np.argmin(term))
        q = int(p_dev[j])
        worst = max(worst, float(term[q] - term[q_ref]) - tol * L[j, j] * gap)
        if q != q_ref:
            differ += 1
        e[j] = c[q] - w[j]
    return worst, differ
