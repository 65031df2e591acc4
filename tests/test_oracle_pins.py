"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a hand-worked
example, brute force, a closed-form identity, or a textbook special case.
CPU only.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_gq_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _spd(rng, d, n=None, diag_boost=0.0):
    n = n or 3 * d
    y = rng.standard_normal((n, d))
    return y.T @ y / n + diag_boost * np.eye(d)


# --------------------------------------------------------------------------
# Hand-worked examples (GuidedQuant blog page: objective equation, LNQ box)
# --------------------------------------------------------------------------

def test_golden_fisher():
    ex = json.load(open(GOLDEN))["fisher"]
    X, G = np.array(ex["X"]), np.array(ex["G"])
    np.testing.assert_allclose(O.fisher(X, G, 1), np.array(ex["groups_1"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(O.fisher(X, G, 2), np.array(ex["groups_2"]), rtol=0, atol=1e-13)


def test_golden_codebook():
    ex = json.load(open(GOLDEN))["codebook"]
    F, w, p = np.array(ex["F"]), np.array(ex["w"]), np.array(ex["p"])
    A, b = O.codebook_system(F, w, p, 2)
    np.testing.assert_allclose(A, np.array(ex["A"]), atol=1e-14)
    np.testing.assert_allclose(b, np.array(ex["b"]), atol=1e-14)
    c = O.codebook_update(F, w, p, np.array(ex["c_old"]))
    np.testing.assert_allclose(c, np.array(ex["c"]), rtol=1e-15)


def test_golden_sweep():
    ex = json.load(open(GOLDEN))["sweep"]
    F, w, c = np.array(ex["F"]), np.array(ex["w"]), np.array(ex["c"])
    p0 = np.array(ex["p_start"])
    assert O.objective(F, w, c, p0) == pytest.approx(ex["objective_start"], abs=1e-14)
    p1 = O.assign_sweep(F, w, c, p0)
    assert list(p1) == ex["p_end"]
    assert O.objective(F, w, c, p1) == pytest.approx(ex["objective_end"], abs=1e-14)


def test_golden_ridge():
    """lambda = rho * mean(diag F) + lam_abs, worked by hand: only the diagonal
    enters, through its mean (not its sum, not the mean of every entry)."""
    ex = json.load(open(GOLDEN))["ridge"]
    for case in ex["cases"]:
        F = np.array(case["F"], dtype=np.float64)
        lam = O.ridge_lambda(F, case["rho"], case["lam_abs"])
        assert lam == pytest.approx(case["lambda"], rel=1e-15, abs=1e-15)
        Fp = O.damped(F, case["rho"], case["lam_abs"])
        np.testing.assert_allclose(np.diag(Fp), case["damped_diag"], rtol=1e-15)
        off = ~np.eye(F.shape[0], dtype=bool)
        np.testing.assert_array_equal(Fp[off], F[off])
    # the default is the relative ridge alone
    F = np.array(ex["cases"][0]["F"])
    assert O.ridge_lambda(F, 0.5) == 1.5


def test_lnq_row_without_trace_takes_the_same_steps():
    rng = _rng(5)
    d, m = 48, 4
    Fp = O.damped(_spd(rng, d), 1e-6)
    w = rng.standard_normal(d)
    c1, p1, t1 = O.lnq_row(Fp, w, m, 3)
    c2, p2, t2 = O.lnq_row(Fp, w, m, 3, trace=False)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(p1, p2)
    assert t2.shape == (1,) and t2[0] == t1[-1]


# --------------------------------------------------------------------------
# Fisher: brute-force sums, the GuidedQuant identity, invariants
# --------------------------------------------------------------------------

def test_fisher_bruteforce_loops():
    rng = _rng(1)
    n, d, d_out = 7, 4, 6
    X = rng.standard_normal((n, d))
    G = rng.laplace(0, 1.0, (n, d_out))
    for groups in (1, 2, 3, 6):
        F = O.fisher(X, G, groups)
        size = d_out // groups
        for g in range(groups):
            for a in range(d):
                for b in range(d):
                    acc = 0.0
                    for t in range(n):
                        s = sum(G[t, j] * G[t, j] for j in range(g * size, (g + 1) * size)) / size
                        acc += s * X[t, a] * X[t, b]
                    assert F[g, a, b] == pytest.approx(acc, rel=1e-12, abs=1e-14)


def test_guidedquant_identity_tiny_workload():
    """|| G (.) (X W^T - X W_hat^T) ||^2 = sum_j e_j^T F_j e_j  (objective equation, no 1/n)."""
    inp = synth.make_inputs("tiny", seed=3)
    X, W, G = (synth.decode(inp[k]) for k in ("X", "W", "G"))
    rng = _rng(2)
    W_hat = W + 0.01 * rng.standard_normal(W.shape)
    lhs = O.guided_loss(X, G, W, W_hat)
    Fj = O.fisher_per_channel(X, G)
    E = W_hat - W
    rhs = sum(E[j] @ Fj[j] @ E[j] for j in range(W.shape[0]))
    assert lhs == pytest.approx(rhs, rel=1e-10)
    # group average of the per-channel blocks equals the grouped Fisher
    for groups in (1, 2, 4):
        Fg = O.fisher(X, G, groups)
        size = W.shape[0] // groups
        for g in range(groups):
            np.testing.assert_allclose(Fg[g], Fj[g * size:(g + 1) * size].mean(0), rtol=1e-12,
                                       atol=1e-12 * np.abs(Fg[g]).max())


def test_layerwise_special_case():
    """G == 1 reduces the guided loss to the layer-wise reconstruction loss (item 1)."""
    rng = _rng(4)
    n, d, d_out = 40, 8, 5
    X = rng.standard_normal((n, d))
    W = rng.standard_normal((d_out, d))
    W_hat = W + 0.1 * rng.standard_normal(W.shape)
    G = np.ones((n, d_out))
    lhs = float(np.sum((X @ W.T - X @ W_hat.T) ** 2))
    F = O.fisher(X, G, 1)[0]
    rhs = sum((W_hat[j] - W[j]) @ F @ (W_hat[j] - W[j]) for j in range(d_out))
    assert lhs == pytest.approx(rhs, rel=1e-12)
    assert O.guided_loss(X, G, W, W_hat) == pytest.approx(lhs, rel=1e-13)


def test_fisher_invariants():
    rng = _rng(5)
    n, d, d_out = 64, 12, 8
    X = rng.standard_normal((n, d))
    G = rng.laplace(0, 1e-3, (n, d_out))
    F = O.fisher(X, G, 2)
    S = O.group_scale(G, 2)
    for g in range(2):
        assert np.abs(F[g] - F[g].T).max() <= 1e-12 * np.abs(F[g]).max()
        assert np.linalg.eigvalsh(F[g]).min() >= -1e-12 * np.abs(F[g]).max()
        assert np.trace(F[g]) == pytest.approx(float(np.sum(S[g] * np.sum(X * X, 1))), rel=1e-12)
    # additivity over token chunks
    F1 = O.fisher(X[:20], G[:20], 2)
    F2 = O.fisher(X[20:], G[20:], 2)
    np.testing.assert_allclose(F1 + F2, F, rtol=1e-12, atol=1e-15)


def test_fisher_entry_matches_definition():
    rng = _rng(6)
    X = rng.standard_normal((50, 6))
    G = rng.standard_normal((50, 4))
    F = O.fisher(X, G, 2)
    S = O.group_scale(G, 2)
    for g, a, b in [(0, 0, 0), (1, 2, 5), (0, 5, 3)]:
        assert O.fisher_entry(X[:, a], X[:, b], S[g]) == pytest.approx(F[g, a, b], rel=1e-13)


# --------------------------------------------------------------------------
# Assignment step: residual-form deltas against brute-force re-evaluation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(4))
def test_sweep_deltas_bruteforce(seed):
    rng = _rng(10 + seed)
    d, m = 9, 4
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p = rng.integers(0, m, d)
    p_end, steps = O.assign_sweep(F, w, c, p, return_steps=True)
    # replay and check every delta by re-evaluating the objective directly
    pc = p.copy()
    for i in range(d):
        base = O.objective(F, w, c, pc)
        for q in range(m):
            trial = pc.copy()
            trial[i] = q
            assert steps[i][q] == pytest.approx(O.objective(F, w, c, trial) - base,
                                                rel=1e-9, abs=1e-12)
        best = int(np.argmin(steps[i]))
        if steps[i][best] < 0:
            pc[i] = best
    assert np.array_equal(pc, p_end)


def test_sweep_is_one_opt_at_fixed_point():
    rng = _rng(20)
    d, m = 8, 3
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p = rng.integers(0, m, d)
    for _ in range(50):
        p_new = O.assign_sweep(F, w, c, p)
        if np.array_equal(p_new, p):
            break
        p = p_new
    base = O.objective(F, w, c, p)
    for i in range(d):
        for q in range(m):
            t = p.copy()
            t[i] = q
            assert O.objective(F, w, c, t) >= base - 1e-12


def test_sweep_diagonal_F_is_global_optimum():
    """Diagonal F: one sweep reaches the brute-force optimum over all m^d assignments."""
    rng = _rng(21)
    d, m = 7, 4
    F = np.diag(rng.uniform(0.5, 2.0, d))
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p0 = rng.integers(0, m, d)
    p = O.assign_sweep(F, w, c, p0)
    best = min(O.objective(F, w, c, np.array(t)) for t in itertools.product(range(m), repeat=d))
    assert O.objective(F, w, c, p) == pytest.approx(best, rel=1e-12, abs=1e-15)


# --------------------------------------------------------------------------
# Codebook step: normal equations, exact minimiser, empty codes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_codebook_normal_equations_and_minimiser(seed):
    rng = _rng(30 + seed)
    d, m = 24, 8
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    p = rng.integers(0, m - 2, d)          # codes m-2, m-1 stay empty
    c_old = np.sort(rng.standard_normal(m))
    c = O.codebook_update(F, w, p, c_old)
    e = c[p] - w
    grad = O.one_hot(p, m).T @ (F @ e)     # P^T F (w_hat - w)
    S = np.bincount(p, minlength=m) > 0
    assert np.abs(grad[S]).max() <= 1e-10 * np.abs(O.one_hot(p, m).T @ F @ w).max()
    np.testing.assert_array_equal(c[~S], c_old[~S])
    base = O.objective(F, w, c, p)
    for q in np.nonzero(S)[0]:
        for eps in (1e-3, -1e-3, 1e-6, -1e-6):
            cc = c.copy()
            cc[q] += eps
            assert O.objective(F, w, cc, p) >= base


def test_codebook_identity_F_is_cluster_mean():
    rng = _rng(40)
    d, m = 30, 4
    w = rng.standard_normal(d)
    p = rng.integers(0, m, d)
    c = O.codebook_update(np.eye(d), w, p, np.zeros(m))
    for q in range(m):
        if np.any(p == q):
            assert c[q] == pytest.approx(float(np.mean(w[p == q])), rel=1e-12, abs=1e-15)


def test_codebook_diagonal_F_is_weighted_mean():
    rng = _rng(41)
    d, m = 30, 4
    f = rng.uniform(0.1, 3.0, d)
    w = rng.standard_normal(d)
    p = rng.integers(0, m, d)
    c = O.codebook_update(np.diag(f), w, p, np.zeros(m))
    for q in range(m):
        sel = p == q
        if np.any(sel):
            assert c[q] == pytest.approx(float(np.sum(f[sel] * w[sel]) / np.sum(f[sel])), rel=1e-12)


# --------------------------------------------------------------------------
# Whole LNQ loop
# --------------------------------------------------------------------------

def _lloyd_1d(w, c, p, iters):
    """Textbook 1-D Lloyd k-means with LNQ's conventions (empty centre kept,
    move only to a strictly closer centre, lowest index among the closest)."""
    c = c.copy()
    p = p.copy()
    for _ in range(iters):
        for q in range(len(c)):
            members = [w[i] for i in range(len(w)) if p[i] == q]
            if members:
                c[q] = sum(members) / len(members)
        for i in range(len(w)):
            dist = [(w[i] - c[q]) ** 2 for q in range(len(c))]
            best = min(range(len(c)), key=lambda q: (dist[q], q))
            if dist[best] < dist[p[i]]:
                p[i] = best
    return c, p


def test_lnq_identity_F_is_lloyd():
    rng = _rng(50)
    d, m = 200, 8
    w = rng.standard_normal(d) * 0.02
    c0, p0 = O.init_quantile(w, m)
    c, p, trace = O.lnq_row(np.eye(d), w, m, 6)
    cl, pl = _lloyd_1d(w, c0, p0, 6)
    assert np.array_equal(p, pl)
    np.testing.assert_allclose(c, cl, rtol=1e-12, atol=1e-16)


def test_lnq_monotone_and_bruteforce_bound():
    rng = _rng(51)
    d, m = 8, 3
    F = _spd(rng, d, n=5)                 # rank-deficient: the ridge keeps F' PD
    Fp = O.damped(F, 1e-6)
    w = rng.standard_normal(d)
    c, p, trace = O.lnq_row(Fp, w, m, 8)
    assert np.all(np.diff(trace) <= 1e-12 * trace[0])
    # joint brute force: for each assignment, the best codebook is the codebook step
    best = np.inf
    for t in itertools.product(range(m), repeat=d):
        t = np.array(t)
        cc = O.codebook_update(Fp, w, t, np.zeros(m))
        best = min(best, O.objective(Fp, w, cc, t))
    assert trace[-1] >= best - 1e-12 * abs(best)


def test_lnq_monotone_on_tiny_workload_rows():
    inp = synth.make_inputs("tiny", seed=0)
    X, W, G = (synth.decode(inp[k]) for k in ("X", "W", "G"))
    Fp = O.damped(O.fisher(X, G, 1)[0], 1e-6)
    for j in range(6):
        c, p, trace = O.lnq_row(Fp, W[j], 8, 5)
        assert np.all(np.diff(trace) <= 1e-12 * trace[0])
        assert trace[-1] < trace[0]


def test_lnq_scale_invariance():
    rng = _rng(52)
    d, m = 40, 4
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    r1 = O.lnq_row(O.damped(F, 1e-6), w, m, 4)
    r2 = O.lnq_row(O.damped(37.5 * F, 1e-6), w, m, 4)
    assert np.array_equal(r1[1], r2[1])
    np.testing.assert_allclose(r1[0], r2[0], rtol=1e-10)


def test_ridge_makes_rank_deficient_fisher_solvable():
    rng = _rng(53)
    d, m = 16, 4
    y = rng.standard_normal((3, d))          # rank 3 < d
    F = y.T @ y
    w = rng.standard_normal(d)
    p = rng.integers(0, m, d)
    c = O.codebook_update(O.damped(F, 1e-6), w, p, np.zeros(m))
    assert np.all(np.isfinite(c))


# --------------------------------------------------------------------------
# Initialisation (reading; pinned to the textbook linear quantile)
# --------------------------------------------------------------------------


def test_zero_fisher_group_keeps_state():
    """A group whose gradients all vanish has F = 0, hence lambda = 0 and F' = 0.
    Every objective is 0, the codebook system P^T F' P = 0 has no unique solution
    (the codebook is kept), no coordinate strictly decreases the objective (no
    move), so LNQ returns its quantile initialisation unchanged."""
    rng = _rng(77)
    d, m = 64, 8
    X = rng.standard_normal((50, d))
    G = np.zeros((50, 4))
    G[:, :2] = rng.standard_normal((50, 2))
    F = O.fisher(X, G, 2)
    assert np.all(F[1] == 0.0) and np.any(F[0] != 0.0)
    Fp = O.damped(F[1], 1e-6)
    assert O.ridge_lambda(F[1], 1e-6) == 0.0 and np.all(Fp == 0.0)
    w = rng.standard_normal(d)
    c0, p0 = O.init_quantile(w, m)
    c, p, tr = O.lnq_row(Fp, w, m, 3)
    np.testing.assert_array_equal(c, c0)
    np.testing.assert_array_equal(p, p0)
    assert np.all(tr == 0.0)
    # with a positive definite F' the same state does move
    c1, p1, _ = O.lnq_row(O.damped(F[0], 1e-6), w, m, 1)
    assert np.any(c1 != c0)


def test_degenerate_rows_init_and_lnq():
    """All-zero and constant rows: every quantile is that constant, every
    coordinate takes code 0 (lowest index on ties), the objective is 0 at the start
    and stays 0; a row with two distinct values is reproduced exactly (each
    coordinate lands on an entry equal to its own value)."""
    rng = _rng(78)
    d, m = 64, 8
    F = _spd(rng, d)
    Fp = O.damped(F, 1e-6)
    for val in (0.0, 0.0137):
        w = np.full(d, val)
        c, p = O.init_quantile(w, m)
        np.testing.assert_array_equal(c, np.full(m, np.float64(np.float32(val))))
        np.testing.assert_array_equal(p, np.zeros(d, np.int64))
        c3, p3, tr = O.lnq_row(Fp, w, m, 3)
        np.testing.assert_array_equal(p3, p)
        assert tr[-1] <= 1e-28 + 1e-12 * (w @ Fp @ w)
    w = np.where(rng.random(d) < 0.3, -0.5, 0.25)
    c, p, tr = O.lnq_row(Fp, w, m, 2)
    assert tr[-1] <= 1e-12 * (w @ Fp @ w)
    dist = np.minimum(np.abs(c[p] + 0.5), np.abs(c[p] - 0.25))
    assert dist.max() <= 1e-12

@pytest.mark.parametrize("N,m", [(128, 8), (4096, 8), (11008, 4), (100, 16), (5, 2)])
def test_init_quantile_is_textbook_linear_quantile(N, m):
    rng = _rng(N + m)
    w = synth.decode(synth.f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32) * 0.02))
    c, p = O.init_quantile(w, m)
    ref = np.quantile(w, (np.arange(m) + 0.5) / m, method="linear").astype(np.float32)
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(c - ref.astype(np.float64)) <= ulp)
    assert np.all(np.diff(c) >= 0)
    for i in range(N):
        dist = np.abs(w[i] - c)
        assert dist[p[i]] == dist.min()
        assert p[i] == int(np.nonzero(dist == dist.min())[0][0])


# --------------------------------------------------------------------------
# Teacher-forced replay (the device-decision checker)
# --------------------------------------------------------------------------

def test_replay_accepts_own_decisions_and_rejects_a_planted_one():
    rng = _rng(60)
    d, m = 64, 8
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p0 = rng.integers(0, m, d)
    p1 = O.assign_sweep(F, w, c, p0)
    worst, differ = O.replay_sweep(F, w, c, p0, p1, 1e-5)
    assert worst <= 0 and differ == 0
    bad = p1.copy()
    # plant a clearly worse choice at the first coordinate
    D = O.assign_deltas(F[0, 0], (F @ (c[p0] - w))[0], c, c[p0[0]])
    bad[0] = int(np.argmax(D))
    worst, differ = O.replay_sweep(F, w, c, p0, bad, 1e-5)
    assert worst > 0 and differ >= 1


# --------------------------------------------------------------------------
# Input generator (not the method): bf16 rounding and determinism
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    import torch
    rng = _rng(70)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_deterministic_and_prefix_stable():
    a = synth.make_inputs("tiny", seed=7)
    b = synth.make_inputs("tiny", seed=7)
    for k in ("X", "W", "G"):
        assert np.array_equal(a[k], b[k])
    c = synth.make_inputs("tiny", seed=7, tokens=100, rows=10)
    assert np.array_equal(c["X"], a["X"][:100])
    assert np.array_equal(c["W"], a["W"][:10])
    wl = synth.workload("tiny")
    X = synth.decode(a["X"])
    # four outlier columns scaled x20
    big = np.sort(np.argsort(np.std(X, 0))[-4:])
    assert np.array_equal(big, a["outlier_cols"])
    assert wl.m == 8


# --------------------------------------------------------------------------
# Fixed-grid backend: uniform min-max grid, assignment passes only
# --------------------------------------------------------------------------

def test_uniform_grid_hand_example():
    """w = (-1, 0.5, 2), m = 4: grid -1, 0, 1, 2; 0.5 is equally far from 0 and 1 and
    takes the lower index; codes (0, 1, 3)."""
    c, p = O.init_uniform_grid(np.array([-1.0, 0.5, 2.0]), 4)
    np.testing.assert_array_equal(c, [-1.0, 0.0, 1.0, 2.0])
    np.testing.assert_array_equal(p, [0, 1, 3])


@pytest.mark.parametrize("m", [2, 4, 8, 16])
def test_uniform_grid_definition(m):
    """Endpoints at the row's minimum and maximum, equal spacing, nearest codes
    (brute force over the grid, lowest index on ties)."""
    rng = _rng(70 + m)
    for _ in range(20):
        w = (rng.standard_normal(257) * 0.02).astype(np.float32).astype(np.float64)
        c, p = O.init_uniform_grid(w, m)
        assert c[0] == w.min()
        ulp = np.spacing(np.float32(abs(w.max())))
        assert abs(c[-1] - w.max()) <= ulp
        assert np.all(np.diff(c) > 0)
        step = (w.max() - w.min()) / (m - 1)
        assert np.max(np.abs(np.diff(c) - step)) <= 2 * np.spacing(np.float32(np.abs(c).max()))
        for i in range(w.shape[0]):
            dist = np.abs(w[i] - c)
            assert dist[p[i]] == dist.min()
            assert p[i] == np.flatnonzero(dist == dist.min())[0]


def test_uniform_grid_constant_row():
    c, p = O.init_uniform_grid(np.full(9, 0.25), 8)
    assert np.all(c == 0.25) and np.all(p == 0)


def test_grid_row_diagonal_F_keeps_nearest_codes():
    """Diagonal F': the objective separates over coordinates and the nearest grid
    point is each coordinate's minimiser, so no pass moves a code."""
    rng = _rng(80)
    d, m = 40, 8
    F = np.diag(rng.uniform(0.1, 3.0, d))
    w = rng.standard_normal(d) * 0.02
    c0, p0 = O.init_uniform_grid(w, m)
    c, p, tr = O.grid_row(F, w, m, 3)
    np.testing.assert_array_equal(p, p0)
    np.testing.assert_array_equal(c, c0)
    assert np.all(tr == tr[0])


def test_grid_row_monotone_local_min_and_bruteforce_bound():
    """Coupled F': the trace never increases; once a pass changes nothing the codes
    are a one-coordinate local minimum (every single change checked), and the
    brute-force optimum over all m^d codes on the same grid is no larger."""
    rng = _rng(81)
    d, m = 6, 4
    for _ in range(5):
        F = _spd(rng, d, n=d + 2)
        w = rng.standard_normal(d)
        c, p, tr = O.grid_row(F, w, m, 12)
        assert np.all(np.diff(tr) <= 1e-15)
        assert np.array_equal(O.assign_sweep(F, w, c, p), p)
        base = O.objective(F, w, c, p)
        for i in range(d):
            for q in range(m):
                t = p.copy()
                t[i] = q
                assert O.objective(F, w, c, t) >= base - 1e-12
        best = min(O.objective(F, w, c, np.array(t)) for t in itertools.product(range(m), repeat=d))
        assert best <= base + 1e-15


# --------------------------------------------------------------------------
# LUT dequantisation GEMV: packing layout and the product
# --------------------------------------------------------------------------

def test_lut_pack_hand_examples():
    """bits 3: ten codes per word at shifts 0, 3, ..., 27:
    1 + 2*2^3 + 3*2^6 + 4*2^9 + 5*2^12 + 6*2^15 + 7*2^18 + 0*2^21 + 5*2^24 + 2*2^27
    = 0x151F58D1; the 11th code opens word 1; rows padded to 4 words.
    bits 4: eight codes per word, 0xA + 0x5*2^4 + 0xF*2^8 + 0x1*2^12 = 0x1F5A."""
    Q = O.lut_pack(np.array([[1, 2, 3, 4, 5, 6, 7, 0, 5, 2, 3]]), 3)
    np.testing.assert_array_equal(Q, [[0x151F58D1, 3, 0, 0]])
    Q = O.lut_pack(np.array([[0xA, 0x5, 0xF, 0x1, 0, 0, 0, 0, 0x3]]), 4)
    np.testing.assert_array_equal(Q, [[0x1F5A, 3, 0, 0]])
    assert [O.lut_codes_per_word(b) for b in (1, 2, 3, 4)] == [32, 16, 10, 8]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lut_pack_roundtrip(bits):
    rng = _rng(90 + bits)
    for d_in in (1, 9, 64, 333, 4096):
        P = rng.integers(0, 1 << bits, size=(5, d_in))
        Q = O.lut_pack(P, bits)
        rw = O.lut_row_words(d_in, bits)
        assert Q.shape == (5, rw) and rw % 4 == 0
        assert rw * 32 >= d_in * bits and (rw - 4) * O.lut_codes_per_word(bits) < d_in
        np.testing.assert_array_equal(O.lut_unpack(Q, d_in, bits), P)
        # every slot past d_in is zero
        cpw = O.lut_codes_per_word(bits)
        full = O.lut_unpack(Q, rw * cpw, bits)
        assert np.all(full[:, d_in:] == 0)


def test_oracle_bf16_round_matches_torch():
    import torch
    rng = _rng(91)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)


@pytest.mark.parametrize("lut_bf16", [False, True])
def test_lut_gemv_one_hot_codebook_gives_masked_sums(lut_bf16):
    """c^(j) = e_q: y_j is the sum of the activations whose code is q."""
    rng = _rng(92)
    d_out, d_in, m = 6, 50, 8
    P = rng.integers(0, m, size=(d_out, d_in))
    x = rng.standard_normal((3, d_in))
    for q in range(m):
        C = np.zeros((d_out, m), np.float32)
        C[:, q] = 1.0
        y = O.lut_gemv(C, P, x, lut_bf16)
        for b in range(3):
            for j in range(d_out):
                assert y[b, j] == pytest.approx(np.sum(x[b][P[j] == q]), rel=1e-15, abs=1e-15)


def test_lut_gemv_bruteforce_loops():
    """Small integer case against plain loops (exact in float64)."""
    rng = _rng(93)
    d_out, d_in, m = 3, 7, 4
    P = rng.integers(0, m, size=(d_out, d_in))
    C = rng.integers(-8, 9, size=(d_out, m)).astype(np.float32)
    x = rng.integers(-5, 6, size=(2, d_in)).astype(np.float64)
    y = O.lut_gemv(C, P, x, True)
    for b in range(2):
        for j in range(d_out):
            s = 0.0
            for i in range(d_in):
                s += float(C[j, P[j, i]]) * x[b, i]
            assert y[b, j] == s


# --------------------------------------------------------------------------
# GANQ-style assignment: back-substitution over F' = L L^T
# --------------------------------------------------------------------------

def test_ganq_hand_example():
    """F' = [[4, 2], [2, 2]] = L L^T with L = [[2, 0], [1, 1]]; w = (0.3, 0.6),
    codebook {0, 1}.  Coordinate 1 first: target 0.6 -> entry 1, e_1 = 0.4; then
    s_0 = L_10 e_1 = 0.4, target 0.3 - 0.4 / 2 = 0.1 -> entry 0, e_0 = -0.3.
    Objective e^T F' e = 0.36 - 0.48 + 0.32 = 0.2."""
    F = np.array([[4.0, 2.0], [2.0, 2.0]])
    p = O.ganq_assign(F, np.array([0.3, 0.6]), np.array([0.0, 1.0]))
    np.testing.assert_array_equal(p, [0, 1])
    assert O.objective(F, np.array([0.3, 0.6]), np.array([0.0, 1.0]), p) == pytest.approx(0.2)


def test_ganq_diagonal_F_gives_nearest_codes():
    rng = _rng(100)
    d, m = 30, 8
    F = np.diag(rng.uniform(0.1, 3.0, d))
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p = O.ganq_assign(F, w, c)
    np.testing.assert_array_equal(p, np.argmin(np.abs(w[:, None] - c[None, :]), axis=1))


@pytest.mark.parametrize("seed", range(4))
def test_ganq_is_the_reverse_lexicographic_minimiser(seed):
    """Brute force over all m^d codes: the assignment minimises |(L^T e)_{d-1}| first,
    then |(L^T e)_{d-2}|, ... down to |(L^T e)_0| (lowest index among exact ties),
    and its objective equals ||L^T e||^2."""
    rng = _rng(110 + seed)
    d, m = 5, 3
    F = _spd(rng, d, n=d + 3)
    L = np.linalg.cholesky(F)
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p = O.ganq_assign(F, w, c)
    best_key, best = None, None
    for t in itertools.product(range(m), repeat=d):
        e = c[np.array(t)] - w
        terms = np.abs(L.T @ e)
        key = tuple(terms[::-1])
        if best_key is None or key < best_key:
            best_key, best = key, np.array(t)
    np.testing.assert_array_equal(p, best)
    e = c[p] - w
    assert O.objective(F, w, c, p) == pytest.approx(float(np.sum((L.T @ e) ** 2)), rel=1e-12)
    opt = min(O.objective(F, w, c, np.array(t)) for t in itertools.product(range(m), repeat=d))
    assert opt <= O.objective(F, w, c, p) + 1e-15


def test_ganq_exact_when_weights_are_codebook_entries():
    rng = _rng(120)
    d, m = 40, 4
    F = _spd(rng, d)
    c = np.sort(rng.standard_normal(m))
    q = rng.integers(0, m, d)
    p = O.ganq_assign(F, c[q], c)
    np.testing.assert_array_equal(p, q)


def test_ganq_row_codebook_steps_do_not_increase():
    rng = _rng(121)
    d, m = 24, 4
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    _, _, tr = O.ganq_row(F, w, m, 4)
    for t in range(1, 5):
        assert tr[2 * t - 1] <= tr[2 * t - 2] * (1 + 1e-12) + 1e-15


def test_ganq_replay_accepts_own_decisions_and_rejects_a_planted_one():
    rng = _rng(122)
    d, m = 60, 8
    F = _spd(rng, d)
    w = rng.standard_normal(d)
    c = np.sort(rng.standard_normal(m))
    p = O.ganq_assign(F, w, c)
    worst, differ = O.ganq_replay(F, w, c, p, 1e-9)
    assert worst <= 0.0 and differ == 0
    bad = p.copy()
    bad[d // 2] = (bad[d // 2] + m // 2) % m
    worst, differ = O.ganq_replay(F, w, c, bad, 1e-9)
    assert worst > 0.0 and differ >= 1
