"""GPU parity of the GANQ-style alternation (ganq_quantize, ganq_factor_damped).

GANQ summary page, "Approach": a closed-form codebook update alternated with an
assignment by Cholesky / back-substitution.  Bars:
  * factor: the float32 L of F'_g within 1e-6 relative Frobenius of numpy's float64
    Cholesky of the same F' (float64 on the GPU, rounded once);
  * assignment, from the GPU's own codebook: every decision within 1e-4 of the
    codebook spacing (in units of the term L_jj e_j + s_j) of the fp64 nearest
    entry with the GPU's later decisions fixed, and >= 99.9 % identical;
  * end to end on the mid-size layer: final objective within 1e-3 of the oracle's
    own run; the trace matches the oracle's objective of the GPU's states;
  * a group whose gradients vanish (F' = 0) is flagged and keeps its codes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _util import f64, rel_fro, to_dev
from test_gpu_lnq import MID, Problem, RHO, _wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mid(device):
    return Problem(device, MID, seed=1)


def _factors(prob):
    return [np.linalg.cholesky(Fp) for Fp in prob.Fp]


def test_ganq_factor_matches_numpy(device, mid):
    L, npd = gq.ganq_factor_damped(mid.F, RHO)
    torch.cuda.synchronize()
    assert npd.cpu().numpy().tolist() == [0] * MID.groups
    Ln = L.cpu().double().numpy()
    for g, Lref in enumerate(_factors(mid)):
        assert np.all(np.triu(Ln[g], 1) == 0.0)
        e = rel_fro(Ln[g], Lref)
        print(f"group {g}: factor rel Frobenius {e:.2e}")
        assert e <= 1e-6


@pytest.mark.parametrize("d,groups", [(64, 1), (128, 2), (192, 3), (320, 1)])
def test_ganq_factor_panel_counts(device, d, groups):
    """One to five 64-wide panels: no trailing update, a column update only, and the
    second-stream rest-updates of the lookahead.  F'_g = F_g + rho mean(diag F_g) I of
    seeded SPD F_g against numpy's float64 Cholesky, within 1e-6 relative Frobenius."""
    rng = np.random.default_rng(d + groups)
    X = rng.standard_normal((groups, 3 * d, d))
    F32 = np.einsum("gni,gnj->gij", X, X).astype(np.float32) / np.float32(3 * d)
    F32 = (F32 + np.transpose(F32, (0, 2, 1))) * np.float32(0.5)
    L, npd = gq.ganq_factor_damped(to_dev(np.ascontiguousarray(F32), "cuda"), RHO)
    torch.cuda.synchronize()
    assert npd.cpu().numpy().tolist() == [0] * groups
    Ln = L.cpu().double().numpy()
    for g in range(groups):
        F64 = F32[g].astype(np.float64)
        Fp = F64 + RHO * np.mean(np.diag(F64)) * np.eye(d)
        e = rel_fro(Ln[g], np.linalg.cholesky(Fp))
        print(f"d={d} group {g}: factor rel Frobenius {e:.2e}")
        assert np.all(np.triu(Ln[g], 1) == 0.0)
        assert e <= 1e-6


def _check_assignment(prob, C1, P1, rows=None, tol=1e-4, frac=0.999):
    Ls = _factors(prob)
    rows = range(prob.wl.d_out) if rows is None else rows
    worst, differ, dec = -np.inf, 0, 0
    for j in rows:
        g = j // prob.rpg
        ex, dif = O.ganq_replay(prob.Fp[g], prob.w[j], C1[j], P1[j], tol, Ls[g])
        worst = max(worst, ex)
        differ += dif
        dec += prob.wl.d_in
    agree = 1.0 - differ / dec
    print(f"assignment: decisions identical {agree:.6f}, worst excess {worst:.3e}")
    assert worst <= 0.0
    assert agree >= frac


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_ganq_assignment_replay(device, mid, bits):
    m = 1 << bits
    C0, P0, _, _ = gq.lnq_quantize(mid.W, mid.F, bits, 0)
    C1, P1, tr, nch, npd = gq.ganq_quantize(mid.W, mid.F, bits, 1, ridge_rel=RHO, C=C0.clone(),
                                            P=P0.clone())
    torch.cuda.synchronize()
    C1, P1 = f64(C1), P1.cpu().numpy()
    assert P1.max() < m
    _check_assignment(mid, C1, P1)
    assert int(nch[0].item()) == int(np.sum(P1 != P0.cpu().numpy()))


def test_ganq_end_to_end_mid(device, mid):
    iters = 3
    C, P, tr, _, npd = gq.ganq_quantize(mid.W, mid.F, 3, iters, ridge_rel=RHO)
    torch.cuda.synchronize()
    C, P, tr = f64(C), P.cpu().numpy(), tr.cpu().numpy()
    gpu = ref = 0.0
    for j in range(MID.d_out):
        Fp = mid.Fp_row(j)
        _, _, t_ref = O.ganq_row(Fp, mid.w[j], 8, iters)
        ref += t_ref[-1]
        gpu += O.objective(Fp, mid.w[j], C[j], P[j])
    print(f"GANQ end to end: gpu {gpu:.6e} oracle {ref:.6e}; trace {tr}")
    assert abs(gpu - ref) <= 1e-3 * ref
    assert abs(tr[-1] - gpu) <= 1e-4 * gpu
    # each codebook step is a closed-form minimiser: it never raises the objective
    for t in range(1, iters + 1):
        assert tr[2 * t - 1] <= tr[2 * t - 2] * (1 + 1e-6)


@pytest.mark.parametrize("d_in,d_out,groups,bits", [
    (576, 200, 2, 2),      # ragged tiles and 16-row groups, a partial last super-block
    (256, 48, 1, 4),       # m = 16
    (1024, 64, 4, 1),      # m = 2, four groups of 16 rows
])
def test_ganq_shapes(device, d_in, d_out, groups, bits):
    wl = _wl("ganq", d_in, d_out, 1536, groups, bits, index=33)
    prob = Problem(device, wl, seed=d_in + 11)
    C0, P0, _, _ = gq.lnq_quantize(prob.W, prob.F, bits, 0)
    C1, P1, _, _, npd = gq.ganq_quantize(prob.W, prob.F, bits, 1, ridge_rel=RHO, C=C0.clone(),
                                         P=P0.clone())
    torch.cuda.synchronize()
    assert npd.cpu().numpy().tolist() == [0] * groups
    _check_assignment(prob, f64(C1), P1.cpu().numpy())


def test_ganq_zero_fisher_group_keeps_codes(device):
    """Group 1's gradients are all zero and ridge_rel = 0: F'_1 = 0 has no factor; the
    group is flagged and its codes stay as they were, group 0 is assigned as usual."""
    wl = _wl("ganq0", 256, 64, 1024, 2, 3, index=34)
    inp = synth.make_inputs(wl, seed=5)
    G = synth.decode(inp["G"]).copy()
    G[:, 32:] = 0.0
    F32 = O.fisher(synth.decode(inp["X"]), G, 2).astype(np.float32)
    F32 = (F32 + np.transpose(F32, (0, 2, 1))) * np.float32(0.5)
    F = to_dev(np.ascontiguousarray(F32), "cuda")
    W = to_dev(inp["W"], "cuda")
    C0, P0, _, _ = gq.lnq_quantize(W, F, 3, 0)
    C1, P1, _, _, npd = gq.ganq_quantize(W, F, 3, 1, ridge_rel=0.0, C=C0.clone(), P=P0.clone())
    torch.cuda.synchronize()
    assert npd.cpu().numpy().tolist() == [0, 1]
    assert torch.equal(P1[32:], P0[32:])


def test_ganq_deterministic(device, mid):
    """The factor runs its trailing updates on a second stream ordered by events; two
    runs of the whole alternation give bitwise identical codebooks, codes, traces and
    factors."""
    a = gq.ganq_quantize(mid.W, mid.F, 3, 3, ridge_rel=RHO)
    b = gq.ganq_quantize(mid.W, mid.F, 3, 3, ridge_rel=RHO)
    La, _ = gq.ganq_factor_damped(mid.F, RHO)
    Lb, _ = gq.ganq_factor_damped(mid.F, RHO)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(La, Lb)


def test_ganq_deterministic_many_panels(device):
    """Twelve 64-wide panels (the lookahead's second stream active for ten of them):
    two factorizations are bitwise identical."""
    rng = np.random.default_rng(99)
    d = 768
    X = rng.standard_normal((2 * d, d))
    F32 = (X.T @ X / (2 * d)).astype(np.float32)
    F32 = np.ascontiguousarray(((F32 + F32.T) * np.float32(0.5))[None])
    F = to_dev(F32, "cuda")
    La, _ = gq.ganq_factor_damped(F, RHO)
    Lb, _ = gq.ganq_factor_damped(F, RHO)
    torch.cuda.synchronize()
    assert torch.equal(La, Lb)
