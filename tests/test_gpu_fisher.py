"""GPU parity of the grouped Fisher (gq_fisher_accumulate) against the fp64 oracle.

Bars, for bfloat16 inputs (bfloat16 operands, float32 accumulation), per group and
on every entry, so an off-diagonal tile cannot hide behind a few large diagonal
entries:
  * |F_gpu[a,b] - F_ref[a,b]| <= (2^-8 + (n + 64) 2^-24) A[a,b] with
    A[a,b] = sum_t s_g[t] |X[t,a] X[t,b]| (the oracle's Fisher of |X|).  The scaled
    operand s_g[t] X[t,b] is rounded once to bfloat16 (8 significant bits: relative
    error below 2^-8), the product with X[t,a] is exact, and float32 sums of n terms
    add at most n 2^-24 of the absolute sum.  This bound holds for any token count;
  * |F_gpu[a,b] - F_ref[a,b]| <= 2e-3 sqrt(F_ref[a,a] F_ref[b,b]) on every entry
    whose effective token count n_eff = A[a,b]^2 / sum_t (s_g[t] X[t,a] X[t,b])^2 is
    at least 64: the rounding errors of many comparable terms average out, while an
    entry carried by a handful of tokens (few tokens, or heavy-tailed per-token
    weights) can be off by up to 2^-8 = 3.9e-3 of its own size from one rounding;
  * ||F_gpu - F_ref||_F / ||F_ref||_F <= 2e-3.
float32 inputs take the float64-accumulating path and must agree to float32
rounding (1e-6).  The result must be exactly symmetric.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _util import f64, rel_fro, to_dev

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-3


def _custom(name, d_in, d_out, n, groups, dtype="bf16", x_kind="normal", outliers=0,
            oscale=1.0, index=20):
    return synth.Workload(name, d_in, d_out, n, groups, 3, 1, 32, dtype, x_kind, outliers,
                          oscale, "normal", 0.02, 1e-3, index)


def _run(device, inp, groups, **kw):
    X, G = to_dev(inp["X"], device), to_dev(inp["G"], device)
    F = gq.gq_fisher_accumulate(X, G, groups, **kw)
    torch.cuda.synchronize()
    return F


def _check_symmetric(F):
    assert torch.equal(F, F.transpose(1, 2)), "F is not exactly symmetric"
    assert torch.isfinite(F).all()


def _check_entries(F64, inp, groups, tol=BF16_TOL):
    """The three bars of the module docstring, against the oracle's Fisher of the
    stored inputs."""
    X, G = synth.decode(inp["X"]), synth.decode(inp["G"])
    n = X.shape[0]
    ref = O.fisher(X, G, groups)
    absref = O.fisher(np.abs(X), G, groups)
    S2 = O.group_scale(G, groups) ** 2
    X2 = X * X
    rigorous = 2.0 ** -8 + (n + 64) * 2.0 ** -24
    worst = worst_abs = 0.0
    checked = 0
    for g in range(groups):
        err = np.abs(F64[g] - ref[g])
        ok = err <= rigorous * absref[g]
        assert ok.all(), ("bound", g, np.argwhere(~ok)[:5], err[~ok][:5], absref[g][~ok][:5])
        nz = absref[g] > 0
        if nz.any():
            worst_abs = max(worst_abs, float(np.max(err[nz] / absref[g][nz])))
        dg = np.sqrt(np.maximum(np.diag(ref[g]), 0.0))
        scale = np.outer(dg, dg)
        sq = X2.T @ (S2[g][:, None] * X2)            # sum_t (s x_a x_b)^2
        with np.errstate(divide="ignore", invalid="ignore"):
            n_eff = np.where(sq > 0, absref[g] ** 2 / sq, 0.0)
        many = n_eff >= 64
        checked += int(many.sum())
        ok = ~many | (err <= tol * scale)
        assert ok.all(), ("entry", g, np.argwhere(~ok)[:5], err[~ok][:5], scale[~ok][:5])
        nz = many & (scale > 0)
        if nz.any():
            worst = max(worst, float(np.max(err[nz] / scale[nz])))
        e = rel_fro(F64[g], ref[g]) if np.any(ref[g]) else float(np.abs(F64[g]).max())
        assert e <= tol, (g, e)
    print(f"n={n}: worst entry error / sqrt(F_aa F_bb) {worst:.3e} over {checked} entries with "
          f"n_eff >= 64; / sum_t s|x_a x_b| {worst_abs:.3e} (bound {rigorous:.3e})")
    return worst


def test_fisher_tiny_f32(device):
    """Tiny single layer (d_in=128, d_out=64, n=256, float32, one group)."""
    inp = synth.make_inputs("tiny", seed=0)
    F = _run(device, inp, 1)
    ref = O.fisher(synth.decode(inp["X"]), synth.decode(inp["G"]), 1)
    _check_symmetric(F)
    assert rel_fro(f64(F), ref) <= 1e-6


def test_fisher_f32_ragged(device):
    """float32 path, d_in not a multiple of 8, three groups."""
    wl = _custom("f32r", 100, 12, 77, 3, dtype="f32", outliers=3, oscale=10.0, index=21)
    inp = synth.make_inputs(wl, seed=1)
    F = _run(device, inp, 3)
    ref = O.fisher(synth.decode(inp["X"]), synth.decode(inp["G"]), 3)
    _check_symmetric(F)
    for g in range(3):
        assert rel_fro(f64(F[g]), ref[g]) <= 1e-6


@pytest.mark.parametrize("d_in,d_out,n,groups,x_kind,outl", [
    (776, 96, 3001, 3, "normal", 4),        # ragged tile (3 x 256 + 8) and ragged token chunk
    (520, 64, 16384, 4, "gated", 2),        # split over tokens, ragged tile
    (256, 8, 64, 2, "normal", 0),           # one tile, one token chunk
    (8, 4, 5, 1, "gated", 0),               # smallest shape the matrix-core path takes
])
def test_fisher_bf16_parity(device, d_in, d_out, n, groups, x_kind, outl):
    wl = _custom("bf", d_in, d_out, n, groups, x_kind=x_kind, outliers=outl, oscale=30.0,
                 index=22)
    inp = synth.make_inputs(wl, seed=d_in)
    F = _run(device, inp, groups)
    _check_symmetric(F)
    _check_entries(f64(F), inp, groups)


def test_fisher_accumulate_streams_tokens(device):
    wl = _custom("acc", 264, 32, 4000, 2, outliers=2, oscale=20.0, index=23)
    inp = synth.make_inputs(wl, seed=5)
    X, G = to_dev(inp["X"], device), to_dev(inp["G"], device)
    F = gq.gq_fisher_accumulate(X[:1500].contiguous(), G[:1500].contiguous(), 2)
    gq.gq_fisher_accumulate(X[1500:].contiguous(), G[1500:].contiguous(), 2, F=F,
                            accumulate=True)
    torch.cuda.synchronize()
    _check_symmetric(F)
    _check_entries(f64(F), inp, 2)


@pytest.mark.parametrize("sigma", [1.0, 2.5])
def test_fisher_token_dependent_gradients(device, sigma):
    """Every token row of G scaled by a log-normal factor exp(sigma z_t): the per-token
    weights s_g[t] then span orders of magnitude (not the few percent of i.i.d.
    Laplace gradients), so F_g is far from a multiple of X^T X and the scaled operand
    carries the guided weighting.  Same element-wise bar."""
    wl = synth.Workload("lognormal", 776, 96, 5000, 3, 3, 1, 32, "bf16", "gated", 4, 30.0,
                        "normal", 0.02, 1e-3, 25, g_row_sigma=sigma)
    inp = synth.make_inputs(wl, seed=7)
    S = O.group_scale(synth.decode(inp["G"]), 3)
    spread = np.percentile(S, 99, axis=1) / np.percentile(S, 1, axis=1)
    print(f"sigma {sigma}: s_g 99th / 1st percentile {spread}")
    assert np.all(spread > 20.0)
    F = _run(device, inp, 3)
    _check_symmetric(F)
    _check_entries(f64(F), inp, 3)


def test_fisher_deterministic(device):
    wl = _custom("det", 520, 64, 9000, 4, x_kind="gated", index=24)
    inp = synth.make_inputs(wl, seed=6)
    F1 = _run(device, inp, 4)
    F2 = _run(device, inp, 4)
    assert torch.equal(F1, F2)
