"""GPU parity of the fixed-grid backend (grid_quantize) against the fp64 oracle.

The backend keeps each row's uniform min-max grid and runs only the assignment
pass on the GuidedQuant objective (GuidedQuant blog page: the objective serves
any layer-wise quantizer; LNQ algorithm box, "(assignment)").  Bars:
  * initial grid (float32) and nearest codes identical to the oracle's;
  * every pass, teacher-forced from the GPU's own state before it: every
    decision valid under the fp64 replay (within 1e-5 |obj_row| of the best
    change) and >= 99.9 % of the decisions identical to the fp64 choice;
  * the trace never increases and its entries match the oracle's objective of
    the GPU's (C, P) within 1e-4 relative;
  * free-running end to end on the mid-size layer: final objective within 1e-3
    of the oracle's own run;
  * splitting the passes over several calls (GIVEN init) reproduces one call
    bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _util import f64, to_dev
from test_gpu_lnq import MID, Problem, RHO, _wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mid(device):
    return Problem(device, MID, seed=1)


def _passes_one_at_a_time(prob, bits, iters, block=gq.DEFAULT_BLOCK):
    """The GPU trajectory pass by pass (each call starts from the previous C, P)."""
    C, P, tr0, _ = gq.grid_quantize(prob.W, prob.F, bits, 0, block=block, ridge_rel=RHO)
    states = [(f64(C), P.cpu().numpy())]
    for _ in range(iters):
        C, P, _, _ = gq.grid_quantize(prob.W, prob.F, bits, 1, block=block, ridge_rel=RHO,
                                      C=C.clone(), P=P.clone())
        states.append((f64(C), P.cpu().numpy()))
    torch.cuda.synchronize()
    return states


def _check_trajectory(prob, bits, iters, rows=None, block=gq.DEFAULT_BLOCK):
    m = 1 << bits
    C, P, tr, nch = gq.grid_quantize(prob.W, prob.F, bits, iters, block=block, ridge_rel=RHO)
    torch.cuda.synchronize()
    tr = tr.cpu().numpy()
    assert np.all(tr[1:] <= tr[:-1] * (1 + 1e-6)), tr
    states = _passes_one_at_a_time(prob, bits, iters, block)
    np.testing.assert_array_equal(states[-1][1], P.cpu().numpy())
    np.testing.assert_array_equal(states[-1][0], f64(C))
    rows = range(prob.wl.d_out) if rows is None else rows
    dec = differ = 0
    worst = -np.inf
    obj = np.zeros(iters + 1)
    for j in rows:
        Fp, w = prob.Fp_row(j), prob.w[j]
        c_init, p_init = O.init_uniform_grid(w, m)
        np.testing.assert_array_equal(states[0][0][j], c_init)
        np.testing.assert_array_equal(states[0][1][j], p_init)
        obj[0] += O.objective(Fp, w, c_init, p_init)
        for t in range(1, iters + 1):
            c = states[t][0][j]
            np.testing.assert_array_equal(c, c_init)              # the grid never moves
            ex, dif = O.replay_sweep(Fp, w, c, states[t - 1][1][j], states[t][1][j], 1e-5)
            worst = max(worst, ex)
            differ += dif
            dec += w.shape[0]
            obj[t] += O.objective(Fp, w, c, states[t][1][j])
    frac = 1.0 - differ / dec
    print(f"grid passes: decisions identical {frac:.6f}, worst replay excess {worst:.2e}; "
          f"trace {tr}; oracle objective of the GPU states {obj}")
    assert worst <= 0.0
    assert frac >= 0.999
    if len(rows) == prob.wl.d_out:
        np.testing.assert_allclose(tr, obj, rtol=1e-4)
        moves = [int(np.sum(states[t][1] != states[t - 1][1])) for t in range(1, iters + 1)]
        assert moves == [int(x) for x in nch.cpu().numpy()]
    return C, P, tr


def test_grid_init_matches_oracle(device, mid):
    for bits in (1, 2, 3, 4):
        m = 1 << bits
        C, P, tr, _ = gq.grid_quantize(mid.W, mid.F, bits, 0)
        torch.cuda.synchronize()
        C, P = C.cpu().numpy(), P.cpu().numpy()
        for j in range(MID.d_out):
            c_ref, p_ref = O.init_uniform_grid(mid.w[j], m)
            np.testing.assert_array_equal(C[j], c_ref.astype(np.float32))
            np.testing.assert_array_equal(P[j], p_ref)


def test_grid_init_float32_and_degenerate_rows(device, mid):
    """float32 weights; a constant row (all codes 0) and a two-valued row."""
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((MID.d_out, MID.d_in)) * 0.02).astype(np.float32)
    W[3] = np.float32(0.125)
    W[7] = np.where(rng.random(MID.d_in) < 0.5, np.float32(-0.5), np.float32(0.25))
    C, P, _, _ = gq.grid_quantize(to_dev(W, device), mid.F, 3, 0)
    torch.cuda.synchronize()
    C, P = C.cpu().numpy(), P.cpu().numpy()
    for j in range(MID.d_out):
        c_ref, p_ref = O.init_uniform_grid(W[j].astype(np.float64), 8)
        np.testing.assert_array_equal(C[j], c_ref.astype(np.float32))
        np.testing.assert_array_equal(P[j], p_ref)
    assert np.all(P[3] == 0)
    assert set(np.unique(P[7])) == {0, 7}


def test_grid_passes_mid(device, mid):
    _check_trajectory(mid, 3, 4)


@pytest.mark.parametrize("d_in,d_out,groups,bits", [
    (576, 200, 2, 2),      # ragged matrix-core tiles, ragged 16-row sweep groups
    (256, 48, 1, 4),       # m = 16
    (1024, 64, 4, 1),      # m = 2, four groups of 16 rows
])
def test_grid_passes_shapes(device, d_in, d_out, groups, bits):
    wl = _wl("grid", d_in, d_out, 1536, groups, bits, index=32)
    _check_trajectory(Problem(device, wl, seed=d_in + 7), bits, 3)


def test_grid_end_to_end_mid(device, mid):
    """Free-running: the final objective within 1e-3 of the oracle's own run."""
    iters = 4
    C, P, tr, _ = gq.grid_quantize(mid.W, mid.F, 3, iters, ridge_rel=RHO)
    torch.cuda.synchronize()
    C, P = f64(C), P.cpu().numpy()
    gpu = ref = 0.0
    for j in range(MID.d_out):
        Fp = mid.Fp_row(j)
        _, _, t_ref = O.grid_row(Fp, mid.w[j], 8, iters)
        ref += t_ref[-1]
        gpu += O.objective(Fp, mid.w[j], C[j], P[j])
    print(f"grid end to end: gpu {gpu:.6e} oracle {ref:.6e}")
    assert abs(gpu - ref) <= 1e-3 * ref


def test_grid_given_resumes_exactly(device, mid):
    C5, P5, t5, _ = gq.grid_quantize(mid.W, mid.F, 3, 5)
    C2, P2, _, _ = gq.grid_quantize(mid.W, mid.F, 3, 2)
    C3, P3, _, _ = gq.grid_quantize(mid.W, mid.F, 3, 3, C=C2.clone(), P=P2.clone())
    torch.cuda.synchronize()
    assert torch.equal(C5, C3) and torch.equal(P5, P3)


def test_lnq_from_uniform_init(device, mid):
    """LNQ started from the uniform grid: the init equals the oracle's grid, the
    trace never increases, the final objective is within 1e-3 of the oracle's run
    from the same start."""
    iters = 3
    C, P, tr, _ = gq.lnq_quantize(mid.W, mid.F, 3, iters, ridge_rel=RHO, init=gq.GQ_INIT_UNIFORM)
    torch.cuda.synchronize()
    tr = tr.cpu().numpy()
    assert np.all(tr[1:] <= tr[:-1] * (1 + 1e-6)), tr
    C, P = f64(C), P.cpu().numpy()
    gpu = ref = start = 0.0
    for j in range(MID.d_out):
        Fp = mid.Fp_row(j)
        c0, p0 = O.init_uniform_grid(mid.w[j], 8)
        _, _, t_ref = O.lnq_row(Fp, mid.w[j], 8, iters, c0=c0, p0=p0)
        ref += t_ref[-1]
        start += t_ref[0]
        gpu += O.objective(Fp, mid.w[j], C[j], P[j])
    print(f"LNQ from the uniform grid: gpu {gpu:.6e} oracle {ref:.6e} start {start:.6e}")
    assert abs(tr[0] - start) <= 1e-4 * start
    assert abs(gpu - ref) <= 1e-3 * ref
