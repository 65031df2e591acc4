"""GPU parity of the grouped Fisher (gq_fisher_accumulate) against the fp64 oracle.

Bar: per group, ||F_gpu - F_ref||_F / ||F_ref||_F <= 2e-3 for bfloat16 inputs
(bfloat16 operands, float32 accumulation); float32 inputs take the
float64-accumulating path and must agree to float32 rounding (1e-6).
The result must be exactly symmetric.
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
    ref = O.fisher(synth.decode(inp["X"]), synth.decode(inp["G"]), groups)
    _check_symmetric(F)
    F64 = f64(F)
    for g in range(groups):
        err = rel_fro(F64[g], ref[g])
        print(f"group {g}: rel Frobenius error {err:.3e}")
        assert err <= BF16_TOL


def test_fisher_accumulate_streams_tokens(device):
    wl = _custom("acc", 264, 32, 4000, 2, outliers=2, oscale=20.0, index=23)
    inp = synth.make_inputs(wl, seed=5)
    X, G = to_dev(inp["X"], device), to_dev(inp["G"], device)
    F = gq.gq_fisher_accumulate(X[:1500].contiguous(), G[:1500].contiguous(), 2)
    gq.gq_fisher_accumulate(X[1500:].contiguous(), G[1500:].contiguous(), 2, F=F,
                            accumulate=True)
    torch.cuda.synchronize()
    ref = O.fisher(synth.decode(inp["X"]), synth.decode(inp["G"]), 2)
    _check_symmetric(F)
    for g in range(2):
        assert rel_fro(f64(F[g]), ref[g]) <= BF16_TOL


def test_fisher_deterministic(device):
    wl = _custom("det", 520, 64, 9000, 4, x_kind="gated", index=24)
    inp = synth.make_inputs(wl, seed=6)
    F1 = _run(device, inp, 4)
    F2 = _run(device, inp, 4)
    assert torch.equal(F1, F2)
