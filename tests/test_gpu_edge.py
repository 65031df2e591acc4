"""Edge cases of the GPU path against the fp64 oracle.

  * Fisher over more tokens than one packing pass holds: the library stages at
    most 16 GiB of packed bfloat16 operands ([tokens][d_in] activations plus
    one gradient-scaled copy per group) per pass, so 4096 columns and 64 groups
    take 32256 tokens per pass; 40003 tokens make two passes, the second one
    ragged.  Sampled entries against the oracle's fp64 sum over every token,
    |F_gpu - F_ref| <= 2e-3 sqrt(F_ref[a,a] F_ref[b,b]).
  * A group whose output gradients are all zero: its Fisher is exactly zero
    (both input dtypes), the other groups keep their parity bar.
  * LNQ with such a group (F' = 0, lambda = 0): every objective is zero, the
    codebook system is singular, so each row of the group keeps its codebook
    and is counted as not positive definite, and no coordinate moves; the rows
    of that group come back bit-identical to their quantile initialisation, as
    in the oracle.  The other group matches the oracle end to end (1e-3).
  * Degenerate weight rows: all-zero rows, constant rows, rows with two or
    three distinct values (fewer than the 2^bits codebook entries).  Initial
    codebooks and codes identical to the oracle's; zero and constant rows stay
    exact (objective 0, codebook unchanged); the final objective of the other
    classes within 1e-3 relative of the oracle's own run, or 1e-9 of the
    objective of quantising every weight to zero where the oracle reaches 0.
  * The widest layer the LNQ entry points take, d_in = 32768 (one group's bf16
    plane of F' is 2 GiB): initial codebooks and codes identical to the
    oracle's on every row, the GPU trace monotone, and one sampled row per group
    within 1e-3 of the oracle's own run (one LNQ iteration).  F is torch's
    float32 product of the seeded activations, made exactly symmetric, so no
    oracle input comes from the library.
"""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _progress import say as _say
from _util import f64, rel_fro, symmetric_f32, to_dev

pytestmark = pytest.mark.gpu

RHO = 1e-6
BF16_TOL = 2e-3


def _progress(msg):
    _say(f"[edge] {msg}")


def _wl(name, d_in, d_out, n, groups, bits=3, dtype="bf16", x_kind="gated", outliers=4,
        index=40):
    return synth.Workload(name, d_in, d_out, n, groups, bits, 4, 64, dtype, x_kind, outliers,
                          30.0, "t4", 0.02, 1e-3, index)


@pytest.mark.timeout(600)
def test_fisher_multi_pass_sampled(device):
    """A call beyond one pass's token limit (2^20 tokens) runs as two passes, the
    second a ragged 4003 tokens, each adding into F; d_in 520 is three tiles, the last
    ragged.  Sampled entries against the oracle's, each to the entry bar."""
    wl = _wl("multipass", 520, 64, (1 << 20) + 4003, 4, index=41)
    inp = synth.make_inputs(wl, seed=0)
    _progress(f"multi-pass Fisher: n={wl.n} d_in={wl.d_in} groups={wl.groups}")
    X, G = to_dev(inp["X"], device), to_dev(inp["G"], device)
    F = gq.gq_fisher_accumulate(X, G, wl.groups)
    torch.cuda.synchronize()
    del X, G
    assert torch.isfinite(F).all()
    S = O.group_scale(synth.decode(inp["G"]), wl.groups)
    rng = np.random.default_rng(3)
    cols = set(int(c) for c in rng.choice(wl.d_in, 16, replace=False))
    cols |= set(int(c) for c in inp["outlier_cols"][:2]) | {0, 255, 256, 511, 512, wl.d_in - 1}
    cols = sorted(cols)
    xc = {c: synth.decode(inp["X"][:, c]) for c in cols}
    idx = torch.tensor(cols, device=device)
    num = den = 0.0
    for g in range(wl.groups):
        sub = F[g].index_select(0, idx).index_select(1, idx).cpu().double().numpy()
        np.testing.assert_array_equal(sub, sub.T)
        diag = {c: O.fisher_entry(xc[c], xc[c], S[g]) for c in cols}
        for ia, a in enumerate(cols):
            for ib in range(ia, len(cols)):
                b = cols[ib]
                ref = diag[a] if a == b else O.fisher_entry(xc[a], xc[b], S[g])
                got = sub[ia, ib]
                assert abs(got - ref) <= BF16_TOL * np.sqrt(diag[a] * diag[b]), (g, a, b, got,
                                                                                  ref)
                num += (got - ref) ** 2
                den += ref ** 2
    rel = np.sqrt(num / den)
    _progress(f"multi-pass Fisher: sampled rel error {rel:.2e}")
    assert rel <= BF16_TOL
    del F
    torch.cuda.empty_cache()


def _zero_group_inputs(wl, zero_group, seed=0):
    inp = synth.make_inputs(wl, seed=seed)
    G = inp["G"].copy()
    rpg = wl.d_out // wl.groups
    G[:, zero_group * rpg:(zero_group + 1) * rpg] = 0
    inp["G"] = G
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fisher_zero_gradient_group(device, dtype):
    wl = _wl("zerog", 256, 64, 1000, 4, dtype=dtype, index=42)
    inp = _zero_group_inputs(wl, 2)
    F = gq.gq_fisher_accumulate(to_dev(inp["X"], device), to_dev(inp["G"], device), 4)
    torch.cuda.synchronize()
    ref = O.fisher(synth.decode(inp["X"]), synth.decode(inp["G"]), 4)
    assert np.all(ref[2] == 0.0)
    got = f64(F)
    assert np.all(got[2] == 0.0)
    tol = BF16_TOL if dtype == "bf16" else 1e-6
    for g in (0, 1, 3):
        assert rel_fro(got[g], ref[g]) <= tol


def _oracle_F(inp, groups):
    return symmetric_f32(O.fisher(synth.decode(inp["X"]), synth.decode(inp["G"]), groups))


def test_lnq_zero_fisher_group(device):
    wl = _wl("zerof", 512, 128, 1500, 2, bits=3, index=43)
    inp = _zero_group_inputs(wl, 1)
    F32 = _oracle_F(inp, 2)
    assert np.all(F32[1] == 0.0)
    F, W = to_dev(F32, device), to_dev(inp["W"], device)
    w = synth.decode(inp["W"])
    m, rpg, iters = wl.m, wl.d_out // 2, 3
    Fp = [O.damped(F32[g].astype(np.float64), RHO) for g in range(2)]
    assert np.all(Fp[1] == 0.0)

    C0, P0, _, _ = gq.lnq_quantize(W, F, wl.bits, 0)
    npd = torch.zeros(1, dtype=torch.int64, device=device)
    C1 = C0.clone()
    gq.lnq_codebook_update(F, W, P0, C1, wl.bits, RHO, n_not_pd=npd)
    torch.cuda.synchronize()
    assert npd.item() == rpg
    assert torch.equal(C1[rpg:], C0[rpg:])

    C, P, tr, _ = gq.lnq_quantize(W, F, wl.bits, iters, ridge_rel=RHO)
    torch.cuda.synchronize()
    assert torch.equal(C[rpg:], C0[rpg:]) and torch.equal(P[rpg:], P0[rpg:])
    C, P, tr = f64(C), P.cpu().numpy(), tr.cpu().numpy()
    assert np.all(tr[1:] <= tr[:-1] * (1 + 1e-6)), tr
    gpu = ref = 0.0
    for j in range(wl.d_out):
        c_ref, p_ref, t_ref = O.lnq_row(Fp[j // rpg], w[j], m, iters)
        if j >= rpg:
            np.testing.assert_array_equal(C[j], c_ref)
            np.testing.assert_array_equal(P[j], p_ref)
            assert t_ref[-1] == 0.0
            continue
        gpu += O.objective(Fp[0], w[j], C[j], P[j])
        ref += t_ref[-1]
    _progress(f"zero-Fisher group: other group gpu {gpu:.6e} oracle {ref:.6e}")
    assert abs(gpu - ref) <= 1e-3 * ref
    assert abs(tr[-1] - gpu) <= 1e-4 * gpu


def _degenerate_W(wl, seed):
    """Seeded W whose first 32 rows are degenerate: 8 all-zero, 8 constant, 8 with
    two distinct values, 8 with three."""
    inp = synth.make_inputs(wl, seed=seed)
    W = synth.decode(inp["W"]).astype(np.float32)
    rng = np.random.default_rng(seed + 500)
    d = wl.d_in
    W[0:8] = 0.0
    W[8:16] = rng.standard_normal((8, 1)).astype(np.float32) * np.float32(0.02)
    for j in range(16, 24):
        v = rng.standard_normal(2).astype(np.float32) * np.float32(0.02)
        W[j] = np.where(rng.random(d) < 0.3, v[0], v[1])
    for j in range(24, 32):
        v = rng.standard_normal(3).astype(np.float32) * np.float32(0.02)
        W[j] = v[rng.integers(0, 3, d)]
    inp["W"] = synth.f32_to_bf16_bits(W)
    return inp


@pytest.mark.parametrize("bits", [1, 3, 4])
def test_lnq_degenerate_rows(device, bits):
    wl = _wl("degen", 512, 64, 1500, 2, bits=bits, index=44)
    inp = _degenerate_W(wl, seed=bits)
    F32 = _oracle_F(inp, 2)
    F, W = to_dev(F32, device), to_dev(inp["W"], device)
    w = synth.decode(inp["W"])
    m, rpg, iters = wl.m, wl.d_out // 2, 3
    Fp = [O.damped(F32[g].astype(np.float64), RHO) for g in range(2)]

    C0, P0, _, _ = gq.lnq_quantize(W, F, bits, 0)
    C, P, tr, _ = gq.lnq_quantize(W, F, bits, iters, ridge_rel=RHO)
    torch.cuda.synchronize()
    C0, P0 = f64(C0), P0.cpu().numpy()
    C, P, tr = f64(C), P.cpu().numpy(), tr.cpu().numpy()
    assert np.all(tr[1:] <= tr[:-1] * (1 + 1e-6)), tr
    for j in range(wl.d_out):
        c_init, p_init = O.init_quantile(w[j], m)
        np.testing.assert_array_equal(C0[j], c_init)
        np.testing.assert_array_equal(P0[j], p_init)
    for j in range(16):                        # zero and constant rows stay exact
        Fj = Fp[j // rpg]
        np.testing.assert_array_equal(C[j], C0[j])
        np.testing.assert_array_equal(P[j], np.zeros(wl.d_in, np.uint8))
        assert O.objective(Fj, w[j], C[j], P[j]) == 0.0
    for lo, hi in ((16, 24), (24, 32), (32, 64)):
        gpu = ref = scale = 0.0
        for j in range(lo, hi):
            Fj = Fp[j // rpg]
            _, _, t_ref = O.lnq_row(Fj, w[j], m, iters)
            gpu += O.objective(Fj, w[j], C[j], P[j])
            ref += t_ref[-1]
            scale += w[j] @ Fj @ w[j]
        _progress(f"degenerate rows {lo}-{hi} bits={bits}: gpu {gpu:.6e} oracle {ref:.6e}")
        assert abs(gpu - ref) <= 1e-3 * ref + 1e-9 * scale


@pytest.mark.timeout(900)
def test_lnq_max_width(device):
    wl = _wl("maxwidth", 32768, 32, 4096, 2, bits=3, index=45)
    inp = synth.make_inputs(wl, seed=0)
    _progress(f"max width: d_in={wl.d_in} d_out={wl.d_out} groups={wl.groups}")
    S = O.group_scale(synth.decode(inp["G"]), wl.groups).astype(np.float32)
    X = to_dev(inp["X"], device).float()
    XT = X.t().contiguous()
    F = torch.empty((wl.groups, wl.d_in, wl.d_in), dtype=torch.float32, device=device)
    for g in range(wl.groups):
        Fg = torch.mm(XT, X * torch.from_numpy(S[g]).to(device)[:, None])
        F[g] = (Fg + Fg.t()) * 0.5
        del Fg
    del X, XT
    W = to_dev(inp["W"], device)
    w = synth.decode(inp["W"])
    m, rpg, iters = wl.m, wl.d_out // wl.groups, 1
    C0, P0, _, _ = gq.lnq_quantize(W, F, wl.bits, 0)
    C, P, tr, _ = gq.lnq_quantize(W, F, wl.bits, iters, ridge_rel=RHO)
    torch.cuda.synchronize()
    _progress("max width: GPU LNQ done")
    C0, P0 = f64(C0), P0.cpu().numpy()
    C, P, tr = f64(C), P.cpu().numpy(), tr.cpu().numpy()
    assert np.all(tr[1:] <= tr[:-1] * (1 + 1e-6)), tr
    for j in range(wl.d_out):
        c_init, p_init = O.init_quantile(w[j], m)
        np.testing.assert_array_equal(C0[j], c_init)
        np.testing.assert_array_equal(P0[j], p_init)
    rng = np.random.default_rng(7)
    for g in range(wl.groups):
        Fp = O.damped(F[g].cpu().double().numpy(), RHO)
        j = g * rpg + int(rng.integers(rpg))
        _, _, t_ref = O.lnq_row(Fp, w[j], m, iters)
        gpu = O.objective(Fp, w[j], C[j], P[j])
        _progress(f"max width: row {j} gpu {gpu:.6e} oracle {t_ref[-1]:.6e}")
        assert abs(gpu - t_ref[-1]) <= 1e-3 * t_ref[-1]
        del Fp
    del F
    torch.cuda.empty_cache()
