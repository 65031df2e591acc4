"""GPU parity of the host-streamed Fisher (gq_fisher_accumulate_host).

F is a sum over tokens (GuidedQuant blog page, objective equation: F_j built from
every calibration token), so chunks of tokens streamed from host memory and added
into F give the Fisher of all tokens.  Bars:
  * against the oracle's fp64 Fisher of the same tokens: relative Frobenius error
    <= 2e-3 per group for bfloat16 inputs (the Fisher's own bar), <= 1e-6 for
    float32 inputs;
  * against one gq_fisher_accumulate call on the same data in device memory:
    relative Frobenius <= 1e-5 (the same products; only the float32 summation of
    the chunks' partials differs), exactly symmetric;
  * chunk sizes that divide n, leave a ragged last chunk, exceed n, and a few
    tokens each (hundreds of chunks); pinned and pageable host memory;
    accumulate = 1 adds to F.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _util import rel_fro, to_dev

pytestmark = pytest.mark.gpu


def _host(arr, pinned):
    arr = np.ascontiguousarray(arr)
    t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if arr.dtype == np.uint16 \
        else torch.from_numpy(arr)
    return t.pin_memory() if pinned else t.clone()


def _inputs(n, d_in, d_out, seed, dtype="bf16"):
    wl = synth.Workload("stream", d_in, d_out, n, 2, 3, 1, 128, dtype, "gated",
                        max(1, d_in // 128), 30.0, "t4", 0.02, 1e-3, 40)
    inp = synth.make_inputs(wl, seed=seed, want=("X", "G"))
    return inp["X"], inp["G"]


@pytest.fixture(scope="module")
def data():
    X, G = _inputs(3000, 256, 64, seed=3)
    ref = O.fisher(synth.decode(X), synth.decode(G), 2)
    return X, G, ref


@pytest.mark.parametrize("chunk", [1000, 1024, 3000, 5000, 7])
def test_stream_matches_oracle_and_device_call(device, data, chunk):
    X, G, ref = data
    F = gq.gq_fisher_accumulate_host(_host(X, True), _host(G, True), 2, chunk_tokens=chunk,
                                     device=device)
    Fd = gq.gq_fisher_accumulate(to_dev(X, device), to_dev(G, device), 2)
    torch.cuda.synchronize()
    assert torch.equal(F, F.transpose(1, 2))
    Fn, Fdn = F.cpu().double().numpy(), Fd.cpu().double().numpy()
    for g in range(2):
        e_ref = rel_fro(Fn[g], ref[g])
        e_dev = rel_fro(Fn[g], Fdn[g])
        print(f"chunk {chunk} group {g}: vs oracle {e_ref:.2e}, vs device call {e_dev:.2e}")
        assert e_ref <= 2e-3
        assert e_dev <= 1e-5


def test_stream_pageable_memory_and_accumulate(device, data):
    X, G, ref = data
    F = gq.gq_fisher_accumulate_host(_host(X, False), _host(G, False), 2, chunk_tokens=900,
                                     device=device)
    F2 = gq.gq_fisher_accumulate_host(_host(X, True), _host(G, True), 2, F=F.clone(),
                                      accumulate=True, chunk_tokens=1100)
    torch.cuda.synchronize()
    Fn, F2n = F.cpu().double().numpy(), F2.cpu().double().numpy()
    for g in range(2):
        assert rel_fro(Fn[g], ref[g]) <= 2e-3
        assert rel_fro(F2n[g], 2 * Fn[g]) <= 1e-6


def test_stream_float32_inputs(device):
    X, G = _inputs(700, 128, 32, seed=4, dtype="f32")
    ref = O.fisher(X.astype(np.float64), G.astype(np.float64), 2)
    F = gq.gq_fisher_accumulate_host(_host(X, True), _host(G, True), 2, chunk_tokens=250,
                                     device=device)
    torch.cuda.synchronize()
    Fn = F.cpu().double().numpy()
    for g in range(2):
        assert rel_fro(Fn[g], ref[g]) <= 1e-6


def test_stream_reused_workspace_back_to_back(device, data):
    """Two calls on one stream sharing one workspace: the second call's copies wait for
    the first call's Fisher (which still reads the workspace) before overwriting it."""
    X, G, ref = data
    ws = torch.empty(gq.fisher_stream_workspace_size(512, 256, 64, 2), dtype=torch.uint8,
                     device=device)
    Xh, Gh = _host(X, True), _host(G, True)
    Xz = torch.zeros_like(Xh).pin_memory()
    Fa = gq.gq_fisher_accumulate_host(Xh, Gh, 2, chunk_tokens=512, ws=ws, device=device)
    Fb = gq.gq_fisher_accumulate_host(Xz, Gh, 2, chunk_tokens=512, ws=ws, device=device)
    torch.cuda.synchronize()
    Fan = Fa.cpu().double().numpy()
    for g in range(2):
        assert rel_fro(Fan[g], ref[g]) <= 2e-3
    assert torch.count_nonzero(Fb).item() == 0
