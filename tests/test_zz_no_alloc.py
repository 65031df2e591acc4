"""lnq_quantize_static (the entry point that allocates nothing) against lnq_quantize.

Two calls in a row on the same device (the second on a smaller layer, so it runs on
scratch the first call left full of its own values): each result is bitwise that of
lnq_quantize with a caller workspace on the same inputs (the same kernels run in the
same order on equal data), and so within every parity bar lnq_quantize meets.  The
trace and move counts match as well.
"""
import numpy as np
import pytest
import torch

import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _util import symmetric_f32, to_dev

pytestmark = pytest.mark.gpu


def _layer(device, d_in, d_out, groups, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((3 * d_in, d_in)).astype(np.float32)
    F = np.stack([(X * rng.uniform(0.5, 2.0, (3 * d_in, 1)).astype(np.float32)).T @ X
                  for _ in range(groups)])
    W = synth.f32_to_bf16_bits((rng.standard_normal((d_out, d_in)) * 0.02).astype(np.float32))
    return to_dev(symmetric_f32(F), device), to_dev(W, device)


@pytest.mark.parametrize("bits", [3, 4])
def test_static_scratch_matches_workspace_entry_point(device, bits):
    shapes = [(1024, 768, 2), (512, 256, 2)]     # second call smaller than the first
    assert gq.lnq_workspace_size(768, 1024, 2, bits) <= gq.lnq_static_scratch_bytes()
    for k, (d_in, d_out, groups) in enumerate(shapes):
        F, W = _layer(device, d_in, d_out, groups, seed=10 * bits + k)
        ref = gq.lnq_quantize(W, F, bits, 4)
        got = gq.lnq_quantize_static(W, F, bits, 4)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), (d_in, d_out, bits)
        tr = got[2].cpu().numpy()
        assert np.all(tr[1:] <= tr[:-1] * (1 + 1e-6)), tr
