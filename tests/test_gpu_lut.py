"""GPU parity of the lookup-table product (lut_pack_codes, lut_gemv) against the oracle.

Bars:
  * packed words bitwise equal to the oracle's packing (integer work);
  * y[b][j] within (d_in / 16 + 32) 2^-24 sum_i |v_ji x_bi| of the oracle's float64
    product, v the codebook entry as the path holds it (bfloat16-rounded for
    bfloat16 activations, float32 otherwise).  Each lane adds about d_in / 128 dot
    products (two roundings at most each), then a 64-lane tree adds 6 more; the
    bound allows twice that many float32 roundings of the absolute sum;
  * sizes: ragged and small shapes of every bit width and batch, LNQ's own output
    on the mid-size layer, and all four Llama-shaped layers at full size (every
    row of the product checked: the oracle's product is one float64 matmul).
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_gq_amd as gq
from post_weight_quantization_gq_amd import synth

from _util import to_dev

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _check(y_gpu, C, P, x_vals, lut_bf16, d_in):
    y_ref = O.lut_gemv(C, P, x_vals, lut_bf16)
    Cv = O.bf16_round(C) if lut_bf16 else np.asarray(C, np.float64)
    absW = np.abs(np.take_along_axis(Cv, np.asarray(P, np.int64), axis=1))
    bound = (np.abs(x_vals) @ absW.T) * (d_in / 16 + 32) * 2.0 ** -24
    err = np.abs(y_gpu - y_ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    print(f"max |y - y_ref| {err.max():.3e}, worst error / bound {worst:.3f}")
    assert np.all(err <= bound)


def _run(device, d_out, d_in, bits, batch, x_dtype, seed=0, C=None, P=None):
    rng = np.random.default_rng(seed)
    m = 1 << bits
    if P is None:
        P = rng.integers(0, m, size=(d_out, d_in), dtype=np.uint8)
    if C is None:
        C = np.sort(rng.standard_normal((d_out, m)).astype(np.float32) * np.float32(0.02), axis=1)
    Q = gq.lut_pack_codes(to_dev(P, device), bits)
    if x_dtype == "bf16":
        xb = _bf16(rng, (batch, d_in))
        x_vals = synth.bf16_bits_to_f32(xb).astype(np.float64)
        x = to_dev(xb, device)
    else:
        xf = rng.standard_normal((batch, d_in)).astype(np.float32)
        x_vals = xf.astype(np.float64)
        x = to_dev(xf, device)
    y = gq.lut_gemv(Q, to_dev(C, device), x, bits)
    torch.cuda.synchronize()
    return Q.cpu().numpy().view(np.uint32), y.cpu().numpy().astype(np.float64), C, P, x_vals


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d_out,d_in", [(5, 1), (37, 333), (64, 4096), (200, 576)])
def test_lut_pack_matches_oracle(device, bits, d_out, d_in):
    rng = np.random.default_rng(bits * 1000 + d_in)
    P = rng.integers(0, 1 << bits, size=(d_out, d_in), dtype=np.uint8)
    Q = gq.lut_pack_codes(to_dev(P, device), bits)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Q.cpu().numpy().view(np.uint32), O.lut_pack(P, bits))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("batch", [1, 3, 8])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_lut_gemv_matches_oracle(device, bits, batch, x_dtype):
    for d_out, d_in in ((37, 333), (200, 576), (64, 1)):
        Q, y, C, P, xv = _run(device, d_out, d_in, bits, batch, x_dtype, seed=bits + 10 * batch)
        _check(y, C, P, xv, x_dtype == "bf16", d_in)


def test_lut_gemv_extreme_codebook_values(device):
    """Codebook entries that round to bfloat16 ties and large magnitudes."""
    rng = np.random.default_rng(3)
    d_out, d_in, bits = 16, 640, 2
    C = np.tile(np.array([1.0 + 2 ** -8, -(1.0 + 3 * 2 ** -8), 3.0e4, -2.0e-30],
                         dtype=np.float32), (d_out, 1))
    Q, y, C, P, xv = _run(device, d_out, d_in, bits, 2, "bf16", C=C)
    _check(y, C, P, xv, True, d_in)


def test_lut_gemv_on_lnq_output(device):
    """LNQ's own (C, P) on the mid-size layer, packed and multiplied."""
    from test_gpu_lnq import MID, Problem
    prob = Problem(device, MID, seed=1)
    C, P, _, _ = gq.lnq_quantize(prob.W, prob.F, 3, 3)
    torch.cuda.synchronize()
    _, y, C_np, P_np, xv = _run(device, MID.d_out, MID.d_in, 3, 4, "bf16", seed=5,
                                C=C.cpu().numpy(), P=P.cpu().numpy())
    _check(y, C_np, P_np, xv, True, MID.d_in)


@pytest.mark.parametrize("name,batch", [("llama2_7b_attn", 8), ("llama2_7b_down", 4),
                                        ("llama3_8b_down", 2), ("llama2_70b_down", 2)])
def test_lut_gemv_full_size(device, name, batch):
    """Every row of the product at the four layers' real shapes and bit widths."""
    wl = synth.workload(name)
    Q, y, C, P, xv = _run(device, wl.d_out, wl.d_in, wl.bits, batch, "bf16", seed=7)
    np.testing.assert_array_equal(Q[:3], O.lut_pack(P[:3], wl.bits))
    _check(y, C, P, xv, True, wl.d_in)


@pytest.mark.parametrize("d_out,d_in,bits,batch", [
    (37, 40000, 3, 8),       # 8 segments of 512 words, the last ragged (416)
    (37, 40001, 3, 3),       # odd d_in: the pair-by-pair staging
    (64, 20000, 2, 8),       # 2-bit: 3 segments, 8 pairs per word
    (40, 28672, 1, 4),       # 1-bit: 32 codes per word
])
def test_lut_gemv_segmented_staging(device, d_out, d_in, bits, batch):
    """Rows too wide for one block's LDS at this batch: x staged in segments of whole
    chunks, each output the sum of its segments' sums."""
    Q, y, C, P, xv = _run(device, d_out, d_in, bits, batch, "bf16", seed=d_in + batch)
    _check(y, C, P, xv, True, d_in)


@pytest.mark.parametrize("batch", [4, 8])
def test_lut_gemv_full_size_segmented(device, batch):
    """Every row of the 28672 -> 8192 4-bit product with 4 and 8 vectors (segments)."""
    wl = synth.workload("llama2_70b_down")
    Q, y, C, P, xv = _run(device, wl.d_out, wl.d_in, wl.bits, batch, "bf16", seed=9)
    _check(y, C, P, xv, True, wl.d_in)


def test_lut_gemv_rejects_oversized_staging(device):
    """1-bit codes with 8 bfloat16 vectors: one 512-word chunk of staged activations
    (513 x 16 pairs x 8 vectors x 4 bytes) exceeds the LDS: an error, before any launch."""
    d_out, d_in, bits = 64, 28672, 1
    Q = torch.zeros((d_out, gq.lut_packed_row_words(d_in, bits)), dtype=torch.int32,
                    device=device)
    C = torch.zeros((d_out, 2), dtype=torch.float32, device=device)
    x = torch.zeros((8, d_in), dtype=torch.bfloat16, device=device)
    with pytest.raises(gq.GQError) as e:
        gq.lut_gemv(Q, C, x, bits)
    assert e.value.status == 8
