"""The measurement definitions in bench.py (CPU only).

bench.py reports each stage's roofline from an algorithmic amount of work per step and
a copy-calibrated traffic figure tied to the kernel's source.  These tests pin the
parts a slip could silently change:
  * the codebook Gram's flops: the kernel covers, for every coordinate a, the
    coordinates k from the start of a's 256-wide tile to the end; the count here is
    taken pair by pair over the coordinates, not by the tile formula bench.py uses;
  * the traffic figure is reported only while the kernel's source digest matches the
    one it was measured with, and is the sum of the bytes read and written;
  * the layer composite is the sum of its terms, divided by the measured time.
"""
import dataclasses
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from post_weight_quantization_gq_amd import synth  # noqa: E402


def _covered_pairs(d):
    """(a, k) pairs of the upper-triangle tiles: k >= the first coordinate of a's tile."""
    return sum(d - 256 * (a // 256) for a in range(d))


@pytest.mark.parametrize("d", [128, 256, 544, 4096, 11008])
def test_gram_flops_count_the_covered_pairs(d):
    wl = dataclasses.replace(synth.WORKLOADS["llama2_7b_attn"], d_in=d)
    nchg = np.full(wl.iters, wl.d_out * d, np.int64)   # every code changed: all steps recomputed
    bound, amount, peak, unit, launches = bench._stage_units("lnq_gram", wl, nchg)
    assert (bound, unit) == ("mfma", "TFLOP/s")
    assert launches == wl.iters
    # two bf16 products (F' hi and lo), 2 flops per multiply-add, every (j, q) column
    assert amount == wl.iters * 2 * 2 * _covered_pairs(d) * wl.d_out * wl.m


def test_gram_launches_skip_the_updated_steps():
    wl = synth.WORKLOADS["llama2_7b_attn"]
    lim = wl.d_out * wl.d_in * (wl.m + 3) * 17 // 10000
    # pass t - 1 precedes step t; the last four passes changed at most the limit
    nchg = np.array([lim * 10] * (wl.iters - 4) + [lim, lim // 2, 1, 0], np.int64)
    incr = bench._incremental_iters(wl, nchg)
    assert incr == [t for t in range(2, wl.iters + 1) if nchg[t - 2] <= lim]
    _, _, _, _, launches = bench._stage_units("lnq_gram", wl, nchg)
    assert launches == wl.iters - len(incr)


def test_traffic_follows_the_source_digest(monkeypatch):
    wl = synth.WORKLOADS["llama2_7b_attn"]
    good = bench._source_digest("gq_lnq.hip")
    monkeypatch.setitem(bench._TRAFFIC, "lnq_sweep", (wl.name, "gq_lnq.hip", good, 700, 300))
    assert bench._traffic("lnq_sweep", wl) == 1000
    monkeypatch.setitem(bench._TRAFFIC, "lnq_sweep", (wl.name, "gq_lnq.hip", "0" * 16, 700, 300))
    assert bench._traffic("lnq_sweep", wl) is None
    # another workload's figure is not this one's
    monkeypatch.setitem(bench._TRAFFIC, "lnq_sweep", ("tiny", "gq_lnq.hip", good, 700, 300))
    assert bench._traffic("lnq_sweep", wl) is None
    assert bench._traffic("no_such_stage", wl) is None


def test_source_digest_covers_the_shared_headers(tmp_path, monkeypatch):
    """A kernel's digest changes when either shared header changes."""
    for f in ("gq_lnq.hip", "gq_common.h", "gq_internal.h"):
        (tmp_path / f).write_bytes(open(os.path.join(bench._CSRC, f), "rb").read())
    monkeypatch.setattr(bench, "_CSRC", str(tmp_path))
    base = bench._source_digest("gq_lnq.hip")
    for f in ("gq_common.h", "gq_internal.h", "gq_lnq.hip"):
        p = tmp_path / f
        orig = p.read_bytes()
        p.write_bytes(orig + b"\n")
        assert bench._source_digest("gq_lnq.hip") != base, f
        p.write_bytes(orig)
    assert bench._source_digest("gq_lnq.hip") == base


def test_layer_composite_is_the_sum_of_its_terms():
    wl = synth.WORKLOADS["llama2_7b_attn"]
    nchg = np.full(wl.iters, 1000, np.int64)
    r = bench._layer_roofline(wl, nchg, 30.0)
    terms = r["terms_ms"]
    assert r["t_roof_ms"] == pytest.approx(sum(terms.values()), rel=1e-12)
    assert r["frac"] == pytest.approx(r["t_roof_ms"] / 30.0, rel=1e-12)
    # the Fisher term: unique entries of every group's symmetric F at the bf16 peak
    n, d, G = wl.n, wl.d_in, wl.groups
    assert terms["fisher"] == pytest.approx(n * d * (d + 1) * G / bench.PEAK_BF16_MFMA * 1e3,
                                            rel=1e-12)
