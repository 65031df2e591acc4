"""Seeded synthetic inputs for the GuidedQuant + LNQ hot path.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic: no Fisher, no codebook, no sweep.
The same bytes feed the fp64 CPU oracle (decoded exactly) and the GPU library.

Workload shapes stand in for the layers the GuidedQuant page (jinukkim.me,
"GuidedQuant" section) and the GANQ summary (atlas.scime.ai, "Experimental
setup") evaluate on: Llama-2-7B attention/MLP projections, a Llama-3-8B MLP
down projection and a Llama-2-70B MLP down projection.  No dataset or trained
weight is used; activations, weights and output gradients are drawn from the
distributions listed per workload.

Draw recipe (fixed order, one counter-based stream per tensor and chunk):
  * stream key (seed, workload index, tensor id, chunk index) via
    numpy SeedSequence, bit generator PCG64;
  * X: N(0,1) rows, or SiLU(a)*b with a,b ~ N(0,1) (gated MLP activations);
    then k outlier columns (chosen without replacement from their own stream)
    are multiplied by a factor;
  * W: N(0, std^2) or Student-t(4) rescaled to standard deviation std;
  * G (end-loss output gradients): Laplace(0, b); optionally every token row
    multiplied by exp(sigma z_t), z_t ~ N(0, 1) from its own stream (a strongly
    token-dependent gradient scale, so the per-token weights of the Fisher vary
    over orders of magnitude instead of a few percent);
  * every value is drawn in float32 (Laplace in float64, then cast) and
    rounded to bfloat16 with round-to-nearest-even where the workload stores
    bfloat16.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_inputs", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "decode",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d_in: int
    d_out: int
    n: int
    groups: int
    bits: int
    iters: int
    block: int
    dtype: str            # storage dtype of X, W, G: "f32" or "bf16"
    x_kind: str           # "normal" or "gated"
    outlier_cols: int
    outlier_scale: float
    w_kind: str           # "normal" or "t4"
    w_std: float
    g_scale: float        # Laplace scale b of the output gradients
    index: int            # position in WORKLOADS (part of the stream key)
    g_row_sigma: float = 0.0   # sigma of the log-normal per-token factor of G (0: none)

    @property
    def m(self) -> int:
        return 1 << self.bits


def _outliers(frac: float, d_in: int) -> int:
    return int(round(frac * d_in))


WORKLOADS = {
    # Tiny single linear layer, float32 throughout.
    "tiny": Workload("tiny", 128, 64, 256, 1, 3, 5, 128, "f32", "normal", 4, 20.0,
                     "normal", 0.02, 1e-3, 0),
    # Llama-2-7B attention projection 4096 -> 4096, 131072 calibration tokens.
    "llama2_7b_attn": Workload("llama2_7b_attn", 4096, 4096, 131072, 4, 3, 10, 128, "bf16",
                               "normal", _outliers(0.005, 4096), 30.0, "normal", 0.02,
                               1e-4, 1),
    # Llama-2-7B MLP down projection 11008 -> 4096.
    "llama2_7b_down": Workload("llama2_7b_down", 11008, 4096, 65536, 4, 2, 10, 128, "bf16",
                               "gated", 0, 1.0, "normal", 0.015, 1e-4, 2),
    # Llama-3-8B MLP down projection 14336 -> 4096.
    "llama3_8b_down": Workload("llama3_8b_down", 14336, 4096, 65536, 4, 3, 10, 128, "bf16",
                               "gated", _outliers(0.002, 14336), 50.0, "t4", 0.02, 1e-4, 3),
    # Llama-2-70B MLP down projection 28672 -> 8192.
    "llama2_70b_down": Workload("llama2_70b_down", 28672, 8192, 32768, 4, 4, 8, 256, "bf16",
                                "gated", _outliers(0.001, 28672), 50.0, "t4", 0.01, 5e-5, 4),
}

_TENSOR_X, _TENSOR_XA, _TENSOR_XB, _TENSOR_OUT, _TENSOR_W, _TENSOR_G, _TENSOR_GROW = range(7)
_CHUNK_ROWS = 4096


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def decode(arr: np.ndarray) -> np.ndarray:
    """Exact float64 values of a stored input (uint16 = bfloat16 bits, else float)."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _gen(seed: int, wl_index: int, tensor: int, chunk: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(wl_index, tensor, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_rows(n_rows: int, n_cols: int, fill, dtype: str, out_dtype) -> np.ndarray:
    out = np.empty((n_rows, n_cols), dtype=out_dtype)
    chunks = [(c, c * _CHUNK_ROWS, min(n_rows, (c + 1) * _CHUNK_ROWS))
              for c in range((n_rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS)]

    def work(ch):
        c, lo, hi = ch
        out[lo:hi] = _store(fill(c, hi - lo), dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, chunks))
    return out


def make_inputs(wl: Workload | str, seed: int = 0, rows: int | None = None,
                tokens: int | None = None, want=("X", "W", "G")) -> dict:
    """Draw the workload's X [n][d_in], W [d_out][d_in], G [n][d_out].

    bfloat16 tensors come back as uint16 bit patterns, float32 ones as float32.
    `tokens` keeps the first `tokens` rows of X and G (a prefix of the same
    draws); `rows` keeps the first `rows` rows of W.  Prefixes are byte-identical
    to the corresponding part of the full draw.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    n = wl.n if tokens is None else min(tokens, wl.n)
    d_out_rows = wl.d_out if rows is None else min(rows, wl.d_out)
    out_dtype = np.uint16 if wl.dtype == "bf16" else np.float32
    res = {"workload": wl}

    if "X" in want:
        cols = None
        if wl.outlier_cols > 0:
            g = _gen(seed, wl.index, _TENSOR_OUT, 0)
            cols = np.sort(g.choice(wl.d_in, size=wl.outlier_cols, replace=False))

        def fill_x(c, k):
            if wl.x_kind == "normal":
                x = _gen(seed, wl.index, _TENSOR_X, c).standard_normal((k, wl.d_in), dtype=np.float32)
            else:
                a = _gen(seed, wl.index, _TENSOR_XA, c).standard_normal((k, wl.d_in), dtype=np.float32)
                b = _gen(seed, wl.index, _TENSOR_XB, c).standard_normal((k, wl.d_in), dtype=np.float32)
                x = (a / (np.float32(1.0) + np.exp(-a))) * b
            if cols is not None:
                x[:, cols] *= np.float32(wl.outlier_scale)
            return x

        res["X"] = _draw_rows(n, wl.d_in, fill_x, wl.dtype, out_dtype)
        res["outlier_cols"] = cols

    if "W" in want:
        def fill_w(c, k):
            g = _gen(seed, wl.index, _TENSOR_W, c)
            if wl.w_kind == "normal":
                return g.standard_normal((k, wl.d_in), dtype=np.float32) * np.float32(wl.w_std)
            t = g.standard_t(4.0, size=(k, wl.d_in))
            return (t * (wl.w_std / np.sqrt(2.0))).astype(np.float32)

        res["W"] = _draw_rows(d_out_rows, wl.d_in, fill_w, wl.dtype, out_dtype)

    if "G" in want:
        def fill_g(c, k):
            g = _gen(seed, wl.index, _TENSOR_G, c)
            x = g.laplace(0.0, wl.g_scale, size=(k, wl.d_out)).astype(np.float32)
            if wl.g_row_sigma > 0:
                z = _gen(seed, wl.index, _TENSOR_GROW, c).standard_normal((k, 1), dtype=np.float32)
                x *= np.exp(np.float32(wl.g_row_sigma) * z)
            return x

        res["G"] = _draw_rows(n, wl.d_out, fill_g, wl.dtype, out_dtype)
    return res
