"""Oracle rows in parallel worker processes (test infrastructure only).

Rows of one Fisher group are independent given F'_g, so the oracle's per-row work
runs in a pool of spawned worker processes: fresh interpreters that import only
numpy and the oracle, and never touch the GPU.  Each group's F'_g is written once
as a float64 .npy file that every worker memory-maps read-only, so the page cache
holds one copy for all of them.  Each worker runs its BLAS on one thread.

This module holds no arithmetic of the method: every task calls oracle functions.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

import oracle as O

_MMAP = {}


def _Fp(path):
    if path not in _MMAP:
        _MMAP.clear()
        _MMAP[path] = np.load(path, mmap_mode="r")
    return _MMAP[path]


def workers() -> int:
    """The machine's CPU share: at most 16 workers, whatever the machine shows."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool(n: int | None = None):
    """A spawn pool whose workers run single-threaded BLAS."""
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        return mp.get_context("spawn").Pool(n or workers())
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


class DampedFisherFile:
    """F'_g = damped(F_g) as a float64 .npy file for the workers; removed on exit.
    Written to /dev/shm when it has room, else to the temporary directory."""

    def __init__(self, F_g: np.ndarray, rho: float, lam_abs: float = 0.0):
        Fp = O.damped(F_g, rho, lam_abs)
        need = Fp.nbytes + (64 << 20)
        base = None
        if os.path.isdir("/dev/shm"):
            try:
                if shutil.disk_usage("/dev/shm").free > 2 * need:
                    base = "/dev/shm"
            except OSError:
                base = None
        self.dir = tempfile.mkdtemp(prefix="gq_oracle_", dir=base)
        self.path = os.path.join(self.dir, "Fp.npy")
        np.save(self.path, Fp)
        del Fp

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        shutil.rmtree(self.dir, ignore_errors=True)
        return False


# ----------------------------------------------------------------------------
# Tasks: each takes one tuple and returns plain numbers
# ----------------------------------------------------------------------------

def lnq_free_running(args):
    """The oracle's own LNQ run of one row (init, iters x (codebook, assignment)) and
    the oracle's objective of the device's final (c, p) for that row.
    Returns (j, oracle final objective, objective of the device result, device init
    identical to the oracle's)."""
    path, j, w, m, iters, c_dev, p_dev, c0_dev, p0_dev = args
    Fp = _Fp(path)
    c_init, p_init = O.init_quantile(w, m)
    same_init = bool(np.array_equal(c0_dev, c_init) and np.array_equal(p0_dev, p_init))
    _, _, tr = O.lnq_row(Fp, w, m, iters, trace=False)
    return j, float(tr[-1]), O.objective(Fp, w, c_dev, p_dev), same_init


def sweep_and_codebook(args):
    """One pass and one codebook step from a random state, checked against the
    device's results: (j, identical codes, decisions that differ, worst replay
    excess, step-relative codebook error, objective excess, empty codes kept)."""
    path, j, w, c0, p0, p_dev, c_dev, m, n_empty = args
    Fp = _Fp(path)
    p_ref = O.assign_sweep(Fp, w, c0, p0)
    same = int(np.sum(p_ref == p_dev))
    ex, differ = O.replay_sweep(Fp, w, c0, p0, p_dev, 1e-5)
    if differ == 0 and not np.array_equal(p_ref, p_dev):
        ex = max(ex, 1.0)                    # no differing decision yet different codes
    ref = O.codebook_update(Fp, w, p0, c0)
    kept = bool(np.array_equal(c_dev[m - n_empty:], c0[m - n_empty:])) if n_empty else True
    scale = max(np.linalg.norm(ref), np.linalg.norm(ref - c0))
    step = float(np.linalg.norm(c_dev - ref) / scale)
    o_ref = O.objective(Fp, w, ref, p0)
    excess = (O.objective(Fp, w, c_dev, p0) - o_ref) / o_ref
    return j, same, differ, float(ex), step, float(excess), kept


def teacher_forced(args):
    """The device's trajectory of one row, one iteration at a time: every codebook
    step against the oracle's closed form from the device's state before it, every
    pass replayed decision by decision.  Returns (j, init identical, worst codebook
    error, worst objective excess, worst replay excess, differing decisions,
    decisions)."""
    path, j, w, m, states = args
    Fp = _Fp(path)
    c_init, p_init = O.init_quantile(w, m)
    same_init = bool(np.array_equal(states[0][0], c_init) and np.array_equal(states[0][1], p_init))
    step = obj = rep = -np.inf
    differ = dec = 0
    for t in range(1, len(states)):
        c_prev, p_prev = states[t - 1]
        c_t, p_t = states[t]
        ref = O.codebook_update(Fp, w, p_prev, c_prev)
        step = max(step, float(np.linalg.norm(c_t - ref) / np.linalg.norm(ref)))
        o_ref = O.objective(Fp, w, ref, p_prev)
        obj = max(obj, (O.objective(Fp, w, c_t, p_prev) - o_ref) / o_ref)
        ex, dif = O.replay_sweep(Fp, w, c_t, p_prev, p_t, 1e-5)
        rep = max(rep, float(ex))
        differ += dif
        dec += w.shape[0]
    return j, same_init, step, float(obj), rep, differ, dec
