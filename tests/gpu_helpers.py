"""Shared helpers of the GPU parity tests: device uploads and the tolerance checks."""

from __future__ import annotations

import os
import sys
import time

import numpy as np

from oracle import moe_oracle as O

# Tolerances for bf16 FFN outputs against the fp64 oracle, per token: normwise maximum
# relative error max|y - ref| / max|ref| <= 2e-2 and cosine >= 0.9995.
NORMWISE_TOL = 2e-2
COSINE_TOL = 0.9995
# Router weights: relative error of the fp32 result against the fp64 value.
WEIGHT_REL_TOL = 2.0 ** -22


def log(msg: str) -> None:
    sys.stdout.write(f"[{time.strftime('%H:%M:%S')}] {msg}\n")
    sys.stdout.flush()


def check_ffn(y_bits: np.ndarray, ref: np.ndarray, label: str = ""):
    """Per-token normwise relative error and cosine of bf16 outputs vs the oracle."""
    y = O.bf16_to_f64(y_bits)
    assert np.all(np.isfinite(y)), f"{label}: non-finite outputs"
    worst_err, worst_cos = 0.0, 1.0
    for t in range(y.shape[0]):
        err = O.normwise_rel_err(y[t], ref[t])
        cos = O.cosine(y[t], ref[t])
        worst_err = max(worst_err, err)
        worst_cos = min(worst_cos, cos)
        assert err <= NORMWISE_TOL, f"{label} token {t}: normwise rel err {err:.3e}"
        assert cos >= COSINE_TOL, f"{label} token {t}: cosine {cos:.6f}"
    return worst_err, worst_cos


def check_route(ids_gpu: np.ndarray, w_gpu: np.ndarray, ids_ref: np.ndarray, w_ref: np.ndarray,
                label: str = ""):
    assert ids_gpu.shape == ids_ref.shape
    bad = np.nonzero(np.any(ids_gpu != ids_ref, axis=1))[0]
    assert bad.size == 0, f"{label}: ids differ at tokens {bad[:10].tolist()}"
    rel = np.abs(w_gpu.astype(np.float64) - w_ref) / np.abs(w_ref)
    assert float(rel.max()) <= WEIGHT_REL_TOL, f"{label}: weight rel err {rel.max():.3e}"


def oracle_workers() -> int:
    """Threads for the oracle on large checks: the host cores this process may use, at most
    16 (a GPU machine's CPU share per GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_ffn_parallel(x_bits, ids, w, src, n_experts, hidden, inter, workers=None):
    """The oracle's expert_ffn for many tokens, run on disjoint expert ranges in threads
    (NumPy releases the interpreter lock in its array work) and summed range by range.
    Each range's call is the plain oracle with the other ranges' ids masked to -1 (ids
    outside [0, E) contribute nothing), so the result is the oracle's up to fp64
    reassociation of the per-token sum across ranges."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    workers = workers or oracle_workers()
    ids = np.asarray(ids)
    parts = max(1, min(workers, n_experts))

    def run(r):
        lo, hi = n_experts * r // parts, n_experts * (r + 1) // parts
        idr = np.where((ids >= lo) & (ids < hi), ids, -1).astype(np.int32)
        if not np.any(idr >= 0):
            return None
        with threadpool_limits(limits=1):
            return O.expert_ffn(x_bits, idr, w, src, n_experts, hidden, inter)

    with ThreadPoolExecutor(parts) as ex:
        outs = list(ex.map(run, range(parts)))
    y = np.zeros((np.asarray(x_bits).shape[0], hidden), dtype=np.float64)
    for o in outs:
        if o is not None:
            y += o
    return y
