"""Parity rules between the HIP path and the oracle.

* Top-k sets are bit-exact, except that an id in the symmetric difference is
  allowed when its oracle (float64) score lies within 1e-6 relative of the
  oracle's k-th score tau (the float32 score-gap rule).  Such swaps are
  counted and reported.
* Floating outputs: per row, max|gpu - ref| / max(max|ref|, 1e-3 * median
  row max) <= tol, with tol = 1e-4 for float32 paths and 2e-2 for bfloat16.
  The worst row, the global max-abs error and the lse error are reported.
"""

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def topk_check(gpu_ids, gpu_cnt, oracle_sel, scores, k, rel_gap=1e-6):
    """Returns (ok, n_swaps, message)."""
    gpu = np.asarray(gpu_ids)[:int(gpu_cnt)]
    if np.any(np.diff(gpu) <= 0):
        return False, 0, "gpu ids not strictly ascending"
    if len(gpu) != len(oracle_sel):
        return False, 0, f"count {len(gpu)} != oracle {len(oracle_sel)}"
    if np.array_equal(gpu, oracle_sel):
        return True, 0, ""
    diff = np.setxor1d(gpu, oracle_sel)
    if diff.size and (diff.min() < 0 or diff.max() >= len(scores)):
        return False, 0, "gpu id outside the visible range"
    tau = np.sort(scores)[::-1][min(k, len(scores)) - 1]
    bad = [int(s) for s in diff if abs(scores[s] - tau) > rel_gap * abs(tau)]
    if bad:
        return False, len(diff), f"ids {bad[:8]} differ with score gaps beyond {rel_gap} (tau={tau})"
    return True, len(diff) // 2, ""


def rel_err_rows(gpu, ref):
    """Per-row relative errors (rows = last axis vectors)."""
    g = np.asarray(gpu, np.float64).reshape(-1, np.shape(gpu)[-1])
    r = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    rowmax = np.abs(r).max(axis=1)
    floor = 1e-3 * np.median(rowmax) if rowmax.size else 0.0
    den = np.maximum(rowmax, max(floor, 1e-30))
    return np.abs(g - r).max(axis=1) / den


def assert_close(gpu, ref, kind, what=""):
    tol = TOL[kind]
    e = rel_err_rows(gpu, ref)
    worst = int(np.argmax(e)) if e.size else 0
    maxabs = float(np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64)).max())
    assert e.size == 0 or e.max() <= tol, (
        f"{what}: worst row {worst} rel err {e.max():.3e} > {tol} (max-abs {maxabs:.3e})")
    return float(e.max()) if e.size else 0.0, maxabs


def bf16_bits_to_f32(bits):
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
