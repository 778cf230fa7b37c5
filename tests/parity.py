"""Comparators of GPU results with the oracle.

fp32 paths: normwise relative error per tensor <= 1e-5 (two fp32 summation
orders differ elementwise by more than that on cancelling sums, so the bound is
read normwise).  bf16 paths: per element |got - ref| <= 2e-2 (|ref| + rms(ref));
the rms term is the floor near zero.  Loss: relative 1e-5 (fp32), 2e-3 (bf16).
"""
import numpy as np

F32_TOL = 1e-5
BF16_TOL = 2e-2
LOSS_TOL = {"f32": 1e-5, "bf16": 2e-3}


def rms(x):
    x = np.asarray(x, np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return num / den if den > 0 else num


def check(got, ref, act, name="", tol=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if act == "f32":
        err = normwise(got, ref)
        assert err <= (tol or F32_TOL), f"{name}: normwise error {err:.3e}"
        return err
    t = tol or BF16_TOL
    bound = t * (np.abs(ref) + rms(ref))
    diff = np.abs(got - ref)
    bad = diff > bound
    assert not np.any(bad), (f"{name}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"worst {float((diff / np.maximum(bound, 1e-300)).max()):.2f}x")
    return float((diff / np.maximum(np.abs(ref) + rms(ref), 1e-300)).max())


def check_weights(got, ref, gref, act, name=""):
    """Post-AdamW weights.  Where the reference gradient is within the tie band
    (|g| <= tau rms(g)) both signs of the first AdamW update are correct, so
    those elements are exempted (and counted)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g = np.asarray(gref, np.float64)
    tau = 1e-3 if act == "f32" else BF16_TOL
    tie = np.abs(g) <= tau * rms(g)
    got = np.where(tie, ref, got)
    check(got, ref, act, name)
    return int(tie.sum())
