"""Comparison gates between the HIP path and the float64 oracle.

Gates (fp32 arithmetic against the float64 definition):
  * no NaN or Inf anywhere in the output;
  * exactly 0 wherever the logit is -inf (fix paragraph of the pull-request
    page "fix(kernel): avoid nan in triton sampling softmax when a chunk starts
    with -inf": a masked entry contributes nothing);
  * max relative error <= 1e-5 over entries whose oracle probability is
    > 1e-6 (the page reports 3.2e-6 for its fixed fp32 kernel on the same
    masked inputs, results table);
  * absolute error <= 1e-11 where the oracle probability is <= 1e-6;
  * every row's float64 sum of the fp32 outputs within 1e-5 of 1.

Token draws (results table, sampling row: every draw lands on an allowed id;
the inverse-CDF rule is this library's reading). Several ids are correct when
a target sits within rounding of a CDF boundary, so the unique part is
checked: the id has a positive weight, and the target lies in the id's
interval of the exact float64 CDF widened by tau of the row total on each
side. tau is a worst-case bound on how far the draw's boundaries can sit from
the exact ones, derived from the float32 arithmetic the draw does:
  * against the probabilities the ids were drawn from (ts_sample, and the draw
    that writes the probabilities, on what it wrote): only the float sums that
    the draw's integer prefix sums are built on are inexact. A boundary at
    level 1 (groups of 4096 ids) is off by at most gamma(G) / 2 of the row
    total, one inside a group (blocks of 64 ids) by at most gamma(K) / 2 more,
    where gamma(n) bounds a float32 sum of tree depth n; inside a block the
    draw is exact. G = 15, K = 8 covers both paths (ts_sample sums at depth 12
    and 6; the draw-sums of the fused softmax at 14 and 7, plus one rounding of
    each written probability): SAMPLE_TAU = 6.9e-7.
  * ids drawn straight from the logits (ts_softmax_sample without
    probabilities), against the oracle's probabilities: the sums (depth 12 and
    6) plus the float32 exponents. An exponent d = (x - gsh) log2(e) / T carries
    at most 3 roundings (difference, scale, product): relative error 3 ln(2) u
    |d| in 2^d, plus 2u for the hardware exp2, in the element and again in its
    group's rescale (where the two |d| add up to the element's distance from
    the row's max), plus u for the rescale's product. A boundary moves by at
    most the mass-weighted mean of those errors, so per row
    tau = (gamma(12) + gamma(6)) / 2 + 3 ln(2) u E_p[|d|] + 5u, with E_p[|d|]
    taken from the oracle (ids_only_tau).
"""
import math

import numpy as np

from oracle import cdf_ref, softmax_ref

REL_TOL = 1e-5
PROB_FLOOR = 1e-6
ABS_TOL_SMALL = 1e-11
ROWSUM_TOL = 1e-5

U32 = 2.0 ** -24          # unit roundoff of float32 (round to nearest)
LN2 = math.log(2.0)


def gamma(n: int) -> float:
    """Bound on the relative error of a float32 sum of non-negative terms
    evaluated as a tree of depth n (Higham's gamma_n = n u / (1 - n u))."""
    return n * U32 / (1.0 - n * U32)


SAMPLE_TAU = (gamma(15) + gamma(8)) / 2


def mean_log2_distance(ref: np.ndarray, logits: np.ndarray, temps: np.ndarray) -> np.ndarray:
    """Per row, E_p[|d|]: the probability-weighted mean of (max z - z) log2(e)
    over the row's entries, z = x / T in float64 (0 where p = 0)."""
    z = logits.astype(np.float64) / temps.astype(np.float64)[:, None]
    zf = np.where(np.isfinite(z), z, -np.inf)
    top = zf.max(axis=1, keepdims=True)
    d = np.where(ref > 0, (top - np.where(np.isfinite(z), z, 0.0)) * math.log2(math.e), 0.0)
    return (ref * d).sum(axis=1)


def ids_only_tau(ref: np.ndarray, logits: np.ndarray, temps: np.ndarray) -> np.ndarray:
    """Per-row band for ids drawn straight from the logits, checked against the
    oracle's probabilities (module docstring)."""
    return (gamma(12) + gamma(6)) / 2 + 3 * LN2 * U32 * mean_log2_distance(ref, logits, temps) + 5 * U32


def softmax_errors(got: np.ndarray, logits: np.ndarray, ref: np.ndarray) -> dict:
    got64 = got.astype(np.float64)
    big = ref > PROB_FLOOR
    rel = np.abs(got64[big] - ref[big]) / ref[big]
    small = ~big
    return {
        "finite": bool(np.all(np.isfinite(got))),
        "masked_nonzero": int(np.count_nonzero(got[~np.isfinite(logits)])),
        "max_rel": float(rel.max()) if rel.size else 0.0,
        "max_abs_small": float(np.abs(got64[small] - ref[small]).max()) if small.any() else 0.0,
        "max_rowsum_dev": float(np.abs(got64.sum(axis=1) - 1.0).max()) if got.shape[0] else 0.0,
    }


def assert_softmax_matches(got: np.ndarray, logits: np.ndarray, temps: np.ndarray, ref=None, what=""):
    if ref is None:
        ref = softmax_ref(logits, temps)
    e = softmax_errors(got, logits, ref)
    assert e["finite"], f"{what}: NaN/Inf in output"
    assert e["masked_nonzero"] == 0, f"{what}: {e['masked_nonzero']} masked entries are not 0"
    assert e["max_rel"] <= REL_TOL, f"{what}: max rel err {e['max_rel']:.3e} > {REL_TOL}"
    assert e["max_abs_small"] <= ABS_TOL_SMALL, f"{what}: small-prob abs err {e['max_abs_small']:.3e}"
    assert e["max_rowsum_dev"] <= ROWSUM_TOL, f"{what}: row sum off by {e['max_rowsum_dev']:.3e}"
    return e


def assert_ids_valid(ids: np.ndarray, probs: np.ndarray, uniforms: np.ndarray, tau=SAMPLE_TAU, what=""):
    """Each id must have p > 0 and own its target in the float64 CDF of `probs`
    up to tau of the row total (tau: a number, or one per row). Returns the
    largest distance, as a fraction of the row total, by which a target fell
    outside its id's exact interval (0 when every target is inside)."""
    p = probs.astype(np.float64)
    c = cdf_ref(p)
    B, K = ids.shape
    assert ids.dtype == np.int32
    assert np.all((ids >= 0) & (ids < p.shape[1])), f"{what}: id out of range"
    rows = np.repeat(np.arange(B), K).reshape(B, K)
    assert np.all(p[rows, ids] > 0), f"{what}: drew an id with probability 0"
    u = np.where(np.isnan(uniforms), 0.0, np.clip(uniforms.astype(np.float64), 0.0, 1.0))
    total = c[:, -1:]
    target = u * total
    hi = c[rows, ids]
    lo = np.where(ids > 0, c[rows, np.maximum(ids - 1, 0)], 0.0)
    dev = np.maximum(np.maximum(lo - target, target - hi), 0.0) / total
    band = np.broadcast_to(np.asarray(tau, np.float64).reshape(-1, 1) if np.ndim(tau) else tau, dev.shape)
    bad = dev > band
    assert not bad.any(), (f"{what}: {np.count_nonzero(bad)} ids do not own their target "
                           f"(worst {dev.max():.3e} of the row total, band {np.min(band):.3e})")
    return float(dev.max()) if dev.size else 0.0


def assert_logit_ids_valid(ids: np.ndarray, logits: np.ndarray, temps: np.ndarray, uniforms: np.ndarray,
                           ref=None, what=""):
    """assert_ids_valid for ids drawn straight from the logits, against the
    oracle's float64 probabilities with the per-row band ids_only_tau. Returns
    (largest deviation, largest band)."""
    if ref is None:
        ref = softmax_ref(logits, temps)
    tau = ids_only_tau(ref, logits, temps)
    return assert_ids_valid(ids, ref, uniforms, tau=tau, what=what), float(tau.max())
