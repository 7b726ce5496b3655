"""Pins for the float64 oracle, checked against facts that do not come from it.

Each test uses a closed form, an invariant, an independent library routine, a
brute force on a tiny input, or the outcomes the pull-request page "fix(kernel):
avoid nan in triton sampling softmax when a chunk starts with -inf" (FreeToken
pull request 654) reports. Together they are chosen so that a plausible slip in
the oracle -- a dropped or inverted temperature, a temperature taken from the
wrong row, a wrong sign, no max shift, a sum over the wrong axis, a
non-strict CDF comparison, a missing clamp, an off-by-one id -- fails at least
one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import cdf_ref, sample_ref, softmax_ref
from temperature_softmax_vocabulary_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG = -np.inf


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# softmax: closed forms
# ----------------------------------------------------------------------------

def test_uniform_finite_logits_give_one_over_count():
    # n equal finite logits (the rest -inf) -> every finite entry is 1/n.
    V = 37
    x = np.full((3, V), NEG, dtype=np.float32)
    counts = [1, 5, 37]
    for r, n in enumerate(counts):
        x[r, V - n:] = np.float32(2.5 * (r + 1))
    p = softmax_ref(x, np.array([0.5, 1.0, 1.4], np.float32))
    for r, n in enumerate(counts):
        assert np.all(p[r, V - n:] == 1.0 / n)
        assert np.all(p[r, : V - n] == 0.0)


@pytest.mark.parametrize("T", [0.5, 0.75, 1.25, 1.5])
def test_rational_weights_closed_form(T):
    # x_j = T * ln(w_j)  =>  p_j = w_j / sum(w). No exponentials in the expectation.
    w = np.array([1, 2, 3, 4, 6, 9, 10], dtype=np.float64)
    x = (T * np.log(w)).astype(np.float32)[None, :]
    p = softmax_ref(x, np.array([T], np.float32))[0]
    expect = w / w.sum()
    # float32 storage of x perturbs p by < |ln w| * 2^-24 relative (~1.4e-7 here)
    np.testing.assert_allclose(p, expect, rtol=5e-7, atol=0)


def test_per_row_temperature_is_taken_from_its_own_row():
    # Three rows, same weights, different temperatures: each row's closed form
    # only holds with its own T (catches temps indexed by column or transposed).
    w = np.array([1, 2, 5, 8], dtype=np.float64)
    Ts = np.array([0.5, 1.0, 1.5], np.float32)
    x = np.stack([(float(T) * np.log(w)).astype(np.float32) for T in Ts])
    p = softmax_ref(x, Ts)
    for r in range(3):
        np.testing.assert_allclose(p[r], w / w.sum(), rtol=5e-7)
    # and with the rows' temperatures rotated the closed form breaks
    q = softmax_ref(x, np.roll(Ts, 1))
    assert np.max(np.abs(q - w / w.sum())) > 1e-2


def test_two_allowed_ids_logistic_form():
    # Two finite logits a, b: p_a = 1 / (1 + exp((b - a) / T)) (scipy's expit).
    V = 151936
    x = np.full((1, V), NEG, dtype=np.float32)
    a, b, T = np.float32(1.75), np.float32(-0.5), np.float32(0.8)
    x[0, 17], x[0, V - 3] = a, b
    p = softmax_ref(x, np.array([T]))[0]
    pa = scipy.special.expit((float(a) - float(b)) / float(T))
    assert abs(p[17] - pa) <= 1e-15
    assert abs(p[V - 3] - (1 - pa)) <= 1e-15
    assert np.count_nonzero(p) == 2


def test_extreme_spread_does_not_overflow():
    # One logit 1e4 above the rest at T = 0.5: exp(2e4) would overflow without
    # the shift; the answer is exactly one-hot.
    x = np.zeros((2, 1000), dtype=np.float32)
    x[0, 123] = 1e4
    x[1, 0] = 1e4
    x[1, 1:] = -1e4
    p = softmax_ref(x, np.array([0.5, 0.5], np.float32))
    assert p[0, 123] == 1.0 and p[1, 0] == 1.0
    assert np.count_nonzero(p) == 2


# ----------------------------------------------------------------------------
# softmax: invariants
# ----------------------------------------------------------------------------

def test_shift_invariance_exact_inputs():
    rng = np.random.default_rng(5)
    x = (rng.integers(-256, 256, size=(4, 513)) / 64.0).astype(np.float32)   # exact in fp32
    x[1, :100] = NEG
    t = np.array([0.5, 0.9, 1.1, 1.4], np.float32)
    p0 = softmax_ref(x, t)
    p1 = softmax_ref(x + np.float32(3.0), t)
    np.testing.assert_allclose(p1, p0, rtol=1e-13, atol=1e-300)


def test_temperature_scaling_equivalence():
    # softmax(x, T) == softmax(x / 2, T / 2); halving is exact in fp32.
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((3, 777)) * 4).astype(np.float32)
    t = np.array([0.6, 1.0, 1.4], np.float32)
    np.testing.assert_allclose(softmax_ref(x / np.float32(2), t / np.float32(2)),
                               softmax_ref(x, t), rtol=1e-13)


def test_rows_sum_to_one_and_masks_are_zero_nonsquare():
    w = workloads.make(5, 3001, "quarters", seed=11)
    p = softmax_ref(w.logits, w.temps)
    assert p.shape == (5, 3001)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)
    assert np.all(p[~np.isfinite(w.logits)] == 0.0)
    assert np.all(p[np.isfinite(w.logits)] > 0.0)


# ----------------------------------------------------------------------------
# softmax: independent library routines
# ----------------------------------------------------------------------------

def test_matches_scipy_softmax():
    w = workloads.make(8, 20011, "block20000", seed=3)
    z = w.logits.astype(np.float64) / w.temps.astype(np.float64)[:, None]
    ref = scipy.special.softmax(z, axis=1)
    p = softmax_ref(w.logits, w.temps)
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)


def test_matches_torch_softmax_float64_cpu():
    # The page's own test compares against torch.softmax (test paragraph).
    torch = pytest.importorskip("torch")
    w = workloads.make_config("B3_V151936_pr_test_rows")
    xt = torch.from_numpy(w.logits).double() / torch.from_numpy(w.temps).double()[:, None]
    ref = torch.softmax(xt, dim=1).numpy()
    p = softmax_ref(w.logits, w.temps)
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)


# ----------------------------------------------------------------------------
# softmax: the page's failure mechanism and outcomes
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1024, 2048, 4096, 8192])
def test_mask_covering_whole_leading_chunks_stays_finite(chunk):
    # Bug paragraph: a chunk whose first block is all -inf produced NaN. The
    # oracle has no chunks; it must simply be finite with exact zeros there.
    V = 4 * chunk + 384
    x = np.random.default_rng(chunk).standard_normal((2, V)).astype(np.float32)
    x[0, :chunk] = NEG                      # first chunk fully masked
    x[1, chunk: 2 * chunk + 1] = NEG        # a chunk start and its whole chunk
    p = softmax_ref(x, np.array([0.7, 1.2], np.float32))
    assert np.all(np.isfinite(p))
    assert np.all(p[0, :chunk] == 0) and np.all(p[1, chunk: 2 * chunk + 1] == 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)


def test_page_masked_case_grid_is_finite():
    g = _load_golden("pr654_cases.json")["masked_case_grid"]
    for kind in g["kinds"]:
        for V in g["V"]:
            B = 3   # every kind/V pair once; B=1 and B=8 are the same rows
            w = workloads.make(B, V, kind)
            p = softmax_ref(w.logits, w.temps)
            assert g["expected"]["every_masked_row_finite"] and np.all(np.isfinite(p))
            assert np.all(p[~np.isfinite(w.logits)] == 0)


def test_oracle_rejects_inputs_outside_the_domain():
    ok = np.zeros((1, 4), np.float32)
    with pytest.raises(ValueError):
        softmax_ref(np.full((1, 4), NEG, np.float32), np.ones(1, np.float32))
    with pytest.raises(ValueError):
        softmax_ref(ok, np.zeros(1, np.float32))
    with pytest.raises(ValueError):
        softmax_ref(ok, np.array([np.nan], np.float32))
    bad = ok.copy(); bad[0, 1] = np.nan
    with pytest.raises(ValueError):
        softmax_ref(bad, np.ones(1, np.float32))
    bad[0, 1] = np.inf
    with pytest.raises(ValueError):
        softmax_ref(bad, np.ones(1, np.float32))


# ----------------------------------------------------------------------------
# sampler
# ----------------------------------------------------------------------------

def _brute_force_id(weights, u):
    """Exact rational inverse CDF by enumeration: smallest j with C_j > u*C_total."""
    fr = [Fraction(float(v)) for v in weights]
    total = sum(fr, Fraction(0))
    uu = Fraction(float(u))
    uu = min(max(uu, Fraction(0)), Fraction(1))
    t = uu * total
    acc = Fraction(0)
    for j, v in enumerate(fr):
        acc += v
        if acc > t:
            return j
    return max(j for j, v in enumerate(fr) if v > 0)


def test_sampler_brute_force_tiny_dyadic_rows():
    # Dyadic weights make every CDF value exact in float64 too, so the oracle
    # must agree with exact enumeration at and around every boundary.
    rows = [
        [0.125, 0.0, 0.375, 0.5],
        [0.0, 0.5, 0.5, 0.0],
        [0.25, 0.25, 0.0, 0.0, 0.5],
        [0.0, 0.0, 1.0, 0.0],
        [0.5, 0.25, 0.125, 0.0625, 0.0625],
    ]
    for wts in rows:
        c = np.cumsum(wts)
        us = {0.0, 1.0, -0.5, 2.0}
        for v in c:
            us |= {float(v), float(np.nextafter(v, 0)), float(np.nextafter(v, 2))}
        us = sorted(u for u in us)
        p = np.array([wts], np.float64)
        got = sample_ref(p, np.array([us]))[0]
        for u, j in zip(us, got):
            assert j == _brute_force_id(wts, u), (wts, u, j)
            assert wts[j] > 0


def test_sampler_strictness_zero_probability_never_drawn():
    p = np.array([[0.25, 0.0, 0.75], [0.0, 0.5, 0.5]])
    ids = sample_ref(p, np.array([[0.25, 0.0], [0.0, 0.5]]))
    assert ids.tolist() == [[2, 0], [1, 2]]


def test_sampler_clamps_out_of_range_and_nan_uniforms():
    p = np.array([[0.0, 0.3, 0.0, 0.7, 0.0]])
    ids = sample_ref(p, np.array([[-1.0, np.nan, 0.0, 1.0, 1.5, np.inf]]))
    assert ids.tolist() == [[1, 1, 1, 3, 3, 3]]


def test_sampler_frequencies_match_weights_on_a_uniform_grid():
    # Defining property of an inverse-CDF draw: with u on a fine uniform grid,
    # the share of draws landing on id j is p_j (up to one grid step per
    # boundary). An off-by-one id or a target not scaled by the total fails.
    rng = np.random.default_rng(9)
    w = rng.random(50) * (rng.random(50) > 0.3)
    w = w / w.sum() * 2.0                    # total 2: the target must scale by it
    n = 200000
    u = (np.arange(n) + 0.5) / n
    ids = sample_ref(w[None, :], u[None, :])[0]
    freq = np.bincount(ids, minlength=50) / n
    np.testing.assert_allclose(freq, w / w.sum(), atol=2.0 / n)
    assert np.all(freq[w == 0] == 0)


def test_sampler_page_draw_case_all_allowed():
    g = _load_golden("pr654_cases.json")["sampling_draws"]
    w = workloads.make(g["rows"], 151936, "allowed3", K=g["draws_per_row"])
    p = softmax_ref(w.logits, w.temps)
    ids = sample_ref(p, w.uniforms)
    allowed = sum(int(np.isin(ids[r], w.allowed[r]).sum()) for r in range(g["rows"]))
    assert allowed == g["expected_allowed_draws"]


def test_cdf_is_inclusive_prefix_sum():
    p = np.array([[0.5, 0.25, 0.25]])
    assert cdf_ref(p).tolist() == [[0.5, 0.75, 1.0]]
    assert math.isclose(cdf_ref(np.ones((1, 10)) / 10)[0, -1], 1.0)


# ----------------------------------------------------------------------------
# allowed-id bitmask (mask producers of the scope paragraph)
# ----------------------------------------------------------------------------

def test_bitmask_bit_order_single_allowed_id_is_one_hot():
    # one allowed id at a word boundary, inside a word, at the row end: the
    # result must be one-hot exactly there (catches bit order / word index slips)
    from oracle import softmax_masked_ref
    V = 100
    for j in (0, 1, 31, 32, 33, 63, 64, 99):
        bits = np.zeros((1, (V + 31) // 32), np.uint32)
        bits[0, j // 32] = np.uint32(1) << np.uint32(j % 32)
        x = np.random.default_rng(j).standard_normal((1, V)).astype(np.float32)
        p = softmax_masked_ref(x, np.ones(1, np.float32), bits)
        assert p[0, j] == 1.0 and np.count_nonzero(p) == 1, j


def test_bitmask_all_ones_and_equivalence_with_pre_masked_logits():
    from oracle import softmax_masked_ref
    w = workloads.make(6, 5003, "quarters", seed=21)
    ones = np.full((6, (5003 + 31) // 32), 0xFFFFFFFF, np.uint32)
    finite = np.where(np.isfinite(w.logits), w.logits, np.float32(0.0))
    np.testing.assert_array_equal(softmax_masked_ref(finite, w.temps, ones), softmax_ref(finite, w.temps))
    # the workload's -inf pattern as bits, applied to different finite values there
    bits = workloads.make_allowed(w)
    x = workloads.unmasked_logits(w)
    assert np.all(np.isfinite(x)) and np.array_equal(x[np.isfinite(w.logits)], w.logits[np.isfinite(w.logits)])
    np.testing.assert_array_equal(softmax_masked_ref(x, w.temps, bits), softmax_ref(w.logits, w.temps))


def test_bitmask_two_allowed_ids_logistic():
    from oracle import softmax_masked_ref
    V = 70
    x = np.random.default_rng(2).standard_normal((1, V)).astype(np.float32) * 4
    keep = np.zeros((1, V), bool)
    keep[0, [5, 66]] = True
    p = softmax_masked_ref(x, np.array([0.7], np.float32), workloads.pack_allowed(keep))
    pa = scipy.special.expit((float(x[0, 5]) - float(x[0, 66])) / float(np.float32(0.7)))
    assert abs(p[0, 5] - pa) <= 1e-15 and abs(p[0, 66] - (1 - pa)) <= 1e-15


def test_pack_allowed_round_trips():
    from oracle import allowed_bits_to_bool
    keep = np.random.default_rng(3).random((4, 1000)) < 0.3
    assert np.array_equal(allowed_bits_to_bool(workloads.pack_allowed(keep), 1000), keep)
    with pytest.raises(ValueError):
        allowed_bits_to_bool(np.zeros((4, 31), np.uint32), 1000)
