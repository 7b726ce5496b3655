"""GPU parity of ts_sample (inverse-CDF draws) against the float64 oracle.

The probabilities fed to both sides come from the oracle (cast to float32),
never from the HIP softmax. Several ids are correct when a target sits within
rounding of a CDF boundary, so the unique part is compared: the id has p > 0
and owns the target in the oracle's CDF of the same probabilities, up to the
band tests/parity.py derives from the draw's float32 sums (6.9e-7 of the row
total; ids drawn from logits: a per-row band that adds the float32 exponents'
error). Where every CDF value is
exact (dyadic weights) the ids must equal the oracle's exactly. The page's
draw case ("fix(kernel): avoid nan in triton sampling softmax when a chunk
starts with -inf", results table, sampling row: 3 allowed ids, 16 rows x 64
draws, all 1024 draws allowed) is reproduced from its golden fixture.
"""
import json
import os

import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from oracle import sample_ref, softmax_ref
from temperature_softmax_vocabulary_amd import workloads
from tests.parity import assert_ids_valid, assert_logit_ids_valid

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pr654_cases.json")


def _sample(p32, u32):
    ids = tsv.ts_sample(torch.from_numpy(p32).to(DEV), torch.from_numpy(u32).to(DEV))
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_configs_sample_matches_oracle(name):
    w = workloads.make_config(name)
    p32 = softmax_ref(w.logits, w.temps).astype(np.float32)
    print(f"[gpu] sample {name}", flush=True)
    ids = _sample(p32, w.uniforms)
    assert_ids_valid(ids, p32, w.uniforms, what=name)
    assert np.all(np.isfinite(w.logits)[np.arange(w.B)[:, None], ids])
    ref = sample_ref(p32, w.uniforms)
    # away from boundaries the id is unique: expect near-total agreement
    assert np.mean(ids == ref) > 0.999


def test_page_draw_case_all_allowed():
    g = json.load(open(GOLDEN))["sampling_draws"]
    w = workloads.make(g["rows"], 151936, "allowed3", K=g["draws_per_row"])
    p32 = softmax_ref(w.logits, w.temps).astype(np.float32)
    ids = _sample(p32, w.uniforms)
    allowed = sum(int(np.isin(ids[r], w.allowed[r]).sum()) for r in range(g["rows"]))
    assert allowed == g["expected_allowed_draws"]
    assert_ids_valid(ids, p32, w.uniforms)


def test_dyadic_rows_match_oracle_exactly_at_boundaries():
    # Every prefix sum of these rows is exact in float32 and float64, so the
    # strict-inequality rule has one answer even at the boundaries.
    V = 4099
    rng = np.random.default_rng(3)
    B = 6
    p = np.zeros((B, V), np.float32)
    for r in range(B):
        ids = rng.choice(V, size=8, replace=False)
        p[r, ids] = np.float32(1.0 / 8)
    p[0, :] = 0
    p[0, [0, 1, V - 1]] = [0.5, 0.25, 0.25]
    c = np.cumsum(p.astype(np.float64), axis=1)
    us = []
    for r in range(B):
        cuts = np.unique(c[r])
        row = np.concatenate([cuts, np.nextafter(cuts.astype(np.float32), np.float32(0)),
                              np.nextafter(cuts.astype(np.float32), np.float32(2)), [0.0, 1.0, -1.0, 2.0, np.nan]])
        us.append(row[:64] if row.size >= 64 else np.pad(row, (0, 64 - row.size), constant_values=0.5))
    u = np.array(us, np.float32)
    ids = _sample(p, u)
    ref = sample_ref(p, u)
    np.testing.assert_array_equal(ids, ref)


def test_extreme_uniforms_clamp_to_allowed_ids():
    w = workloads.make(4, 201088, "allowed3", K=8)
    p32 = softmax_ref(w.logits, w.temps).astype(np.float32)
    u = np.tile(np.array([0.0, 1.0 - 2.0 ** -24, 1.0, np.nan, -1.0, 2.0, np.inf, -np.inf], np.float32), (4, 1))
    ids = _sample(p32, u)
    for r in range(4):
        assert set(ids[r].tolist()) <= set(w.allowed[r].tolist())
        first, last = w.allowed[r][0], w.allowed[r][-1]
        assert ids[r, 0] == first and ids[r, 3] == first and ids[r, 4] == first and ids[r, 7] == first
        assert ids[r, 2] == last and ids[r, 5] == last and ids[r, 6] == last


@pytest.mark.parametrize("V,K", [(151937, 64), (7, 300), (262144, 2500), (1, 5)])
def test_odd_shapes_and_many_targets(V, K):
    w = workloads.make(3, V, "block20000" if V > 20000 else "none", K=K)
    p32 = softmax_ref(w.logits, w.temps).astype(np.float32)
    ids = _sample(p32, w.uniforms)
    assert_ids_valid(ids, p32, w.uniforms, what=f"V={V} K={K}")


def test_misaligned_probs_pointer():
    w = workloads.make_config("B3_V151936_pr_test_rows")
    p32 = softmax_ref(w.logits, w.temps).astype(np.float32)
    base = torch.empty(p32.size + 1, dtype=torch.float32, device=DEV)
    pt = base[1:].view(p32.shape)
    pt.copy_(torch.from_numpy(p32))
    ids = tsv.ts_sample(pt, torch.from_numpy(w.uniforms).to(DEV)).cpu().numpy()
    assert_ids_valid(ids, p32, w.uniforms)


@pytest.mark.parametrize("K", [4, 4100])   # one wave per target; rows sharing level 1 (4100 % 16 = 4)
def test_row_without_mass_gives_minus_one(K):
    p = np.zeros((2, 1000), np.float32)
    p[1, 10] = 1.0
    u = np.full((2, K), 0.5, np.float32)
    ids = _sample(p, u)
    assert np.all(ids[0] == -1) and np.all(ids[1] == 10)


def test_unnormalised_weights_scale_by_total():
    # ts_sample scales the target by the row total, so weights need not sum to 1
    rng = np.random.default_rng(12)
    p = (rng.random((4, 3000)) * (rng.random((4, 3000)) > 0.5)).astype(np.float32) * 7
    u = rng.random((4, 256)).astype(np.float32)
    ids = _sample(p, u)
    assert_ids_valid(ids, p, u)


@pytest.mark.parametrize("V,K", [
    (3 * 4096 + 100, 64),       # one wave per target, each doing level 1
    (3 * 4096 + 100, 1030),     # 16 targets per workgroup share level 1 (grid >= the CUs; 1030 % 16 = 6)
    (193 * 4096 - 5, 1030),     # the same over 4 tiles of 64 groups
])
def test_dyadic_rows_exact_across_groups_and_blocks(V, K):
    # Weights 2^-e spread over several 4096-id groups and 64-id blocks (some
    # blocks and groups empty): every float sum is exact, so every level of the
    # draw is exact and the ids must equal the oracle's, at and next to every
    # CDF boundary.
    rng = np.random.default_rng(21)
    B = 4
    p = np.zeros((B, V), np.float32)
    for r in range(B):
        ids = np.sort(rng.choice(V, size=16, replace=False))
        p[r, ids] = np.float32(2.0) ** -rng.integers(1, 6, size=16).astype(np.float32)
    p[0, :] = 0
    p[0, [5, 4096 + 64, 2 * 4096 + 63, V - 1]] = [0.5, 0.25, 0.125, 0.125]   # one id per group, block edges
    c = np.cumsum(p.astype(np.float64), axis=1)
    us = []
    for r in range(B):
        t = c[r, -1]
        cuts = np.unique(c[r]) / t
        row = np.concatenate([cuts, np.nextafter(cuts.astype(np.float32), np.float32(0)),
                              np.nextafter(cuts.astype(np.float32), np.float32(2)), [0.0, 1.0]])
        us.append(np.resize(row, K))
    u = np.array(us, np.float32)
    ids = _sample(p, u)
    np.testing.assert_array_equal(ids, sample_ref(p, u))


def test_nan_and_negative_entries_are_never_drawn():
    # entries that are not > 0 hold no mass: they are skipped whatever the
    # uniform, and they do not poison the rest of the row
    rng = np.random.default_rng(22)
    V = 9000
    p = rng.random((3, V)).astype(np.float32)
    bad = rng.random((3, V)) < 0.3
    p[bad] = np.where(rng.random(int(bad.sum())) < 0.5, np.float32(np.nan), np.float32(-1.0))
    u = rng.random((3, 512)).astype(np.float32)
    ids = _sample(p, u)
    clean = np.where(p > 0, p, 0).astype(np.float32)
    assert_ids_valid(ids, clean, u, what="nan/negative")
    assert not bad[np.arange(3)[:, None], ids].any()


@pytest.mark.parametrize("ng,K", [(8191, 64), (8191, 4096), (8193, 4096)])
def test_rows_at_the_shared_prefix_limit(ng, K):
    # With enough targets (here 4096 on one row: 256 workgroups) the resolve
    # keeps a row's level-1 prefix sums in LDS (8 bytes per 4096-id group,
    # plus the total) while they fit 64 KiB: 8191 groups just do (128 tiles of
    # 64 groups); at 8193, and with few targets, every target's wave does
    # level 1 itself. Dyadic weights in a few groups far apart: ids exact at
    # and next to every boundary. The same row as logits (-inf elsewhere)
    # through the ids-only draw: ids valid against the oracle.
    V = ng * 4096 - 7
    print(f"[gpu] long row: {ng} groups, V={V}, K={K}", flush=True)
    rng = np.random.default_rng(ng)
    cols = np.unique(np.concatenate([rng.choice(V, size=24, replace=False), [0, 4095, 4096, V - 1]]))
    w = np.float32(2.0) ** -rng.integers(1, 8, size=cols.size).astype(np.float32)
    p = np.zeros((1, V), np.float32)
    p[0, cols] = w
    c = np.cumsum(w.astype(np.float64))
    cuts = c / c[-1]
    row = np.concatenate([cuts, np.nextafter(cuts.astype(np.float32), np.float32(0)), [0.0, 1.0]])
    u = np.resize(row, (1, K)).astype(np.float32)
    np.testing.assert_array_equal(_sample(p, u), sample_ref(p, u))
    x = np.full((1, V), -np.inf, np.float32)
    x[0, cols] = np.log(w)
    t = np.ones(1, np.float32)
    ids, _ = tsv.ts_softmax_sample(torch.from_numpy(x).to(DEV), torch.from_numpy(t).to(DEV),
                                   torch.from_numpy(u).to(DEV))
    torch.cuda.synchronize()
    assert_logit_ids_valid(ids.cpu().numpy(), x, t, u, what=f"{ng} groups, logits")
    assert np.all(np.isin(ids.cpu().numpy(), cols))
    assert tsv.ts_device_errors() == 0


@pytest.mark.parametrize("B,V,K", [(1024, 4096 + 100, 40), (512, 3 * 4096 + 7, 96),
                                   (1024, 8 * 4096, 40), (1024, 8 * 4096 + 1, 40)])   # 8 groups: level 2 shared; 9: not
def test_two_targets_per_wave_exact_and_ragged(B, V, K):
    # Grids of at least 4 workgroups per compute unit put two targets on each
    # wave of the shared-level-1 resolve (K = 40: the second tile has live
    # targets only in part of its first half). Dyadic rows: every level is
    # exact, so the ids must equal the oracle's, at and next to every CDF
    # boundary; a row without mass gives -1 for every target; the ids-only
    # draw from the logits, with an allowed mask, lands on allowed ids.
    rng = np.random.default_rng(B + V + K)
    p = np.zeros((B, V), np.float32)
    for r in range(B):
        ids = np.sort(rng.choice(V, size=12, replace=False))
        p[r, ids] = np.float32(2.0) ** -rng.integers(1, 6, size=12).astype(np.float32)
    p[3, :] = 0
    c = np.cumsum(p.astype(np.float64), axis=1)
    us = np.zeros((B, K), np.float32)
    for r in range(B):
        t = c[r, -1] if c[r, -1] > 0 else 1.0
        cuts = np.unique(c[r]) / t
        row = np.concatenate([cuts, np.nextafter(cuts.astype(np.float32), np.float32(0)), [0.0, 1.0]])
        us[r] = np.resize(rng.permutation(row), K)
    print(f"[gpu] two targets per wave B={B} V={V} K={K}", flush=True)
    ids = _sample(p, us)
    rows = np.arange(B) != 3   # the oracle takes rows with mass only
    np.testing.assert_array_equal(ids[rows], sample_ref(p[rows], us[rows]))
    assert np.all(ids[3] == -1)
    w = workloads.make(B, V, "quarters", K=K, seed=B + K)
    xm = torch.from_numpy(workloads.unmasked_logits(w)).to(DEV)
    bits = torch.from_numpy(workloads.make_allowed(w).view(np.int32).copy()).to(DEV)
    got, _ = tsv.ts_softmax_sample(xm, torch.from_numpy(w.temps).to(DEV), torch.from_numpy(w.uniforms).to(DEV),
                                   allowed=bits)
    torch.cuda.synchronize()
    assert_logit_ids_valid(got.cpu().numpy(), w.logits, w.temps, w.uniforms, what="two per wave, masked")
    assert tsv.ts_device_errors() == 0
