"""GPU parity of ts_softmax_sample (softmax and inverse-CDF draw in one call).

The probabilities must pass the same gates as ts_softmax against the float64
oracle. The ids are checked for the unique part (p > 0 and the target inside
the id's interval of the exact CDF): those drawn with the probabilities written
against the CDF of what was written, within the band the draw's float32 sums
allow; those drawn straight from the logits against the oracle's probabilities,
within a per-row band that adds the float32 exponents' error (tests/parity.py
derives both). The two modes weigh groups and
blocks from different float sums, so they agree except within rounding of a
boundary. The page's draw case ("fix(kernel): avoid nan in triton sampling
softmax when a chunk starts with -inf", results table, sampling row) must give
1024 allowed draws out of 1024.
"""
import json
import os

import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from oracle import sample_ref, softmax_ref
from temperature_softmax_vocabulary_amd import workloads
from tests.parity import SAMPLE_TAU, assert_ids_valid, assert_logit_ids_valid, assert_softmax_matches

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pr654_cases.json")


def _dev(a):
    return torch.from_numpy(a).to(DEV)


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_configs_probs_and_ids(name):
    w = workloads.make_config(name)
    ref = softmax_ref(w.logits, w.temps)
    x, t, u = _dev(w.logits), _dev(w.temps), _dev(w.uniforms)
    print(f"[gpu] softmax_sample {name}", flush=True)
    ids, probs = tsv.ts_softmax_sample(x, t, u, probs_out=True)
    ids_only, none = tsv.ts_softmax_sample(x, t, u)
    torch.cuda.synchronize()
    assert none is None
    p = probs.cpu().numpy()
    assert_softmax_matches(p, w.logits, w.temps, ref, what=name)
    ids = ids.cpu().numpy()
    ids_only = ids_only.cpu().numpy()
    # ids-only draws from group partials of the logits, the other from the
    # written probabilities: both follow the rule (each against what it drew
    # from, within its derived band), and can differ only for a target within
    # float rounding of a boundary
    dev_p = assert_ids_valid(ids, p, w.uniforms, what=f"{name} with probs")
    dev_l, tau_l = assert_logit_ids_valid(ids_only, w.logits, w.temps, w.uniforms, ref, what=f"{name} ids only")
    print(f"[gpu] {name}: largest target outside its exact interval: with probs {dev_p:.2e} "
          f"(band {SAMPLE_TAU:.2e}), ids only {dev_l:.2e} (band up to {tau_l:.2e})", flush=True)
    for got in (ids, ids_only):
        assert np.all(np.isfinite(w.logits)[np.arange(w.B)[:, None], got])
    assert np.mean(ids == ids_only) > 0.99
    # The draw uses the GPU's fp32 probabilities (relative error ~1e-6), so a
    # target within that distance of a CDF boundary may fall on either side:
    # assert_ids_valid above is the gate; this only guards against a gross shift.
    agree = np.mean(ids == sample_ref(ref, w.uniforms))
    assert agree > 0.95, agree
    assert tsv.ts_device_errors() == 0


def test_matches_separate_softmax_then_sample():
    w = workloads.make_config("B64_V262144_masked_quarters")
    x, t, u = _dev(w.logits), _dev(w.temps), _dev(w.uniforms)
    ids_f, probs_f = tsv.ts_softmax_sample(x, t, u, probs_out=True)
    probs_s = tsv.ts_softmax(x, t)
    ids_s = tsv.ts_sample(probs_s, u)
    torch.cuda.synchronize()
    # both paths meet the oracle's gates; the probabilities agree to float
    # rounding (the work split may differ), and the ids can differ only where a
    # target sits within rounding of a block or group boundary
    ref = softmax_ref(w.logits, w.temps)
    assert_softmax_matches(probs_f.cpu().numpy(), w.logits, w.temps, ref, what="fused with draw")
    assert_softmax_matches(probs_s.cpu().numpy(), w.logits, w.temps, ref, what="separate")
    a, b = ids_f.cpu().numpy(), ids_s.cpu().numpy()
    assert_ids_valid(a, probs_f.cpu().numpy(), w.uniforms, what="fused")
    assert_ids_valid(b, probs_s.cpu().numpy(), w.uniforms, what="separate")
    assert np.mean(a == b) > 0.99


def test_page_draw_case_all_allowed():
    g = json.load(open(GOLDEN))["sampling_draws"]
    w = workloads.make(g["rows"], 151936, "allowed3", K=g["draws_per_row"])
    ids, _ = tsv.ts_softmax_sample(_dev(w.logits), _dev(w.temps), _dev(w.uniforms))
    ids = ids.cpu().numpy()
    allowed = sum(int(np.isin(ids[r], w.allowed[r]).sum()) for r in range(g["rows"]))
    assert allowed == g["expected_allowed_draws"]


@pytest.mark.parametrize("B,V,K", [(3, 7, 5), (2, 1025, 64), (5, 151937, 64), (1, 262144, 3000),
                                   (4, 2097152, 16)])
def test_odd_shapes(B, V, K):
    w = workloads.make(B, V, "block20000" if V > 20000 else "none", K=K)
    ref = softmax_ref(w.logits, w.temps)
    ids, probs = tsv.ts_softmax_sample(_dev(w.logits), _dev(w.temps), _dev(w.uniforms), probs_out=True)
    torch.cuda.synchronize()
    p = probs.cpu().numpy()
    assert_softmax_matches(p, w.logits, w.temps, ref, what=f"B={B} V={V}")
    assert_ids_valid(ids.cpu().numpy(), p, w.uniforms, what=f"B={B} V={V} K={K}")


def test_in_place_probs_and_extreme_uniforms():
    w = workloads.make(4, 201088, "allowed3", K=8)
    ref = softmax_ref(w.logits, w.temps)
    u = np.tile(np.array([0.0, 1.0 - 2.0 ** -24, 1.0, np.nan, -1.0, 2.0, np.inf, -np.inf], np.float32), (4, 1))
    x = _dev(w.logits)
    ids, probs = tsv.ts_softmax_sample(x, _dev(w.temps), _dev(u), probs_out=x)
    torch.cuda.synchronize()
    assert probs.data_ptr() == x.data_ptr()
    assert_softmax_matches(x.cpu().numpy(), w.logits, w.temps, ref, what="in place")
    ids = ids.cpu().numpy()
    for r in range(4):
        first, last = w.allowed[r][0], w.allowed[r][-1]
        # u = 0, NaN, -1, -inf clamp to 0: the first allowed id; u = 1, 2, inf: the last one
        assert [ids[r][i] for i in (0, 3, 4, 7)] == [first] * 4
        assert [ids[r][i] for i in (2, 5, 6)] == [last] * 3
        assert set(ids[r].tolist()) <= set(w.allowed[r].tolist())


def test_zero_draws_and_limits():
    w = workloads.make(2, 5000, "none", K=0)
    x, t = _dev(w.logits), _dev(w.temps)
    u = torch.empty((2, 0), dtype=torch.float32, device=DEV)
    ids, probs = tsv.ts_softmax_sample(x, t, u, probs_out=True)
    torch.cuda.synchronize()
    assert ids.shape == (2, 0)
    assert_softmax_matches(probs.cpu().numpy(), w.logits, w.temps, what="K=0")


def test_long_rows_draw_from_logits():
    # more groups than one wave's tile (256 groups of 1024): the draw's CDF
    # walks several tiles with a carry; masked ids are never drawn
    w = workloads.make(2, 2097152 + 4099, "block20000", K=32)
    ref = softmax_ref(w.logits, w.temps)
    ids = tsv.ts_softmax_sample(_dev(w.logits), _dev(w.temps), _dev(w.uniforms))[0].cpu().numpy()
    assert_logit_ids_valid(ids, w.logits, w.temps, w.uniforms, ref, what="long rows")


def test_with_probs_ids_agree_with_ts_sample_on_them():
    # the draw with probs_out reads the written probabilities; its block and
    # group weights come from the fused kernel (summed before scaling), so the
    # ids equal ts_sample's on the same probabilities except within float
    # rounding of a boundary
    for name in ("B3_V151936_pr_test_rows", "B64_V262144_masked_quarters"):
        w = workloads.make_config(name)
        x, t, u = _dev(w.logits), _dev(w.temps), _dev(w.uniforms)
        ids, probs = tsv.ts_softmax_sample(x, t, u, probs_out=True)
        again = tsv.ts_sample(probs, u)
        torch.cuda.synchronize()
        p = probs.cpu().numpy()
        a, b = ids.cpu().numpy(), again.cpu().numpy()
        assert_ids_valid(a, p, w.uniforms, what=f"{name} fused")
        assert_ids_valid(b, p, w.uniforms, what=f"{name} ts_sample")
        assert np.mean(a == b) > 0.99, name


def test_sample_long_rows():
    # rows of more than 256 groups of 1024 ids: the draw's CDF spans several tiles
    B, V, K = 2, 2097152 + 4099, 32
    rng = np.random.default_rng(4)
    p = (rng.random((B, V)) * (rng.random((B, V)) < 0.01)).astype(np.float32)
    u = rng.random((B, K)).astype(np.float32)
    ids = tsv.ts_sample(_dev(p), _dev(u)).cpu().numpy()
    assert_ids_valid(ids, p, u, what="fallback")


@pytest.mark.parametrize("K", [64, 256])   # one wave per target; 16 targets of a row per workgroup
@pytest.mark.parametrize("with_probs", [True, False], ids=["with_probs", "ids_only"])
def test_graph_capture_softmax_sample(with_probs, K):
    B, V = 16, 201088
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(B, V, device=DEV, stream=s)
    x = torch.zeros((B, V), dtype=torch.float32, device=DEV)
    t = torch.ones((B,), dtype=torch.float32, device=DEV)
    u = torch.zeros((B, K), dtype=torch.float32, device=DEV)
    ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
    probs = torch.empty_like(x)
    po = probs if with_probs else None
    with torch.cuda.stream(s):
        tsv.ts_softmax_sample(x, t, u, out_ids=ids, probs_out=po)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tsv.ts_softmax_sample(x, t, u, out_ids=ids, probs_out=po)
    for rep in range(3):
        w = workloads.make(B, V, "quarters", K=K, seed=500 + rep)
        x.copy_(_dev(w.logits))
        t.copy_(_dev(w.temps))
        u.copy_(_dev(w.uniforms))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = softmax_ref(w.logits, w.temps)
        if with_probs:
            p = probs.cpu().numpy()
            assert_softmax_matches(p, w.logits, w.temps, ref, what=f"replay {rep}")
            assert_ids_valid(ids.cpu().numpy(), p, w.uniforms, what=f"replay {rep}")
        else:
            assert_logit_ids_valid(ids.cpu().numpy(), w.logits, w.temps, w.uniforms, ref, what=f"replay {rep}")
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0


@pytest.mark.parametrize("B,V,chunk", [(3, 1000, 4096), (8, 4096, 4096), (64, 16384, 4096), (128, 20480, 8192),
                                       (2048, 32768, 8192)])
def test_probs_of_row_kernel_shapes_come_from_the_fused_split(B, V, chunk):
    # shapes the work-split table gives the one-workgroup-per-row kernel: the
    # draw that also writes the probabilities takes the fused split there (it
    # leaves the draw's group sums): its probabilities are that split's bit for
    # bit, ts_softmax's within the tolerance, and its ids follow the rule
    w = workloads.make(B, V, "quarters" if B >= 4 else "first16384", K=8)
    assert tsv.ts_plan(B, V)[0] == tsv.TS_VARIANT_ROWWISE
    x, t, u = _dev(w.logits), _dev(w.temps), _dev(w.uniforms)
    print(f"[gpu] with-probs draw plan B={B} V={V}", flush=True)
    ids, probs = tsv.ts_softmax_sample(x, t, u, probs_out=True)
    fused = tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_FUSED, chunk)
    torch.cuda.synchronize()
    assert torch.equal(probs, fused)
    assert_softmax_matches(probs.cpu().numpy(), w.logits, w.temps, what=f"with probs B={B} V={V}")
    assert_softmax_matches(tsv.ts_softmax(x, t).cpu().numpy(), w.logits, w.temps, what=f"rowwise B={B} V={V}")
    assert_ids_valid(ids.cpu().numpy(), probs.cpu().numpy(), w.uniforms, what=f"with probs B={B} V={V}")
    assert tsv.ts_device_errors() == 0
