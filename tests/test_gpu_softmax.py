"""GPU parity of ts_softmax against the float64 oracle, element by element.

Every workload is seeded and synthetic (temperature_softmax_vocabulary_amd.
workloads), at the full sizes the bench uses, in every work split the library
has. The edge grid follows the failure mechanism of the pull-request page "fix(kernel):
avoid nan in triton sampling softmax when a chunk starts with -inf" (bug
paragraph): -inf placed at exact chunk starts, whole masked chunks, and a
chunk whose first vector is masked, for every chunk size.
"""
import functools

import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from oracle import softmax_ref
from temperature_softmax_vocabulary_amd import workloads
from tests.parity import assert_softmax_matches

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SPLITS = [(tsv.TS_VARIANT_SPLIT, c) for c in tsv.CHUNKS] + \
         [(tsv.TS_VARIANT_FUSED, c) for c in tsv.CHUNKS] + [(tsv.TS_VARIANT_ROWWISE, 0)]
SPLIT_IDS = [f"{tsv.VARIANT_NAMES[v]}-{c}" for v, c in SPLITS]


@functools.lru_cache(maxsize=None)
def _config(name):
    w = workloads.make_config(name)
    return w, softmax_ref(w.logits, w.temps)


def _run(logits, temps, variant=tsv.TS_VARIANT_AUTO, chunk=0, out=None):
    x = torch.from_numpy(logits).to(DEV) if isinstance(logits, np.ndarray) else logits
    t = torch.from_numpy(temps).to(DEV) if isinstance(temps, np.ndarray) else temps
    if variant == tsv.TS_VARIANT_AUTO and chunk == 0:
        y = tsv.ts_softmax(x, t, out=out)
    else:
        y = tsv.ts_softmax_variant(x, t, variant, chunk, out=out)
    torch.cuda.synchronize()
    return y


def _no_device_errors():
    assert tsv.ts_device_errors() == 0


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_configs_default_plan(name):
    w, ref = _config(name)
    print(f"[gpu] default plan {name} plan={tsv.ts_plan(w.B, w.V)}", flush=True)
    y = _run(w.logits, w.temps).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, ref, what=name)
    _no_device_errors()


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=SPLIT_IDS)
@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_configs_every_split(name, variant, chunk):
    w, ref = _config(name)
    print(f"[gpu] {name} variant={variant} chunk={chunk}", flush=True)
    y = _run(w.logits, w.temps, variant, chunk).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, ref, what=f"{name}/{variant}/{chunk}")
    _no_device_errors()


def _edge_rows(V, C, rng):
    """Rows whose masks hit the chunk grid of chunk size C."""
    x = (rng.standard_normal((8, V)) * 4).astype(np.float32)
    NEG = np.float32(-np.inf)
    n = (V + C - 1) // C
    x[0, :min(C, V - 1)] = NEG                       # first chunk fully masked
    x[1, C: min(2 * C, V)] = NEG                     # a later chunk fully masked
    x[2, min(C, V - 1): C + C // 2] = NEG            # half a chunk from its start
    for c in range(n):                               # first float4 of every chunk
        x[3, c * C: c * C + 4] = NEG
    x[4, :] = NEG                                    # one finite id, in the tail chunk
    x[4, V - 1] = np.float32(0.25)
    x[5, :] = NEG                                    # 3 ids in three different chunks
    for j in (0, min(C + 5, V - 1), V - 2):
        x[5, j] = np.float32(rng.standard_normal() * 4)
    x[6, :] = NEG                                    # every chunk but the last masked
    x[6, (n - 1) * C:] = (rng.standard_normal(V - (n - 1) * C) * 4).astype(np.float32)
    x[7, 0] = x[7].max() + np.float32(1e4)           # extreme spread
    t = np.array([0.5, 0.8, 1.0, 1.2, 0.7, 1.4, 0.9, 0.5], np.float32)
    return x, t


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=SPLIT_IDS)
@pytest.mark.parametrize("V", [151936, 151937, 40000, 16384, 5003])
def test_edge_grid(V, variant, chunk):
    C = chunk or 1024
    rng = np.random.default_rng(V * 31 + C)
    x, t = _edge_rows(V, C, rng)
    print(f"[gpu] edge V={V} variant={variant} chunk={chunk}", flush=True)
    y = _run(x, t, variant, chunk).cpu().numpy()
    assert_softmax_matches(y, x, t, what=f"edge V={V} {variant}/{chunk}")
    assert y[7, 0] == 1.0
    _no_device_errors()


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=SPLIT_IDS)
def test_tiny_and_odd_shapes(variant, chunk):
    rng = np.random.default_rng(1)
    for B, V in [(1, 1), (3, 7), (2, 1023), (5, 1025), (1, 4097)]:
        x = (rng.standard_normal((B, V)) * 4).astype(np.float32)
        t = (rng.random(B) + 0.5).astype(np.float32)
        y = _run(x, t, variant, chunk).cpu().numpy()
        assert_softmax_matches(y, x, t, what=f"B={B} V={V}")
        if V == 1:
            assert np.all(y == 1.0)
    _no_device_errors()


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=SPLIT_IDS)
def test_misaligned_pointers_take_scalar_path(variant, chunk):
    # logits and out start 4 bytes past a 16-byte boundary
    w, ref = _config("B3_V151936_pr_test_rows")
    B, V = w.B, w.V
    base = torch.empty(B * V + 4, dtype=torch.float32, device=DEV)
    x = base[1: 1 + B * V].view(B, V)
    x.copy_(torch.from_numpy(w.logits))
    obase = torch.full((B * V + 4,), 7.0, dtype=torch.float32, device=DEV)
    out = obase[1: 1 + B * V].view(B, V)
    t = torch.from_numpy(w.temps).to(DEV)
    y = _run(x, t, variant, chunk, out=out).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, ref, what="misaligned")
    o = obase.cpu().numpy()
    assert o[0] == 7.0 and np.all(o[1 + B * V:] == 7.0), "wrote outside out"


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=SPLIT_IDS)
def test_in_place(variant, chunk):
    w, ref = _config("B8_V201088_block_and_head")
    x = torch.from_numpy(w.logits).to(DEV)
    t = torch.from_numpy(w.temps).to(DEV)
    y = _run(x, t, variant, chunk, out=x)
    assert y.data_ptr() == x.data_ptr()
    assert_softmax_matches(x.cpu().numpy(), w.logits, w.temps, ref, what="in place")


def test_output_does_not_spill_past_rows():
    # out is a window of a larger buffer: nothing outside it may change
    w, ref = _config("B16_V201088_unmasked")
    big = torch.full((w.B + 2, w.V), -3.0, dtype=torch.float32, device=DEV)
    out = big[1: 1 + w.B]
    for v, c in SPLITS:
        _run(w.logits, w.temps, v, c, out=out)
        b = big.cpu().numpy()
        assert np.all(b[0] == -3.0) and np.all(b[-1] == -3.0), (v, c)


def test_bitwise_deterministic():
    w, _ = _config("B64_V262144_masked_quarters")
    x = torch.from_numpy(w.logits).to(DEV)
    t = torch.from_numpy(w.temps).to(DEV)
    for v, c in SPLITS:
        a = _run(x, t, v, c).clone()
        b = _run(x, t, v, c)
        assert torch.equal(a, b), (v, c)


def test_zero_rows_is_noop():
    x = torch.empty((0, 100), dtype=torch.float32, device=DEV)
    t = torch.empty((0,), dtype=torch.float32, device=DEV)
    assert tsv.ts_softmax(x, t).shape == (0, 100)


def test_plan_for_configs_is_legal():
    for name in workloads.CONFIG_ORDER:
        c = workloads.CONFIGS[name]
        v, ch = tsv.ts_plan(c["B"], c["V"])
        assert v in (tsv.TS_VARIANT_FUSED, tsv.TS_VARIANT_SPLIT, tsv.TS_VARIANT_ROWWISE)
        assert v == tsv.TS_VARIANT_ROWWISE or ch in tsv.CHUNKS


@pytest.mark.parametrize("V", [2 * 1024 * 1024 + 4099, 4 * 1024 * 1024 + 1000])
def test_long_rows_default_plan(V):
    # rows beyond 256 chunks of 8192 (fused at 16384) and of 16384 columns
    # (the split pair): the plan's upper branches, with masks at chunk starts
    w = workloads.make(2, V, "block_and_head")
    ref = softmax_ref(w.logits, w.temps)
    plan = tsv.ts_plan(2, V)
    print(f"[gpu] long rows V={V} plan={plan}", flush=True)
    y = tsv.ts_softmax(torch.from_numpy(w.logits).to(DEV), torch.from_numpy(w.temps).to(DEV)).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, ref, what=f"V={V}")
    expect = tsv.TS_VARIANT_FUSED if V <= 256 * 16384 else tsv.TS_VARIANT_SPLIT
    assert plan[0] == expect


@pytest.mark.parametrize("B,V", [(4, 16384), (4, 16385), (767, 16384), (768, 16384), (2048, 4096), (2049, 4096),
                                 (127, 20480), (128, 20480), (128, 20484), (2047, 32768), (2048, 32768),
                                 (2048, 32772), (4, 262144), (4, 262148), (64, 32768), (65, 32768),
                                 (2, 256 * 8192), (2, 256 * 8192 + 4)])
def test_default_plan_at_thresholds(B, V):
    # each side of every edge of the work-split table: rowwise up to 16384
    # columns (but fused for 768..2048 rows of 4096..16384 columns), and up
    # to 32768 columns from 128 rows (20480 columns) or 2048 rows, fused
    # 4096 up to 2^20 elements (2^21 for rows of at most 65536 columns), fused
    # 8192 up to 256 chunks a row
    w = workloads.make(B, V, "quarters" if B >= 4 else "first16384")
    plan = tsv.ts_plan(B, V)
    print(f"[gpu] threshold B={B} V={V} plan={plan}", flush=True)
    y = _run(w.logits, w.temps).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, what=f"B={B} V={V} plan={plan}")
    _no_device_errors()


def _sampled_rows_match(y, w, rows):
    """The oracle on a sample of rows; every row's invariants on the device."""
    got = y[torch.from_numpy(rows).to(y.device)].cpu().numpy()
    assert_softmax_matches(got, w.logits[rows], w.temps[rows], what=f"rows {rows[:4]}...")
    assert bool(torch.isfinite(y).all())
    dev = (y.double().sum(dim=1) - 1.0).abs().max().item()
    assert dev <= 1e-5, dev
    masked = torch.from_numpy(~np.isfinite(w.logits)).to(y.device)
    assert int(torch.count_nonzero(y[masked])) == 0


def test_many_rounds_of_the_persistent_grid():
    # B=1024 rows of 151936: about 19 items per workgroup of the fused grid, so
    # every workgroup waits on rows many times and the slot tags flip on every
    # row; rows are checked against the oracle on a sample, and all rows for
    # finiteness, exact zeros under -inf and their sums
    w = workloads.make(1024, 151936, "quarters")
    assert tsv.ts_plan(w.B, w.V) == (tsv.TS_VARIANT_FUSED, 8192)
    x = torch.from_numpy(w.logits).to(DEV)
    t = torch.from_numpy(w.temps).to(DEV)
    print("[gpu] many rounds B=1024 V=151936", flush=True)
    for rep in range(2):   # twice on one stream: tags carry over between calls
        y = tsv.ts_softmax(x, t)
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(rep).choice(w.B, 24, replace=False))
        rows[0], rows[-1] = 0, w.B - 1
        _sampled_rows_match(y, w, rows)
        del y
    _no_device_errors()


def test_rowwise_many_short_rows():
    # the one-workgroup-per-row kernel at a large batch of short rows
    w = workloads.make(4096, 4096, "none")
    assert tsv.ts_plan(w.B, w.V)[0] == tsv.TS_VARIANT_ROWWISE
    w.logits[::7, :64] = -np.inf    # leading masked columns on some rows
    y = tsv.ts_softmax(torch.from_numpy(w.logits).to(DEV), torch.from_numpy(w.temps).to(DEV))
    torch.cuda.synchronize()
    rows = np.arange(0, w.B, 97)
    _sampled_rows_match(y, w, rows)


@pytest.mark.parametrize("B,V", [(3, 16385), (5, 20000), (2, 32000), (3, 32767), (4, 32768), (2, 32772)])
def test_rowwise_forced_register_edges(B, V):
    # the forced one-workgroup-per-row kernel on each side of its register
    # limits (8 values a lane up to 32768 columns, streamed above), aligned
    # and not, plain and with an allowed-id mask
    w = workloads.make(B, V, "quarters" if B >= 4 else "first16384")
    print(f"[gpu] rowwise forced B={B} V={V}", flush=True)
    y = _run(w.logits, w.temps, tsv.TS_VARIANT_ROWWISE, 0).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, what=f"rowwise B={B} V={V}")
    xm = torch.from_numpy(workloads.unmasked_logits(w)).to(DEV)
    bits = torch.from_numpy(workloads.make_allowed(w).view(np.int32).copy()).to(DEV)
    ym = tsv.ts_softmax_variant(xm, torch.from_numpy(w.temps).to(DEV), tsv.TS_VARIANT_ROWWISE, 0, allowed=bits)
    torch.cuda.synchronize()
    assert_softmax_matches(ym.cpu().numpy(), w.logits, w.temps, what=f"rowwise masked B={B} V={V}")
    _no_device_errors()


def test_extreme_temperatures():
    # a denormal temperature (k = log2(e)/T beyond the float range) gives the
    # one-hot limit, as the float64 definition does; a huge one the uniform
    # limit; both through every split
    rng = np.random.default_rng(41)
    V = 20000
    x = (rng.standard_normal((5, V)) * 4).astype(np.float32)
    x[1, 100:200] = -np.inf
    x[3, 7] = x[3].max() + np.float32(0.5)
    t = np.array([1e-45, 2e-39, 1e-30, 1e30, 3.4e38], np.float32)
    ref = softmax_ref(x, t)
    for v, c in SPLITS:
        y = _run(x, t, v, c).cpu().numpy()
        assert_softmax_matches(y, x, t, ref, what=f"extreme T {v}/{c}")
        for r in (0, 1, 2):
            assert y[r].max() == 1.0 and np.count_nonzero(y[r]) == 1, (v, c, r)
    _no_device_errors()


@pytest.mark.parametrize("n,offset", [(1 << 20, 0), ((1 << 20) + 3, 0), (4099, 1), (1, 0)])
def test_measurement_copy_is_exact(n, offset):
    # the same-bytes copy is the bandwidth ceiling and the counter calibration:
    # it must move exactly n floats, aligned or not, and nothing past them
    src = torch.randn(n + 8, device=DEV)
    dst = torch.full((n + 8,), 7.0, device=DEV)
    tsv.ts_copy_f32(src[offset: offset + n], dst[offset: offset + n])
    torch.cuda.synchronize()
    assert torch.equal(dst[offset: offset + n], src[offset: offset + n])
    assert torch.all(dst[:offset] == 7.0) and torch.all(dst[offset + n:] == 7.0)


def test_memory_params_for_the_recomputed_peak():
    clock_khz, bus_bits = tsv.ts_device_memory_params(DEV)
    assert clock_khz > 0 and bus_bits > 0


@pytest.mark.parametrize("chunk", [1024, 2048])   # 293 chunks per row (row kernel), 147 (each workgroup)
def test_split_rows_of_many_chunks(chunk):
    # Rows of more than 256 chunks have their partials combined once per row
    # by a kernel between the split's two passes; shorter rows combine them in
    # every write workgroup. Rows masked from the start over 100 chunks, over
    # one whole chunk, and everywhere but two ids (one in the last chunk).
    rng = np.random.default_rng(61)
    V = 293 * 1024 - 5
    x = (rng.standard_normal((4, V)) * 4).astype(np.float32)
    NEG = np.float32(-np.inf)
    x[0, :100 * 1024] = NEG
    x[1, 1024: 2 * 1024] = NEG
    x[2, :] = NEG
    x[2, [5000, V - 7]] = [0.5, 1.0]
    t = np.array([0.5, 1.0, 1.3, 0.7], np.float32)
    y = _run(x, t, tsv.TS_VARIANT_SPLIT, chunk).cpu().numpy()
    assert_softmax_matches(y, x, t, what=f"split {chunk}")
    _no_device_errors()


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=SPLIT_IDS)
def test_closed_forms_on_the_gpu(variant, chunk):
    # Closed forms of the definition (test paragraph) applied to the GPU
    # itself, with no oracle in between:
    #  - n equal finite logits (the rest -inf) give exactly 1/n: every
    #    exponential is exp2(0) = 1 and a float sum of at most 2^24 ones is
    #    exact, so each entry is 1/n within one rounding; masked entries are 0;
    #  - two allowed ids give the logistic 1 / (1 + exp((b - a) / T)).
    rng = np.random.default_rng(71)
    V = 3 * 8192 + 389                      # several chunks and a ragged tail at every chunk size
    NEG = np.float32(-np.inf)
    x = np.full((7, V), NEG, np.float32)
    x[0, :] = 2.5                                                   # the whole row
    x[1, rng.choice(V, size=1000, replace=False)] = -3.0            # scattered ids
    x[2, V - 300:] = 7.0                                            # the ragged tail only
    x[3, :100] = 0.0                                                # the first chunk only
    x[4, 12345] = 1.0                                               # a single id
    a, b = 1.75, -0.5
    x[5, [10, V - 10]] = [a, b]                                     # two ids, first and last chunk
    x[6, [2047, 2048]] = [b, a]                                     # two ids across a chunk boundary
    t = np.array([0.5, 1.0, 1.5, 0.7, 1.2, 0.8, 1.3], np.float32)
    y = _run(x, t, variant, chunk).cpu().numpy()
    fin = np.isfinite(x)
    assert np.all(y[~fin] == 0)
    for r in range(5):
        want = np.float32(1.0) / np.float32(fin[r].sum())
        got = y[r, fin[r]]
        assert np.all(np.abs(got - want) <= np.spacing(want)), (r, got.min(), got.max(), want)
    for r, (ia, ib) in ((5, (10, V - 10)), (6, (2048, 2047))):
        pa = 1.0 / (1.0 + np.exp((np.float64(b) - np.float64(a)) / np.float64(t[r])))
        np.testing.assert_allclose(y[r, ia], pa, rtol=1e-5)
        np.testing.assert_allclose(y[r, ib], 1.0 - pa, rtol=1e-5)
