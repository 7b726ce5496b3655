"""The seeded input generator follows the recipe it states (host only)."""
import numpy as np
import pytest

from temperature_softmax_vocabulary_amd import workloads


def test_seed_formula_and_determinism():
    a = workloads.make_config("B3_V151936_pr_test_rows")
    b = workloads.make_config("B3_V151936_pr_test_rows")
    assert a.seed == 3 * 7 + 151936
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.temps, b.temps)
    assert np.array_equal(a.uniforms, b.uniforms)


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_config_shapes_dtypes_and_ranges(name):
    w = workloads.make_config(name)
    c = workloads.CONFIGS[name]
    assert w.logits.shape == (c["B"], c["V"]) and w.logits.dtype == np.float32
    assert w.logits.flags["C_CONTIGUOUS"]
    assert w.temps.dtype == np.float32 and np.all((w.temps >= 0.5) & (w.temps < 1.5))
    assert w.uniforms.shape == (c["B"], 64) and np.all((w.uniforms >= 0) & (w.uniforms < 1))
    fin = np.isfinite(w.logits)
    assert np.all(fin.any(axis=1))
    assert not np.any(np.isnan(w.logits)) and not np.any(w.logits == np.inf)
    # unmasked entries are N(0,1)*4 draws
    vals = w.logits[fin]
    assert abs(vals.std() - 4.0) < 0.1 and abs(vals.mean()) < 0.1


def test_pr_test_rows_layout():
    w = workloads.make_config("B3_V151936_pr_test_rows")
    fin = np.isfinite(w.logits)
    assert not fin[0, :16384].any() and fin[0, 16384:].all()
    assert fin[1].sum() == 3 and sorted(np.nonzero(fin[1])[0]) == list(w.allowed[1])
    assert fin[2].all()


def test_block_and_head_layout():
    w = workloads.make_config("B8_V201088_block_and_head")
    for r in range(8):
        masked = ~np.isfinite(w.logits[r])
        if r % 2 == 0:
            assert masked[:16384].all()
        # a contiguous 20000-column run exists
        runs = np.diff(np.concatenate([[0], masked.astype(np.int8), [0]]))
        starts, ends = np.nonzero(runs == 1)[0], np.nonzero(runs == -1)[0]
        assert (ends - starts).max() >= 20000


def test_quarters_layout():
    w = workloads.make_config("B64_V262144_masked_quarters")
    fin = np.isfinite(w.logits)
    for r in range(64):
        kind = workloads.MASK_KINDS[r % 4]
        n_masked = (~fin[r]).sum()
        expect = {"none": 0, "first16384": 16384, "block20000": 20000, "allowed3": 262144 - 3}[kind]
        assert n_masked == expect, (r, kind)
