"""What the -inf guard changes, shown with a build of the same sources without it.

The pull-request page "fix(kernel): avoid nan in triton sampling softmax when a
chunk starts with -inf" claims two things about its fix:
  * finite rows are bit-identical with and without it (A/B list: every
    autotune config on four finite-row shapes, 48 cases);
  * without it, a column chunk that starts with an all -inf block turns the
    whole row into NaN (bug paragraph; results table: every masked row NaN).
libtsoftmax_noguard.so is built from the same sources with TS_NO_INF_GUARD,
which removes the guard's selects. Here every work split and chunk size of the
library (11) runs on the page's four finite-row shapes (44 cases) in both
builds, bit for bit; and rows masked from a chunk start are finite with the
guard and NaN without it in every chunked split.
"""
import ctypes

import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from temperature_softmax_vocabulary_amd import binding, workloads
from tests.parity import assert_softmax_matches

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SPLITS = [(tsv.TS_VARIANT_SPLIT, c) for c in tsv.CHUNKS] + \
         [(tsv.TS_VARIANT_FUSED, c) for c in tsv.CHUNKS] + [(tsv.TS_VARIANT_ROWWISE, 0)]
IDS = [f"{tsv.VARIANT_NAMES[v]}-{c}" for v, c in SPLITS]
PAGE_SHAPES = [(1, 151936), (4, 151936), (16, 201088), (64, 262144)]   # A/B list and timing table

_noguard = None


def _lib_noguard():
    global _noguard
    if _noguard is None:
        _noguard = binding.load_library(binding.NOGUARD_LIB_PATH)
    return _noguard


def _run(L, x, t, variant, chunk):
    y = torch.empty_like(x)
    st = torch.cuda.current_stream().cuda_stream
    assert L.ts_softmax_variant(x.data_ptr(), t.data_ptr(), None, x.shape[0], x.shape[1], y.data_ptr(),
                                variant, chunk, st) == 0
    torch.cuda.synchronize()
    return y


def _errors(L):
    f = ctypes.c_uint32()
    assert L.ts_device_errors(torch.cuda.current_stream().cuda_stream, ctypes.byref(f)) == 0
    return f.value


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=IDS)
def test_finite_rows_bitwise_identical_with_and_without_guard(variant, chunk):
    for B, V in PAGE_SHAPES:
        w = workloads.make(B, V, "none")            # seed B*7+V, as in the page's A/B script
        x = torch.from_numpy(w.logits).to(DEV)
        t = torch.from_numpy(w.temps).to(DEV)
        a = _run(binding.lib(), x, t, variant, chunk)
        b = _run(_lib_noguard(), x, t, variant, chunk)
        print(f"[gpu] A/B B={B} V={V} {tsv.VARIANT_NAMES[variant]}-{chunk}", flush=True)
        assert torch.equal(a, b), (B, V, variant, chunk)
    assert _errors(_lib_noguard()) == 0


@pytest.mark.parametrize("variant,chunk", [s for s in SPLITS if s[0] != tsv.TS_VARIANT_ROWWISE],
                         ids=[i for s, i in zip(SPLITS, IDS) if s[0] != tsv.TS_VARIANT_ROWWISE])
def test_chunk_start_mask_is_nan_without_guard_and_finite_with_it(variant, chunk):
    B, V = 3, 151936
    w = workloads.make(B, V, "none")
    x = w.logits.copy()
    x[0, :chunk] = -np.inf                 # the first chunk of row 0 is all -inf
    x[1, chunk: 2 * chunk] = -np.inf       # a later chunk of row 1 is all -inf
    xd = torch.from_numpy(x).to(DEV)
    t = torch.from_numpy(w.temps).to(DEV)
    good = _run(binding.lib(), xd, t, variant, chunk).cpu().numpy()
    bad = _run(_lib_noguard(), xd, t, variant, chunk).cpu().numpy()
    assert_softmax_matches(good, x, w.temps, what="guarded")
    assert np.all(np.isnan(bad[0])) and np.all(np.isnan(bad[1])), "masked rows should be NaN without the guard"
    assert np.all(np.isfinite(bad[2])) and np.array_equal(bad[2], good[2]), "the unmasked row is unaffected"
    _errors(_lib_noguard())
