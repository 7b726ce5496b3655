"""Seeded random cases against the float64 oracle.

Each case draws a shape (B up to 70, V from 1 to 300000, odd and even, rows
aligned or not), temperatures over two decades, and per-row masks from the
families that matter to the method (pull-request page "fix(kernel): avoid nan
in triton sampling softmax when a chunk starts with -inf", bug and fix
paragraphs): -inf over whole chunks of every chunk size, from a chunk start,
around the row's last columns, a few allowed ids, or none. Every case runs the
default plan, one forced work split, the allowed-id bitmask path, and both draw
modes. The cases are fixed by their seeds, so a failure names its case.
"""
import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from oracle import softmax_ref
from temperature_softmax_vocabulary_amd import workloads
from tests.parity import assert_ids_valid, assert_logit_ids_valid, assert_softmax_matches

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SPLITS = [(tsv.TS_VARIANT_SPLIT, c) for c in tsv.CHUNKS] + \
         [(tsv.TS_VARIANT_FUSED, c) for c in tsv.CHUNKS] + [(tsv.TS_VARIANT_ROWWISE, 0)]
N_CASES = 48
MAX_ELEMS = 2_000_000   # keeps each float64 oracle call well under a second


def _case(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.choice([1, 2, 3, 5, 63, 1023, 1024, 4097, 16383, 16384, 16385])) if rng.random() < 0.3 \
        else int(rng.integers(1, 300001))
    B = int(rng.integers(1, max(2, min(70, MAX_ELEMS // V)) + 1))
    x = (rng.standard_normal((B, V)) * rng.choice([1.0, 4.0, 20.0])).astype(np.float32)
    NEG = np.float32(-np.inf)
    for r in range(B):
        kind = rng.integers(0, 7)
        if kind == 1 and V > 1:     # whole chunks of a random chunk size, from their start
            C = int(rng.choice(tsv.CHUNKS))
            for c0 in range(0, V, C):
                if rng.random() < 0.5:
                    x[r, c0: min(V, c0 + C)] = NEG
        elif kind == 2 and V > 1:   # from a chunk start to a random end
            c0 = int(rng.choice(tsv.CHUNKS)) * int(rng.integers(0, 4))
            c0 = min(c0, V - 1)
            x[r, c0: int(rng.integers(c0 + 1, V + 1))] = NEG
        elif kind == 3 and V > 4:   # around the row's last columns (the partial float4)
            x[r, V - int(rng.integers(1, 5)):] = NEG
        elif kind == 4:             # a few allowed ids
            keep = rng.choice(V, size=min(V, int(rng.integers(1, 4))), replace=False)
            vals = x[r, keep].copy()
            x[r, :] = NEG
            x[r, keep] = vals
        elif kind == 5 and V > 1:   # everything but the last column
            x[r, :V - 1] = NEG
        if not np.isfinite(x[r]).any():
            x[r, int(rng.integers(0, V))] = np.float32(rng.standard_normal())
    t = (10.0 ** rng.uniform(-1.3, 1.0, size=B)).astype(np.float32)
    K = int(rng.integers(1, 70))
    u = rng.random((B, K), dtype=np.float32)
    split = SPLITS[int(rng.integers(0, len(SPLITS)))]
    offset = bool(rng.random() < 0.3)   # rows 4 bytes past a 16-byte boundary
    return x, t, u, split, offset


def _dev(a, offset):
    if not offset:
        return torch.from_numpy(a).to(DEV)
    base = torch.empty(a.size + 4, dtype=torch.float32, device=DEV)
    d = base[1: 1 + a.size].view(a.shape)
    d.copy_(torch.from_numpy(a))
    return d


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    x, t, u, (variant, chunk), offset = _case(seed)
    B, V = x.shape
    print(f"[gpu] random case {seed}: B={B} V={V} split={variant}/{chunk} offset={offset}", flush=True)
    ref = softmax_ref(x, t)
    xd, td, ud = _dev(x, offset), torch.from_numpy(t).to(DEV), torch.from_numpy(u).to(DEV)
    y = tsv.ts_softmax(xd, td)
    fused_ok = not (variant == tsv.TS_VARIANT_FUSED and -(-V // chunk) > 256)
    ys = tsv.ts_softmax_variant(xd, td, variant, chunk) if fused_ok else None
    bits = workloads.pack_allowed(np.isfinite(x)).view(np.int32)
    xm = np.where(np.isfinite(x), x, np.float32(0.0)).astype(np.float32)
    ym = tsv.ts_softmax_masked(_dev(xm, offset), td, torch.from_numpy(bits).to(DEV))
    ids_p = tsv.ts_sample(y, ud)
    ids_l, _ = tsv.ts_softmax_sample(xd, td, ud)
    ids_w, yw = tsv.ts_softmax_sample(xd, td, ud, probs_out=True)
    torch.cuda.synchronize()
    what = f"case {seed} B={B} V={V}"
    got = y.cpu().numpy()
    assert_softmax_matches(got, x, t, ref, what=what)
    if ys is not None:
        assert_softmax_matches(ys.cpu().numpy(), x, t, ref, what=f"{what} split {variant}/{chunk}")
    assert torch.equal(ym, y), what   # bitmask = -inf in the logits, bit for bit
    ywh = yw.cpu().numpy()
    assert_softmax_matches(ywh, x, t, ref, what=f"{what} with draw")
    assert_ids_valid(ids_p.cpu().numpy(), got, u, what=f"{what} sample")
    assert_ids_valid(ids_w.cpu().numpy(), ywh, u, what=f"{what} with probs")
    assert_logit_ids_valid(ids_l.cpu().numpy(), x, t, u, ref, what=f"{what} ids only")
    for ids, w in ((ids_p, "sample"), (ids_l, "ids only"), (ids_w, "with probs")):
        assert np.all(np.isfinite(x)[np.arange(B)[:, None], ids.cpu().numpy()]), f"{what} {w}"
    assert tsv.ts_device_errors() == 0


def _many_rows_case(seed):
    """Many short rows and many draws: B up to 2048 (around the 768..2048 rows
    that take the fused split for 4096..16384 columns), V up to 20000,
    K up to 1100 (the resolve that shares level 1 across a row's targets)."""
    rng = np.random.default_rng(10_000 + seed)
    V = int(rng.choice([4096, 4097, 8191, 8192, 12000, 16384, 16383])) if rng.random() < 0.5 \
        else int(rng.integers(1, 20001))
    B = int(rng.choice([767, 768, 1024, 2048, 2049])) if rng.random() < 0.4 else int(rng.integers(1, 2049))
    B = max(1, min(B, 4_000_000 // V))
    x = (rng.standard_normal((B, V)) * rng.choice([1.0, 4.0])).astype(np.float32)
    NEG = np.float32(-np.inf)
    kinds = rng.integers(0, 5, size=B)
    for r in np.nonzero(kinds == 1)[0]:                      # masked from the start
        x[r, : int(rng.integers(1, V + 1))] = NEG
    for r in np.nonzero(kinds == 2)[0]:                      # three allowed ids
        keep = rng.choice(V, size=min(V, 3), replace=False)
        vals = x[r, keep].copy()
        x[r, :] = NEG
        x[r, keep] = vals
    for r in np.nonzero(kinds == 3)[0]:                      # the row's last columns
        x[r, V - int(rng.integers(1, min(V, 5) + 1)):] = NEG
    x[~np.isfinite(x).any(axis=1), 0] = 1.0
    t = (10.0 ** rng.uniform(-1.0, 0.7, size=B)).astype(np.float32)
    K = int(rng.choice([1, 16, 64, 300, 1100]))
    return x, t, rng.random((B, K), dtype=np.float32)


@pytest.mark.parametrize("seed", range(16))
def test_random_many_rows_case(seed):
    x, t, u = _many_rows_case(seed)
    B, V = x.shape
    what = f"many-rows case {seed} B={B} V={V} K={u.shape[1]} plan={tsv.ts_plan(B, V)}"
    print(f"[gpu] {what}", flush=True)
    ref = softmax_ref(x, t)
    xd, td, ud = (torch.from_numpy(a).to(DEV) for a in (x, t, u))
    y = tsv.ts_softmax(xd, td)
    bits = workloads.pack_allowed(np.isfinite(x)).view(np.int32)
    xm = np.where(np.isfinite(x), x, np.float32(0.0)).astype(np.float32)
    ym = tsv.ts_softmax_masked(torch.from_numpy(xm).to(DEV), td, torch.from_numpy(bits).to(DEV))
    ids = tsv.ts_sample(y, ud)
    ids2, yp = tsv.ts_softmax_sample(xd, td, ud, probs_out=True)
    ids3, _ = tsv.ts_softmax_sample(xd, td, ud)
    torch.cuda.synchronize()
    yh, yph = y.cpu().numpy(), yp.cpu().numpy()
    assert_softmax_matches(yh, x, t, ref, what=what)
    assert torch.equal(ym, y), what
    assert_softmax_matches(yph, x, t, ref, what=f"{what} with draw")
    assert_ids_valid(ids.cpu().numpy(), yh, u, what=f"{what} sample")
    assert_ids_valid(ids2.cpu().numpy(), yph, u, what=f"{what} with probs")
    assert_logit_ids_valid(ids3.cpu().numpy(), x, t, u, ref, what=f"{what} ids only")
    assert tsv.ts_device_errors() == 0
