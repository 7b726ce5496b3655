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
from tests.parity import assert_ids_valid, assert_softmax_matches

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
    assert_softmax_matches(yw.cpu().numpy(), x, t, ref, what=f"{what} with draw")
    p32 = ref.astype(np.float32)
    for ids, w in ((ids_p, "sample"), (ids_l, "ids only"), (ids_w, "with probs")):
        assert_ids_valid(ids.cpu().numpy(), p32, u, what=f"{what} {w}")
        assert np.all(np.isfinite(x)[np.arange(B)[:, None], ids.cpu().numpy()]), f"{what} {w}"
    assert tsv.ts_device_errors() == 0
