"""The largest calls: the longest row the boundary accepts (V = 2^31 - 1) and
calls of more than 2^31 elements, through the fused, split and draw kernels.

At these sizes the float64 oracle cannot take whole rows, so the checks are
properties the definition fixes at any size (pull-request page "fix(kernel):
avoid nan in triton sampling softmax when a chunk starts with -inf", test
paragraph for the definition, bug and fix paragraphs for masked chunks):
  - every output is finite, and masked entries are exactly 0;
  - every row sums to 1 (float64 sum of the float32 outputs);
  - for ids i, j of one row p_i / p_j = exp((x_i - x_j) / T), checked in
    float64 on the row's logits within 5 T of its max (where the exponent's
    rounding error is smallest, whatever the row's length);
  - each drawn id has a finite logit and holds its target in the row's CDF,
    taken in float64 from the logits with torch's own operations (u = 0, 1
    and two inside), up to the worst-case band tests/parity.py derives: the
    draw's float32 sums plus the float32 exponents' error, weighted by the
    row's probabilities (E_p[|d|], computed here the same way).
Inputs are drawn on the device by torch's seeded generator (normal * 4,
temperatures in [0.5, 1.5), seed B * 7 + V), with the masks of the pages'
workloads: the first 16384 columns of row 0, a 20000-column block of the last
row. The with-probabilities draw must write exactly ts_softmax's
probabilities, and an all-ones allowed mask must change nothing.
"""
import math

import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from tests.parity import LN2, SAMPLE_TAU, U32, gamma

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RATIO_RTOL = 2e-5   # two probabilities, each within the 1e-5 gate


def _inputs(B, V):
    g = torch.Generator(device=DEV)
    g.manual_seed(B * 7 + V)
    x = torch.randn((B, V), generator=g, device=DEV).mul_(4.0)
    t = torch.rand((B,), generator=g, device=DEV).add_(0.5)
    x[0, :16384] = -math.inf
    off = V // 3
    x[B - 1, off: off + 20000] = -math.inf
    return x, t, off


def _check_rows(x, t, y, off, rows):
    B, V = x.shape
    assert bool(torch.isfinite(y).all())
    assert bool((y[0, :16384] == 0).all()) and bool((y[B - 1, off: off + 20000] == 0).all())
    sums = y.sum(dim=1, dtype=torch.float64).cpu().numpy()
    assert np.max(np.abs(sums - 1.0)) <= 1e-5, sums
    for r in rows:
        T = float(t[r])
        xmax = float(x[r].max())
        top = torch.nonzero(x[r] >= xmax - 5.0 * T).flatten()[:64]   # within e^-5 of the row's max
        xs = x[r, top].double().cpu().numpy()
        ps = y[r, top].double().cpu().numpy()
        i, j = np.meshgrid(np.arange(len(xs)), np.arange(len(xs)))
        assert len(xs) >= 2 and np.all(ps > 0)
        np.testing.assert_allclose(ps[i] / ps[j], np.exp((xs[i] - xs[j]) / T), rtol=RATIO_RTOL)


def _mass(xr, T, xmax, lo, hi, step=1 << 27):
    """sum of exp((x_j - xmax) / T) over j in [lo, hi), float64, in slices (torch ops)."""
    tot = 0.0
    for a in range(lo, hi, step):
        b = min(hi, a + step)
        tot += float(torch.exp((xr[a:b].double() - xmax) / T).sum())
    return tot


def _mean_log2_distance(xr, T, xmax, total, step=1 << 27):
    """E_p[|d|] of the row: sum of p_j (xmax - x_j) log2(e) / T, float64, in slices."""
    acc = 0.0
    for a in range(0, xr.shape[0], step):
        z = (xr[a:a + step].double() - xmax) / T
        fin = torch.isfinite(z)
        acc += float((torch.exp(torch.where(fin, z, -math.inf)) * torch.where(fin, -z, 0.0)).sum())
    return acc / total * math.log2(math.e)


def _check_draws(x, t, ids, us, rows, from_logits):
    # each id has a finite logit and holds its target u * C[V-1] in the exact
    # CDF up to the row's band tau: C[id - 1] - tau <= u <= C[id] + tau (C
    # normalised to 1). Drawn from the written probabilities: their float32
    # error plus the draw's sums; straight from the logits: the ids-only band.
    V = x.shape[1]
    for r in rows:
        xr, T = x[r], float(t[r])
        xmax = float(xr.max())
        total = _mass(xr, T, xmax, 0, V)
        e = _mean_log2_distance(xr, T, xmax, total)
        if from_logits:
            tau = (gamma(12) + gamma(6)) / 2 + 3 * LN2 * U32 * e + 5 * U32
        else:
            tau = SAMPLE_TAU + 3 * LN2 * U32 * e + 7 * U32
        for k, u in enumerate(us):
            j = int(ids[r, k])
            assert 0 <= j < V and bool(torch.isfinite(xr[j])), (r, k, j)
            before = _mass(xr, T, xmax, 0, j) / total
            upto = before + math.exp((float(xr[j]) - xmax) / T) / total
            assert before - tau <= u <= upto + tau, (r, u, j, before, upto)


@pytest.mark.parametrize("B,V", [
    (1, 2**31 - 1),     # the longest row: 131072 chunks, split; V % 4 = 3 (unaligned rows)
    (513, 4194304),     # 2.15e9 elements; fused at 16384 columns, ~256 items per workgroup
    (5, 2**29 + 5),     # 2.68e9 elements; split; offsets past 2^31 elements
])
def test_largest_calls(B, V):
    print(f"[gpu] large call B={B} V={V} plan={tsv.ts_plan(B, V)}", flush=True)
    x, t, off = _inputs(B, V)
    y = tsv.ts_softmax(x, t)
    rows = sorted({0, B // 2, B - 1})
    _check_rows(x, t, y, off, rows)
    us = [0.0, 1.0, 0.5, 0.999]
    u = torch.tensor([us], device=DEV).repeat(B, 1)
    _check_draws(x, t, tsv.ts_sample(y, u).cpu(), us, rows, from_logits=False)
    _check_draws(x, t, tsv.ts_softmax_sample(x, t, u)[0].cpu(), us, rows, from_logits=True)
    # the draw that also writes the probabilities writes ts_softmax's, bit for bit
    ids3, p3 = tsv.ts_softmax_sample(x, t, u, probs_out=True)
    assert torch.equal(p3, y)
    _check_draws(x, t, ids3.cpu(), us, rows, from_logits=False)
    del p3
    # an all-ones allowed mask (2^26 words per row at the longest) changes nothing
    ones = torch.full((B, (V + 31) // 32), -1, dtype=torch.int32, device=DEV)
    assert torch.equal(tsv.ts_softmax_masked(x, t, ones), y)
    assert tsv.ts_device_errors() == 0
    del y
    torch.cuda.empty_cache()
