"""The fused kernel's partial exchange across calls, and its bounded wait.

The fused kernel keeps per-row tagged slots in the stream's workspace from one
call to the next (their parity tag flips every call). These tests change the
chunk count per row, the row count and the vocabulary between calls on one
stream and check every result against the oracle. They also force the bounded
wait to run out from the host (a one-poll limit): the kernel then forms the
missing chunk partials from the logits itself, so every such call must give
the bits of a call whose waits never ran out (for every chunk size, unaligned
rows, an allowed-id mask, in place, and with the draw's sums), the library
must report the slow path, and the next call must be clean. No kernel faults
or hangs in any of them: a timed-out wait always finishes the row.
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


def _case(B, V, seed):
    w = workloads.make(B, V, "quarters", seed=seed)
    return w, torch.from_numpy(w.logits).to(DEV), torch.from_numpy(w.temps).to(DEV)


def test_slot_tags_survive_changing_shapes_on_one_stream():
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(32, 262144, device=DEV, stream=s)
    seq = [(8, 151936, 4096), (8, 151936, 16384), (32, 201088, 1024), (3, 262144, 2048),
           (32, 201088, 8192), (8, 151936, 4096), (1, 20000, 1024), (32, 262144, 16384)]
    with torch.cuda.stream(s):
        for i, (B, V, chunk) in enumerate(seq):
            w, x, t = _case(B, V, 77 + i)
            y = tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_FUSED, chunk)
            s.synchronize()
            print(f"[gpu] call {i}: B={B} V={V} chunk={chunk}", flush=True)
            assert_softmax_matches(y.cpu().numpy(), w.logits, w.temps, what=f"call {i}")
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0


def _timeouts(s):
    """1 if a wait on stream s ran out since the last check, else 0."""
    try:
        tsv.ts_device_errors(device=DEV, stream=s)
        return 0
    except tsv.TsError as e:
        assert e.status == tsv.TS_ERR_SYNC_TIMEOUT
        return 1


def test_forced_wait_timeout_gives_the_exact_result_and_is_reported():
    w, x, t = _case(64, 262144, 5)
    u = torch.from_numpy(w.uniforms).to(DEV)
    xm = torch.from_numpy(workloads.unmasked_logits(w)).to(DEV)
    bits = torch.from_numpy(workloads.make_allowed(w).view(np.int32).copy()).to(DEV)
    wo, xo, to = _case(8, 151937, 6)   # V % 4 = 1: unaligned rows
    ref = softmax_ref(w.logits, w.temps)
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(64, 262144, device=DEV, stream=s)

    def calls():
        with torch.cuda.stream(s):
            out = {f"fused {c}": tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_FUSED, c) for c in (4096, 8192, 16384)}
            out["masked 8192"] = tsv.ts_softmax_variant(xm, t, tsv.TS_VARIANT_FUSED, 8192, allowed=bits)
            out["unaligned 4096"] = tsv.ts_softmax_variant(xo, to, tsv.TS_VARIANT_FUSED, 4096)
            y = x.clone()
            tsv.ts_softmax_variant(y, t, tsv.TS_VARIANT_FUSED, 8192, out=y)
            out["in place 8192"] = y
            ids, yp = tsv.ts_softmax_sample(x, t, u, probs_out=True)
            out["with draw sums"], out["draw ids"] = yp, ids
        s.synchronize()
        return out

    clean = calls()
    assert _timeouts(s) == 0
    seen = 0
    try:
        tsv.ts_debug_set_spin_limit(1)
        for rep in range(2):
            got = calls()
            seen += _timeouts(s)
            for name, y in got.items():
                print(f"[gpu] one-poll limit, call {rep}: {name}", flush=True)
                assert torch.equal(y, clean[name]), f"{name}: differs from the call whose waits never ran out"
    finally:
        tsv.ts_debug_set_spin_limit(0)
    assert seen >= 1, "a one-poll wait limit never ran out"
    for name in ("fused 8192", "in place 8192", "with draw sums"):
        assert_softmax_matches(got[name].cpu().numpy(), w.logits, w.temps, ref, what=name)
    assert_ids_valid(got["draw ids"].cpu().numpy(), got["with draw sums"].cpu().numpy(), w.uniforms)
    # and the next calls run clean
    with torch.cuda.stream(s):
        y = tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_FUSED, 4096)
        y2 = tsv.ts_softmax(x, t)
    s.synchronize()
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0
    assert torch.equal(y, clean["fused 4096"]) and torch.equal(y2, clean["fused 8192"])


def test_two_streams_have_independent_workspaces():
    w1, x1, t1 = _case(16, 201088, 1)
    w2, x2, t2 = _case(16, 201088, 2)
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            a = tsv.ts_softmax_variant(x1, t1, tsv.TS_VARIANT_FUSED, 8192)
        with torch.cuda.stream(s2):
            b = tsv.ts_softmax_variant(x2, t2, tsv.TS_VARIANT_FUSED, 8192)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert_softmax_matches(a.cpu().numpy(), w1.logits, w1.temps, what="stream 1")
        assert_softmax_matches(b.cpu().numpy(), w2.logits, w2.temps, what="stream 2")
    assert tsv.ts_device_errors(device=DEV, stream=s1) == 0
    assert tsv.ts_device_errors(device=DEV, stream=s2) == 0


def test_fused_rejects_rows_with_too_many_chunks():
    # 300000 columns at 1024 per chunk is 293 chunks: more than the 256 slots a row has
    x = torch.zeros((1, 300000), dtype=torch.float32, device=DEV)
    t = torch.ones((1,), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_FUSED, 1024)
    y = tsv.ts_softmax(x, t)          # the default plan picks a legal split
    torch.cuda.synchronize()
    assert np.allclose(y.cpu().numpy(), 1.0 / 300000, rtol=1e-6)



F8, F16 = (tsv.TS_VARIANT_FUSED, 8192), (tsv.TS_VARIANT_FUSED, 16384)


@pytest.mark.parametrize("cap,plan", [
    (0, F8),          # the device's own capacity (1024 workgroups of 8192 columns on MI355X)
    (48, F8),         # 48 workgroups loop over 2048 items
    (32, F8),         # exactly one row's 32 chunks resident: the smallest legal grid
    (31, F16),        # a row of 8192-column chunks no longer fits: 16 chunks of 16384
    (16, F16),
    (15, (tsv.TS_VARIANT_SPLIT, 16384)),   # nothing fused fits: the split pair, which never waits
])
def test_plan_and_grid_follow_the_resident_capacity(cap, plan):
    # A device that holds fewer workgroups at once (simulated from the host by
    # lowering the capacity the planner counts on; the grid still fits the
    # real device) must never get a fused grid that cannot hold a whole row.
    w, x, t = _case(64, 262144, 11)
    u = torch.from_numpy(w.uniforms).to(DEV)
    try:
        tsv.ts_debug_set_resident_cap(cap)
        assert tsv.ts_plan(64, 262144) == plan
        if 0 < cap < 32:
            with pytest.raises(ValueError):
                tsv.ts_softmax_variant(x, t, *F8)
        y = tsv.ts_softmax(x, t)
        ids, yp = tsv.ts_softmax_sample(x, t, u, probs_out=True)
        torch.cuda.synchronize()
    finally:
        tsv.ts_debug_set_resident_cap(0)
    print(f"[gpu] resident cap {cap}: plan {plan}", flush=True)
    # the per-item arithmetic does not depend on the grid: bitwise the same as
    # the same split on the full device
    assert torch.equal(y, tsv.ts_softmax_variant(x, t, *plan))
    ref = softmax_ref(w.logits, w.temps)
    assert_softmax_matches(y.cpu().numpy(), w.logits, w.temps, ref, what=f"cap {cap}")
    assert_softmax_matches(yp.cpu().numpy(), w.logits, w.temps, ref, what=f"cap {cap} with draw")
    assert_ids_valid(ids.cpu().numpy(), yp.cpu().numpy(), w.uniforms, what=f"cap {cap}")
    assert tsv.ts_device_errors() == 0


def test_concurrent_full_grids_on_two_streams():
    # Two calls whose grids each fill the device (B=64 x 262144: 1024
    # workgroups apiece), issued on two streams at once, ten times. Their
    # workgroups may share the device; every row must still complete (no
    # bounded wait runs out) and give the single-stream result bit for bit.
    w, x1, t = _case(64, 262144, 9)
    x2 = x1.clone()
    ref = tsv.ts_softmax(x1, t)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(64, 262144, device=DEV, stream=s1)
    tsv.ts_reserve(64, 262144, device=DEV, stream=s2)
    for it in range(10):
        a = tsv.ts_softmax(x1, t, stream=s1)
        b = tsv.ts_softmax(x2, t, stream=s2)
        torch.cuda.synchronize()
        assert tsv.ts_device_errors(device=DEV, stream=s1) == 0, it
        assert tsv.ts_device_errors(device=DEV, stream=s2) == 0, it
        assert torch.equal(a, ref) and torch.equal(b, ref), it
