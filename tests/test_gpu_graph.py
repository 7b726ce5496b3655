"""HIP-graph capture of ts_softmax and ts_sample, replayed with fresh inputs.

Pattern: capture once into static buffers, then several replays, each with new
inputs copied in and checked against the oracle, with eager work and
synchronisations between the replays. The workspace is reserved before the
capture so that the captured calls allocate nothing.
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


@pytest.mark.parametrize("variant,chunk", [(tsv.TS_VARIANT_AUTO, 0), (tsv.TS_VARIANT_SPLIT, 4096),
                                           (tsv.TS_VARIANT_FUSED, 8192), (tsv.TS_VARIANT_ROWWISE, 0)])
def test_capture_and_replay_softmax_then_sample(variant, chunk):
    B, V, K = 16, 201088, 64
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(B, V, device=DEV, stream=s)
    x = torch.zeros((B, V), dtype=torch.float32, device=DEV)
    t = torch.ones((B,), dtype=torch.float32, device=DEV)
    u = torch.zeros((B, K), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        # warm-up on the capture stream, outside capture
        tsv.ts_softmax_variant(x, t, variant, chunk, out=y) if variant else tsv.ts_softmax(x, t, out=y)
        tsv.ts_sample(y, u, out_ids=ids)
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        if variant:
            tsv.ts_softmax_variant(x, t, variant, chunk, out=y)
        else:
            tsv.ts_softmax(x, t, out=y)
        tsv.ts_sample(y, u, out_ids=ids)
    for rep in range(3):
        w = workloads.make(B, V, "quarters", K=K, seed=1000 + rep)
        x.copy_(torch.from_numpy(w.logits))
        t.copy_(torch.from_numpy(w.temps))
        u.copy_(torch.from_numpy(w.uniforms))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert_softmax_matches(got, w.logits, w.temps, what=f"replay {rep}")
        assert_ids_valid(ids.cpu().numpy(), got, w.uniforms, what=f"replay {rep}")
        # eager work between replays
        _ = (x * 2).sum().item()
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0


@pytest.mark.parametrize("B,V", [(8, 4096), (128, 20480)])
def test_capture_short_rows_softmax_and_draw_with_probs(B, V):
    # shapes the work-split table gives the row kernel: ts_softmax runs it (no
    # workspace), the with-probabilities draw runs the fused split (workspace
    # rows and partials); the reservation alone, with no call on the stream
    # before the capture, must cover both
    K = 16
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(B, V, device=DEV, stream=s)
    x = torch.zeros((B, V), dtype=torch.float32, device=DEV)
    t = torch.ones((B,), dtype=torch.float32, device=DEV)
    u = torch.zeros((B, K), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    yp = torch.empty_like(x)
    ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tsv.ts_softmax(x, t, out=y)
        tsv.ts_softmax_sample(x, t, u, out_ids=ids, probs_out=yp)
    for rep in range(3):
        w = workloads.make(B, V, "quarters", K=K, seed=2000 + rep)
        x.copy_(torch.from_numpy(w.logits))
        t.copy_(torch.from_numpy(w.temps))
        u.copy_(torch.from_numpy(w.uniforms))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_softmax_matches(y.cpu().numpy(), w.logits, w.temps, what=f"rowwise replay {rep}")
        got = yp.cpu().numpy()
        assert_softmax_matches(got, w.logits, w.temps, what=f"with-probs replay {rep}")
        assert_ids_valid(ids.cpu().numpy(), got, w.uniforms, what=f"with-probs replay {rep}")
        _ = (x * 2).sum().item()
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0


# the refused call launches nothing, so the graph torch captures is empty (by design)
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
@pytest.mark.parametrize("variant,chunk", [(tsv.TS_VARIANT_FUSED, 8192), (tsv.TS_VARIANT_SPLIT, 2048)])
def test_capture_without_reserve_is_refused(variant, chunk):
    # a fresh stream has no workspace: a captured call must not allocate one
    B, V = 8, 300000
    s = torch.cuda.Stream(device=DEV)
    x = torch.zeros((B, V), dtype=torch.float32, device=DEV)
    t = torch.ones((B,), dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=s):
        try:
            tsv.ts_softmax_variant(x, t, variant, chunk)
        except tsv.TsError as e:
            err = e
    assert err is not None and err.status == tsv.TS_ERR_NOT_RESERVED


def test_graph_survives_later_workspace_growth():
    # A graph captured on a stream keeps pointing at that stream's workspace.
    # A later, larger eager call on the same stream grows the workspace; the
    # outgrown one stays allocated, so the graph's replays still run on it,
    # interleaved with eager calls on the new one.
    B, V, K = 8, 201088, 16
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(B, V, device=DEV, stream=s)
    x = torch.zeros((B, V), dtype=torch.float32, device=DEV)
    t = torch.ones((B,), dtype=torch.float32, device=DEV)
    u = torch.zeros((B, K), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    ids = torch.empty((B, K), dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        tsv.ts_softmax(x, t, out=y)
        tsv.ts_sample(y, u, out_ids=ids)
    s.synchronize()
    with torch.cuda.graph(g, stream=s):
        tsv.ts_softmax(x, t, out=y)
        tsv.ts_sample(y, u, out_ids=ids)
    big = workloads.make(64, 262144, "quarters", seed=7)
    xb, tb = torch.from_numpy(big.logits).to(DEV), torch.from_numpy(big.temps).to(DEV)
    for rep in range(3):
        # a larger call on the capture stream: the first one grows its workspace
        with torch.cuda.stream(s):
            yb = tsv.ts_softmax(xb, tb, stream=s)
        s.synchronize()
        assert_softmax_matches(yb.cpu().numpy(), big.logits, big.temps, what=f"eager {rep}")
        w = workloads.make(B, V, "quarters", K=K, seed=2000 + rep)
        x.copy_(torch.from_numpy(w.logits))
        t.copy_(torch.from_numpy(w.temps))
        u.copy_(torch.from_numpy(w.uniforms))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert_softmax_matches(got, w.logits, w.temps, what=f"replay {rep}")
        assert_ids_valid(ids.cpu().numpy(), got, w.uniforms, what=f"replay {rep}")
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0


def test_capture_split_with_row_combine():
    # rows of more than 256 chunks: the split runs three kernels (partials,
    # one row-combine workgroup per row, write); all three are captured
    B, V, chunk = 3, 293 * 1024 - 5, 1024
    s = torch.cuda.Stream(device=DEV)
    tsv.ts_reserve(B, V, device=DEV, stream=s)
    x = torch.zeros((B, V), dtype=torch.float32, device=DEV)
    t = torch.ones((B,), dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    with torch.cuda.stream(s):
        tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_SPLIT, chunk, out=y)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        tsv.ts_softmax_variant(x, t, tsv.TS_VARIANT_SPLIT, chunk, out=y)
    for rep in range(3):
        w = workloads.make(B, V, "first16384", seed=700 + rep)
        x.copy_(torch.from_numpy(w.logits))
        t.copy_(torch.from_numpy(w.temps))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_softmax_matches(y.cpu().numpy(), w.logits, w.temps, what=f"replay {rep}")
        _ = (x * 2).sum().item()   # eager work between replays
    assert tsv.ts_device_errors(device=DEV, stream=s) == 0
