"""The Python binding's argument checks, and the library's own alias and size
checks behind it: every malformed call raises ValueError and writes nothing.

The binding only marshals arguments; what it cannot see (overlapping buffers,
an unsupported work split) the C ABI rejects with TS_ERR_INVALID_ARGUMENT
before any launch, which the binding also turns into ValueError.
"""
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
B, V, K = 2, 100, 4


def _x(dtype=torch.float32):
    return torch.randn(B, V, device=DEV, dtype=dtype)


def _t(n=B):
    return torch.ones(n, device=DEV)


def _u(rows=B):
    return torch.rand(rows, K, device=DEV)


def _bits(rows=B, words=(V + 31) // 32, dtype=torch.int32):
    return torch.full((rows, words), -1, dtype=dtype, device=DEV)


CASES = {
    "logits float64": lambda: tsv.ts_softmax(_x(torch.float64), _t()),
    "logits 1-D": lambda: tsv.ts_softmax(torch.randn(V, device=DEV), _t(1)),
    "logits not contiguous": lambda: tsv.ts_softmax(torch.randn(V, B, device=DEV).t(), _t()),
    "logits on the host": lambda: tsv.ts_softmax(torch.randn(B, V), _t()),
    "temps of the wrong length": lambda: tsv.ts_softmax(_x(), _t(B + 1)),
    "out of the wrong shape": lambda: tsv.ts_softmax(_x(), _t(), out=torch.empty(B, V - 1, device=DEV)),
    "out float16": lambda: tsv.ts_softmax(_x(), _t(), out=torch.empty(B, V, device=DEV, dtype=torch.float16)),
    "allowed of the wrong shape": lambda: tsv.ts_softmax_masked(_x(), _t(), _bits(words=3)),
    "allowed float32": lambda: tsv.ts_softmax_masked(_x(), _t(), _bits(dtype=torch.float32)),
    "allowed not a tensor": lambda: tsv.ts_softmax_masked(_x(), _t(), [[-1] * 4] * B),
    "allowed missing": lambda: tsv.ts_softmax_masked(_x(), _t(), None),
    "variant out of range": lambda: tsv.ts_softmax_variant(_x(), _t(), 7, 0),
    "chunk not a multiple of 1024": lambda: tsv.ts_softmax_variant(_x(), _t(), tsv.TS_VARIANT_FUSED, 1000),
    "chunk of 32768": lambda: tsv.ts_softmax_variant(_x(), _t(), tsv.TS_VARIANT_SPLIT, 32768),
    "uniforms of the wrong rows": lambda: tsv.ts_sample(_x(), _u(B + 1)),
    "uniforms float64": lambda: tsv.ts_sample(_x(), _u().double()),
    "out_ids int64": lambda: tsv.ts_sample(_x(), _u(), out_ids=torch.empty(B, K, dtype=torch.int64, device=DEV)),
    "out_ids of the wrong shape": lambda: tsv.ts_softmax_sample(
        _x(), _t(), _u(), out_ids=torch.empty(B, K + 1, dtype=torch.int32, device=DEV)),
    "probs_out of the wrong shape": lambda: tsv.ts_softmax_sample(
        _x(), _t(), _u(), probs_out=torch.empty(B + 1, V, device=DEV)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_malformed_call_raises_value_error(name):
    with pytest.raises(ValueError):
        CASES[name]()


def test_overlapping_buffers_are_refused_before_any_write():
    # out overlapping the logits other than exactly (in place), or the
    # temperatures: the library refuses before launching anything
    buf = torch.randn(4 * B * V, device=DEV)
    x = buf[: B * V].view(B, V)
    shifted = buf[V: V + B * V].view(B, V)
    before = buf.clone()
    with pytest.raises(ValueError):
        tsv.ts_softmax(x, _t(), out=shifted)
    t_in_out = buf[2 * B * V: 2 * B * V + B]
    out = buf[2 * B * V: 3 * B * V].view(B, V)
    with pytest.raises(ValueError):
        tsv.ts_softmax(x, t_in_out, out=out)
    with pytest.raises(ValueError):   # out_ids inside the uniforms
        u = torch.rand(B * K * 2, device=DEV)
        tsv.ts_sample(x, u[: B * K].view(B, K), out_ids=u[B * K // 2: B * K // 2 + B * K].view(torch.int32).view(B, K))
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    # in place is allowed and normalises the rows
    y = tsv.ts_softmax(x, _t(), out=x)
    torch.cuda.synchronize()
    assert torch.allclose(y.sum(dim=1).double(), torch.ones(B, dtype=torch.float64, device=DEV), atol=1e-5)
