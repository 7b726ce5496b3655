"""GPU parity of the allowed-id bitmask applied while the logits are read.

The pull-request page "fix(kernel): avoid nan in triton sampling softmax when a
chunk starts with -inf" names the producers of -inf logits: allowed-token-ids,
min-tokens and grammar masks (scope paragraph). ts_softmax_masked takes such a
mask as bits and treats a disallowed id exactly as a -inf logit. Checked here:
against the float64 oracle (softmax_masked_ref), and bit for bit against the
same work split run on logits with the -inf already written, for every split;
plus one allowed id at word boundaries, odd V, misaligned pointers, and the
one-pass softmax-and-draw with a mask (every id drawn is allowed).
"""
import numpy as np
import pytest
import torch

import temperature_softmax_vocabulary_amd as tsv
from oracle import softmax_masked_ref, softmax_ref
from temperature_softmax_vocabulary_amd import workloads
from tests.parity import assert_ids_valid, assert_logit_ids_valid, assert_softmax_matches

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SPLITS = [(tsv.TS_VARIANT_SPLIT, c) for c in tsv.CHUNKS] + \
         [(tsv.TS_VARIANT_FUSED, c) for c in tsv.CHUNKS] + [(tsv.TS_VARIANT_ROWWISE, 0)]
IDS = [f"{tsv.VARIANT_NAMES[v]}-{c}" for v, c in SPLITS]


def _bits(keep_or_bits):
    a = keep_or_bits if keep_or_bits.dtype == np.uint32 else workloads.pack_allowed(keep_or_bits)
    return torch.from_numpy(a.view(np.int32).copy()).to(DEV)


def _case(name):
    w = workloads.make_config(name)
    return w, workloads.unmasked_logits(w), workloads.make_allowed(w)


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_configs_masked_matches_oracle_and_premasked(name):
    w, x, bits = _case(name)
    ref = softmax_masked_ref(x, w.temps, bits)
    xd, td, bd = torch.from_numpy(x).to(DEV), torch.from_numpy(w.temps).to(DEV), _bits(bits)
    y = tsv.ts_softmax_masked(xd, td, bd)
    y_pre = tsv.ts_softmax(torch.from_numpy(w.logits).to(DEV), td)
    torch.cuda.synchronize()
    print(f"[gpu] masked {name}", flush=True)
    assert_softmax_matches(y.cpu().numpy(), w.logits, w.temps, ref, what=name)
    assert torch.equal(y, y_pre), "masking at load must equal -inf written beforehand"
    assert tsv.ts_device_errors() == 0


@pytest.mark.parametrize("variant,chunk", SPLITS, ids=IDS)
def test_every_split_masked_equals_premasked(variant, chunk):
    for name in ("B3_V151936_pr_test_rows", "B64_V262144_masked_quarters"):
        w, x, bits = _case(name)
        td = torch.from_numpy(w.temps).to(DEV)
        y = tsv.ts_softmax_variant(torch.from_numpy(x).to(DEV), td, variant, chunk, allowed=_bits(bits))
        y_pre = tsv.ts_softmax_variant(torch.from_numpy(w.logits).to(DEV), td, variant, chunk)
        torch.cuda.synchronize()
        assert torch.equal(y, y_pre), (name, variant, chunk)
    assert tsv.ts_device_errors() == 0


@pytest.mark.parametrize("V", [151936, 151937, 100, 33])
def test_single_allowed_id_at_word_boundaries(V):
    ids = sorted({0, 1, 31, 32, 33, 63, 64, V - 2, V - 1} & set(range(V)))
    B = len(ids)
    x = (np.random.default_rng(V).standard_normal((B, V)) * 4).astype(np.float32)
    keep = np.zeros((B, V), bool)
    keep[np.arange(B), ids] = True
    t = np.full(B, 0.9, np.float32)
    for variant, chunk in SPLITS:
        y = tsv.ts_softmax_variant(torch.from_numpy(x).to(DEV), torch.from_numpy(t).to(DEV), variant, chunk,
                                   allowed=_bits(keep)).cpu().numpy()
        assert np.array_equal(y, keep.astype(np.float32)), (V, variant, chunk)


def test_misaligned_logits_with_mask():
    w, x, bits = _case("B8_V201088_block_and_head")
    B, V = x.shape
    base = torch.empty(B * V + 1, dtype=torch.float32, device=DEV)
    xd = base[1:].view(B, V)
    xd.copy_(torch.from_numpy(x))
    y = tsv.ts_softmax_masked(xd, torch.from_numpy(w.temps).to(DEV), _bits(bits)).cpu().numpy()
    assert_softmax_matches(y, w.logits, w.temps, what="misaligned masked")


def test_mask_and_inf_logits_combine():
    # ids masked by the bits and ids already -inf in the logits both give 0
    w = workloads.make(16, 201088, "quarters", seed=9)
    rng = np.random.default_rng(9)
    keep = rng.random(w.logits.shape) < 0.7
    keep[:, 16384 + 7] = True                         # keep a finite id in every row
    x = w.logits.copy()
    x[:, 16384 + 7] = 1.0
    ref = softmax_masked_ref(x, w.temps, workloads.pack_allowed(keep))
    y = tsv.ts_softmax_masked(torch.from_numpy(x).to(DEV), torch.from_numpy(w.temps).to(DEV), _bits(keep)).cpu().numpy()
    assert_softmax_matches(y, np.where(keep, x, -np.inf).astype(np.float32), w.temps, ref, what="combined")


def test_softmax_sample_with_mask_draws_only_allowed_ids():
    w, x, bits = _case("B64_V262144_masked_quarters")
    ref = softmax_ref(w.logits, w.temps)
    xd, td = torch.from_numpy(x).to(DEV), torch.from_numpy(w.temps).to(DEV)
    ids, probs = tsv.ts_softmax_sample(xd, td, torch.from_numpy(w.uniforms).to(DEV), probs_out=True,
                                       allowed=_bits(bits))
    torch.cuda.synchronize()
    p = probs.cpu().numpy()
    assert_softmax_matches(p, w.logits, w.temps, ref, what="masked softmax_sample")
    ids = ids.cpu().numpy()
    assert_ids_valid(ids, p, w.uniforms, what="masked draw")
    keep = np.isfinite(w.logits)
    assert np.all(keep[np.arange(w.B)[:, None], ids])


def test_ids_only_draw_with_mask_draws_only_allowed_ids():
    # the draw straight from the logits applies the bits in both of its kernels
    # (group and block partials, then the chosen block's entries)
    for name in ("B3_V151936_pr_test_rows", "B64_V262144_masked_quarters"):
        w, x, bits = _case(name)
        ref = softmax_ref(w.logits, w.temps)
        ids, none = tsv.ts_softmax_sample(torch.from_numpy(x).to(DEV), torch.from_numpy(w.temps).to(DEV),
                                          torch.from_numpy(w.uniforms).to(DEV), allowed=_bits(bits))
        torch.cuda.synchronize()
        assert none is None
        ids = ids.cpu().numpy()
        assert_logit_ids_valid(ids, w.logits, w.temps, w.uniforms, ref, what=f"{name} ids only, masked")
        assert np.all(np.isfinite(w.logits)[np.arange(w.B)[:, None], ids])
