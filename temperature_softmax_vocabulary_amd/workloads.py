"""Seeded synthetic workloads for the temperature softmax and the sampler.

This module only draws random inputs and writes -inf masks. It holds none of
the method's arithmetic and is the one piece of code that both the oracle's
tests and the HIP path's tests/bench use.

Recipe (from the pull-request page "fix(kernel): avoid nan in triton sampling
softmax when a chunk starts with -inf", FreeToken pull request 654):

* A/B script: logits are standard normal times 4, temperatures uniform on
  [0.5, 1.5), and the generator seed for a (B, V) shape is B*7 + V. The page
  uses torch's CUDA generator; a host numpy PCG64 generator with the same
  seed formula and the same distributions stands in for it.
* Results table, masked cases: three mask kinds -- the first 16384 columns
  masked, everything masked except 3 allowed ids, or a 20000-column block
  masked inside the row -- over B in {1, 3, 8} and V in
  {151936, 201088, 262144}.
* Test paragraph: 3 rows of 151936 logits, row 0 with its first 16384
  columns masked, row 1 with all but 3 ids masked, row 2 unmasked, with
  per-row temperatures.

Draw order for every workload: logits, temperatures, masks (row by row),
uniforms. Masked entries are float32 -inf. Every row keeps at least one
finite logit (asserted).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

NEG_INF = np.float32(-np.inf)

# The five workloads the library is measured and checked on. ``masks`` names the
# per-row mask kind; "quarters" means row r takes kind r % 4 from
# (none, first16384, block20000, allowed3).
CONFIGS = {
    "B1_V151936_unmasked": dict(B=1, V=151936, masks="none"),
    "B3_V151936_pr_test_rows": dict(B=3, V=151936, masks="pr_test_rows"),
    "B8_V201088_block_and_head": dict(B=8, V=201088, masks="block_and_head"),
    "B16_V201088_unmasked": dict(B=16, V=201088, masks="none"),
    "B64_V262144_masked_quarters": dict(B=64, V=262144, masks="quarters"),
}
CONFIG_ORDER = list(CONFIGS)

MASK_KINDS = ("none", "first16384", "block20000", "allowed3")
HEAD_COLS = 16384
BLOCK_COLS = 20000
N_ALLOWED = 3


@dataclass
class Workload:
    name: str
    logits: np.ndarray            # [B, V] float32, row-major contiguous
    temps: np.ndarray             # [B] float32
    uniforms: np.ndarray          # [B, K] float32
    seed: int
    row_kinds: list = field(default_factory=list)
    allowed: dict = field(default_factory=dict)   # row -> sorted allowed ids (allowed3 rows)

    @property
    def B(self) -> int:
        return self.logits.shape[0]

    @property
    def V(self) -> int:
        return self.logits.shape[1]


def seed_for(B: int, V: int) -> int:
    """Seed formula of the page's A/B script: B*7 + V."""
    return B * 7 + V


def _apply_mask(rng: np.random.Generator, row: np.ndarray, kind: str, allowed: dict, r: int) -> None:
    V = row.shape[0]
    if kind == "none":
        return
    if kind == "first16384":
        row[: min(HEAD_COLS, V - 1)] = NEG_INF          # keep >= 1 finite logit
        return
    if kind == "block20000":
        w = min(BLOCK_COLS, V - 1)
        off = int(rng.integers(0, V - w + 1))
        row[off: off + w] = NEG_INF
        return
    if kind == "allowed3":
        k = min(N_ALLOWED, V)
        ids = np.sort(rng.choice(V, size=k, replace=False))
        keep = row[ids].copy()
        row[:] = NEG_INF
        row[ids] = keep
        allowed[r] = ids
        return
    raise ValueError(f"unknown mask kind {kind!r}")


def _row_kinds(masks: str, B: int) -> list:
    if masks in MASK_KINDS:
        return [masks] * B
    if masks == "pr_test_rows":
        base = ["first16384", "allowed3", "none"]
        return [base[r % 3] for r in range(B)]
    if masks == "block_and_head":
        # every row: a 20000-column block; even rows also the first 16384 columns
        return ["block_and_head" if r % 2 == 0 else "block20000" for r in range(B)]
    if masks == "quarters":
        return [MASK_KINDS[r % 4] for r in range(B)]
    raise ValueError(f"unknown mask recipe {masks!r}")


def make(B: int, V: int, masks: str = "none", K: int = 64, seed: Optional[int] = None,
         name: Optional[str] = None, scale: float = 4.0) -> Workload:
    """Draw one workload. ``masks`` is a kind from MASK_KINDS or a recipe name."""
    if B < 0 or V < 1 or K < 0:
        raise ValueError("need B >= 0, V >= 1, K >= 0")
    seed = seed_for(B, V) if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((B, V), dtype=np.float32) * np.float32(scale)
    temps = rng.random(B, dtype=np.float32) + np.float32(0.5)
    kinds = _row_kinds(masks, B)
    allowed: dict = {}
    for r, kind in enumerate(kinds):
        if kind == "block_and_head":
            _apply_mask(rng, logits[r], "block20000", allowed, r)
            _apply_mask(rng, logits[r], "first16384", allowed, r)
        else:
            _apply_mask(rng, logits[r], kind, allowed, r)
    if B:
        assert np.all(np.any(np.isfinite(logits), axis=1)), "a row lost every finite logit"
    uniforms = rng.random((B, K), dtype=np.float32)
    return Workload(name=name or f"B{B}_V{V}_{masks}", logits=np.ascontiguousarray(logits),
                    temps=temps, uniforms=uniforms, seed=seed, row_kinds=kinds, allowed=allowed)


def make_config(name: str, K: int = 64) -> Workload:
    c = CONFIGS[name]
    return make(c["B"], c["V"], c["masks"], K=K, name=name)


def pack_allowed(keep: np.ndarray) -> np.ndarray:
    """[B, V] bool -> [B, ceil(V/32)] uint32, bit (j % 32) of word j // 32 = keep[:, j]."""
    B, V = keep.shape
    W = (V + 31) // 32
    pad = np.zeros((B, W * 32), dtype=bool)
    pad[:, :V] = keep
    bits = pad.reshape(B, W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=2).astype(np.uint32)


def make_allowed(w: Workload) -> np.ndarray:
    """The workload's -inf pattern as an allowed-id bitmask (1 = allowed)."""
    return pack_allowed(np.isfinite(w.logits))


def unmasked_logits(w: Workload, seed: int = 0) -> np.ndarray:
    """The workload's logits with every -inf replaced by a fresh finite draw,
    so that the same pattern can be applied through a bitmask instead."""
    rng = np.random.Generator(np.random.PCG64(w.seed ^ 0x5EED ^ seed))
    x = w.logits.copy()
    bad = ~np.isfinite(x)
    x[bad] = rng.standard_normal(int(bad.sum()), dtype=np.float32) * np.float32(4.0)
    return x
