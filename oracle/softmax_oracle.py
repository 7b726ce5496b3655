"""Float64 CPU oracle for the temperature softmax over a vocabulary and for the
inverse-CDF draw that consumes it.

TEST INFRASTRUCTURE. This module is what the tests compare against, not the
product. Only code under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it. The HIP library
never calls it, never links it, and shares no code, table or helper with it;
the product path has no CPU fallback.

It is deliberately plain and slow: numpy float64, one library primitive per
step, no blocking, no chunking, no fusion.

Source: the pull-request page "fix(kernel): avoid nan in triton sampling
softmax when a chunk starts with -inf" (FreeToken pull request 654).

* What is computed (test paragraph of that page): each row b of the logits is
  divided by its own temperature t[b] and passed through a softmax over the
  whole vocabulary, checked there against torch.softmax.
* Masking (bug and fix paragraphs): masked logits are -inf; the result must be
  finite for every row that keeps at least one finite logit, and a masked
  entry's probability is exactly 0.
* Mask producers (scope paragraph): allowed-token-ids, min-tokens and grammar
  masks are what write -inf into the logits. softmax_masked_ref takes such a
  mask as an allowed-id bitmask and applies it as -inf before the softmax.
* Sampling (scope paragraph and the sampling row of the results table): the
  probabilities feed a draw of token ids, and every draw must be an allowed
  (finite-logit) id. The page does not spell out the draw rule; the reading
  taken here is the textbook inverse-CDF rule on caller-supplied uniforms.

Parity pins: every function below is pinned by tests under ``tests/`` that do
not reuse its arithmetic (closed forms, invariants, library routines and brute
force on tiny inputs).
"""
from __future__ import annotations

import numpy as np

__all__ = ["softmax_ref", "sample_ref", "cdf_ref", "check_softmax_inputs", "allowed_bits_to_bool",
           "softmax_masked_ref"]


def check_softmax_inputs(logits: np.ndarray, temps: np.ndarray) -> None:
    """Raise ValueError for inputs outside the method's domain.

    The page guarantees a finite result only for a row that keeps a finite
    logit (fix paragraph); temperatures on the page are positive (its A/B
    script draws them from [0.5, 1.5)). NaN and +inf logits are not part of
    the method; masking is written as -inf only.
    """
    if logits.ndim != 2:
        raise ValueError(f"logits must be [B, V], got shape {logits.shape}")
    if temps.ndim != 1 or temps.shape[0] != logits.shape[0]:
        raise ValueError(f"temps must be [B] with B={logits.shape[0]}, got {temps.shape}")
    if logits.shape[1] < 1:
        raise ValueError("V must be >= 1")
    t = np.asarray(temps, dtype=np.float64)
    if not np.all(np.isfinite(t)) or np.any(t <= 0):
        raise ValueError("every temperature must be finite and > 0")
    x = np.asarray(logits)
    if np.any(np.isnan(x)) or np.any(x == np.inf):
        raise ValueError("logits must be finite or -inf")
    if x.shape[0] and not np.all(np.any(np.isfinite(x), axis=1)):
        raise ValueError("every row needs at least one finite logit")


def softmax_ref(logits: np.ndarray, temps: np.ndarray) -> np.ndarray:
    """probs[b, j] = exp(x[b, j] / t[b]) / sum_i exp(x[b, i] / t[b]), in float64.

    This is the plain definition the page tests against (test paragraph:
    torch.softmax of the temperature-scaled logits, one temperature per row).
    The usual max subtraction is part of the definition's safe evaluation and
    changes nothing mathematically; exp(-inf) is exactly 0, so masked entries
    come out exactly 0 (fix paragraph).

    Args:
      logits: [B, V] array (any float dtype; converted exactly to float64).
      temps:  [B] array of positive temperatures.
    Returns:
      [B, V] float64 probabilities.
    """
    check_softmax_inputs(logits, temps)
    z = np.asarray(logits, dtype=np.float64) / np.asarray(temps, dtype=np.float64)[:, None]
    m = np.max(z, axis=1, keepdims=True)       # finite: each row has a finite logit
    e = np.exp(z - m)                           # -inf - m = -inf -> exactly 0
    s = np.sum(e, axis=1, keepdims=True)        # >= 1 (the max term is exp(0) = 1)
    return e / s


def cdf_ref(probs: np.ndarray) -> np.ndarray:
    """Inclusive cumulative sums C[b, j] = sum_{i <= j} probs[b, i] in float64."""
    p = np.asarray(probs, dtype=np.float64)
    if p.ndim != 2:
        raise ValueError("probs must be [B, V]")
    return np.cumsum(p, axis=1)


def sample_ref(probs: np.ndarray, uniforms: np.ndarray) -> np.ndarray:
    """Inverse-CDF draws: ids[b, k] for uniforms[b, k].

    Reading taken (the page names the draw, not its rule): with the row's
    inclusive CDF C and total C[V-1], a uniform u is clamped to [0, 1] (NaN
    counts as 0), the target is u * C[V-1], and the id is the smallest j with
    C[j] > target. The comparison is strict, so an entry with probability 0
    never owns a target and a masked id is never drawn (results table,
    sampling row: every draw must be an allowed id). If no j qualifies
    (u = 1), the id is the last j with probs[b, j] > 0.

    Args:
      probs:    [B, V] non-negative weights (softmax rows).
      uniforms: [B, K] floats.
    Returns:
      [B, K] int64 ids.
    """
    p = np.asarray(probs, dtype=np.float64)
    u = np.asarray(uniforms, dtype=np.float64)
    if p.ndim != 2 or u.ndim != 2 or u.shape[0] != p.shape[0]:
        raise ValueError("probs must be [B, V] and uniforms [B, K]")
    if np.any(~(p >= 0)):
        raise ValueError("probs must be non-negative and not NaN")
    B, K = u.shape
    ids = np.empty((B, K), dtype=np.int64)
    c = cdf_ref(p)
    for b in range(B):
        nz = np.nonzero(p[b] > 0)[0]
        if nz.size == 0:
            raise ValueError(f"row {b} has no positive probability")
        uc = np.where(np.isnan(u[b]), 0.0, np.clip(u[b], 0.0, 1.0))
        target = uc * c[b, -1]
        j = np.searchsorted(c[b], target, side="right")   # first C[j] > target
        ids[b] = np.where(j < p.shape[1], j, nz[-1])
    return ids


def allowed_bits_to_bool(allowed: np.ndarray, V: int) -> np.ndarray:
    """[B, ceil(V/32)] uint32 words -> [B, V] bool: id j of row b is allowed
    when bit (j % 32) of word j // 32 is 1. Written as the plain per-id rule."""
    w = np.asarray(allowed)
    if w.ndim != 2 or w.dtype != np.uint32 or w.shape[1] != (V + 31) // 32:
        raise ValueError(f"allowed must be uint32 [B, {(V + 31) // 32}]")
    j = np.arange(V)
    return ((w[:, j // 32] >> (j % 32).astype(np.uint32)) & np.uint32(1)).astype(bool)


def softmax_masked_ref(logits: np.ndarray, temps: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """softmax_ref of the logits with every disallowed id set to -inf."""
    x = np.asarray(logits)
    keep = allowed_bits_to_bool(allowed, x.shape[1])
    return softmax_ref(np.where(keep, x, np.float32(-np.inf)), temps)
