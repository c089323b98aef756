"""Seeded synthetic inputs of the accept / rollback step.

Logits stand in for the LM head of the LoopSpec summary's looped models
(rit.work blog): the target rows come from the full-depth verify pass, the
draft rows from shallower states, which the pages describe as already close
to the final distribution.  Here:

* target rows z ~ N(0, sharpness^2) per vocabulary entry;
* draft rows = target row + N(0, draft_noise^2), so drafts agree often but
  not always; the fallback's first draft row (the deeper state) uses half
  that noise, being closer to the final one;
* tokens are drawn from their draft rows by the Gumbel-max trick (arg max of
  z / tau + Gumbel noise), or as arg max of the row for greedy; the
  fallback's first token is drawn from its deeper-state row;
* random words are uniform 32-bit integers.

Nothing here accepts, rejects or forms residuals: that is the method.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

__all__ = ["AcceptInputs", "accept_inputs"]


class AcceptInputs(NamedTuple):
    target: np.ndarray       # float32 [B][2][k+1][V]
    draft: np.ndarray        # float32 [B][2][k][V]
    tokens: np.ndarray       # int32 [B][2][k]
    has_fallback: np.ndarray # uint8 [B]
    rand: np.ndarray         # uint32 [B][2k+1]


def accept_inputs(seed: int, B: int, k: int, V: int, temperature: float, fallback_frac: float = 0.4,
                  sharpness: float = 2.0, draft_noise: float = 0.5) -> AcceptInputs:
    rng = np.random.default_rng(seed)
    target = (rng.standard_normal((B, 2, k + 1, V), dtype=np.float32) * sharpness).astype(np.float32)
    noise = rng.standard_normal((B, 2, k, V), dtype=np.float32) * draft_noise
    noise[:, 1, 0] *= 0.5
    draft = np.empty((B, 2, k, V), np.float32)
    draft[:, :, :] = target[:, :, :k] + noise
    draft[:, 1, 0] = target[:, 0, 0] + noise[:, 1, 0]  # deeper state of position 0 (shared prefix)
    tau = float(np.float32(temperature))
    if tau > 0:
        g = -np.log(-np.log(rng.random((B, 2, k, V))))
        tokens = np.argmax(draft.astype(np.float64) / tau + g, axis=-1).astype(np.int32)
    else:
        tokens = np.argmax(draft, axis=-1).astype(np.int32)
    has_fallback = (rng.random(B) < fallback_frac).astype(np.uint8)
    rand = rng.integers(0, 1 << 32, size=(B, 2 * k + 1), dtype=np.uint64).astype(np.uint32)
    return AcceptInputs(target, draft, tokens, has_fallback, rand)
