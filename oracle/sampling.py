"""Reference temperature / nucleus (top-p) sampling of one position (test infrastructure).

Only the tests use this module; the product path never imports it. The pages name the method
and nothing more: the MoE model's server offers greedy or temperature/top-p generation
("tpu-megakernels README", section "OpenAI-compatible servers"). It is written here from its plain
definition, in float64, by sorting:

- probabilities p = softmax(logits / temperature);
- the nucleus: sort p in descending order and take the shortest prefix whose sum reaches top_p;
  tau is the smallest probability in it, and the kept set is every token with p >= tau (tokens
  tied with tau are all kept, so the kept set does not depend on how ties were ordered);
- the draw: with the caller's uniform number u in [0, 1), the token is the first, in index order,
  at which the running sum of the kept probabilities exceeds u times their total.

The random number is an input: the method draws nothing itself.
"""
from __future__ import annotations

import numpy as np


def probabilities(logits: np.ndarray, temperature: float) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    e = np.exp(z - z.max())
    return e / e.sum()


def nucleus_threshold(p: np.ndarray, top_p: float) -> float:
    """tau: the smallest probability of the shortest descending prefix with mass >= top_p."""
    srt = np.sort(p)[::-1]
    cum = np.cumsum(srt)
    k = int(np.searchsorted(cum, top_p * cum[-1], side="left"))  # first prefix length - 1 reaching it
    return float(srt[min(k, len(srt) - 1)])


def sample(logits: np.ndarray, temperature: float, top_p: float, u: float) -> dict:
    """One position. Returns the token and the pieces a check of another implementation needs:
    the kept mask, the kept mass, tau and the running kept mass before and after the token."""
    p = probabilities(logits, temperature)
    tau = nucleus_threshold(p, top_p)
    kept = p >= tau
    kp = np.where(kept, p, 0.0)
    run = np.cumsum(kp)
    mass = run[-1]
    target = u * mass
    idx = np.nonzero(kept & (run > target))[0]
    tok = int(idx[0]) if len(idx) else int(np.nonzero(kept)[0][-1])
    return {"token": tok, "p": p, "kept": kept, "tau": tau, "mass": mass, "target": target,
            "before": run[tok] - kp[tok], "after": run[tok]}
