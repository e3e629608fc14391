"""Reference greedy selection and draft acceptance for the tests (plain definitions, host only).

A verify step's new tokens are an anchor followed by drafts; draft j is accepted while it equals
the target's greedy token at the position before it, for every draft up to it. The step then
yields the accepted drafts plus the target's greedy token after them."""
import numpy as np


def greedy_tokens(logits: np.ndarray) -> np.ndarray:
    """[..., V] -> [...] index of the largest logit, the lowest index on ties."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def accepted_drafts(tokens: np.ndarray, greedy: np.ndarray) -> np.ndarray:
    """tokens, greedy: [B][T]. Number of drafts (tokens[b][1:]) accepted per sequence."""
    B, T = tokens.shape
    out = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n + 1 < T and tokens[b, n + 1] == greedy[b, n]:
            n += 1
        out[b] = n
    return out
