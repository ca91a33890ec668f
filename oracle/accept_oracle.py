"""CPU oracle of greedy MTP verify/accept (test infrastructure only).

Only tests, the smoke check and the bench's CPU baseline use this module.
It follows the verify and accept steps of the data-flow trace in "Support
Step3.5/3.7 flash mtp3" (overview, trace of one MTP step, steps 4 and 5):
the target decodes the verify batch [id_last, draft1, ..., draft_{M-1}]
with logits for every row. Row j's logits predict the token after batch
token j. Drafts are accepted while the target's own token at row j equals
draft j+1. The first row that disagrees gives the token that replaces the
draft (the resample). If every draft agrees, the last row gives one more
token. The accepted list is the agreeing drafts followed by that token.
n_accepted counts the agreeing drafts. The hidden state kept for the next
round is the verify row n_accepted (pending_h = verify_h[n_accepted]).

Greedy sampling: the token of a row is the index of its largest logit, the
lower index on ties (reading taken; the pages fix no tie rule). Logits are
taken to be finite.
"""

from __future__ import annotations

import numpy as np


def greedy_token(row) -> int:
    """Index of the largest entry of one row of logits; ties -> lower index."""
    r = np.asarray(row, dtype=np.float64)
    best = int(np.argmax(r))  # argmax returns the first of equal maxima
    return best


def verify_accept(logits, drafts, verify_h=None) -> dict:
    """logits [M][V], drafts [M-1] (draft j+1 at index j), verify_h [M][Hh] or None.

    Returns tokens (greedy token per row), n_accepted, accepted (length
    n_accepted + 1) and pending_h (row n_accepted of verify_h, or None).
    """
    L = np.atleast_2d(np.asarray(logits))
    M = L.shape[0]
    d = [int(t) for t in np.asarray(drafts).reshape(-1)]
    if len(d) != M - 1:
        raise ValueError("need one draft per verify row after the first")
    tokens = [greedy_token(L[j]) for j in range(M)]
    n = 0
    while n < M - 1 and tokens[n] == d[n]:
        n += 1
    accepted = d[:n] + [tokens[n]]
    pending = None
    if verify_h is not None:
        pending = np.array(np.asarray(verify_h)[n], copy=True)
    return dict(tokens=tokens, n_accepted=n, accepted=accepted, pending_h=pending)
