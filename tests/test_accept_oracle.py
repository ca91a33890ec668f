"""Pins of the verify/accept oracle (CPU), each independent of its code.

* The worked example of the pages' MTP trace (tests/golden/accept_trace.txt).
* Closed cases: every draft right, the first draft wrong, a mismatch at a
  chosen row, equal maxima (lower index), a vocabulary permutation.
* The greedy token against a brute-force scan on random rows.
* Planted mistakes in a copy of the oracle are caught by these pins.
"""

import os

import numpy as np
import pytest

from oracle import accept_oracle as ao

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "accept_trace.txt")


def _read_trace():
    kv = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                kv[line[0]] = [int(t) for t in line[1:]]
    return kv


def _onehot_logits(tokens, V):
    L = np.zeros((len(tokens), V), dtype=np.float32)
    for j, t in enumerate(tokens):
        L[j, t] = 1.0
    return L


def _pins(fn):
    """Run every pin against `fn` (same signature as verify_accept)."""
    kv = _read_trace()
    V = kv["vocab"][0]
    L = _onehot_logits(kv["row_argmax"], V)
    H = np.arange(4 * 8, dtype=np.float32).reshape(4, 8)
    r = fn(L, kv["drafts"], H)
    assert r["n_accepted"] == kv["expect_n_accepted"][0]
    assert r["accepted"] == kv["expect_accepted"]
    assert np.array_equal(r["pending_h"], H[kv["expect_pending_row"][0]])
    assert r["accepted"][-1] == 44  # the token carried into the next round is T_new

    rng = np.random.default_rng(3)
    for M in (1, 2, 3, 4, 7):
        toks = [int(t) for t in rng.integers(0, 50, M)]
        H = rng.standard_normal((M, 5)).astype(np.float32)
        # Every draft right: all accepted, plus the last row's own token.
        r = fn(_onehot_logits(toks, 50), toks[:-1], H)
        assert r["n_accepted"] == M - 1 and r["accepted"] == toks
        assert np.array_equal(r["pending_h"], H[M - 1])
        if M > 1:
            # The first draft wrong: nothing accepted, the resample is row 0's token.
            bad = [(toks[0] + 1) % 50] + toks[1:-1]
            r = fn(_onehot_logits(toks, 50), bad, H)
            assert r["n_accepted"] == 0 and r["accepted"] == [toks[0]]
            assert np.array_equal(r["pending_h"], H[0])
            # A mismatch at row j accepts j drafts; later rows do not matter.
            for j in range(M - 1):
                dr = toks[:j] + [(toks[j] + 7) % 50] + [toks[i] for i in range(j + 1, M - 1)]
                r = fn(_onehot_logits(toks, 50), dr, H)
                assert r["n_accepted"] == j and r["accepted"] == toks[:j + 1]
                assert np.array_equal(r["pending_h"], H[j])

    # Equal maxima: the lower index wins.
    L = np.zeros((2, 10), dtype=np.float32)
    L[0, [3, 7]] = 2.5
    L[1, [9, 1]] = -0.5
    L[1, [0, 2, 3, 4, 5, 6, 7, 8]] = -1.0
    r = fn(L, [3], None)
    assert r["tokens"] == [3, 1] and r["n_accepted"] == 1 and r["accepted"] == [3, 1]

    # Permuting the vocabulary permutes the tokens.
    L = rng.standard_normal((4, 40)).astype(np.float32)
    perm = rng.permutation(40)
    inv = np.argsort(perm)
    base = fn(L, [1, 2, 3], None)
    Lp = L[:, inv]  # column c of Lp is column inv[c] of L: token t of L is token perm[t] of Lp
    rp = fn(Lp, [int(perm[t]) for t in (1, 2, 3)], None)
    assert rp["tokens"] == [int(perm[t]) for t in base["tokens"]]
    assert rp["n_accepted"] == base["n_accepted"]

    # Greedy token of random rows vs a brute-force scan.
    for _ in range(20):
        row = rng.integers(-3, 4, 33).astype(np.float32)  # many equal maxima
        best, idx = -np.inf, -1
        for i, v in enumerate(row.tolist()):
            if v > best:
                best, idx = v, i
        r = fn(row[None, :], [], None)
        assert r["tokens"] == [idx]


def test_oracle_meets_the_pins():
    _pins(ao.verify_accept)


def _m_ties_high(logits, drafts, verify_h=None):
    L = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    M = L.shape[0]
    toks = [int(L.shape[1] - 1 - np.argmax(L[j, ::-1])) for j in range(M)]
    n = 0
    while n < M - 1 and toks[n] == drafts[n]:
        n += 1
    return dict(tokens=toks, n_accepted=n, accepted=list(drafts[:n]) + [toks[n]],
                pending_h=None if verify_h is None else np.asarray(verify_h)[n])


def _m_pending_off_by_one(logits, drafts, verify_h=None):
    r = ao.verify_accept(logits, drafts, verify_h)
    if verify_h is not None:
        r["pending_h"] = np.asarray(verify_h)[max(r["n_accepted"] - 1, 0)]
    return r


def _m_keeps_accepting(logits, drafts, verify_h=None):
    r = ao.verify_accept(logits, drafts, None)
    toks = r["tokens"]
    n = sum(1 for j in range(len(drafts)) if toks[j] == drafts[j])
    r["n_accepted"] = n
    r["accepted"] = [d for j, d in enumerate(drafts) if toks[j] == d] + [toks[n]]
    r["pending_h"] = None if verify_h is None else np.asarray(verify_h)[n]
    return r


def _m_resample_is_draft(logits, drafts, verify_h=None):
    r = ao.verify_accept(logits, drafts, verify_h)
    n = r["n_accepted"]
    if n < len(drafts):
        r["accepted"] = list(drafts[:n + 1])
    return r


@pytest.mark.parametrize("mutant", [_m_ties_high, _m_pending_off_by_one, _m_keeps_accepting,
                                    _m_resample_is_draft])
def test_planted_mistake_is_caught(mutant):
    with pytest.raises(AssertionError):
        _pins(mutant)
