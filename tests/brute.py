"""Brute-force definitions used to pin the oracle on tiny inputs.

Nothing here sorts.  A Top-N set under a total order is found by enumerating
every N-subset and keeping the one whose members all beat every non-member,
which is the defining property of a Top-N selection.  Block keys use exact
rational means (``fractions.Fraction``) and Python's built-in ``round``, whose
ties go to the even integer.
"""
from __future__ import annotations

import itertools
from fractions import Fraction


def block_key_exact(k_seq, B, j, t):
    """Rounded mean (ties to even) of block j's rows visible at position t."""
    rows = [list(map(int, k_seq[p])) for p in range(j * B, min(j * B + B - 1, t) + 1)]
    d = len(rows[0])
    return [round(Fraction(sum(r[c] for r in rows), len(rows))) for c in range(d)]


def dot(a, b):
    return sum(int(x) * int(y) for x, y in zip(a, b))


def beats(a, b):
    """(score, id) pairs: a beats b if its score is higher, or equal with a lower id."""
    return a[0] > b[0] or (a[0] == b[0] and a[1] < b[1])


def top_n_by_enumeration(items, n):
    """items: list of (score, id).  Returns the ids of the unique n-subset whose
    members all beat every other item (all ids if len(items) <= n)."""
    if len(items) <= n:
        return sorted(i for _, i in items)
    found = []
    for subset in itertools.combinations(range(len(items)), n):
        inside = set(subset)
        if all(beats(items[a], items[b]) for a in inside for b in range(len(items)) if b not in inside):
            found.append(sorted(items[a][1] for a in subset))
    assert len(found) == 1, "a total order has exactly one Top-n set"
    return found[0]


def select_brute(q_idx, k_seq, t, B, P, K, tail=0):
    """Pool and Top-K for one query by enumeration (tiny inputs only).
    ``tail`` is the reading of a partial own block: 0 keyed by its visible
    rows, 1 not eligible, 2 keyed by all of its rows in k_seq (future ones
    too).  Candidates are always positions <= t."""
    n_elig = (t + 1) // B if tail == 1 else t // B + 1
    last_row = len(k_seq) - 1 if tail == 2 else t
    blocks = [(dot(q_idx, block_key_exact(k_seq, B, j, last_row)), j) for j in range(n_elig)]
    pool = top_n_by_enumeration(blocks, P)
    cands = [(dot(q_idx, k_seq[p]), p) for j in pool for p in range(j * B, j * B + B) if p <= t]
    return pool, top_n_by_enumeration(cands, K)
