"""Brute-force scalar oracle for tiny inputs (pure Python, no NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/paged_attention.py``). It restates
the attention definition one query, one head and one key at a time with
``math.exp`` and ``math.fsum``, and the block pool as the lab page's sorted
free list, so the vectorised oracle can be checked against code with no
shared structure.
"""
from __future__ import annotations

import math


def attention_row(q, keys, values, scale, t):
    """Output and log-sum-exp for one query vector at absolute position ``t``.

    ``keys``/``values`` are lists of vectors (lists of floats), one per key
    position ``0..L-1``; only positions ``j <= t`` take part (lab page,
    ``forward``: causal mask, max-subtracted softmax, weighted sum of V).
    """
    scores = []
    for j, k in enumerate(keys):
        if j <= t:
            scores.append(scale * math.fsum(a * b for a, b in zip(q, k)))
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    z = math.fsum(e)
    d = len(values[0])
    out = [math.fsum(e[j] / z * values[j][c] for j in range(len(e))) for c in range(d)]
    return out, m + math.log(z), [x / z for x in e]


def lab_free_list_model(num_blocks, script):
    """The lab's pool bookkeeping, literally: a sorted Python list, ``pop(0)``
    per block taken, re-sort on release (lab page, ``KVPool``).

    ``script`` is a list of ("take", n) / ("give", [ids]) steps; returns the
    ids taken by each "take" and the final free list.
    """
    free = list(range(num_blocks))
    taken = []
    for op, arg in script:
        if op == "take":
            got = []
            for _ in range(arg):
                got.append(free.pop(0))
            taken.append(got)
        else:
            free = sorted(free + list(arg))
    return taken, free
