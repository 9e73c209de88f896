"""Bucket composition of a prompt -- TEST INFRASTRUCTURE ONLY (as the rest of ``oracle``).

guanjiawei.ai "AIMA AMD395 Qwen3.6-35B-A3B": the data-path section says any
prompt is decomposed into optimised 8192-token tiles, 1024-token tiles and a
tail; the runtime section says the process keeps 1024/2048/4096/8192-token
buckets resident, covers each prompt with the smallest bucket total and pads
only the final segment when no exact composition exists.

Reading (the pages fix the smallest total; the rest is the plainest rule that
makes the answer unique): among the covers with that total, the fewest
segments; among those, the lexicographically largest sequence when the
segments are listed largest first.  Segments are listed largest first, so the
only partial one is the last.

Written as a brute force over every count vector of bucket sizes: slow and
plain, for small T.
"""
from __future__ import annotations

import itertools
from typing import List, Sequence, Tuple


def bucket_plan(T: int, buckets: Sequence[int]) -> Tuple[List[int], List[int]]:
    """(segment bucket sizes, real tokens per segment) covering T tokens."""
    if T < 0:
        raise ValueError("T < 0")
    if T == 0:
        return [], []
    bs = sorted(set(int(b) for b in buckets), reverse=True)
    if len(bs) != len(buckets) or bs[-1] < 1:
        raise ValueError("bucket sizes must be positive and distinct")
    best = None
    # a cover with more than ceil(T / b) buckets of size b is not of smallest total
    ranges = [range(-(-T // b) + 1) for b in bs]
    for counts in itertools.product(*ranges):
        total = sum(c * b for c, b in zip(counts, bs))
        if total < T:
            continue
        seq = [b for b, c in zip(bs, counts) for _ in range(c)]
        key = (total, len(seq), [-v for v in seq])
        if best is None or key < best[0]:
            best = (key, seq)
    seq = best[1]
    lens, left = [], T
    for b in seq:
        lens.append(min(left, b))
        left -= lens[-1]
    return seq, lens
