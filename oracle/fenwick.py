"""Fenwick-tree level function of log-linear attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: this package is imported by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``;
the product path never imports it.

Source: log-linear attention write-up (yoousoft.com/industry/3746), section
"special structure: tree partition" (特殊结构：树划分).  The page rejects
levels from absolute position (too coarse for recent tokens) and instead
splits the prefix seen by query t the way a Fenwick tree (树状数组) does:
power-of-two segments, each summarised at the position where it ends, finest
for the most recent tokens, so a query touches O(log T) buckets.  The exact
level function, whose formula the extracted page lost, is taken as
    level(t, s) = 0 if s == t, else 1 + floor(log2(t XOR s)),
i.e. the bit length of t XOR s.

Two independent computations are given so each can pin the other:
``levels`` uses integer bit length of t XOR s; ``fenwick_buckets`` walks the
textbook Fenwick prefix decomposition (strip the lowest set bit).
"""
from __future__ import annotations

import numpy as np


def bit_length(x: np.ndarray) -> np.ndarray:
    """Exact integer bit length of non-negative integers (0 -> 0)."""
    v = np.asarray(x, dtype=np.int64).copy()
    if (v < 0).any():
        raise ValueError("bit_length of a negative integer")
    out = np.zeros(v.shape, dtype=np.int64)
    while v.any():
        out += v > 0
        v >>= 1
    return out


def levels(t, s) -> np.ndarray:
    """Fenwick level of key position s for query position t (s <= t).

    Broadcasts over integer arrays.  Levels of s > t are not defined (the
    mask is causal); callers mask them out.
    """
    t = np.asarray(t, dtype=np.int64)
    s = np.asarray(s, dtype=np.int64)
    return bit_length(np.bitwise_xor(t, s))


def fenwick_buckets(t: int):
    """Textbook Fenwick decomposition of the prefix [0, t] seen by query t.

    Returns a list of ``(level, first, last)`` with inclusive bounds.  Level 0
    is the query position itself.  The remaining prefix [0, t) is split by
    repeatedly removing the lowest set bit of the running end i: the block
    [i - lowbit(i), i) has 2**(level-1) elements, level = log2(lowbit(i)) + 1.
    """
    out = [(0, t, t)]
    i = t
    while i > 0:
        low = i & (-i)
        lev = low.bit_length()  # log2(low) + 1
        out.append((lev, i - low, i - 1))
        i -= low
    return out


def max_level(seqlen: int) -> int:
    """Largest level that occurs in a sequence of length T: ceil(log2 T)."""
    return (max(seqlen, 1) - 1).bit_length()
