"""fp64 log-sum-exp merge of partial softmax triples -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this module; the product path never imports it.

A triple (m, l, O) summarises a set of keys for one query row in the natural
exp domain: m = max score, l = sum exp(s - m), O = sum exp(s - m) * v (not
divided by l).  Source: kernbench2 page "_gqa_attention_decode_long.py",
function `_merge_running` (new max; each side rescaled by exp(its max - new
max); l and O summed), and its reduce section ("Level-2 row chain",
"Level-1 inter-CUBE reduce" with the 1-D chain and the centre-root mesh
reduce) for the two merge orders.

Reading where the page is silent: the page names the identity (-inf, 0, 0) as
the seed of a single loop but never merges it.  exp(-inf - (-inf)) is NaN, so
a side whose max is -inf gets scale 0; merging two identities gives the
identity.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

Triple = Tuple[float, float, np.ndarray]


def identity(d: int) -> Triple:
    return (-math.inf, 0.0, np.zeros(d, dtype=np.float64))


def merge_pair(local: Triple, other: Triple) -> Triple:
    """The page's `_merge_running(local, other)` in fp64, with the identity guard."""
    m_a, l_a, O_a = local
    m_b, l_b, O_b = other
    m_new = max(m_a, m_b)
    scale_a = 0.0 if m_a == -math.inf else math.exp(m_a - m_new)
    scale_b = 0.0 if m_b == -math.inf else math.exp(m_b - m_new)
    return (m_new, l_a * scale_a + l_b * scale_b, O_a * scale_a + O_b * scale_b)


def finish(t: Triple) -> np.ndarray:
    """Final normalise: O / l (an all-empty triple gives zeros)."""
    m, l, O = t
    if l == 0.0:
        return np.zeros_like(O)
    return O / l


def chain(parts: Sequence[Triple]) -> Triple:
    """1-D chain toward rank 0: the last rank sends west, every other rank merges
    what arrives from the east into its own triple and forwards the result."""
    acc = parts[-1]
    for p in reversed(parts[:-1]):
        acc = merge_pair(p, acc)
    return acc


def _converge_line(parts: Sequence[Triple], root: int) -> Triple:
    """Bidirectional reduce along one line of ranks, converging at index `root`:
    ranks west of the root chain eastward, ranks east of it chain westward, and
    the root merges the western result, then the eastern one, into its own."""
    n = len(parts)
    west = None
    for i in range(0, root):
        west = parts[i] if west is None else merge_pair(parts[i], west)
    east = None
    for i in range(n - 1, root, -1):
        east = parts[i] if east is None else merge_pair(parts[i], east)
    acc = parts[root]
    if west is not None:
        acc = merge_pair(acc, west)
    if east is not None:
        acc = merge_pair(acc, east)
    return acc


def center_root(parts: Sequence[Triple], sub_w: int) -> Triple:
    """Centre-root mesh reduce over a sub_w x sub_h grid (rank = row*sub_w + col):
    phase 1 converges every row at column sub_w//2, phase 2 converges that
    column at row sub_h//2.  Requires sub_w >= 2, sub_h >= 2, sub_w*sub_h == len(parts),
    as the page's launch-argument check does."""
    C = len(parts)
    sub_h = C // sub_w if sub_w else 0
    if sub_w < 2 or sub_h < 2 or sub_w * sub_h != C:
        raise ValueError("centre-root reduce needs sub_w >= 2, sub_h >= 2, sub_w*sub_h == C")
    root_col = sub_w // 2
    root_row = sub_h // 2
    rows: List[Triple] = []
    for r in range(sub_h):
        rows.append(_converge_line(parts[r * sub_w:(r + 1) * sub_w], root_col))
    return _converge_line(rows, root_row)
