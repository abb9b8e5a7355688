"""50-digit decimal brute force of GQA decode for tiny inputs -- TEST INFRASTRUCTURE.

Only the test suite and the script that writes tests/golden/ use this module.
It computes the same plain definition as oracle.c (softmax of scale * q.k_t over
the keys of a sequence, applied to its V rows; query head h reads kv head
h // G), but in Python's decimal arithmetic with 50 significant digits and a
correctly rounded exp, so that it pins the fp64 oracle to within its own
rounding.  Every input is converted exactly (bf16 bits, fp16 or fp32 -> float -> Decimal).

Source: kernbench2 page "_gqa_attention_decode_long.py", "Tile 0" block over all
keys and the final normalise-and-store block.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np


def _exact(a: np.ndarray):
    if a.dtype == np.uint16:
        f = (a.astype(np.uint32) << 16).view(np.float32)
    elif a.dtype in (np.float32, np.float16):
        f = a
    else:
        raise TypeError(a.dtype)
    return [[Decimal(float(x)) for x in row] for row in f.reshape(-1, f.shape[-1])]


def brute_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_lens, scale: float,
                 digits: int = 50):
    """Returns a nested list [batch][h_q][d] of Decimal outputs; for q of shape
    [batch, t_q, h_q, d], [batch][t_q][h_q][d] with query token t seeing keys
    0 .. S - t_q + t."""
    if q.ndim == 4:
        return _brute_tq(q, k, v, seq_lens, scale, digits)
    batch, h_q, d = q.shape
    h_kv = k.shape[1]
    G = h_q // h_kv
    qd = _exact(q)            # rows indexed b*h_q + h
    kd = _exact(k)            # rows indexed row*h_kv + j
    vd = _exact(v)
    out = []
    with localcontext() as ctx:
        ctx.prec = digits
        sc = Decimal(float(scale))
        base = 0
        for b in range(batch):
            S = max(int(seq_lens[b]), 0)
            ob = []
            for h in range(h_q):
                j = h // G
                if S == 0:
                    ob.append([Decimal(0)] * d)
                    continue
                qrow = qd[b * h_q + h]
                s = []
                for t in range(S):
                    krow = kd[(base + t) * h_kv + j]
                    s.append(sc * sum(qi * ki for qi, ki in zip(qrow, krow)))
                m = max(s)
                w = [(x - m).exp() for x in s]
                l = sum(w)
                o = []
                for i in range(d):
                    o.append(sum(w[t] * vd[(base + t) * h_kv + j][i] for t in range(S)) / l)
                ob.append(o)
            out.append(ob)
            base += S
    return out


def _brute_tq(q, k, v, seq_lens, scale, digits):
    batch, t_q, h_q, d = q.shape
    out = []
    base = 0
    for b in range(batch):
        S = max(int(seq_lens[b]), 0)
        ob = []
        for t in range(t_q):
            St = min(S, max(0, S - t_q + t + 1))
            # query token t alone against the first St keys of its sequence
            r = brute_decode(q[b:b + 1, t], k[base:base + St], v[base:base + St], [St], scale, digits)
            ob.append(r[0])
        out.append(ob)
        base += S
    return out
