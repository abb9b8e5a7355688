"""fp64 CPU oracle for grouped-query-attention decode -- TEST INFRASTRUCTURE.

Only the test suite (tests/), the smoke check (__graft_entry__.smoke) and the
benchmark's CPU-baseline leg (bench.py) may import this package.  The product
path -- the HIP library in gqa_split_kv_amd/ and its Python binding -- never
imports, loads or calls anything here, and this package imports nothing from
it.  The two share no code.

Contents
  gqa_decode_f64     direct softmax(scale * q K^T) V per query head (oracle.c)
  gqa_prefill_f64    causal prefill: every token of a sequence as a query over
                     its own prefix (the multi-token rule with t_q = S)
  gqa_prefill_rows_f64  chosen rows of gqa_prefill_f64, one token at a time
  softmax_weights    the normalised weights of one (sequence, head)
  partial_f64        the (m, l, O) triple of one (sequence, head) over a key range
  merge              (merge.py) the log-sum-exp merge of two triples, and the
                     chain / centre-root merge orders
  brute              (brute.py) 50-digit decimal brute force for tiny inputs

Source: kernbench2 page "_gqa_attention_decode_long.py": the "Tile 0" block
(one tile over all keys), `_merge_running`, and the final normalise-and-store
block.  Readings where that page is silent are listed in oracle.c's header.

Inputs are numpy arrays: bf16 tensors travel as their raw bits in uint16
arrays (dtype code 0), fp32 tensors as float32 arrays (dtype code 1), IEEE fp16
tensors as float16 arrays (dtype code 2).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

BF16 = 0
F32 = 1
F16 = 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.oracle_gqa_decode_f64.argtypes = [P, P, P, P, i32, i32, i32, i32, ctypes.c_double, i32, P]
    lib.oracle_gqa_decode_f64.restype = ctypes.c_int
    lib.oracle_gqa_decode_tq_f64.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_double,
                                             i32, P]
    lib.oracle_gqa_decode_tq_f64.restype = ctypes.c_int
    lib.oracle_softmax_weights_f64.argtypes = [P, P, P, i32, i32, i32, i32, ctypes.c_double, i32,
                                               i32, i32, P]
    lib.oracle_softmax_weights_f64.restype = ctypes.c_int
    lib.oracle_partial_f64.argtypes = [P, P, P, P, i32, i32, i32, i32, ctypes.c_double, i32, i32,
                                       i32, i32, i32, P, P, P]
    lib.oracle_partial_f64.restype = ctypes.c_int
    lib.oracle_widen_f64.argtypes = [P, ctypes.c_int64, i32, P]
    lib.oracle_widen_f64.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all host cores)."""
    return int(_load().oracle_num_threads())


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise TypeError("oracle inputs are uint16 (bf16 bits), float16 or float32, got %s" % a.dtype)


def widen(a: np.ndarray) -> np.ndarray:
    """The exact widening to float64 the oracle applies to its inputs."""
    a = np.ascontiguousarray(a)
    out = np.empty(a.shape, dtype=np.float64)
    _load().oracle_widen_f64(_ptr(a), a.size, _dtype_code(a), _ptr(out))
    return out


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _prep(q, k, v, seq_lens):
    """Single-query inputs: q [batch, h_q, d]."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v) if v is not None else None
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    code = _dtype_code(q)
    if _dtype_code(k) != code or (v is not None and _dtype_code(v) != code):
        raise TypeError("q, k, v must share one dtype")
    if q.ndim != 3:
        raise ValueError("q must be [batch, h_q, d]")
    batch, h_q, d = q.shape
    if k.ndim != 3 or k.shape[2] != d:
        raise ValueError("k must be [sum(seq_lens), h_kv, d]")
    h_kv = k.shape[1]
    total = int(np.clip(sl, 0, None).sum())
    if k.shape[0] < total or (v is not None and v.shape != k.shape):
        raise ValueError("k/v hold fewer rows than sum(seq_lens), or differ in shape")
    if sl.shape != (batch,):
        raise ValueError("seq_lens must be [batch]")
    return q, k, v, sl, code, batch, h_q, h_kv, d


def gqa_decode_f64(q, k, v, seq_lens, scale: float) -> np.ndarray:
    """o[b, h, :] = softmax(scale * q[b,h] K_j^T) V_j, j = h // (h_q // h_kv); float64.

    With q of shape [batch, t_q, h_q, d] (t_q query tokens per sequence, the last
    t_q key rows being theirs) query token t sees keys 0 .. S - t_q + t and the
    result is [batch, t_q, h_q, d]."""
    q = np.ascontiguousarray(q)
    if q.ndim == 4:
        batch, t_q, h_q, d = q.shape
        _, k, v, sl, code, _, _, h_kv, _ = _prep(q.reshape(batch, t_q * h_q, d), k, v, seq_lens)
        out = np.empty((batch, t_q, h_q, d), dtype=np.float64)
        rc = _load().oracle_gqa_decode_tq_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), batch, t_q, h_q,
                                              h_kv, d, float(scale), code, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_gqa_decode_tq_f64 failed (%d)" % rc)
        return out
    q, k, v, sl, code, batch, h_q, h_kv, d = _prep(q, k, v, seq_lens)
    out = np.empty((batch, h_q, d), dtype=np.float64)
    rc = _load().oracle_gqa_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), batch, h_q, h_kv, d,
                                       float(scale), code, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_gqa_decode_f64 failed (%d)" % rc)
    return out


def gqa_prefill_f64(q, k, v, seq_lens, scale: float) -> np.ndarray:
    """Causal prefill, float64: q, k, v packed [sum(S), heads, d]; row base_b + t,
    head h = softmax over keys 0 .. t of sequence b (the multi-token decode of
    gqa_decode_f64 with t_q = S_b: the query tokens are the sequence itself).
    Source: kernbench2 page "_gqa_attention_decode_long.py", commit description
    (prefill panel, T_q = S_kv); the causal rule is this package's reading."""
    q = np.ascontiguousarray(q)
    sl = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, None)
    if q.ndim != 3 or q.shape[0] != int(sl.sum()):
        raise ValueError("q must be [sum(seq_lens), h_q, d]")
    out = np.zeros(q.shape, dtype=np.float64)
    base = 0
    for S in sl:
        S = int(S)
        if S:
            qb = np.ascontiguousarray(q[base:base + S])[None]
            out[base:base + S] = gqa_decode_f64(qb, k[base:base + S], v[base:base + S], [S], scale)[0]
        base += S
    return out


def gqa_prefill_rows_f64(q, k, v, seq_lens, scale: float, tokens) -> np.ndarray:
    """Rows `tokens` (indices into the packed token axis) of gqa_prefill_f64, each
    computed as a single-token decode of that token over its sequence's keys
    0 .. itself; float64 [len(tokens), h_q, d]."""
    sl = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, None)
    ends = np.cumsum(sl)
    out = np.empty((len(tokens),) + tuple(q.shape[1:]), dtype=np.float64)
    for n, r in enumerate(tokens):
        r = int(r)
        b = int(np.searchsorted(ends, r, side="right"))
        base = int(ends[b] - sl[b])
        t = r - base
        qr = np.ascontiguousarray(q[r:r + 1])
        out[n] = gqa_decode_f64(qr, k[base:base + t + 1], v[base:base + t + 1], [t + 1], scale)[0]
    return out


def softmax_weights(q, k, seq_lens, scale: float, b: int, h: int) -> np.ndarray:
    """Normalised softmax weights of sequence b, query head h (float64[seq_lens[b]])."""
    q, k, _, sl, code, batch, h_q, h_kv, d = _prep(q, k, None, seq_lens)
    w = np.zeros(max(int(sl[b]), 0), dtype=np.float64)
    rc = _load().oracle_softmax_weights_f64(_ptr(q), _ptr(k), _ptr(sl), batch, h_q, h_kv, d,
                                            float(scale), code, b, h, _ptr(w) if w.size else None)
    if rc != 0:
        raise ValueError("oracle_softmax_weights_f64 failed (%d)" % rc)
    return w


def partial_f64(q, k, v, seq_lens, scale: float, b: int, h: int, t0: int, t1: int):
    """(m, l, O) of sequence b, head h over keys [t0, t1) in the natural-exp domain."""
    q, k, v, sl, code, batch, h_q, h_kv, d = _prep(q, k, v, seq_lens)
    m = ctypes.c_double()
    l = ctypes.c_double()
    O = np.zeros(d, dtype=np.float64)
    rc = _load().oracle_partial_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), batch, h_q, h_kv, d,
                                    float(scale), code, b, h, t0, t1, ctypes.byref(m),
                                    ctypes.byref(l), _ptr(O))
    if rc != 0:
        raise ValueError("oracle_partial_f64 failed (%d)" % rc)
    return m.value, l.value, O
