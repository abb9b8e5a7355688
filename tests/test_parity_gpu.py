"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle, on an MI355X.

Every test calls libgqa_decode.so via the ctypes binding and compares with
oracle.gqa_decode_f64 on the same seeded inputs:
  * fp32 results: max |err| <= 2e-3 and relative L2 <= 1e-3;
  * bf16 results: every element within one bf16 ulp of the nearest-even bf16
    rounding of the oracle, and relative L2 <= 1e-3 against that rounding.
Outputs are NaN-poisoned before each call so an unwritten element fails.
Every test runs twice: with the pieces of cut sequences merged by a second
kernel, and with the merge fused into the sweep kernel.
"""
import numpy as np
import pytest

import helpers
from gqa_split_kv_amd import binding as B
from gqa_split_kv_amd.inputs import (WORKLOADS, device_workload, host_case, host_workload,
                                     to_host_bits)

from helpers import compare, oracle_of, run_hip, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=[B.GQA_MERGE_KERNEL, B.GQA_MERGE_FUSED], ids=["kernel", "fused"])
def merge_form(request):
    """The merge form every decode call of the test requests."""
    helpers.MERGE = request.param
    yield request.param
    helpers.MERGE = B.GQA_MERGE_AUTO


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need an MI355X GPU"
    B.lib()   # raises if the library is not built: there is no fallback path
    yield
    B.gqa_release()


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ the named workloads


def test_tiny_fp32_workload():
    import torch
    w = WORKLOADS[1]
    c = host_workload(w)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    for nc, mc in [(0, 0), (1, 1), (16, 1), (4096, 1), (7, 33)]:
        _say("tiny fp32, num_chunks", nc, "min_chunk", mc)
        out = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc)
        e, r = compare(out, ref, "cfg1 nc=%d mc=%d" % (nc, mc))
        assert e < 1e-5 and r < 1e-5, (e, r)   # fp32 in and out: fp32-level agreement
        hinted = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc, max_seq_len=int(c.seq_lens.max()))
        assert torch.equal(hinted, out), "cfg1 with the length bound"


@pytest.mark.parametrize("cfg", [2, 3])
def test_single_sequence_bf16_workloads(cfg):
    import torch
    w = WORKLOADS[cfg]
    c = host_workload(w)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    plans = [(0, 0), (0, 1024), (1 << 16, 1024), (333, 1)]
    for nc, mc in plans:
        _say("cfg", cfg, "num_chunks", nc, "min_chunk", mc)
        out32 = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
        e, r = compare(out32, ref, "cfg%d f32 out" % cfg)
        assert e < 1e-4 and r < 1e-4, (e, r)
        out16 = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc)
        compare(out16, ref, "cfg%d bf16 out" % cfg)
        # The benchmark's call: the longest length as the max_seq_len bound (the merge
        # then reads the pieces before the length arrives); the same bits.
        hinted = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc, max_seq_len=int(c.seq_lens.max()))
        assert torch.equal(hinted, out16), "cfg%d with the length bound" % cfg


def _full_size(cfg):
    import torch
    w = WORKLOADS[cfg]
    _say("generating", w.name)
    d = device_workload(w)
    torch.cuda.synchronize()
    _say("decode (automatic plan, as the benchmark runs it)")
    out16 = run_hip(d.q, d.k, d.v, d.seq_lens, d.scale)
    out32 = run_hip(d.q, d.k, d.v, d.seq_lens, d.scale, out_dtype=torch.float32)
    _say("copying inputs to the host and running the oracle")
    qh, kh, vh = to_host_bits(d.q), to_host_bits(d.k), to_host_bits(d.v)
    import oracle
    ref = oracle.gqa_decode_f64(qh, kh, vh, d.seq_lens_host, d.scale)
    return out16, out32, ref


def test_70b_shaped_ragged_workload_full_size():
    out16, out32, ref = _full_size(4)
    e, r = compare(out32, ref, "cfg4 f32 out")
    _say("cfg4 fp32 out: max|err| %.3g rel-L2 %.3g" % (e, r))
    u, r16, r16raw = compare(out16, ref, "cfg4 bf16 out")
    _say("cfg4 bf16 out: max ulps %d rel-L2 vs bf16(oracle) %.3g vs oracle %.3g" % (u, r16, r16raw))


def test_long_context_peaked_workload_full_size():
    out16, out32, ref = _full_size(5)
    e, r = compare(out32, ref, "cfg5 f32 out")
    _say("cfg5 fp32 out: max|err| %.3g rel-L2 %.3g" % (e, r))
    compare(out16, ref, "cfg5 bf16 out")


def test_sequence_beyond_2_pow_25_keys():
    """A sequence of 2^25 + 3 keys between two short ones (d 64, one kv head, G 2):
    the long one is cut into many ranges and merged, and the short one after it
    starts past 2^25 key rows, at the offset the kernels' table of lengths gives."""
    import torch
    from gqa_split_kv_amd.inputs import device_case
    import oracle
    lens = [5, (1 << 25) + 3, 7]
    _say("generating 3 sequences, %d keys" % sum(lens))
    d = device_case(3, 2, 1, 64, lens, "bf16", seed=2525)
    o32 = run_hip(d.q, d.k, d.v, d.seq_lens, d.scale, out_dtype=torch.float32)
    o16 = run_hip(d.q, d.k, d.v, d.seq_lens, d.scale)
    _say("copying inputs to the host and running the oracle")
    ref = oracle.gqa_decode_f64(to_host_bits(d.q), to_host_bits(d.k), to_host_bits(d.v), d.seq_lens_host,
                                d.scale)
    e, r = compare(o32, ref, "2^25+3 keys f32 out")
    _say("fp32 out: max|err| %.3g rel-L2 %.3g" % (e, r))
    compare(o16, ref, "2^25+3 keys bf16 out")


# ------------------------------------------------------------------ shapes and plans


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G,h_kv", [(1, 4), (2, 2), (3, 1), (4, 2), (8, 1), (8, 2), (16, 1), (5, 3)])
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"),
                                       ("f16", "f16"), ("f16", "f32")])
def test_heads_dims_dtypes(d, G, h_kv, dtype, out):
    import torch
    lens = [37, 0, 300, 16, 1]
    c = host_case(len(lens), G * h_kv, h_kv, d, lens, dtype, seed=G * 100 + h_kv * 10 + d)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    odt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    for nc, mc in [(0, 0), (5, 1), (64, 16)]:
        o = run_hip(q, k, v, sl, c.scale, out_dtype=odt, num_chunks=nc, min_chunk=mc)
        compare(o, ref, "G=%d h_kv=%d d=%d %s->%s nc=%d mc=%d" % (G, h_kv, d, dtype, out, nc, mc))


@pytest.mark.parametrize("lens", [[0], [1], [15], [16], [17], [31], [33], [1024], [1025],
                                  [0, 0, 5], [-2, 3], [0, 0], [5, 0, 0, 0, 7], list(range(0, 70))])
def test_edge_lengths(lens):
    import torch
    c = host_case(len(lens), 8, 2, 128, lens, "bf16", seed=len(lens) + 7)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    for nc, mc in [(0, 0), (1, 1), (3, 1), (1000, 1), (2, 16)]:
        o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
        compare(o, ref, "lens=%s nc=%d mc=%d" % (lens[:8], nc, mc))
        for b, L in enumerate(lens):
            if L <= 0:
                assert (o[b] == 0).all().item()


@pytest.mark.parametrize("h_q,h_kv,d,t_q,dtype", [(32, 8, 128, 0, "bf16"), (8, 1, 128, 0, "bf16"),
                                                  (16, 2, 128, 4, "bf16"), (8, 1, 64, 0, "f32")])
def test_single_sequence_length_bound(h_q, h_kv, d, t_q, dtype):
    """One sequence with the caller's max_seq_len bound: the merge reads its pieces
    for the length the bound predicts and falls back when the stored length differs
    (bound above the length, a bound below it, an empty or negative length).  Each
    result matches the oracle and, bit for bit, the same call without a bound."""
    import torch
    out_dtype = torch.float32
    for L in [1, 33, 1000, 8192, 0, -3]:
        c = host_case(1, h_q, h_kv, d, [L], dtype, seed=L + 1000 * h_kv + t_q, t_q=t_q)
        ref = oracle_of(c)
        q, k, v, sl = upload(c)
        for nc, mc in [(0, 0), (4096, 1), (64, 1)]:
            _say("h_q", h_q, "h_kv", h_kv, "d", d, "t_q", t_q, dtype, "len", L, "no bound", "nc", nc, "mc", mc)
            base = run_hip(q, k, v, sl, c.scale, out_dtype=out_dtype, num_chunks=nc, min_chunk=mc)
            for hint in sorted({max(L, 0), max(L, 0) + 1, 2 * max(L, 0) + 7, max(L - 1, 0), 5}):
                _say("  bound", hint)
                o = run_hip(q, k, v, sl, c.scale, out_dtype=out_dtype, num_chunks=nc, min_chunk=mc,
                            max_seq_len=hint)
                compare(o, ref, "len=%d bound=%d nc=%d mc=%d" % (L, hint, nc, mc))
                # (the merge form is forced here, so the bound cannot change the plan)
                assert torch.equal(o, base), "len=%d bound=%d nc=%d mc=%d" % (L, hint, nc, mc)
                if L <= 0:
                    assert (o == 0).all().item()


@pytest.mark.parametrize("nc,mc", [(1, 1), (2, 1), (3, 7), (64, 1), (4096, 1), (100000, 1),
                                   (7, 1024), (1 << 20, 16), (0, 17)])
def test_forced_chunking_ragged_batch(nc, mc):
    import torch
    lens = [513, 1, 2000, 0, 77, 1024, 16, 3333]
    c = host_case(len(lens), 64, 8, 128, lens, "bf16", seed=55)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
    compare(o, ref, "nc=%d mc=%d" % (nc, mc))
    o16 = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc)
    compare(o16, ref, "bf16 nc=%d mc=%d" % (nc, mc))


# ------------------------------------------------------------------ multi-token decode


@pytest.mark.parametrize("G,h_kv,t_q", [(8, 1, 2), (4, 2, 4), (1, 4, 16), (2, 8, 8), (3, 1, 5),
                                        (16, 1, 1), (5, 2, 3)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"),
                                       ("f16", "f16")])
def test_multi_token_heads_dims_dtypes(G, h_kv, t_q, d, dtype, out):
    import torch
    lens = [37, 0, 300, 2, 1, 16, 129]
    c = host_case(len(lens), G * h_kv, h_kv, d, lens, dtype, seed=G * 31 + t_q * 7 + d, t_q=t_q)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    odt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    for nc, mc in [(0, 0), (5, 1), (64, 16), (1000, 1)]:
        _say("t_q", t_q, "G", G, "h_kv", h_kv, "d", d, dtype, "->", out, "nc", nc, "mc", mc)
        o = run_hip(q, k, v, sl, c.scale, out_dtype=odt, num_chunks=nc, min_chunk=mc)
        assert o.shape == (len(lens), t_q, G * h_kv, d)
        compare(o, ref, "t_q=%d G=%d h_kv=%d d=%d %s->%s nc=%d mc=%d" % (t_q, G, h_kv, d, dtype, out,
                                                                         nc, mc))


@pytest.mark.parametrize("nc,mc", [(0, 0), (1, 1), (3, 7), (64, 1), (4096, 1), (7, 1024)])
def test_multi_token_ragged_70b_heads(nc, mc):
    import torch
    lens = [513, 1, 2000, 0, 77, 1024, 3, 3333]
    c = host_case(len(lens), 64, 8, 128, lens, "bf16", seed=56, t_q=2)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    _say("t_q 2 ragged, nc", nc, "mc", mc)
    o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
    compare(o, ref, "t_q=2 nc=%d mc=%d" % (nc, mc))
    o16 = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc)
    compare(o16, ref, "t_q=2 bf16 nc=%d mc=%d" % (nc, mc))


def test_multi_token_70b_shaped_ragged_full_size():
    """Two query tokens per sequence on the 70B-shaped ragged workload at full size
    (64 sequences of 1K-32K keys, G 8 x t_q 2 = 16 rows), automatic plan as the
    benchmark runs the decode; the oracle checks every sequence whole."""
    import torch
    import oracle
    from gqa_split_kv_amd.inputs import device_case
    w = WORKLOADS[4]
    sl_host = w.seq_lens()
    _say("generating the 70B-shaped ragged workload with t_q = 2")
    d = device_case(w.batch, w.h_q, w.h_kv, w.d, sl_host, w.dtype, seed=w.seed + 50, t_q=2)
    out32 = run_hip(d.q, d.k, d.v, d.seq_lens, d.scale, out_dtype=torch.float32)
    out16 = run_hip(d.q, d.k, d.v, d.seq_lens, d.scale)
    _say("copying inputs to the host and running the oracle over all 64 sequences")
    ref = oracle.gqa_decode_f64(to_host_bits(d.q), to_host_bits(d.k), to_host_bits(d.v), sl_host, d.scale)
    e, r = compare(out32, ref, "t_q=2 full size fp32")
    _say("t_q=2 fp32 out: max|err| %.3g rel-L2 %.3g" % (e, r))
    compare(out16, ref, "t_q=2 full size bf16")


@pytest.mark.parametrize("form", ["t_q8", "G64"])
def test_64_rows_70b_shaped_ragged_full_size(form):
    """The two 64-row forms the benchmark times on the 70B-shaped ragged workload's
    keys and values (64 sequences of 1K-32K keys), with its query blocks: eight
    query tokens on 64 query heads (G 8 x t_q 8), and one token on 512 query heads
    (G 64); automatic plan; the oracle checks 16 of the 64 sequences whole (every
    fourth, so short and long ones alike) and every output is finite."""
    import torch
    import oracle
    from gqa_split_kv_amd.inputs import device_queries
    w = WORKLOADS[4]
    sl_host = w.seq_lens()
    _say("generating the 70B-shaped ragged workload's K/V and the", form, "queries")
    d = device_workload(w)
    if form == "t_q8":
        q = device_queries(w.batch, 8, w.h_q, w.d, "bf16", seed=w.seed + 11)
    else:
        q = device_queries(w.batch, 1, 64 * w.h_kv, w.d, "bf16", seed=w.seed + 13)[:, 0].contiguous()
    out32 = run_hip(q, d.k, d.v, d.seq_lens, d.scale, out_dtype=torch.float32)
    out16 = run_hip(q, d.k, d.v, d.seq_lens, d.scale)
    assert torch.isfinite(out32).all().item() and torch.isfinite(out16.float()).all().item()
    pick = list(range(0, w.batch, 4))
    _say("copying the inputs of sequences", pick[0], "...", pick[-1], "to the host and running the oracle")
    kh, vh = to_host_bits(d.k), to_host_bits(d.v)
    starts = np.concatenate([[0], np.cumsum(sl_host)])
    qs, ks, vs = [], [], []
    for b in pick:
        qs.append(to_host_bits(q[b:b + 1]))
        ks.append(kh[starts[b]:starts[b + 1]])
        vs.append(vh[starts[b]:starts[b + 1]])
    ref = oracle.gqa_decode_f64(np.concatenate(qs), np.concatenate(ks), np.concatenate(vs),
                                sl_host[pick].astype(np.int32), d.scale)
    idx = torch.tensor(pick, device=out32.device)
    e, r = compare(out32.index_select(0, idx), ref, "%s full size fp32" % form)
    _say("%s fp32 out: max|err| %.3g rel-L2 %.3g" % (form, e, r))
    compare(out16.index_select(0, idx), ref, "%s full size bf16" % form)


@pytest.mark.parametrize("G,h_kv,t_q", [(8, 2, 4), (16, 1, 3), (8, 1, 8), (32, 2, 1), (64, 1, 1),
                                        (24, 1, 2), (17, 1, 1), (3, 3, 7)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"),
                                       ("f16", "f16")])
def test_more_than_16_rows_per_kv_head(G, h_kv, t_q, d, dtype, out):
    """G * t_q from 17 to 64 rows per kv head: a wavefront holds two or four 16-row
    tiles and computes each step once per tile on one load of the keys; short
    sequences leave tokens that see no key (output 0)."""
    import torch
    lens = [37, 0, 300, 2, 1, 16, 129]
    c = host_case(len(lens), G * h_kv, h_kv, d, lens, dtype, seed=G * 37 + t_q * 5 + d + h_kv, t_q=t_q)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    odt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[out]
    for nc, mc in [(0, 0), (5, 1), (64, 16), (1000, 1)]:
        _say("rows", G * t_q, "t_q", t_q, "G", G, "h_kv", h_kv, "d", d, dtype, "->", out, "nc", nc, "mc", mc)
        o = run_hip(q, k, v, sl, c.scale, out_dtype=odt, num_chunks=nc, min_chunk=mc)
        assert o.shape == (len(lens), t_q, G * h_kv, d)
        compare(o, ref, "rows=%d t_q=%d G=%d h_kv=%d d=%d %s->%s nc=%d mc=%d" % (G * t_q, t_q, G, h_kv, d,
                                                                                 dtype, out, nc, mc))


def test_more_than_16_rows_70b_heads_ragged_batch():
    """Four speculative tokens on the 70B grouping (G 8, h_kv 8: 32 rows per kv
    head) over a ragged batch of 12 sequences up to 3000 keys, and one token on 64
    query heads over one kv head (G 64), against the oracle."""
    import torch
    rng = np.random.default_rng(4)
    lens = [int(x) for x in rng.integers(0, 3001, size=12)]
    for h_q, h_kv, t_q in ((64, 8, 4), (64, 1, 1)):
        c = host_case(len(lens), h_q, h_kv, 128, lens, "bf16", seed=400 + h_kv + t_q, t_q=t_q)
        ref = oracle_of(c)
        q, k, v, sl = upload(c)
        for nc, mc in [(0, 0), (7, 1), (4096, 1)]:
            _say("70B heads ragged, h_q", h_q, "h_kv", h_kv, "t_q", t_q, "nc", nc)
            o32 = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
            compare(o32, ref, "h_q=%d h_kv=%d t_q=%d nc=%d f32" % (h_q, h_kv, t_q, nc))
            o16 = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=mc)
            compare(o16, ref, "h_q=%d h_kv=%d t_q=%d nc=%d bf16" % (h_q, h_kv, t_q, nc))


def test_more_than_16_rows_more_than_64_sequences():
    """Four 16-row tiles per wavefront (G 48) over 90 sequences, where the
    kernels take the lengths from seq_lens block by block instead of one register
    table, with the automatic and forced plans."""
    import torch
    rng = np.random.default_rng(90)
    lens = [int(x) for x in rng.integers(0, 400, size=90)]
    lens[0] = 0
    lens[64] = 1
    c = host_case(len(lens), 96, 2, 128, lens, "bf16", seed=90, t_q=1)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    for nc, mc in [(0, 0), (6, 1), (2000, 1)]:
        _say("90 sequences, G 48, nc", nc, "mc", mc)
        o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
        compare(o, ref, "90 sequences G=48 nc=%d mc=%d" % (nc, mc))


def test_multi_token_short_sequences_give_zero_for_unseen_tokens():
    import torch
    lens = [0, 1, 2, 3, 4, 5]
    t_q = 4
    c = host_case(len(lens), 8, 2, 128, lens, "bf16", seed=9, t_q=t_q)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    for nc, mc in [(0, 0), (2, 1), (12, 1)]:
        o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
        compare(o, ref, "short t_q=4 nc=%d" % nc)
        for b, L in enumerate(lens):
            for t in range(t_q):
                if L - t_q + t < 0:
                    assert (o[b, t] == 0).all().item(), (b, t)


def test_multi_token_one_token_matches_single_token_call():
    import torch
    lens = [700, 33, 0, 4096]
    c = host_case(len(lens), 32, 8, 128, lens, "bf16", seed=11, t_q=1)
    q, k, v, sl = upload(c)
    o4 = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32)
    o3 = run_hip(q[:, 0].contiguous(), k, v, sl, c.scale, out_dtype=torch.float32)
    assert torch.equal(o4[:, 0], o3)


def test_peaked_keys_exercise_running_max():
    import torch
    lens = [4096, 8192]
    c = host_case(2, 16, 2, 128, lens, "bf16", seed=77, peaked_frac=0.001, peak_factor=8.0)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    for nc, mc in [(0, 0), (257, 1), (9, 16)]:
        o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
        compare(o, ref, "peaked nc=%d mc=%d" % (nc, mc))


def test_scale_one_is_the_pages_unscaled_kernel():
    import torch
    c = host_case(1, 8, 1, 64, [256], "f32", seed=3, scale=1.0)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    o = run_hip(q, k, v, sl, 1.0, out_dtype=torch.float32)
    compare(o, ref, "scale 1")


@pytest.mark.parametrize("scale", [-0.09, 0.0, -1.3])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_negative_and_zero_scale(scale, dtype):
    """A negative scale (the kernels negate q and scale by |scale|) and scale 0
    (every visible key weighs the same), with one to four 16-row tiles per
    wavefront: 8, 32, 48 and 64 rows per kv head (G 8 with 1, 4, 6 and 8 query
    tokens), over sequences long enough for steps with no masked key."""
    import torch
    lens = [300, 0, 1, 129, 2000, 65]
    for t_q in (1, 4, 6, 8):
        c = host_case(len(lens), 16, 2, 128, lens, dtype, seed=500 + t_q, scale=scale, t_q=t_q)
        ref = oracle_of(c)
        q, k, v, sl = upload(c)
        for nc, mc in [(0, 0), (9, 1)]:
            _say("scale", scale, dtype, "t_q", t_q, "nc", nc)
            o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
            compare(o, ref, "scale=%g %s t_q=%d nc=%d" % (scale, dtype, t_q, nc))


# ------------------------------------------------------------------ boundary behaviour


def test_caller_workspace_poisoned_and_reused(merge_form):
    """A caller workspace whose partial slots hold NaN (only the counter reserve at
    its start is zero, as the header asks) gives the oracle's result twice in a
    row, and the counters read zero again after each call."""
    import torch
    lens = [900, 50, 3000]
    c = host_case(3, 32, 8, 128, lens, "bf16", seed=91)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    args = B.make_args(q, k, v, q, sl, 3, 32, 8, 128, c.scale, 0, 1, num_chunks=300, min_chunk=1, merge=merge_form)
    nbytes = B.gqa_decode_workspace_bytes(args)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    ws[:B.GQA_DECODE_COUNTER_BYTES // 4].zero_()
    for _ in range(2):
        o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=300, min_chunk=1,
                    workspace=ws)
        compare(o, ref, "caller workspace")
        assert (ws[:B.GQA_DECODE_COUNTER_BYTES // 4].view(torch.int32) == 0).all().item()


def test_fused_merge_over_thousands_of_pieces_is_deterministic():
    """One sequence of 48,000 keys cut into 4,000 ranges of 12 keys (1,000
    workgroup-level pieces, a three-level tree of fan-in 16), and a ragged batch
    cut as finely: bit-identical outputs over repeated calls, the oracle's result,
    and counters back at zero after every call."""
    import torch
    for lens, h_q, h_kv in (([48000], 8, 1), ([9000, 0, 30000, 5, 9001], 16, 2)):
        c = host_case(len(lens), h_q, h_kv, 128, lens, "bf16", seed=1000 + len(lens))
        ref = oracle_of(c)
        q, k, v, sl = upload(c)
        nc = 4000 * h_kv
        args = B.make_args(q, k, v, q, sl, len(lens), h_q, h_kv, 128, c.scale, 0, 1, num_chunks=nc, min_chunk=1,
                           merge=B.GQA_MERGE_FUSED)
        st, plan = B.gqa_decode_make_plan(args, 256, 4)
        assert st == B.GQA_OK and plan.fused and plan.num_chunks == nc and plan.fold_levels == 3, plan.fold_levels
        ws = torch.zeros(B.gqa_decode_workspace_bytes(args), dtype=torch.uint8, device="cuda")
        outs = []
        for rep in range(3):
            _say("fused merge, lens", lens, "rep", rep)
            o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=1, workspace=ws,
                        merge=B.GQA_MERGE_FUSED)
            outs.append(o)
            assert (ws[:B.GQA_DECODE_COUNTER_BYTES].view(torch.int32) == 0).all().item()
        compare(outs[0], ref, "fused, 1000 pieces")
        assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
        o16 = run_hip(q, k, v, sl, c.scale, num_chunks=nc, min_chunk=1, merge=B.GQA_MERGE_FUSED)
        compare(o16, ref, "fused, 1000 pieces, bf16 out")


def test_too_small_workspace_is_rejected_and_output_untouched():
    import torch
    c = host_case(1, 8, 1, 128, [100], "bf16", seed=92)
    q, k, v, sl = upload(c)
    ws = torch.zeros(64, dtype=torch.float32, device="cuda")
    o = torch.full((1, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.GqaError) as ei:
        B.decode(q, k, v, sl, out=o, num_chunks=10, workspace=ws, merge=helpers.MERGE)
    assert ei.value.status == B.GQA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (o == 7.0).all().item()


def test_invalid_arguments_leave_output_untouched():
    import torch
    c = host_case(1, 8, 2, 128, [10], "bf16", seed=93)
    q, k, v, sl = upload(c)
    o = torch.full((1, 8, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    for kw, status in [(dict(h_q=7), B.GQA_ERR_SHAPE), (dict(d_head=96), B.GQA_ERR_UNSUPPORTED),
                       (dict(scale=float("nan")), B.GQA_ERR_SCALE)]:
        base = dict(q=q, k=k, v=v, o=o, seq_lens=sl, batch=1, h_q=8, h_kv=2, d_head=128,
                    scale=c.scale, in_dtype=0, out_dtype=0, merge=helpers.MERGE)
        base.update(kw)
        args = B.make_args(**base)
        with pytest.raises(B.GqaError) as ei:
            B.gqa_decode_ex(args)
        assert ei.value.status == status
    torch.cuda.synchronize()
    assert (o == 3.0).all().item()


def test_c_names_and_f32_entry_point():
    import torch
    c = host_case(2, 8, 2, 64, [40, 9], "f32", seed=94)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    o = torch.full((2, 8, 64), float("nan"), dtype=torch.float32, device="cuda")
    B.gqa_decode_f32(q, k, v, o, sl, 2, 8, 2, 64, c.scale)
    torch.cuda.synchronize()
    compare(o, ref, "gqa_decode_f32")
    cb = host_case(2, 8, 2, 64, [40, 9], "bf16", seed=95)
    refb = oracle_of(cb)
    q, k, v, sl = upload(cb)
    ob = torch.full((2, 8, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    B.gqa_decode(q, k, v, ob, sl, 2, 8, 2, 64, cb.scale)
    torch.cuda.synchronize()
    compare(ob, refb, "gqa_decode")


def test_f16_entry_point_and_70b_shape():
    """fp16 (the pages' element type) through gqa_decode_f16 and gqa_decode_ex, on the
    70B-shaped head layout with ragged lengths, peaked keys included."""
    import torch
    lens = [4000, 1, 17, 9001, 1024, 33]
    c = host_case(len(lens), 64, 8, 128, lens, "f16", seed=97, peaked_frac=0.001, peak_factor=8.0)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    o = torch.full((len(lens), 64, 128), float("nan"), dtype=torch.float16, device="cuda")
    B.gqa_decode_f16(q, k, v, o, sl, len(lens), 64, 8, 128, c.scale)
    torch.cuda.synchronize()
    compare(o, ref, "gqa_decode_f16")
    for nc, mc in [(0, 0), (64, 1), (8, 16)]:
        o32 = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32, num_chunks=nc, min_chunk=mc)
        e, r = compare(o32, ref, "f16 -> f32 nc=%d" % nc)
        assert e < 1e-4 and r < 1e-4, (e, r)


def test_f16_small_weights_keep_their_mass():
    """A long sequence whose weights are mostly far below fp16's range relative to
    the maximum: the sum of the small weights must not be lost."""
    import torch
    S = 20000
    c = host_case(1, 8, 1, 128, [S], "f16", seed=98, scale=1.0)
    qf = np.zeros_like(c.q)
    qf[0, :, 0] = 3.0                                   # scores = 3 * k[:, 0]
    k = c.k.copy()
    k[:, 0, 0] = np.float16(0.0)
    k[7, 0, 0] = np.float16(6.0)                        # one key leads by 18 (weight ratio e^-18)
    ref = oracle_of(type(c)(qf, k, c.v, c.seq_lens, 1.0, "f16"))
    q_, k_, v_, sl = upload(type(c)(qf, k, c.v, c.seq_lens, 1.0, "f16"))
    o32 = run_hip(q_, k_, v_, sl, 1.0, out_dtype=torch.float32)
    e, r = compare(o32, ref, "f16 small weights")
    assert e < 1e-4, e


def test_runs_on_the_given_stream_and_is_deterministic():
    import torch
    lens = [5000, 123, 7001]
    c = host_case(3, 64, 8, 128, lens, "bf16", seed=96)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(2):
        o = torch.full((3, 64, 128), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.current_stream().synchronize()
        with torch.cuda.stream(s):
            B.decode(q, k, v, sl, out=o, stream=s, merge=helpers.MERGE)
            ev = torch.cuda.Event()
            ev.record(s)
        ev.synchronize()
        outs.append(o.clone())
    compare(outs[0], ref, "side stream")
    assert torch.equal(outs[0], outs[1])


# ------------------------------------------------------------------ measurement probes


@pytest.mark.parametrize("n", [16, 1024 + 48, (37 << 20) + 48])
def test_probe_copy_and_read_are_exact(n):
    import torch
    src = torch.randint(0, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")     # GQA_PROBE_SINK_WORDS
    B.gqa_probe_copy(src, dst, n)
    B.gqa_probe_read(src, n, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))) == int(want)


def test_decode_after_prefill_on_library_workspaces(merge_form):
    """Decode and prefill keep separate library-owned workspaces: a prefill's copy
    of V must not land on the decode's merge counters (which must read zero)."""
    import torch
    from gqa_split_kv_amd.inputs import host_prefill_case
    pc = host_prefill_case(2, 8, 1, 128, [3000, 500], "bf16", seed=1234)
    pq, pk, pv, psl = upload(pc)
    B.prefill(pq, pk, pv, psl, scale=pc.scale)
    lens = [4000, 77]
    c = host_case(len(lens), 8, 1, 128, lens, "bf16", seed=1235)
    ref = oracle_of(c)
    q, k, v, sl = upload(c)
    for rep in range(2):
        o = run_hip(q, k, v, sl, c.scale, out_dtype=torch.float32)
        compare(o, ref, "decode after prefill, rep %d" % rep)
        B.prefill(pq, pk, pv, psl, scale=pc.scale)
