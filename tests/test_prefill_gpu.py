"""Parity of the causal prefill (gqa_prefill_ex through the C ABI) with the fp64
CPU oracle, on an MI355X.

Every token of a sequence is a query over its sequence's keys up to itself.  The
HIP result is compared with oracle.gqa_prefill_f64 (or, at the 32K-token size,
with oracle.gqa_prefill_rows_f64 on sampled tokens):
  * fp32 results: max |err| <= 2e-3 and relative L2 <= 1e-3, in both precision
    modes;
  * 16-bit results: relative L2 <= 1e-3 against the nearest-even rounding of the
    oracle, and every element within one ulp of it or within the method's error
    bound -- 2e-3 for the default fp16 P V product (P keeps 11 significant bits,
    so its error, ~1e-4, can exceed an ulp of small outputs), 1e-5 with
    split_pv = 1 (P split into two 16-bit parts, fp32-level error).
Outputs are NaN-poisoned before each call so an unwritten element fails.
"""
import numpy as np
import pytest

import oracle
from gqa_split_kv_amd import binding as B
from gqa_split_kv_amd.inputs import PREFILL_32K, host_prefill_case

from helpers import MAX_ABS, compare, upload

pytestmark = pytest.mark.gpu

_TORCH_DT = {"bf16": "bfloat16", "f16": "float16", "f32": "float32"}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need an MI355X GPU"
    B.lib()
    yield


def _say(*a):
    print(*a, flush=True)


def _run(q, k, v, sl, scale, out_dtype=None, num_blocks=0, split_pv=0):
    import torch
    out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    out.fill_(float("nan"))
    B.prefill(q, k, v, sl, scale=scale, out=out, num_blocks=num_blocks, split_pv=split_pv)
    torch.cuda.synchronize()
    return out


def _check(o, ref, what, split_pv=0):
    """The rules of the module docstring for a result of either precision mode."""
    return compare(o, ref, what, slack=None if split_pv else MAX_ABS)


@pytest.mark.parametrize("G,h_kv", [(8, 1), (4, 2), (1, 2), (16, 1), (3, 2), (2, 1), (32, 1), (64, 1), (24, 2)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f16", "f32")])
def test_prefill_heads_dims_dtypes(G, h_kv, d, dtype, out):
    import torch
    lens = [300, 1, 0, 77, 33]
    c = host_prefill_case(len(lens), G * h_kv, h_kv, d, lens, dtype, seed=G * 13 + h_kv + d)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    odt = getattr(torch, _TORCH_DT[out])
    for nb, sp in ((0, 0), (1, 0), (5, 0), (0, 1)):
        _say("prefill G", G, "h_kv", h_kv, "d", d, dtype, "->", out, "num_blocks", nb, "split_pv", sp)
        o = _run(q, k, v, sl, c.scale, odt, nb, sp)
        _check(o, ref, "prefill G=%d h_kv=%d d=%d %s->%s nb=%d split=%d" % (G, h_kv, d, dtype, out, nb, sp), sp)


def test_prefill_longer_ragged_batch_and_grid_independence():
    import torch
    lens = [1500, 2, 700, 0, 1025]
    c = host_prefill_case(len(lens), 16, 2, 128, lens, "bf16", seed=21)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    for sp in (0, 1):
        outs = []
        for nb in (0, 3, 64, 4096):
            _say("prefill ragged, num_blocks", nb, "split_pv", sp)
            o = _run(q, k, v, sl, c.scale, torch.float32, nb, sp)
            e, r = _check(o, ref, "ragged nb=%d split=%d" % (nb, sp), sp)
            _say("  max|err| %.3g rel-L2 %.3g" % (e, r))
            outs.append(o)
        # every row is computed by one workgroup in a fixed order: the grid size
        # does not change a single bit
        for o in outs[1:]:
            assert torch.equal(o, outs[0])


def test_prefill_batch_of_more_than_64_sequences():
    """150 sequences (lengths 0 .. 400, some empty, some past a 64-key step):
    the work-item count and the search for a tile's sequence run over several
    64-sequence blocks, and the V copy's step blocks follow every sequence."""
    import torch
    rng = np.random.default_rng(150)
    lens = [int(x) for x in rng.integers(0, 401, size=150)]
    lens[3] = 0
    lens[70] = 0
    lens[64] = 65
    c = host_prefill_case(len(lens), 8, 2, 128, lens, "bf16", seed=150)
    _say("oracle: 150 sequences, %d tokens" % sum(lens))
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    for nb, sp in ((0, 0), (7, 0), (0, 1)):
        _say("prefill 150 sequences, num_blocks", nb, "split_pv", sp)
        o = _run(q, k, v, sl, c.scale, torch.float32, nb, sp)
        e, r = _check(o, ref, "150 sequences nb=%d split=%d" % (nb, sp), sp)
        _say("  max|err| %.3g rel-L2 %.3g" % (e, r))
    o16 = _run(q, k, v, sl, c.scale)
    _check(o16, ref, "150 sequences bf16 out")


def test_prefill_70b_heads_long_sequences():
    """64 query heads over 8 kv heads (the 70B grouping), two sequences long
    enough for dozens of fast-loop steps per tile, both P V modes."""
    import torch
    lens = [2500, 640]
    c = host_prefill_case(2, 64, 8, 128, lens, "bf16", seed=33)
    _say("oracle: 70B heads, lens", lens)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    for sp in (0, 1):
        o = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp)
        e, r = _check(o, ref, "70B heads split=%d" % sp, sp)
        _say("  split_pv %d max|err| %.3g rel-L2 %.3g" % (sp, e, r))


def test_prefill_peaked_keys():
    import torch
    lens = [2048, 600]
    c = host_prefill_case(2, 8, 1, 128, lens, "bf16", seed=23, peaked_frac=0.01, peak_factor=8.0)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    for sp in (0, 1):
        o = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp)
        _check(o, ref, "peaked split=%d" % sp, sp)


def _scaled_v(c, exp2, rows=None):
    """c with V rows `rows` (all if None) multiplied by 2^exp2 -- exact in bf16 for these values."""
    from gqa_split_kv_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    v = bf16_bits_to_f32(c.v).copy()
    sel = slice(None) if rows is None else rows
    v[sel] *= np.float32(2.0 ** exp2)
    c.v = f32_to_bf16_bits(v)
    assert np.array_equal(bf16_bits_to_f32(c.v), v)
    return c


@pytest.mark.parametrize("exp2", [20, -14, -8])
def test_prefill_v_scaled_outside_and_inside_fp16_range(exp2):
    """V far above fp16's range (2^20), far below it (2^-14: every tile takes the
    exact bf16 path) and small but inside it (2^-8: the fp16 path with subnormals):
    the result scales with V, so it is compared after dividing by 2^exp2."""
    import torch
    lens = [700, 300]
    c = _scaled_v(host_prefill_case(2, 8, 1, 128, lens, "bf16", seed=27), exp2)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale) / 2.0 ** exp2
    q, k, v, sl = upload(c)
    for sp in (0, 1):
        o = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp)
        _check(o / 2.0 ** exp2, ref, "V x 2^%d split=%d" % (exp2, sp), sp)


def test_prefill_v_band_beyond_fp16_range():
    """A band of 64 key rows with values up to ~2^22 in the middle of a long
    sequence: the steps before it take the fp16 path, the rest of every tile that
    reaches it the exact one.  Errors are measured against each output row's scale."""
    import torch
    lens = [1200, 90]
    c = _scaled_v(host_prefill_case(2, 8, 1, 128, lens, "bf16", seed=28), 20, rows=slice(500, 564))
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    o = _run(q, k, v, sl, c.scale, torch.float32).cpu().numpy().astype(np.float64)
    row_scale = np.maximum(np.abs(ref).max(axis=-1, keepdims=True), 1.0)
    err = np.abs(o - ref) / row_scale
    assert np.isfinite(o).all()
    assert err.max() <= 2e-3, err.max()
    assert np.sqrt(((o - ref) ** 2).sum() / (ref ** 2).sum()) <= 1e-3


def test_prefill_v_band_in_unaligned_sequences():
    """Sequences that start off the 128-token blocks of the fp16 copy's range
    flags (offsets 77 and 1077), with two key rows of magnitude ~2^20 inside the
    second sequence: every stage that overlaps the flagged block must take the
    exact product, the stages before it the fp16 one."""
    import torch
    lens = [77, 1000, 333]
    c = _scaled_v(host_prefill_case(3, 8, 2, 128, lens, "bf16", seed=29), 20, rows=slice(600, 602))
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    row_scale = np.maximum(np.abs(ref).max(axis=-1, keepdims=True), 1.0)
    for sp in (0, 1):
        o = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp).cpu().numpy().astype(np.float64)
        assert np.isfinite(o).all()
        err = np.abs(o - ref) / row_scale
        assert err.max() <= 2e-3, (sp, err.max())


def test_prefill_caller_workspace_poisoned_and_reused():
    """A caller workspace filled with NaN patterns gives the same bits as the
    library's own, on two calls in a row (the second smaller, other values)."""
    import torch
    cases = [host_prefill_case(3, 16, 2, 128, [900, 333, 1], "bf16", seed=30),
             host_prefill_case(2, 8, 1, 64, [129, 64], "bf16", seed=31)]
    a0 = B.make_prefill_args(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 3, 16, 2, 128, 0.1, B.GQA_DTYPE_BF16,
                             B.GQA_DTYPE_BF16, total_tokens=1234)
    need = B.gqa_prefill_workspace_bytes(a0)
    nvb = -(-1234 // 64) + 3                          # 64-key blocks: ceil(total / 64) + batch
    # transposed copy, one flag byte per block and head, the tile queue's counter
    assert need == 2 * nvb * 128 * 64 * 2 + 256 + 256
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for c in cases:
        q, k, v, sl = upload(c)
        ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
        own = _run(q, k, v, sl, c.scale, torch.float32)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        B.prefill(q, k, v, sl, scale=c.scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, own)
        _check(out, ref, "caller workspace")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_unknown_total_tokens_uses_split_product(dtype):
    """total_tokens = 0 makes no copy of V: the result is bit-identical to
    split_pv = 1."""
    import torch
    c = host_prefill_case(2, 8, 2, 128, [500, 260], dtype, seed=32)
    q, k, v, sl = upload(c)
    o0 = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    B.prefill(q, k, v, sl, scale=c.scale, out=o0, total_tokens=0)
    o1 = _run(q, k, v, sl, c.scale, torch.float32, split_pv=1)
    assert torch.equal(o0, o1)
    o2 = _run(q, k, v, sl, c.scale, torch.float32)
    assert not torch.equal(o2, o1)                    # the default does take the fp16 path


def test_prefill_empty_and_single_token_sequences():
    import torch
    lens = [0, 1, 0, 1, 2]
    c = host_prefill_case(len(lens), 8, 2, 64, lens, "bf16", seed=24)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    for sp in (0, 1):
        o = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp)
        _check(o, ref, "tiny split=%d" % sp, sp)


def test_prefill_32k_single_kv_group_sampled_rows():
    """The long-context prefill panel at full size: 32768 tokens, h_q 8, h_kv 1,
    d 128, bf16; one random token in every 128-token span (256 tokens), the edges
    of the kernel's 32-token tiles and 64-key steps at both ends and in the middle,
    against the oracle one token at a time, in both P V modes, plus finiteness of
    every output."""
    import torch
    w = PREFILL_32K
    c = host_prefill_case(w.batch, w.h_q, w.h_kv, w.d, w.seq_lens(), w.dtype, seed=w.seed)
    q, k, v, sl = upload(c)
    rng = np.random.default_rng(5)
    edges = [0, 1, 31, 32, 33, 63, 64, 65, 1023, 1024, 4095, 16383, 16384, 16385, 32703, 32704, 32735, 32736,
             32766, 32767]
    spans = [128 * i + int(rng.integers(0, 128)) for i in range(32768 // 128)]
    rows = sorted(set(edges + spans))
    assert len(rows) >= 256
    _say("oracle on", len(rows), "sampled tokens")
    ref = oracle.gqa_prefill_rows_f64(c.q, c.k, c.v, c.seq_lens, c.scale, rows)
    for sp in (0, 1):
        _say("prefill 32K: bf16 and fp32 outputs, split_pv", sp)
        o16 = _run(q, k, v, sl, c.scale, split_pv=sp)
        o32 = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp)
        assert torch.isfinite(o32).all().item() and torch.isfinite(o16.float()).all().item()
        idx = torch.tensor(rows, device=o32.device)
        e, r = _check(o32.index_select(0, idx), ref, "32K fp32 rows split=%d" % sp, sp)
        _say("  fp32 max|err| %.3g rel-L2 %.3g" % (e, r))
        _check(o16.index_select(0, idx), ref, "32K bf16 rows split=%d" % sp, sp)


@pytest.mark.parametrize("G", [32, 64])
def test_prefill_wide_groups_long_sequence(G):
    """32 and 64 query heads per kv head (8 and 4 tokens per 256-row tile) over a
    4096-token sequence: one random token in every 64-token span, the tile and
    64-key step edges, against the oracle one token at a time, in both P V modes."""
    import torch
    S = 4096
    c = host_prefill_case(1, G, 1, 128, [S], "bf16", seed=40 + G)
    q, k, v, sl = upload(c)
    tt = 256 // G
    rng = np.random.default_rng(G)
    edges = [0, 1, tt - 1, tt, tt + 1, 63, 64, 65, 2047, 2048, S - tt - 1, S - tt, S - 65, S - 64, S - 1]
    spans = [64 * i + int(rng.integers(0, 64)) for i in range(S // 64)]
    rows = sorted(set(edges + spans))
    _say("G", G, ": oracle on", len(rows), "sampled tokens")
    ref = oracle.gqa_prefill_rows_f64(c.q, c.k, c.v, c.seq_lens, c.scale, rows)
    idx = None
    for sp in (0, 1):
        o32 = _run(q, k, v, sl, c.scale, torch.float32, split_pv=sp)
        assert torch.isfinite(o32).all().item()
        idx = torch.tensor(rows, device=o32.device)
        e, r = _check(o32.index_select(0, idx), ref, "G %d fp32 rows split=%d" % (G, sp), sp)
        _say("  split_pv %d: fp32 max|err| %.3g rel-L2 %.3g" % (sp, e, r))
        o16 = _run(q, k, v, sl, c.scale, split_pv=sp)
        _check(o16.index_select(0, idx), ref, "G %d bf16 rows split=%d" % (G, sp), sp)


def test_prefill_invalid_arguments_leave_output_untouched():
    import torch
    c = host_prefill_case(2, 8, 2, 64, [5, 7], "bf16", seed=25)
    q, k, v, sl = upload(c)
    out = torch.full(q.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    a = B.make_prefill_args(q, k, v, out, sl, 2, 8, 2, 64, c.scale, B.GQA_DTYPE_F32, B.GQA_DTYPE_F32)
    assert B.gqa_prefill_validate(a) == B.GQA_ERR_UNSUPPORTED
    with pytest.raises(B.GqaError):
        B.gqa_prefill_ex(a)
    a = B.make_prefill_args(q, k, v, out, sl, 2, 8, 2, 96, c.scale, B.GQA_DTYPE_BF16, B.GQA_DTYPE_BF16)
    with pytest.raises(B.GqaError):
        B.gqa_prefill_ex(a)
    torch.cuda.synchronize()
    assert (out == 7.0).all().item()


def test_prefill_c_names():
    import torch
    c = host_prefill_case(2, 8, 2, 128, [100, 40], "bf16", seed=26)
    ref = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    q, k, v, sl = upload(c)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    B.gqa_prefill(q, k, v, out, sl, 2, 140, 8, 2, 128, c.scale)
    torch.cuda.synchronize()
    _check(out, ref, "gqa_prefill")
    c16 = host_prefill_case(2, 8, 2, 128, [100, 40], "f16", seed=26)
    ref16 = oracle.gqa_prefill_f64(c16.q, c16.k, c16.v, c16.seq_lens, c16.scale)
    q, k, v, sl = upload(c16)
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda")
    B.gqa_prefill_f16(q, k, v, out, sl, 2, 140, 8, 2, 128, c16.scale)
    torch.cuda.synchronize()
    _check(out, ref16, "gqa_prefill_f16")
