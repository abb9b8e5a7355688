"""Pins of the fp64 CPU oracle to things other than itself (CPU only).

The oracle (oracle/oracle.c) computes o = softmax(scale * q K^T) V per query head
(kernbench2 page "_gqa_attention_decode_long.py": "Tile 0" block over all keys,
then the final normalise-and-store block).  These tests hold it to:
  * a 50-digit decimal brute force (oracle/brute.py) and stored brute-force values
    (tests/golden/tiny_brute.json);
  * a library routine: torch's float64 scaled_dot_product_attention with the kv
    heads repeated G times (GQA == textbook MHA with shared K/V; G = 1 is MHA,
    h_kv = 1 is MQA);
  * closed forms (q = 0 or identical keys -> mean of V; constant V -> V; one key ->
    its V row; a key that leads by > 40 -> its V row);
  * invariants (weights sum to 1; permuting (k_t, v_t) pairs; linearity in V);
  * partition invariance: any partition of the keys into ranges, each reduced to
    its (m, l, O) triple and merged with the page's `_merge_running` rule in the
    page's two merge orders (1-D chain and centre-root mesh), gives the direct
    result.
Multi-token decode (t_q query tokens per sequence, the last t_q key rows being
theirs; token t sees keys 0 .. S - t_q + t) is pinned the same way: brute force
per token, torch's float64 SDPA with the matching boolean mask, t_q = 1 equal to
the single-token call, and the last token equal to a single-token decode over
all S keys.
Causal prefill (every token of a sequence a query over its own prefix) is
pinned to brute force per sequence, to torch's float64 SDPA with is_causal, and
to closed forms (the first token returns its own V row; the last token is the
single-token decode over the whole sequence).
A final test plants plausible mistakes in copies of the definition and checks
that the pins used here catch every one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import merge as M
from oracle.brute import brute_decode
from gqa_split_kv_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, host_case, host_prefill_case

HERE = os.path.dirname(os.path.abspath(__file__))


def _f64(a):
    return bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def test_input_widening_is_exact_for_every_16_bit_pattern():
    # Library routines fix the values: numpy's IEEE half conversion, and bf16 as
    # the upper half of a float32.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    w = oracle.widen(h)
    ref = h.astype(np.float64)
    assert ((w == ref) | (np.isnan(w) & np.isnan(ref))).all()
    wb = oracle.widen(bits)
    refb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert ((wb == refb) | (np.isnan(wb) & np.isnan(refb))).all()
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.widen(x), x.astype(np.float64))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("G,h_kv", [(1, 2), (2, 1), (4, 1), (2, 2)])
@pytest.mark.parametrize("seq_lens", [[0], [1], [2, 5], [16, 0, 3]])
def test_oracle_matches_decimal_brute_force(dtype, G, h_kv, seq_lens):
    d = 8 if G != 4 else 4
    c = host_case(len(seq_lens), G * h_kv, h_kv, d, seq_lens, dtype, seed=G * 7 + h_kv,
                  scale=0.37)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    ref = np.array(brute_decode(c.q, c.k, c.v, c.seq_lens, c.scale), dtype=np.float64)
    assert got.shape == ref.shape
    assert np.abs(got - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())


def test_oracle_matches_stored_brute_force_values():
    with open(os.path.join(HERE, "golden", "tiny_brute.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 4
    for cs in cases:
        npdt = np.uint16 if cs["dtype"] == "bf16" else np.float32
        b, hq, hkv, d = cs["batch"], cs["h_q"], cs["h_kv"], cs["d"]
        rows = sum(max(x, 0) for x in cs["seq_lens"])
        q = np.array(cs["q"], dtype=npdt).reshape(b, hq, d)
        k = np.array(cs["k"], dtype=npdt).reshape(rows, hkv, d)
        v = np.array(cs["v"], dtype=npdt).reshape(rows, hkv, d)
        want = np.array([[[float(x) for x in r] for r in ob] for ob in cs["o"]])
        got = oracle.gqa_decode_f64(q, k, v, np.array(cs["seq_lens"], np.int32), cs["scale"])
        assert np.abs(got - want).max() <= 1e-13 * max(1.0, np.abs(want).max()), cs["name"]


# ---------------------------------------------------------------- library routine


def _sdpa_reference(c, G):
    import torch
    out = []
    base = 0
    q = torch.from_numpy(_f64(c.q))
    k = torch.from_numpy(_f64(c.k))
    v = torch.from_numpy(_f64(c.v))
    for b, S in enumerate(c.seq_lens):
        S = int(S)
        kb = k[base:base + S].permute(1, 0, 2).repeat_interleave(G, dim=0)   # [h_q, S, d]
        vb = v[base:base + S].permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = q[b].unsqueeze(1)                                                # [h_q, 1, d]
        o = torch.nn.functional.scaled_dot_product_attention(
            qb.unsqueeze(0), kb.unsqueeze(0).contiguous(), vb.unsqueeze(0).contiguous(),
            scale=c.scale)
        out.append(o[0, :, 0, :].numpy())
        base += S
    return np.stack(out)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("G,h_kv,d", [(1, 4, 16), (8, 1, 64), (4, 2, 32), (16, 1, 32), (8, 8, 128)])
def test_gqa_equals_mha_with_repeated_kv_heads(G, h_kv, d, dtype):
    c = host_case(3, G * h_kv, h_kv, d, [37, 1, 130], dtype, seed=100 + G, scale=d ** -0.5)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    ref = _sdpa_reference(c, G)
    assert np.abs(got - ref).max() <= 1e-12


# ---------------------------------------------------------------- multi-token decode


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("t_q", [2, 3])
@pytest.mark.parametrize("seq_lens", [[0], [1], [2, 5], [3, 0, 9]])
def test_multi_token_oracle_matches_decimal_brute_force(dtype, t_q, seq_lens):
    c = host_case(len(seq_lens), 4, 2, 8, seq_lens, dtype, seed=70 + t_q, scale=0.41, t_q=t_q)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    ref = np.array(brute_decode(c.q, c.k, c.v, c.seq_lens, c.scale), dtype=np.float64)
    assert got.shape == ref.shape == c.q.shape
    assert np.abs(got - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())


def _sdpa_masked_reference(c, G):
    """torch float64 SDPA, kv heads repeated G times, boolean mask keeping key s
    for query token t iff s <= S - t_q + t.  Tokens whose mask is empty (S < t_q)
    are set to NaN here: SDPA's value for an all-masked row differs between torch
    versions, and the definition's value for them (0) is checked separately."""
    import torch
    batch, t_q, h_q, d = c.q.shape
    q = torch.from_numpy(_f64(c.q))
    k = torch.from_numpy(_f64(c.k))
    v = torch.from_numpy(_f64(c.v))
    out = np.full((batch, t_q, h_q, d), np.nan)
    base = 0
    for b, S in enumerate(c.seq_lens):
        S = int(S)
        if S > 0:
            kb = k[base:base + S].permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
            vb = v[base:base + S].permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
            qb = q[b].permute(1, 0, 2).contiguous()                            # [h_q, t_q, d]
            t = torch.arange(t_q).unsqueeze(1)
            s = torch.arange(S).unsqueeze(0)
            mask = s <= S - t_q + t                                            # [t_q, S]
            o = torch.nn.functional.scaled_dot_product_attention(
                qb.unsqueeze(0), kb.unsqueeze(0), vb.unsqueeze(0), attn_mask=mask, scale=c.scale)
            out[b] = o[0].permute(1, 0, 2).numpy()
            for tt in range(t_q):
                if S - t_q + tt < 0:
                    out[b, tt] = np.nan
        base += S
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("G,h_kv,d,t_q", [(8, 1, 64, 2), (4, 2, 32, 4), (1, 4, 16, 16), (2, 8, 128, 8)])
def test_multi_token_equals_masked_sdpa(G, h_kv, d, t_q, dtype):
    c = host_case(3, G * h_kv, h_kv, d, [37, 3, 130], dtype, seed=200 + t_q, scale=d ** -0.5,
                  t_q=t_q)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    ref = _sdpa_masked_reference(c, G)
    seen = ~np.isnan(ref)
    assert np.abs(got[seen] - ref[seen]).max() <= 1e-12
    # a token that sees no key (S < t_q) gives 0
    assert (got[~seen] == 0).all()
    assert (~seen).any() == (t_q > 3)


def test_multi_token_with_one_token_is_the_single_token_decode():
    c = host_case(3, 8, 2, 32, [17, 0, 64], "bf16", seed=5, t_q=1)
    one = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    flat = oracle.gqa_decode_f64(c.q[:, 0], c.k, c.v, c.seq_lens, c.scale)
    assert one.shape == (3, 1, 8, 32)
    assert np.array_equal(one[:, 0], flat)


def test_last_token_sees_every_key_and_earlier_tokens_see_a_prefix():
    c = host_case(2, 8, 2, 32, [40, 7], "f32", seed=6, t_q=4)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    last = oracle.gqa_decode_f64(np.ascontiguousarray(c.q[:, 3]), c.k, c.v, c.seq_lens, c.scale)
    assert np.array_equal(got[:, 3], last)
    # token 1 of sequence 0 equals a single-token decode over its first 40 - 4 + 2 keys
    sub = oracle.gqa_decode_f64(np.ascontiguousarray(c.q[:1, 1]), c.k[:38], c.v[:38], [38], c.scale)
    assert np.array_equal(got[0, 1], sub[0])


# ---------------------------------------------------------------- causal prefill


def _brute_prefill(c):
    out = []
    base = 0
    for S in c.seq_lens:
        S = int(S)
        if S:
            r = brute_decode(np.ascontiguousarray(c.q[base:base + S])[None], c.k[base:base + S],
                             c.v[base:base + S], [S], c.scale)
            out.append(np.array(r, dtype=np.float64)[0])
        base += S
    return np.concatenate(out) if out else np.zeros(c.q.shape)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("seq_lens", [[1], [3], [2, 0, 4]])
def test_prefill_oracle_matches_decimal_brute_force(dtype, seq_lens):
    c = host_prefill_case(len(seq_lens), 4, 2, 8, seq_lens, dtype, seed=80, scale=0.45)
    got = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    ref = _brute_prefill(c)
    assert got.shape == ref.shape == c.q.shape
    assert np.abs(got - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())


def _sdpa_causal_reference(c, G):
    """torch float64 SDPA per sequence with is_causal=True (query t sees keys <= t),
    kv heads repeated G times."""
    import torch
    q = torch.from_numpy(_f64(c.q))
    k = torch.from_numpy(_f64(c.k))
    v = torch.from_numpy(_f64(c.v))
    out = np.zeros(c.q.shape)
    base = 0
    for S in c.seq_lens:
        S = int(S)
        if S:
            qb = q[base:base + S].permute(1, 0, 2).contiguous()
            kb = k[base:base + S].permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
            vb = v[base:base + S].permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
            o = torch.nn.functional.scaled_dot_product_attention(qb[None], kb[None], vb[None],
                                                                 is_causal=True, scale=c.scale)
            out[base:base + S] = o[0].permute(1, 0, 2).numpy()
        base += S
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("G,h_kv,d", [(8, 1, 64), (4, 2, 32), (1, 4, 16), (16, 1, 32), (3, 2, 16)])
def test_prefill_equals_causal_sdpa(G, h_kv, d, dtype):
    c = host_prefill_case(3, G * h_kv, h_kv, d, [37, 1, 90], dtype, seed=300 + G, scale=d ** -0.5)
    got = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    assert np.abs(got - _sdpa_causal_reference(c, G)).max() <= 1e-12


def test_prefill_rows_equal_full_prefill():
    c = host_prefill_case(3, 8, 2, 32, [40, 1, 70], "bf16", seed=81)
    full = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    rows = [0, 39, 40, 41, 110, 75, 1]
    part = oracle.gqa_prefill_rows_f64(c.q, c.k, c.v, c.seq_lens, c.scale, rows)
    assert np.abs(part - full[rows]).max() <= 1e-15


def test_prefill_first_and_last_tokens():
    c = host_prefill_case(2, 8, 2, 32, [25, 9], "f32", seed=82)
    got = oracle.gqa_prefill_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    v = _f64(c.v)
    for base in (0, 25):
        # the first token sees only its own key: its V row, per kv group
        for h in range(8):
            assert np.array_equal(got[base, h], v[base, h // 4])
    # the last token sees the whole sequence: the single-token decode
    last = oracle.gqa_decode_f64(np.ascontiguousarray(c.q[[24, 33]]), c.k, c.v, c.seq_lens, c.scale)
    assert np.abs(got[[24, 33]] - last).max() <= 1e-15


# ---------------------------------------------------------------- closed forms


def test_zero_query_gives_mean_of_v():
    c = host_case(2, 8, 2, 16, [50, 9], "f32", seed=3)
    q = np.zeros_like(c.q)
    got = oracle.gqa_decode_f64(q, c.k, c.v, c.seq_lens, c.scale)
    v = _f64(c.v)
    assert np.allclose(got[0, :4], v[:50, 0].mean(0), rtol=0, atol=1e-14)
    assert np.allclose(got[0, 4:], v[:50, 1].mean(0), rtol=0, atol=1e-14)
    assert np.allclose(got[1, 4:], v[50:, 1].mean(0), rtol=0, atol=1e-14)


def test_identical_keys_give_mean_of_v():
    c = host_case(1, 4, 1, 16, [33], "bf16", seed=4)
    k = np.repeat(c.k[:1], 33, axis=0)
    got = oracle.gqa_decode_f64(c.q, k, c.v, c.seq_lens, c.scale)
    assert np.allclose(got[0], _f64(c.v)[:, 0].mean(0), rtol=0, atol=1e-14)


def test_constant_v_rows_return_that_row():
    c = host_case(1, 8, 2, 32, [77], "bf16", seed=5)
    v = np.repeat(c.v[:1], 77, axis=0)
    got = oracle.gqa_decode_f64(c.q, c.k, v, c.seq_lens, c.scale)
    row = _f64(c.v)[0]
    assert np.allclose(got[0, :4], row[0], rtol=0, atol=1e-13)
    assert np.allclose(got[0, 4:], row[1], rtol=0, atol=1e-13)


def test_single_key_returns_its_v_row_and_empty_returns_zero():
    c = host_case(3, 4, 2, 8, [1, 0, 1], "f32", seed=6)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    v = _f64(c.v)
    assert np.array_equal(got[0, :2], np.repeat(v[0:1, 0], 2, 0))
    assert np.array_equal(got[0, 2:], np.repeat(v[0:1, 1], 2, 0))
    assert np.array_equal(got[1], np.zeros((4, 8)))
    assert np.array_equal(got[2, 2:], np.repeat(v[1:2, 1], 2, 0))


def test_negative_length_counts_as_empty():
    c = host_case(2, 2, 1, 8, [0, 5], "f32", seed=7)
    sl = np.array([-3, 5], np.int32)
    got = oracle.gqa_decode_f64(c.q, c.k, c.v, sl, c.scale)
    ref = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    assert np.array_equal(got, ref)


def test_dominant_key_returns_its_v_row():
    # q = e_0 * 64, k_t[0] in [-0.5, 0.5] except one key with k[0] = 1: its score
    # leads every other by >= 64*0.5*scale*... > 40, so o = v_t* to within e^-40.
    d, S, t_star = 16, 200, 123
    c = host_case(1, 1, 1, d, [S], "f32", seed=8, scale=1.0)
    q = np.zeros_like(c.q)
    q[0, 0, 0] = 100.0
    rng = np.random.default_rng(0)
    k = np.zeros_like(c.k)
    k[:, 0, 0] = rng.uniform(-0.5, 0.5, S).astype(np.float32)
    k[t_star, 0, 0] = 1.0
    got = oracle.gqa_decode_f64(q, k, c.v, c.seq_lens, 1.0)
    assert np.abs(got[0, 0] - _f64(c.v)[t_star, 0]).max() <= 1e-15 * 200 * 10


# ---------------------------------------------------------------- invariants


def test_softmax_weights_sum_to_one_and_match_output():
    c = host_case(2, 8, 2, 64, [300, 17], "bf16", seed=9)
    out = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    v = _f64(c.v)
    base = [0, 300]
    for b in range(2):
        for h in (0, 5):
            w = oracle.softmax_weights(c.q, c.k, c.seq_lens, c.scale, b, h)
            assert abs(w.sum() - 1.0) <= 1e-14
            assert (w > 0).all()
            S = int(c.seq_lens[b])
            o = w @ v[base[b]:base[b] + S, h // 4]
            assert np.abs(o - out[b, h]).max() <= 1e-14


def test_permuting_key_value_pairs_leaves_output_unchanged():
    c = host_case(1, 4, 1, 32, [97], "bf16", seed=10)
    perm = np.random.default_rng(1).permutation(97)
    a = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    b = oracle.gqa_decode_f64(c.q, c.k[perm], c.v[perm], c.seq_lens, c.scale)
    assert np.abs(a - b).max() <= 1e-14


def test_output_is_linear_in_v():
    c = host_case(1, 4, 2, 16, [41], "f32", seed=11)
    rng = np.random.default_rng(2)
    v1 = rng.integers(-8, 8, c.v.shape).astype(np.float32)
    v2 = rng.integers(-8, 8, c.v.shape).astype(np.float32)
    v3 = (3 * v1 - 2 * v2).astype(np.float32)          # exact in float32
    o1 = oracle.gqa_decode_f64(c.q, c.k, v1, c.seq_lens, c.scale)
    o2 = oracle.gqa_decode_f64(c.q, c.k, v2, c.seq_lens, c.scale)
    o3 = oracle.gqa_decode_f64(c.q, c.k, v3, c.seq_lens, c.scale)
    assert np.abs(o3 - (3 * o1 - 2 * o2)).max() <= 1e-12


# ---------------------------------------------------------------- partition invariance


def _random_partition(S, parts, rng):
    cuts = np.sort(rng.choice(np.arange(0, S + 1), size=parts - 1, replace=True))
    edges = [0] + cuts.tolist() + [S]
    return list(zip(edges[:-1], edges[1:]))


@pytest.mark.parametrize("S,C,sub_w", [(1024, 8, 4), (37, 4, 2), (5, 6, 3), (3000, 16, 4), (64, 8, 2)])
def test_merged_partials_equal_direct_result(S, C, sub_w):
    c = host_case(1, 8, 1, 32, [S], "bf16", seed=S + C, scale=32 ** -0.5)
    direct = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, c.scale)
    rng = np.random.default_rng(S * C)
    for h in (0, 3, 7):
        for trial in range(3):
            ranges = _random_partition(S, C, rng)     # may contain empty ranges
            parts = [oracle.partial_f64(c.q, c.k, c.v, c.seq_lens, c.scale, 0, h, a, b)
                     for a, b in ranges]
            for red in (M.chain(parts), M.center_root(parts, sub_w)):
                assert np.abs(M.finish(red) - direct[0, h]).max() <= 1e-12


def test_tile_sweep_of_1024_keys_equals_direct_result():
    # The page's own sweep: tile 0 establishes (m, l, O), tiles 1..n-1 fold in with
    # the running merge; 1024-key tiles with a ragged last tile.
    S = 3 * 1024 + 77
    c = host_case(1, 8, 1, 64, [S], "bf16", seed=21, scale=1.0)
    direct = oracle.gqa_decode_f64(c.q, c.k, c.v, c.seq_lens, 1.0)
    for h in (0, 7):
        run = oracle.partial_f64(c.q, c.k, c.v, c.seq_lens, 1.0, 0, h, 0, 1024)
        for t in range(1024, S, 1024):
            tile = oracle.partial_f64(c.q, c.k, c.v, c.seq_lens, 1.0, 0, h, t, min(S, t + 1024))
            run = M.merge_pair(run, tile)
        assert np.abs(M.finish(run) - direct[0, h]).max() <= 1e-12


def test_merge_identity_and_order():
    d = 4
    rng = np.random.default_rng(3)
    a = (0.3, 2.0, rng.standard_normal(d))
    b = (1.7, 0.5, rng.standard_normal(d))
    e = M.identity(d)
    for x in (M.merge_pair(a, e), M.merge_pair(e, a)):
        assert x[0] == a[0] and x[1] == a[1] and np.array_equal(x[2], a[2])
    ee = M.merge_pair(e, e)
    assert ee[0] == -math.inf and ee[1] == 0.0 and not np.isnan(ee[2]).any()
    ab, ba = M.merge_pair(a, b), M.merge_pair(b, a)
    assert abs(ab[0] - ba[0]) == 0 and abs(ab[1] - ba[1]) <= 1e-15
    assert np.allclose(ab[2], ba[2], rtol=0, atol=1e-15)
    # by hand: m = 1.7, l = 2 e^{-1.4} + 0.5
    assert abs(ab[1] - (2.0 * math.exp(-1.4) + 0.5)) <= 1e-15
    with pytest.raises(ValueError):
        M.center_root([a] * 4, 4)        # 4x1 is degenerate


# ---------------------------------------------------------------- planted mistakes


def _definition(q, k, v, seq_lens, scale, mutate=None):
    """Plain numpy copy of the definition with optional planted mistakes (test only)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    batch, h_q, d = q.shape
    h_kv = k.shape[1]
    G = h_q // h_kv
    out = np.zeros((batch, h_q, d))
    base = 0
    for b in range(batch):
        S = int(seq_lens[b])
        for h in range(h_q):
            j = h % h_kv if mutate == "head_modulo" else h // G
            if S == 0:
                continue
            K = k[base:base + S, j]
            V = v[base:base + S, j]
            if mutate == "reshape_k":
                K = K.reshape(-1).reshape(d, S).T
            s = K @ q[b, h]
            if mutate != "no_scale":
                s = s * scale
            if mutate == "sign":
                s = -s
            w = np.exp(s - s.max())
            if mutate == "drop_last_key":
                w[-1] = 0.0
            if mutate == "normalise_by_count":
                out[b, h] = (w @ V) / S
            else:
                out[b, h] = (w @ V) / w.sum()
        base += S
    return out


def _pins(fn):
    """Pins from this file applied to an implementation; True if all hold."""
    ok = True
    c = host_case(2, 4, 2, 8, [5, 3], "f32", seed=31, scale=0.7)
    ok &= np.abs(fn(c.q, c.k, c.v, c.seq_lens, c.scale)
                 - np.array(brute_decode(c.q, c.k, c.v, c.seq_lens, c.scale), float)).max() < 1e-12
    c2 = host_case(2, 8, 2, 16, [19, 4], "bf16", seed=32, scale=0.25)
    ok &= np.abs(fn(c2.q, c2.k, c2.v, c2.seq_lens, c2.scale) - _sdpa_reference(c2, 4)).max() < 1e-12
    return bool(ok)


def test_pins_catch_planted_mistakes():
    assert _pins(_definition)
    assert _pins(lambda *a: oracle.gqa_decode_f64(*a))
    for mut in ("head_modulo", "reshape_k", "no_scale", "sign", "drop_last_key",
                "normalise_by_count"):
        assert not _pins(lambda *a, m=mut: _definition(*a, mutate=m)), mut


def _definition_tq(q, k, v, seq_lens, scale, mutate=None):
    """Multi-token definition built on _definition, with planted mistakes (test only)."""
    batch, t_q = q.shape[:2]
    out = np.zeros(q.shape)
    base = 0
    for b in range(batch):
        S = int(seq_lens[b])
        for t in range(t_q):
            if mutate == "mask_off_by_one":
                St = max(0, min(S, S - t_q + t))
            elif mutate == "mask_reversed":
                St = max(0, min(S, S - t)) if S >= t_q else max(0, min(S, S - t_q + t + 1))
            elif mutate == "no_mask":
                St = S
            else:
                St = max(0, min(S, S - t_q + t + 1))
            qt = q[b:b + 1, t]
            if mutate == "token_swap":
                qt = q[b:b + 1, t_q - 1 - t]
            out[b, t] = _definition(qt, k[base:base + St], v[base:base + St], [St], scale)[0]
        base += S
    return out


def _pins_tq(fn):
    c = host_case(2, 4, 2, 8, [6, 2], "f32", seed=41, scale=0.6, t_q=3)
    ok = np.abs(fn(c.q, c.k, c.v, c.seq_lens, c.scale)
                - np.array(brute_decode(c.q, c.k, c.v, c.seq_lens, c.scale), float)).max() < 1e-12
    c2 = host_case(3, 8, 2, 16, [37, 3, 130], "bf16", seed=42, scale=0.25, t_q=4)
    ref = _sdpa_masked_reference(c2, 4)
    got = fn(c2.q, c2.k, c2.v, c2.seq_lens, c2.scale)
    seen = ~np.isnan(ref)
    ok &= np.abs(got[seen] - ref[seen]).max() < 1e-12 and (got[~seen] == 0).all()
    return bool(ok)


def _definition_prefill(q, k, v, seq_lens, scale, mutate=None):
    """Causal prefill from _definition_tq (t_q = S per sequence), with planted mistakes."""
    out = np.zeros(q.shape)
    base = 0
    for S in seq_lens:
        S = int(S)
        if S:
            qb = q[base:base + S][None]
            out[base:base + S] = _definition_tq(qb, k[base:base + S], v[base:base + S], [S], scale,
                                                mutate=mutate)[0]
        base += S
    return out


def _pins_prefill(fn):
    c = host_prefill_case(2, 4, 2, 8, [5, 3], "f32", seed=51, scale=0.6)
    ok = np.abs(fn(c.q, c.k, c.v, c.seq_lens, c.scale) - _brute_prefill(c)).max() < 1e-12
    c2 = host_prefill_case(3, 8, 2, 16, [37, 1, 60], "bf16", seed=52, scale=0.25)
    ok &= np.abs(fn(c2.q, c2.k, c2.v, c2.seq_lens, c2.scale) - _sdpa_causal_reference(c2, 4)).max() < 1e-12
    return bool(ok)


def test_prefill_pins_catch_planted_mistakes():
    assert _pins_prefill(_definition_prefill)
    assert _pins_prefill(lambda *a: oracle.gqa_prefill_f64(*a))
    for mut in ("mask_off_by_one", "mask_reversed", "no_mask", "token_swap"):
        assert not _pins_prefill(lambda *a, m=mut: _definition_prefill(*a, mutate=m)), mut


def test_multi_token_pins_catch_planted_mistakes():
    assert _pins_tq(_definition_tq)
    assert _pins_tq(lambda *a: oracle.gqa_decode_f64(*a))
    for mut in ("mask_off_by_one", "mask_reversed", "no_mask", "token_swap"):
        assert not _pins_tq(lambda *a, m=mut: _definition_tq(*a, mutate=m)), mut


def test_bf16_rounding_helper_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    want = np.array([1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5, 2.9996e38], np.float32)
    assert np.array_equal(got[:5], want[:5])
    import torch
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(4096).astype(np.float32))
    assert np.array_equal(f32_to_bf16_bits(t.numpy()),
                          t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
