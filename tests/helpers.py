"""Shared helpers of the GPU tests: run the HIP path through the C ABI, run the
oracle on the same inputs, and compare them to the tolerance stated for the
method (16-bit inputs, fp32 accumulation: max |err| <= 2e-3 and relative L2 <=
1e-3 on the fp32 result; a bf16 or fp16 result is held to the nearest-even
rounding of the oracle in its format: within one ulp of it or 1e-5, and
relative L2 <= 1e-3).
"""
from __future__ import annotations

import numpy as np

import oracle
from gqa_split_kv_amd import binding as B
from gqa_split_kv_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, from_host_bits, to_host_bits

MAX_ABS = 2e-3
REL_L2 = 1e-3


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.sqrt((b * b).sum())
    return float(np.sqrt(((a - b) ** 2).sum()) / den) if den > 0 else float(np.sqrt((a * a).sum()))


def bf16_ordinal(bits: np.ndarray) -> np.ndarray:
    """Maps bf16 bit patterns to integers that step by one per representable value."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_f32(got: np.ndarray, ref: np.ndarray, what: str = ""):
    err = np.abs(got.astype(np.float64) - ref)
    r = rel_l2(got, ref)
    assert np.isfinite(got).all(), what + ": non-finite output"
    assert err.max() <= MAX_ABS and r <= REL_L2, "%s: max|err| %.3g rel-L2 %.3g" % (what, err.max(), r)
    return float(err.max()), r


BF16_ABS_SLACK = 1e-5


def check_bf16(got_bits: np.ndarray, ref: np.ndarray, what: str = "", slack: float = None):
    """Each element within one bf16 ulp of RNE-bf16(oracle), or within `slack`
    (default 1e-5) of it (near zero the fp32 accumulation error, ~1e-7, exceeds
    the bf16 spacing, so a one-ulp rule alone would reject correct results);
    rel-L2 <= 1e-3.  A path whose fp32 result carries more error than fp32
    accumulation alone passes its own error bound as the slack."""
    slack = BF16_ABS_SLACK if slack is None else slack
    want = f32_to_bf16_bits(ref.astype(np.float32))
    steps = np.abs(bf16_ordinal(got_bits) - bf16_ordinal(want))
    got = bf16_bits_to_f32(got_bits).astype(np.float64)
    want_f = bf16_bits_to_f32(want).astype(np.float64)
    assert np.isfinite(got).all(), what + ": non-finite output"
    ok = (steps <= 1) | (np.abs(got - want_f) <= slack)
    r = rel_l2(got, want_f)
    bad = int((~ok).sum())
    assert bad == 0 and r <= REL_L2, "%s: %d elements beyond 1 ulp and %.0e; rel-L2 %.3g" % (
        what, bad, slack, r)
    big = np.abs(want_f) >= 1e-3
    return int(steps[big].max()) if big.any() else 0, r, rel_l2(got, ref)


# Merge form the decode helpers request (B.GQA_MERGE_*); a test module may set it
# per test to run its cases through both the two-kernel and the fused form.
MERGE = B.GQA_MERGE_AUTO


def run_hip(q, k, v, seq_lens, scale, out_dtype=None, num_chunks=0, min_chunk=0, poison=True,
            workspace=None, stream=None, merge=None, max_seq_len=0):
    """Device tensors in; the decode output tensor (synchronised) out."""
    import torch
    out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if poison:
        out.fill_(float("nan"))
    B.decode(q, k, v, seq_lens, scale=scale, out=out, num_chunks=num_chunks, min_chunk=min_chunk,
             workspace=workspace, stream=stream, merge=MERGE if merge is None else merge,
             max_seq_len=max_seq_len)
    torch.cuda.synchronize()
    return out


def upload(case, device="cuda"):
    """Host case -> device tensors.  An all-empty batch still gets one (unread) K/V
    row so the pointers are real allocations."""
    import torch
    k, v = case.k, case.v
    if k.shape[0] == 0:
        k = np.zeros((1,) + k.shape[1:], k.dtype)
        v = np.zeros((1,) + v.shape[1:], v.dtype)
    return (from_host_bits(case.q, device), from_host_bits(k, device), from_host_bits(v, device),
            torch.from_numpy(np.ascontiguousarray(case.seq_lens, np.int32)).to(device))


def out_host(t) -> np.ndarray:
    """Device output as float32 values, or uint16 bits for bf16."""
    return to_host_bits(t)


def oracle_of(case) -> np.ndarray:
    return oracle.gqa_decode_f64(case.q, case.k, case.v, case.seq_lens, case.scale)


def check_f16(got: np.ndarray, ref: np.ndarray, what: str = "", slack: float = None):
    """fp16 result: each element within one fp16 ulp of the nearest-even fp16
    rounding of the oracle, or within `slack` (default 1e-5) of it; rel-L2 <= 1e-3
    against it."""
    slack = BF16_ABS_SLACK if slack is None else slack
    want = ref.astype(np.float16)              # one rounding, nearest even
    steps = np.abs(bf16_ordinal(got.view(np.uint16)) - bf16_ordinal(want.view(np.uint16)))
    g = got.astype(np.float64)
    wf = want.astype(np.float64)
    assert np.isfinite(g).all(), what + ": non-finite output"
    ok = (steps <= 1) | (np.abs(g - wf) <= slack)
    r = rel_l2(g, wf)
    bad = int((~ok).sum())
    assert bad == 0 and r <= REL_L2, "%s: %d elements beyond 1 ulp and %.0e; rel-L2 %.3g" % (
        what, bad, slack, r)
    big = np.abs(wf) >= 1e-3
    return int(steps[big].max()) if big.any() else 0, r, rel_l2(g, ref)


def compare(out_t, ref: np.ndarray, what: str = "", slack: float = None):
    """Checks a device result against the oracle with the rule of its dtype;
    `slack` widens the 16-bit per-element rule (see check_bf16)."""
    import torch
    h = out_host(out_t)
    if out_t.dtype == torch.bfloat16:
        return check_bf16(h, ref, what, slack)
    if out_t.dtype == torch.float16:
        return check_f16(h, ref, what, slack)
    return check_f32(h, ref, what)
