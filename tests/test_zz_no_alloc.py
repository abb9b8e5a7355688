"""gqa_decode_noalloc -- the decode entry point that allocates nothing (its
partials live in the library's own device scratch array) -- against
gqa_decode_ex on the same inputs and plan, through the C ABI, on an MI355X.

Two calls in a row, the second with a smaller input, each bit-identical to
gqa_decode_ex (same kernels, same plan) and within the method's tolerance of the
fp64 oracle; the scratch array keeps the first call's contents, so the second
call also shows that nothing in it has to be cleared.  Oversized plans and a
caller workspace are refused before anything is enqueued.
"""
import numpy as np
import pytest

from gqa_split_kv_amd import binding as B
from gqa_split_kv_amd.inputs import host_case, to_host_bits

from helpers import compare, oracle_of, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need an MI355X GPU"
    B.lib()
    yield


def _say(*a):
    print(*a, flush=True)


def _run(fn, c, q, k, v, sl, out_dtype, num_chunks, min_chunk, t_q):
    import torch
    stream = int(torch.cuda.current_stream().cuda_stream)
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=q.device)
    code_in = {torch.bfloat16: B.GQA_DTYPE_BF16, torch.float16: B.GQA_DTYPE_F16, torch.float32: B.GQA_DTYPE_F32}
    a = B.make_args(q, k, v, out, sl, q.shape[0], q.shape[-2], k.shape[1], q.shape[-1], c.scale,
                    code_in[q.dtype], code_in[out_dtype], num_chunks, min_chunk, None, 0, stream, t_q=t_q)
    fn(a)
    torch.cuda.synchronize()
    return out


CASES = [
    # (batch, h_q, h_kv, d, lengths, dtype, t_q, out dtype, num_chunks, min_chunk)
    (5, 32, 8, 128, [3000, 17, 0, 800, 4100], "bf16", 0, "bf16", 0, 0),
    (2, 32, 8, 128, [100, 37], "bf16", 2, "f32", 0, 0),
]


@pytest.mark.parametrize("plan", [(0, 0), (64, 16)])
def test_noalloc_matches_decode_ex_on_two_calls(plan):
    import torch
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}
    for i, (batch, h_q, h_kv, d, lens, dtype, t_q, odt, _, _) in enumerate(CASES):
        nc, mc = plan
        _say("noalloc call %d: batch %d h_q %d h_kv %d d %d lens %s t_q %d out %s plan %s" %
             (i, batch, h_q, h_kv, d, lens, t_q, odt, plan))
        c = host_case(batch, h_q, h_kv, d, lens, dtype, seed=4100 + i, t_q=t_q)
        ref = oracle_of(c)
        q, k, v, sl = upload(c)
        got = _run(B.gqa_decode_noalloc, c, q, k, v, sl, dt[odt], nc, mc, t_q)
        want = _run(B.gqa_decode_ex, c, q, k, v, sl, dt[odt], nc, mc, t_q)
        g, w = to_host_bits(got), to_host_bits(want)
        assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), "call %d: not bit-identical to gqa_decode_ex" % i
        compare(got, ref, "noalloc call %d" % i)


def test_noalloc_f32_and_f16():
    import torch
    for dtype, tdt in (("f32", torch.float32), ("f16", torch.float16)):
        _say("noalloc", dtype)
        c = host_case(3, 16, 2, 64, [513, 1, 2049], dtype, seed=4200)
        ref = oracle_of(c)
        q, k, v, sl = upload(c)
        got = _run(B.gqa_decode_noalloc, c, q, k, v, sl, tdt, 0, 0, 0)
        want = _run(B.gqa_decode_ex, c, q, k, v, sl, tdt, 0, 0, 0)
        assert np.array_equal(to_host_bits(got).view(np.uint8), to_host_bits(want).view(np.uint8))
        compare(got, ref, "noalloc " + dtype)


def test_noalloc_refuses_what_it_cannot_hold():
    import torch
    c = host_case(2, 64, 8, 128, [300, 200], "bf16", seed=4300, t_q=4)   # 32 rows per kv head
    q, k, v, sl = upload(c)
    stream = int(torch.cuda.current_stream().cuda_stream)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    a = B.make_args(q, k, v, out, sl, 2, 64, 8, 128, c.scale, B.GQA_DTYPE_BF16, B.GQA_DTYPE_BF16, 0, 0, None, 0,
                    stream, t_q=4)
    st = B.lib().gqa_decode_noalloc(a)
    assert st == B.GQA_ERR_WORKSPACE, B.status_str(st)
    assert "scratch" in B.last_error_message()
    # a smaller wavefront count fits, and gives gqa_decode_ex's result
    a.num_chunks = 256
    B.gqa_decode_noalloc(a)
    torch.cuda.synchronize()
    want = _run(B.gqa_decode_ex, c, q, k, v, sl, torch.bfloat16, 256, 0, 4)
    assert np.array_equal(to_host_bits(out), to_host_bits(want))
    compare(out, oracle_of(c), "noalloc 32 rows, 256 wavefronts")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    before = to_host_bits(out).copy()
    assert B.lib().gqa_decode_noalloc(a) == B.GQA_ERR_ARG
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(out), before)
