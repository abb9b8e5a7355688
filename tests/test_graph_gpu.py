"""Decode and prefill captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI).

The headers state that a call with a caller-provided workspace enqueues only
kernel launches, so it can be captured.  Each test captures one call, then
replays the graph several times with eager work in between (new query values
written in place, an eager call of the same operation, synchronisations), and
requires every replay's output to equal, bit for bit, the eager call on the
same inputs: both run the same kernels with the same plan, and neither has a
data-dependent reduction order.  The eager calls themselves are held to the
oracle by the parity tests.
"""
import pytest

from gqa_split_kv_amd import binding as B
from gqa_split_kv_amd.inputs import device_case, device_prefill_case, device_queries

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "these tests need an MI355X GPU"
    B.lib()
    yield


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("merge", [B.GQA_MERGE_KERNEL, B.GQA_MERGE_FUSED], ids=["kernel", "fused"])
@pytest.mark.parametrize("t_q", [0, 2])
def test_decode_graph_replays_equal_eager(t_q, merge):
    import torch
    lens = [3000, 1, 0, 777, 65]
    c = device_case(len(lens), 32, 4, 128, lens, "bf16", seed=41, t_q=t_q)
    _say("decode graph: lens", lens, "t_q", t_q, "merge", merge)
    out = torch.empty(c.q.shape, dtype=torch.float32, device="cuda")
    args = B.make_args(c.q, c.k, c.v, out, c.seq_lens, len(lens), 32, 4, 128, c.scale, B.GQA_DTYPE_BF16,
                       B.GQA_DTYPE_F32, t_q=t_q, merge=merge)
    # Zero-filled once: the fused merge's counters must read zero before the first call.
    ws = torch.zeros(B.gqa_decode_workspace_bytes(args), dtype=torch.uint8, device="cuda")
    # Eager call first: the library caches the device's shape outside the capture.
    B.decode(c.q, c.k, c.v, c.seq_lens, scale=c.scale, out=out, workspace=ws, merge=merge)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.decode(c.q, c.k, c.v, c.seq_lens, scale=c.scale, out=out, workspace=ws, merge=merge)
    torch.cuda.synchronize()
    qshape = (len(lens), max(t_q, 1), 32, 128)
    for r in range(REPLAYS):
        c.q.copy_(device_queries(len(lens), max(t_q, 1), 32, 128, "bf16", seed=100 + r).reshape(c.q.shape))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = B.decode(c.q, c.k, c.v, c.seq_lens, scale=c.scale, out_dtype=torch.float32, merge=merge)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), "replay %d left unwritten outputs" % r
        assert torch.equal(out, ref), "replay %d differs from the eager call (%s)" % (r, qshape)
        assert (ws[:B.GQA_DECODE_COUNTER_BYTES].view(torch.int32) == 0).all().item()
    del g


@pytest.mark.parametrize("split_pv,num_blocks", [(0, 0), (1, 0), (0, 16)])
def test_prefill_graph_replays_equal_eager(split_pv, num_blocks):
    """With 16 workgroups the 60 tiles take four rounds, the last from the tile
    queue's counter, which every replay's V copy must zero again."""
    import torch
    lens = [1500, 77, 300]
    c = device_prefill_case(len(lens), 8, 1, 128, lens, "bf16", seed=43)
    _say("prefill graph: lens", lens, "split_pv", split_pv, "num_blocks", num_blocks)
    out = torch.empty(c.q.shape, dtype=torch.float32, device="cuda")
    total = c.q.shape[0]
    args = B.make_prefill_args(c.q, c.k, c.v, out, c.seq_lens, len(lens), 8, 1, 128, c.scale, B.GQA_DTYPE_BF16,
                               B.GQA_DTYPE_F32, split_pv=split_pv, total_tokens=total)
    ws = torch.empty(max(B.gqa_prefill_workspace_bytes(args), 1), dtype=torch.uint8, device="cuda")
    B.prefill(c.q, c.k, c.v, c.seq_lens, scale=c.scale, out=out, split_pv=split_pv, workspace=ws,
              num_blocks=num_blocks)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.prefill(c.q, c.k, c.v, c.seq_lens, scale=c.scale, out=out, split_pv=split_pv, workspace=ws,
                  num_blocks=num_blocks)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        # New queries and new values (the replay must rebuild the transposed V copy).
        c.q.copy_(device_prefill_case(len(lens), 8, 1, 128, lens, "bf16", seed=200 + r).q)
        c.v.copy_(device_prefill_case(len(lens), 8, 1, 128, lens, "bf16", seed=300 + r).v)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = B.prefill(c.q, c.k, c.v, c.seq_lens, scale=c.scale, out_dtype=torch.float32, split_pv=split_pv)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), "replay %d left unwritten outputs" % r
        assert torch.equal(out, ref), "replay %d differs from the eager call" % r
    del g
