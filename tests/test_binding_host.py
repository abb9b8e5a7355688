"""The convenience wrappers' tensor checks (binding.decode / binding.prefill), on
the host: every malformed call raises before the library is called.  CPU tensors
stand in for device tensors by switching the accepted device type to "cpu"; the
library entry points are replaced by a recorder, so nothing reaches a device.
"""
import pytest
import torch

from gqa_split_kv_amd import binding as B


@pytest.fixture
def host_binding(monkeypatch):
    calls = []
    monkeypatch.setattr(B, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(B, "_stream", lambda s: 0)
    monkeypatch.setattr(B, "gqa_decode_ex", lambda a: calls.append(("decode", a)) or 0)
    monkeypatch.setattr(B, "gqa_prefill_ex", lambda a: calls.append(("prefill", a)) or 0)
    return calls


def _decode_case(dtype=torch.bfloat16, batch=3, h_q=8, h_kv=2, d=128, rows=40, t_q=0):
    qshape = (batch, t_q, h_q, d) if t_q else (batch, h_q, d)
    q = torch.zeros(qshape, dtype=dtype)
    k = torch.zeros((rows, h_kv, d), dtype=dtype)
    v = torch.zeros((rows, h_kv, d), dtype=dtype)
    sl = torch.tensor([10, 20, 10][:batch] + [0] * max(0, batch - 3), dtype=torch.int32)
    return q, k, v, sl


def test_decode_well_formed_call_reaches_the_library(host_binding):
    q, k, v, sl = _decode_case()
    out = B.decode(q, k, v, sl)
    assert out.shape == q.shape and out.dtype == q.dtype
    out32 = B.decode(q, k, v, sl, out_dtype=torch.float32)
    assert out32.dtype == torch.float32
    q4, k4, v4, sl4 = _decode_case(t_q=3)
    B.decode(q4, k4, v4, sl4, out=torch.empty(q4.shape, dtype=torch.float32))
    assert [c[0] for c in host_binding] == ["decode"] * 3
    assert host_binding[2][1].t_q == 3


@pytest.mark.parametrize("mutate, match", [
    (lambda q, k, v, sl: (q.float(), k, v, sl), "one dtype"),
    (lambda q, k, v, sl: (q, k.half(), v, sl), "one dtype"),
    (lambda q, k, v, sl: (q.to(torch.int16), k.to(torch.int16), v.to(torch.int16), sl), "bfloat16, float16 or float32"),
    (lambda q, k, v, sl: (q, k[:, :1].contiguous(), v, sl), "one shape"),
    (lambda q, k, v, sl: (q, k[:, :, :64].contiguous(), v[:, :, :64].contiguous(), sl), "d_head"),
    (lambda q, k, v, sl: (q, k.transpose(0, 1).contiguous().transpose(0, 1), v, sl), "contiguous"),
    (lambda q, k, v, sl: (q.transpose(0, 1).contiguous().transpose(0, 1), k, v, sl), "contiguous"),
    (lambda q, k, v, sl: (q, k, v, sl.long()), "int32"),
    (lambda q, k, v, sl: (q, k, v, [10, 20, 10]), "int32"),
    (lambda q, k, v, sl: (q, k, v, sl[:2]), "holds 2 lengths"),
    (lambda q, k, v, sl: (q, k, v, torch.tensor([1, 2, 3, 4, 5, 6], dtype=torch.int32)[::2]), "contiguous"),
])
def test_decode_rejects_malformed_tensors(host_binding, mutate, match):
    q, k, v, sl = mutate(*_decode_case())
    with pytest.raises((ValueError, TypeError), match=match):
        B.decode(q, k, v, sl)
    assert host_binding == []


def test_decode_rejects_a_bad_out(host_binding):
    q, k, v, sl = _decode_case()
    for out, match in [(torch.empty((3, 8, 64), dtype=q.dtype), "q's shape"),
                       (torch.empty(q.shape, dtype=torch.float16), "float32"),
                       (torch.empty((8, 3, 128), dtype=q.dtype).transpose(0, 1), "contiguous"),
                       ("not a tensor", "torch.Tensor")]:
        with pytest.raises((ValueError, TypeError), match=match):
            B.decode(q, k, v, sl, out=out)
    with pytest.raises(ValueError, match="out_dtype"):
        B.decode(q, k, v, sl, out_dtype=torch.float16)
    assert host_binding == []


def test_decode_rejects_tensors_off_the_device(monkeypatch, host_binding):
    q, k, v, sl = _decode_case()
    monkeypatch.setattr(B, "_DEVICE_TYPE", "cuda")
    with pytest.raises(ValueError, match="HIP device"):
        B.decode(q, k, v, sl)
    assert host_binding == []


def test_decode_rejects_a_bad_workspace(host_binding):
    q, k, v, sl = _decode_case()
    with pytest.raises(TypeError, match="workspace"):
        B.decode(q, k, v, sl, workspace=12345)
    with pytest.raises(ValueError, match="workspace"):
        B.decode(q, k, v, sl, workspace=torch.zeros(512, dtype=torch.uint8)[::2])
    assert host_binding == []


def _prefill_case(dtype=torch.bfloat16, h_q=8, h_kv=1, d=128, lens=(30, 10)):
    rows = sum(lens)
    q = torch.zeros((rows, h_q, d), dtype=dtype)
    k = torch.zeros((rows, h_kv, d), dtype=dtype)
    v = torch.zeros((rows, h_kv, d), dtype=dtype)
    return q, k, v, torch.tensor(lens, dtype=torch.int32)


def test_prefill_checks(host_binding):
    q, k, v, sl = _prefill_case()
    B.prefill(q, k, v, sl)
    assert host_binding[-1][1].total_tokens == 40
    B.prefill(q, k, v, sl, total_tokens=0)
    n = len(host_binding)
    bad = [
        (lambda: B.prefill(q, k.float(), v, sl), "one dtype"),
        (lambda: B.prefill(q[:20], k, v, sl), "rows"),
        (lambda: B.prefill(q, k, v[:, :, :64].contiguous(), sl), "one shape"),
        (lambda: B.prefill(q, k, v, sl.long()), "int32"),
        (lambda: B.prefill(q, k, v, sl, out=torch.empty((40, 8, 64), dtype=q.dtype)), "q's shape"),
        (lambda: B.prefill(q, k, v, sl, total_tokens=41), "total_tokens"),
        (lambda: B.prefill(q, k, v, sl, total_tokens=-1), "total_tokens"),
        (lambda: B.prefill(q.transpose(0, 1).contiguous().transpose(0, 1), k, v, sl), "contiguous"),
        (lambda: B.prefill(q, k, v, sl, out_dtype=torch.float16), "out_dtype"),
    ]
    for call, match in bad:
        with pytest.raises((ValueError, TypeError), match=match):
            call()
    assert len(host_binding) == n
