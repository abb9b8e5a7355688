"""ctypes binding of libgqa_decode.so (include/gqa_decode.h, include/gqa_prefill.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and every step of the decode runs in the HIP
kernels behind the C ABI.  There is no fallback: if the library is missing or
was not built, calls raise.

Functions with the C names take raw pointers or tensors exactly as the C ABI
does; `decode` and `prefill` are the convenience wrappers that allocate the
output tensor.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgqa_decode.so")

GQA_DTYPE_BF16 = 0
GQA_DTYPE_F32 = 1
GQA_DTYPE_F16 = 2

GQA_MERGE_AUTO = 0
GQA_MERGE_KERNEL = 1
GQA_MERGE_FUSED = 2
GQA_DECODE_COUNTER_BYTES = 64 * 1024

GQA_OK = 0
GQA_ERR_NULL = 1
GQA_ERR_SHAPE = 2
GQA_ERR_UNSUPPORTED = 3
GQA_ERR_ALIGN = 4
GQA_ERR_SCALE = 5
GQA_ERR_WORKSPACE = 6
GQA_ERR_HIP = 7
GQA_ERR_ARG = 8

# Every function include/gqa_decode.h, include/gqa_prefill.h and include/gqa_probe.h declare.
EXPORTS = ("gqa_decode", "gqa_decode_f32", "gqa_decode_f16", "gqa_decode_ex", "gqa_decode_noalloc",
           "gqa_decode_validate",
           "gqa_decode_make_plan", "gqa_decode_workspace_bytes", "gqa_status_str",
           "gqa_last_error_message", "gqa_release", "gqa_prefill", "gqa_prefill_f16", "gqa_prefill_ex",
           "gqa_prefill_validate", "gqa_prefill_workspace_bytes", "gqa_probe_copy", "gqa_probe_read")


class GqaArgs(ctypes.Structure):
    """Mirror of gqa_decode_args."""
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("d_head", ctypes.c_int32), ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("num_chunks", ctypes.c_int32), ("min_chunk", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("sweep_events", ctypes.c_void_p * 2),
        ("t_q", ctypes.c_int32),
        ("merge", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
    ]


class GqaPlan(ctypes.Structure):
    """Mirror of gqa_decode_plan."""
    _fields_ = [
        ("num_chunks", ctypes.c_int32), ("min_chunk", ctypes.c_int32),
        ("split_blocks", ctypes.c_int32), ("merge_blocks", ctypes.c_int32),
        ("merge_threads", ctypes.c_int32), ("merge_slices", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("fused", ctypes.c_int32), ("fold_fanin", ctypes.c_int32), ("fold_levels", ctypes.c_int32),
    ]


class GqaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (status_str(status), message))
        self.status = status


_lib = None


class GqaPrefillArgs(ctypes.Structure):
    """Mirror of gqa_prefill_args."""
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("d_head", ctypes.c_int32), ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("stream", ctypes.c_void_p),
        ("split_pv", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgqa_decode.so is not built: run `python -m gqa_split_kv_amd.build` "
                           "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    sig = [P, P, P, P, P, i32, i32, i32, i32, ctypes.c_float, P]
    L.gqa_decode.argtypes = sig
    L.gqa_decode.restype = ctypes.c_int
    L.gqa_decode_f32.argtypes = sig
    L.gqa_decode_f32.restype = ctypes.c_int
    L.gqa_decode_f16.argtypes = sig
    L.gqa_decode_f16.restype = ctypes.c_int
    L.gqa_decode_ex.argtypes = [ctypes.POINTER(GqaArgs)]
    L.gqa_decode_ex.restype = ctypes.c_int
    L.gqa_decode_noalloc.argtypes = [ctypes.POINTER(GqaArgs)]
    L.gqa_decode_noalloc.restype = ctypes.c_int
    L.gqa_decode_validate.argtypes = [ctypes.POINTER(GqaArgs)]
    L.gqa_decode_validate.restype = ctypes.c_int
    L.gqa_decode_make_plan.argtypes = [ctypes.POINTER(GqaArgs), i32, i32, ctypes.POINTER(GqaPlan)]
    L.gqa_decode_make_plan.restype = ctypes.c_int
    L.gqa_decode_workspace_bytes.argtypes = [ctypes.POINTER(GqaArgs), ctypes.POINTER(ctypes.c_size_t)]
    L.gqa_decode_workspace_bytes.restype = ctypes.c_int
    L.gqa_status_str.argtypes = [ctypes.c_int]
    L.gqa_status_str.restype = ctypes.c_char_p
    L.gqa_last_error_message.argtypes = []
    L.gqa_last_error_message.restype = ctypes.c_char_p
    L.gqa_release.argtypes = []
    L.gqa_release.restype = None
    L.gqa_prefill.argtypes = [P, P, P, P, P, i32, ctypes.c_int64, i32, i32, i32, ctypes.c_float, P]
    L.gqa_prefill.restype = ctypes.c_int
    L.gqa_prefill_f16.argtypes = [P, P, P, P, P, i32, ctypes.c_int64, i32, i32, i32, ctypes.c_float, P]
    L.gqa_prefill_f16.restype = ctypes.c_int
    L.gqa_prefill_ex.argtypes = [ctypes.POINTER(GqaPrefillArgs)]
    L.gqa_prefill_ex.restype = ctypes.c_int
    L.gqa_prefill_validate.argtypes = [ctypes.POINTER(GqaPrefillArgs)]
    L.gqa_prefill_validate.restype = ctypes.c_int
    L.gqa_prefill_workspace_bytes.argtypes = [ctypes.POINTER(GqaPrefillArgs), ctypes.POINTER(ctypes.c_size_t)]
    L.gqa_prefill_workspace_bytes.restype = ctypes.c_int
    L.gqa_probe_copy.argtypes = [P, P, ctypes.c_size_t, P]
    L.gqa_probe_copy.restype = ctypes.c_int
    L.gqa_probe_read.argtypes = [P, ctypes.c_size_t, P, P]
    L.gqa_probe_read.restype = ctypes.c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().gqa_status_str(int(status)).decode()


def last_error_message() -> str:
    return lib().gqa_last_error_message().decode()


def _check(status: int) -> None:
    if status != GQA_OK:
        raise GqaError(status, last_error_message())


def _ptr(x) -> Optional[int]:
    """A tensor's device address, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GQA_DTYPE_BF16
    if t.dtype == torch.float32:
        return GQA_DTYPE_F32
    if t.dtype == torch.float16:
        return GQA_DTYPE_F16
    raise TypeError("q/k/v/o must be bfloat16, float16 or float32 tensors, got %s" % t.dtype)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# ------------------------------------------------------------------ the C names


def gqa_decode(q, k, v, o, seq_lens, batch: int, h_q: int, h_kv: int, d_head: int, scale: float,
               stream=None) -> int:
    """bf16 in / bf16 out.  Raises GqaError on a non-zero status; returns 0."""
    st = lib().gqa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens), batch, h_q, h_kv,
                          d_head, float(scale), _stream(stream))
    _check(st)
    return st


def gqa_decode_f32(q, k, v, o, seq_lens, batch: int, h_q: int, h_kv: int, d_head: int,
                   scale: float, stream=None) -> int:
    """fp32 in / fp32 out."""
    st = lib().gqa_decode_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens), batch, h_q, h_kv,
                              d_head, float(scale), _stream(stream))
    _check(st)
    return st


def gqa_decode_f16(q, k, v, o, seq_lens, batch: int, h_q: int, h_kv: int, d_head: int,
                   scale: float, stream=None) -> int:
    """fp16 in / fp16 out."""
    st = lib().gqa_decode_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens), batch, h_q, h_kv,
                              d_head, float(scale), _stream(stream))
    _check(st)
    return st


def make_args(q, k, v, o, seq_lens, batch, h_q, h_kv, d_head, scale, in_dtype, out_dtype,
              num_chunks=0, min_chunk=0, workspace=None, workspace_bytes=0, stream=0,
              sweep_events=None, t_q=0, merge=GQA_MERGE_AUTO, max_seq_len=0) -> GqaArgs:
    a = GqaArgs()
    a.q, a.k, a.v, a.o, a.seq_lens = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens)
    a.batch, a.h_q, a.h_kv, a.d_head = int(batch), int(h_q), int(h_kv), int(d_head)
    a.scale = float(scale)
    a.in_dtype, a.out_dtype = int(in_dtype), int(out_dtype)
    a.num_chunks, a.min_chunk = int(num_chunks), int(min_chunk)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes)
    a.stream = stream
    if sweep_events is not None:
        a.sweep_events[0] = int(sweep_events[0])
        a.sweep_events[1] = int(sweep_events[1])
    a.t_q = int(t_q)
    a.merge = int(merge)
    a.max_seq_len = int(max_seq_len)
    return a


def gqa_decode_ex(args: GqaArgs) -> int:
    st = lib().gqa_decode_ex(ctypes.byref(args))
    _check(st)
    return st


GQA_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


def gqa_decode_noalloc(args: GqaArgs) -> int:
    """gqa_decode_ex without allocation: the library's own device scratch array
    holds the partials (args.workspace must be NULL).  Raises GqaError."""
    st = lib().gqa_decode_noalloc(ctypes.byref(args))
    _check(st)
    return st


def gqa_decode_validate(args: GqaArgs) -> int:
    """Host-side checks only; returns the status (does not raise)."""
    return int(lib().gqa_decode_validate(ctypes.byref(args)))


def gqa_decode_make_plan(args: GqaArgs, num_cus: int, waves_per_cu: int):
    """(status, GqaPlan) -- pure host arithmetic."""
    plan = GqaPlan()
    st = lib().gqa_decode_make_plan(ctypes.byref(args), int(num_cus), int(waves_per_cu),
                                    ctypes.byref(plan))
    return int(st), plan


def gqa_decode_workspace_bytes(args: GqaArgs) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqa_decode_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return int(n.value)


def gqa_status_str(status: int) -> str:
    return status_str(status)


def gqa_last_error_message() -> str:
    return last_error_message()


def gqa_release() -> None:
    lib().gqa_release()


# ------------------------------------------------------------------ convenience


# Device type the convenience wrappers accept (the library's kernels need HIP
# device memory; torch names that device type "cuda").
_DEVICE_TYPE = "cuda"


def _check_tensors(what: str, q, k, v, seq_lens, out, workspace, batch: int) -> None:
    """Host-side checks of the tensors a convenience call hands to the library.

    The C ABI takes bare pointers, so it cannot see a dtype, a device, strides or
    a tensor's size; a mismatch there would make the kernels read or write outside
    the caller's buffers.  Everything checked here is tensor metadata: no device
    access, no synchronisation (the lengths in seq_lens stay unread, so k and v
    must hold at least sum(seq_lens) rows, as the header states)."""
    import torch
    names = ("q", "k", "v")
    for name, t in zip(names, (q, k, v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: %s must be a torch.Tensor" % (what, name))
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("%s: q, k and v must share one dtype (got %s, %s, %s)" % (what, q.dtype, k.dtype, v.dtype))
    _dtype_code(q)
    dev = q.device
    if dev.type != _DEVICE_TYPE:
        raise ValueError("%s: q must be a %s (HIP device) tensor, got device %s" % (what, _DEVICE_TYPE, dev))
    for name, t in zip(names, (q, k, v)):
        if t.device != dev:
            raise ValueError("%s: %s is on %s, q on %s" % (what, name, t.device, dev))
        if not t.is_contiguous():
            raise ValueError("%s: %s must be contiguous" % (what, name))
    if k.shape != v.shape:
        raise ValueError("%s: k %s and v %s must have one shape" % (what, tuple(k.shape), tuple(v.shape)))
    if k.shape[2] != q.shape[-1]:
        raise ValueError("%s: d_head of k (%d) differs from q's (%d)" % (what, k.shape[2], q.shape[-1]))
    if not isinstance(seq_lens, torch.Tensor) or seq_lens.dtype != torch.int32:
        raise ValueError("%s: seq_lens must be an int32 tensor" % what)
    if seq_lens.device != dev or not seq_lens.is_contiguous():
        raise ValueError("%s: seq_lens must be a contiguous tensor on %s" % (what, dev))
    if seq_lens.numel() != batch:
        raise ValueError("%s: seq_lens holds %d lengths, the batch is %d" % (what, seq_lens.numel(), batch))
    if out is not None:
        if not isinstance(out, torch.Tensor):
            raise TypeError("%s: out must be a torch.Tensor" % what)
        if out.shape != q.shape:
            raise ValueError("%s: out %s must have q's shape %s" % (what, tuple(out.shape), tuple(q.shape)))
        if out.dtype not in (q.dtype, torch.float32):
            raise ValueError("%s: out must be %s or float32, got %s" % (what, q.dtype, out.dtype))
        if out.device != dev or not out.is_contiguous():
            raise ValueError("%s: out must be a contiguous tensor on %s" % (what, dev))
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("%s: workspace must be a torch.Tensor" % what)
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("%s: workspace must be a contiguous tensor on %s" % (what, dev))


def decode(q, k, v, seq_lens, scale: Optional[float] = None, out=None, out_dtype=None,
           num_chunks: int = 0, min_chunk: int = 0, workspace=None, stream=None, merge: int = GQA_MERGE_AUTO,
           max_seq_len: int = 0):
    """o = GQA decode of q [batch, h_q, d] (or [batch, t_q, h_q, d] for t_q query
    tokens per sequence) against packed k, v [sum(seq_lens), h_kv, d].

    q, k and v share one dtype and one CUDA device and are contiguous; seq_lens
    is a contiguous int32 tensor on that device with one length per sequence.
    out_dtype defaults to q's dtype; pass torch.float32 with 16-bit inputs for the
    fp32 result.  merge is GQA_MERGE_AUTO, GQA_MERGE_KERNEL or GQA_MERGE_FUSED;
    max_seq_len (0 = unknown) is the plan's hint of the longest sequence; a
    caller workspace must read zero in its first GQA_DECODE_COUNTER_BYTES bytes
    before its first use (torch.zeros).  Raises ValueError/TypeError before any
    device work when the tensors do not fit these rules.  Returns `out`.
    """
    import torch
    if q.dim() not in (3, 4) or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [batch, h_q, d] or [batch, t_q, h_q, d]; k, v [sum(seq_lens), h_kv, d]")
    t_q = q.shape[1] if q.dim() == 4 else 0
    batch, h_q, d = q.shape[0], q.shape[-2], q.shape[-1]
    h_kv = k.shape[1]
    _check_tensors("decode", q, k, v, seq_lens, out, workspace, batch)
    if out is None and out_dtype not in (None, q.dtype, torch.float32):
        raise ValueError("decode: out_dtype must be %s or float32, got %s" % (q.dtype, out_dtype))
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    args = make_args(q, k, v, out, seq_lens, batch, h_q, h_kv, d, scale, _dtype_code(q),
                     _dtype_code(out), num_chunks, min_chunk, workspace, ws_bytes, _stream(stream),
                     t_q=t_q, merge=merge, max_seq_len=max_seq_len)
    gqa_decode_ex(args)
    return out


def gqa_prefill(q, k, v, o, seq_lens, batch: int, total_tokens: int, h_q: int, h_kv: int, d_head: int,
                scale: float, stream=None) -> int:
    """Causal prefill, bf16 in / bf16 out.  Raises GqaError on a non-zero status."""
    st = lib().gqa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens), batch, int(total_tokens), h_q,
                           h_kv, d_head, float(scale), _stream(stream))
    _check(st)
    return st


def gqa_prefill_f16(q, k, v, o, seq_lens, batch: int, total_tokens: int, h_q: int, h_kv: int, d_head: int,
                    scale: float, stream=None) -> int:
    """Causal prefill, fp16 in / fp16 out."""
    st = lib().gqa_prefill_f16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens), batch, int(total_tokens), h_q,
                               h_kv, d_head, float(scale), _stream(stream))
    _check(st)
    return st


def make_prefill_args(q, k, v, o, seq_lens, batch, h_q, h_kv, d_head, scale, in_dtype, out_dtype,
                      num_blocks=0, stream=0, split_pv=0, total_tokens=0, workspace=None,
                      workspace_bytes=0) -> GqaPrefillArgs:
    a = GqaPrefillArgs()
    a.q, a.k, a.v, a.o, a.seq_lens = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seq_lens)
    a.batch, a.h_q, a.h_kv, a.d_head = int(batch), int(h_q), int(h_kv), int(d_head)
    a.scale = float(scale)
    a.in_dtype, a.out_dtype = int(in_dtype), int(out_dtype)
    a.num_blocks = int(num_blocks)
    a.stream = stream
    a.split_pv = int(split_pv)
    a.total_tokens = int(total_tokens)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace_bytes)
    return a


def gqa_prefill_ex(args: GqaPrefillArgs) -> int:
    st = lib().gqa_prefill_ex(ctypes.byref(args))
    _check(st)
    return st


def gqa_prefill_validate(args: GqaPrefillArgs) -> int:
    """Host-side checks only; returns the status (does not raise)."""
    return int(lib().gqa_prefill_validate(ctypes.byref(args)))


def gqa_prefill_workspace_bytes(args: GqaPrefillArgs) -> int:
    """Workspace bytes the prefill call needs (0 where it uses none)."""
    n = ctypes.c_size_t()
    _check(lib().gqa_prefill_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return int(n.value)


def prefill(q, k, v, seq_lens, scale: Optional[float] = None, out=None, out_dtype=None,
            num_blocks: int = 0, stream=None, split_pv: int = 0, workspace=None, total_tokens=None):
    """o = causal GQA prefill of q [sum(seq_lens), h_q, d] against k, v
    [sum(seq_lens), h_kv, d] (each token sees its sequence's keys up to itself).
    q, k, v share one dtype and CUDA device, are contiguous and hold the same rows;
    seq_lens is a contiguous int32 tensor on that device; total_tokens defaults to
    q's row count (and may not exceed it); workspace (a device byte tensor)
    defaults to the library's own.  Raises ValueError/TypeError before any device
    work when the tensors do not fit these rules.  Returns `out`."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [sum(seq_lens), h_q, d]; k, v [sum(seq_lens), h_kv, d]")
    h_q, d = q.shape[1], q.shape[2]
    h_kv = k.shape[1]
    batch = int(seq_lens.numel()) if isinstance(seq_lens, torch.Tensor) else -1
    _check_tensors("prefill", q, k, v, seq_lens, out, workspace, batch)
    if k.shape[0] != q.shape[0]:
        raise ValueError("prefill: q holds %d rows, k and v %d (the sequences are packed the same way)"
                         % (q.shape[0], k.shape[0]))
    if out is None and out_dtype not in (None, q.dtype, torch.float32):
        raise ValueError("prefill: out_dtype must be %s or float32, got %s" % (q.dtype, out_dtype))
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if total_tokens is None:
        total_tokens = q.shape[0]
    if not 0 <= int(total_tokens) <= q.shape[0]:
        raise ValueError("prefill: total_tokens %d outside [0, %d] (the rows q holds)" % (int(total_tokens), q.shape[0]))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = make_prefill_args(q, k, v, out, seq_lens, batch, h_q, h_kv, d, scale, _dtype_code(q),
                             _dtype_code(out), num_blocks, _stream(stream), split_pv, total_tokens, workspace,
                             ws_bytes)
    gqa_prefill_ex(args)
    return out


def gqa_probe_copy(src, dst, nbytes: int, stream=None) -> int:
    """Plain device copy of nbytes (measurement reference)."""
    st = lib().gqa_probe_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_probe_copy failed")
    return st


GQA_PROBE_SINK_WORDS = 256


def gqa_probe_read(src, nbytes: int, sink, stream=None) -> int:
    """Plain device read of nbytes folded into GQA_PROBE_SINK_WORDS uint32 words at sink."""
    st = lib().gqa_probe_read(_ptr(src), int(nbytes), _ptr(sink), _stream(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_probe_read failed")
    return st
