"""The C-ABI library on the host (no GPU needed): it loads, exports every function
include/gqa_decode.h declares, and its host-side validation and planning follow
the documented rules.  Nothing here launches a kernel.
"""
import ctypes
import math
import os
import re

import pytest

from gqa_split_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from gqa_split_kv_amd import build
        build.build()
    return B.lib()


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?(?:int|void|size_t|char)\s*\*?\s*(gqa_\w+)\s*\(",
                                text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert set(declared) == set(B.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _args(**kw):
    base = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, seq_lens=0x50000, batch=4, h_q=32,
                h_kv=8, d_head=128, scale=0.088, in_dtype=B.GQA_DTYPE_BF16,
                out_dtype=B.GQA_DTYPE_BF16)
    base.update(kw)
    return B.make_args(**base)


def _validate(**kw):
    return B.gqa_decode_validate(_args(**kw))


def test_valid_arguments_pass(lib):
    assert _validate() == B.GQA_OK
    assert _validate(in_dtype=B.GQA_DTYPE_F32, out_dtype=B.GQA_DTYPE_F32, d_head=64) == B.GQA_OK
    assert _validate(out_dtype=B.GQA_DTYPE_F32) == B.GQA_OK
    assert _validate(in_dtype=B.GQA_DTYPE_F16, out_dtype=B.GQA_DTYPE_F16) == B.GQA_OK
    assert _validate(in_dtype=B.GQA_DTYPE_F16, out_dtype=B.GQA_DTYPE_F32) == B.GQA_OK
    for G, h_kv in [(1, 8), (2, 4), (4, 8), (8, 8), (16, 1), (3, 2), (5, 1)]:
        assert _validate(h_q=G * h_kv, h_kv=h_kv) == B.GQA_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "seq_lens"])
def test_null_pointer(lib, field):
    assert _validate(**{field: None}) == B.GQA_ERR_NULL
    assert field in B.last_error_message() or "NULL" in B.last_error_message()


def test_null_args_block(lib):
    assert lib.gqa_decode_validate(None) == B.GQA_ERR_NULL


@pytest.mark.parametrize("kw", [dict(batch=0), dict(batch=-1), dict(h_q=0), dict(h_kv=0),
                                dict(h_q=30, h_kv=8), dict(h_q=7, h_kv=2)])
def test_shape_errors(lib, kw):
    assert _validate(**kw) == B.GQA_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(d_head=96), dict(d_head=256), dict(d_head=0),
                                dict(h_q=65 * 8, h_kv=8), dict(h_q=65, h_kv=1),
                                dict(in_dtype=B.GQA_DTYPE_F32, out_dtype=B.GQA_DTYPE_BF16),
                                dict(in_dtype=B.GQA_DTYPE_F32, out_dtype=B.GQA_DTYPE_F16),
                                dict(in_dtype=B.GQA_DTYPE_F16, out_dtype=B.GQA_DTYPE_BF16),
                                dict(in_dtype=B.GQA_DTYPE_BF16, out_dtype=B.GQA_DTYPE_F16),
                                dict(in_dtype=7), dict(out_dtype=3), dict(h_q=70000, h_kv=70000)])
def test_unsupported(lib, kw):
    assert _validate(**kw) == B.GQA_ERR_UNSUPPORTED


def test_multi_token_limits(lib):
    assert _validate(t_q=2, h_q=64, h_kv=8) == B.GQA_OK          # G 8 x 2 tokens = 16 rows
    assert _validate(t_q=8, h_q=64, h_kv=8) == B.GQA_OK          # 64 rows: 4 wavefronts per range
    assert _validate(t_q=9, h_q=64, h_kv=8) == B.GQA_ERR_UNSUPPORTED
    assert _validate(t_q=64, h_q=8, h_kv=8) == B.GQA_OK
    assert _validate(t_q=65, h_q=8, h_kv=8) == B.GQA_ERR_UNSUPPORTED
    assert _validate(h_q=64, h_kv=1) == B.GQA_OK                 # G 64
    assert _validate(t_q=-1) == B.GQA_ERR_SHAPE
    st, p1 = B.gqa_decode_make_plan(_args(num_chunks=64), 256, 4)
    st2, p4 = B.gqa_decode_make_plan(_args(num_chunks=64, t_q=4), 256, 4)
    assert st == st2 == B.GQA_OK
    C = B.GQA_DECODE_COUNTER_BYTES
    assert p4.workspace_bytes - C >= 4 * (p1.workspace_bytes - C) - 256


def test_more_than_16_rows_plan(lib):
    """More than 16 rows per kv head: still one wavefront per (token range, kv
    head) -- it holds two or four 16-row tiles -- so the plan's wavefront count does
    not change, and the workspace grows with the rows."""
    st, p = B.gqa_decode_make_plan(_args(h_q=64, h_kv=8, t_q=4), 256, 4)       # 32 rows
    assert st == B.GQA_OK and p.num_chunks == 1024 and p.split_blocks == 256
    st, p = B.gqa_decode_make_plan(_args(h_q=48, h_kv=1, t_q=1, num_chunks=11, merge=B.GQA_MERGE_KERNEL), 256, 4)
    assert st == B.GQA_OK and p.num_chunks == 11 and not p.fused              # 48 rows
    st, p = B.gqa_decode_make_plan(_args(h_q=48, h_kv=1, t_q=1, num_chunks=11, max_seq_len=200), 256, 4)
    assert st == B.GQA_OK and p.num_chunks == 8 and p.fused                   # 4 units, short: fused
    st, p64 = B.gqa_decode_make_plan(_args(h_q=64, h_kv=1, num_chunks=64), 256, 4)
    st, p16 = B.gqa_decode_make_plan(_args(h_q=16, h_kv=1, num_chunks=64), 256, 4)
    C = B.GQA_DECODE_COUNTER_BYTES
    assert p64.workspace_bytes - C >= 4 * (p16.workspace_bytes - C) - 256


@pytest.mark.parametrize("field", ["q", "k", "v", "o"])
def test_alignment_16_bytes(lib, field):
    assert _validate(**{field: 0x10008}) == B.GQA_ERR_ALIGN
    assert _validate(**{field: 0x10010}) == B.GQA_OK


def test_seq_lens_alignment(lib):
    assert _validate(seq_lens=0x50002) == B.GQA_ERR_ALIGN
    assert _validate(seq_lens=0x50004) == B.GQA_OK


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_non_finite_scale(lib, scale):
    assert _validate(scale=scale) == B.GQA_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(num_chunks=-1), dict(min_chunk=-5), dict(num_chunks=(1 << 24) + 1),
                                dict(min_chunk=(1 << 30) + 1)])
def test_tuning_ranges(lib, kw):
    assert _validate(**kw) == B.GQA_ERR_ARG


def test_workspace_size_checked_with_explicit_chunks(lib):
    st, plan = B.gqa_decode_make_plan(_args(num_chunks=100), 256, 8)
    assert st == B.GQA_OK
    need = plan.workspace_bytes
    G, D = 4, 128
    assert plan.num_chunks == 96          # rounded down to a multiple of h_kv = 8
    assert need >= 96 * 2 * G * (D + 2) * 4
    assert need % 256 == 0
    assert _validate(num_chunks=100, workspace=0x100000, workspace_bytes=need) == B.GQA_OK
    assert _validate(num_chunks=100, workspace=0x100000, workspace_bytes=need - 1) == B.GQA_ERR_WORKSPACE
    assert _validate(num_chunks=100, workspace=0x100010, workspace_bytes=need) == B.GQA_ERR_WORKSPACE
    # automatic num_chunks: the size needs the device, so validation skips it
    assert _validate(workspace=0x100000, workspace_bytes=1) == B.GQA_OK


def test_plan_automatic_and_explicit(lib):
    st, plan = B.gqa_decode_make_plan(_args(), 256, 8)
    assert st == B.GQA_OK
    assert plan.num_chunks == 256 * 4                       # one wavefront per SIMD
    assert plan.split_blocks == 256                         # 4-wave workgroups
    assert plan.merge_blocks == 4 * 8                       # batch * h_kv (G = 4 heads per block)
    assert plan.merge_threads == 256                        # 128 ranges / batch 4 = 32 pieces
    assert plan.min_chunk > 0
    st, plan = B.gqa_decode_make_plan(_args(num_chunks=7, min_chunk=1024), 256, 8)
    assert st == B.GQA_OK
    assert (plan.num_chunks, plan.min_chunk, plan.split_blocks) == (8, 1024, 2)   # at least h_kv
    assert plan.merge_slices == 1
    kernel = B.GQA_MERGE_KERNEL
    st, plan = B.gqa_decode_make_plan(_args(batch=1, h_kv=1, h_q=8, merge=kernel), 256, 8)
    assert (st, plan.merge_threads) == (B.GQA_OK, 1024)     # one sequence cut into 1024 ranges
    # ... and only 8 rows: each row's d is split over 4 workgroups
    assert (plan.merge_slices, plan.merge_blocks) == (4, 8 * 4)
    st, plan = B.gqa_decode_make_plan(_args(batch=64, h_kv=1, h_q=8, num_chunks=64 * 64), 256, 8)
    assert (plan.merge_threads, plan.merge_slices, plan.merge_blocks) == (1024, 1, 64 * 8)
    st, plan = B.gqa_decode_make_plan(_args(num_chunks=7, h_kv=1, h_q=8, merge=kernel), 256, 8)
    assert (st, plan.num_chunks, plan.split_blocks) == (B.GQA_OK, 7, 2)
    st, plan = B.gqa_decode_make_plan(_args(h_kv=6, h_q=48), 256, 12)
    assert st == B.GQA_OK and plan.num_chunks == 1024 // 6 * 6     # capped at 4 waves per CU
    st, plan = B.gqa_decode_make_plan(_args(), 256, 2)
    assert st == B.GQA_OK and plan.num_chunks == 512                # occupancy below the cap
    st, _ = B.gqa_decode_make_plan(_args(), 0, 8)
    assert st == B.GQA_ERR_ARG
    st, _ = B.gqa_decode_make_plan(_args(h_q=30), 256, 8)
    assert st == B.GQA_ERR_SHAPE


def test_status_strings(lib):
    names = {B.GQA_OK: "GQA_OK", B.GQA_ERR_NULL: "GQA_ERR_NULL", B.GQA_ERR_SHAPE: "GQA_ERR_SHAPE",
             B.GQA_ERR_UNSUPPORTED: "GQA_ERR_UNSUPPORTED", B.GQA_ERR_ALIGN: "GQA_ERR_ALIGN",
             B.GQA_ERR_SCALE: "GQA_ERR_SCALE", B.GQA_ERR_WORKSPACE: "GQA_ERR_WORKSPACE",
             B.GQA_ERR_HIP: "GQA_ERR_HIP", B.GQA_ERR_ARG: "GQA_ERR_ARG"}
    for code, name in names.items():
        assert B.status_str(code) == name
    assert B.status_str(99) == "GQA_ERR_UNKNOWN"


def test_error_message_is_cleared_on_success(lib):
    assert _validate(batch=0) == B.GQA_ERR_SHAPE
    assert B.last_error_message() != ""
    assert _validate() == B.GQA_OK
    assert B.last_error_message() == ""


def test_struct_mirrors_match_header_sizes(lib):
    # gqa_decode_args: 5 pointers, 4 int32 + float, 4 more int32, pointer, size_t, pointer,
    # 2 event pointers, t_q and merge
    assert ctypes.sizeof(B.GqaArgs) == 5 * 8 + 4 * 4 + 4 + 4 * 4 + 4 + 8 + 8 + 8 + 2 * 8 + 4 + 4 + 4 + 4
    # gqa_decode_plan: 6 int32, size_t, 3 int32 (+4 padding)
    assert ctypes.sizeof(B.GqaPlan) == 6 * 4 + 8 + 3 * 4 + 4


# ------------------------------------------------------------------ prefill


def _pargs(**kw):
    base = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, seq_lens=0x50000, batch=1, h_q=8,
                h_kv=1, d_head=128, scale=0.088, in_dtype=B.GQA_DTYPE_BF16,
                out_dtype=B.GQA_DTYPE_BF16)
    base.update(kw)
    return B.make_prefill_args(**base)


def _pvalidate(**kw):
    return B.gqa_prefill_validate(_pargs(**kw))


def test_prefill_validation(lib):
    assert _pvalidate() == B.GQA_OK
    assert _pvalidate(out_dtype=B.GQA_DTYPE_F32) == B.GQA_OK
    assert _pvalidate(in_dtype=B.GQA_DTYPE_F16, out_dtype=B.GQA_DTYPE_F16, d_head=64) == B.GQA_OK
    assert _pvalidate(in_dtype=B.GQA_DTYPE_F16, out_dtype=B.GQA_DTYPE_F32) == B.GQA_OK
    assert _pvalidate(in_dtype=B.GQA_DTYPE_F32, out_dtype=B.GQA_DTYPE_F32) == B.GQA_ERR_UNSUPPORTED
    assert _pvalidate(in_dtype=B.GQA_DTYPE_BF16, out_dtype=B.GQA_DTYPE_F16) == B.GQA_ERR_UNSUPPORTED
    assert _pvalidate(q=0) == B.GQA_ERR_NULL
    assert _pvalidate(seq_lens=0) == B.GQA_ERR_NULL
    assert B.lib().gqa_prefill_validate(None) == B.GQA_ERR_NULL
    assert _pvalidate(batch=0) == B.GQA_ERR_SHAPE
    assert _pvalidate(h_q=12, h_kv=8) == B.GQA_ERR_SHAPE
    assert _pvalidate(h_q=64, h_kv=1) == B.GQA_OK                   # G = 64
    assert _pvalidate(h_q=65, h_kv=1) == B.GQA_ERR_UNSUPPORTED      # G = 65
    assert _pvalidate(h_q=70000, h_kv=70000) == B.GQA_ERR_UNSUPPORTED
    assert _pvalidate(d_head=96) == B.GQA_ERR_UNSUPPORTED
    assert _pvalidate(o=0x40008) == B.GQA_ERR_ALIGN
    assert _pvalidate(seq_lens=0x50002) == B.GQA_ERR_ALIGN
    assert _pvalidate(scale=float("inf")) == B.GQA_ERR_SCALE
    assert _pvalidate(num_blocks=-1) == B.GQA_ERR_ARG
    assert _pvalidate(num_blocks=(1 << 20) + 1) == B.GQA_ERR_ARG
    assert _pvalidate(num_blocks=(1 << 20) + 1) == B.GQA_ERR_ARG and "num_blocks" in B.last_error_message()
    assert _pvalidate(num_blocks=1 << 20) == B.GQA_OK
    assert _pvalidate(split_pv=1) == B.GQA_OK
    assert _pvalidate(split_pv=2) == B.GQA_ERR_ARG and "split_pv" in B.last_error_message()


def test_prefill_args_struct_size(lib):
    # ... stream, split_pv (+4 bytes padding), total_tokens, workspace, workspace_bytes
    assert ctypes.sizeof(B.GqaPrefillArgs) == 5 * 8 + 4 * 4 + 4 + 3 * 4 + 8 + 8 + 8 + 8 + 8
    assert B.GqaPrefillArgs.total_tokens.offset == 88


def test_prefill_total_tokens_and_workspace_rules(lib):
    assert _pvalidate(total_tokens=-1) == B.GQA_ERR_ARG and "total_tokens" in B.last_error_message()
    assert _pvalidate(total_tokens=1 << 37, split_pv=1) == B.GQA_OK           # h_kv 1
    assert _pvalidate(total_tokens=(1 << 37) + 1) == B.GQA_ERR_ARG
    assert _pvalidate(total_tokens=1 << 34, h_q=64, h_kv=8, split_pv=1) == B.GQA_OK
    assert _pvalidate(total_tokens=(1 << 34) + 1, h_q=64, h_kv=8) == B.GQA_ERR_ARG
    # Workspace: V transposed in 64-key blocks, nvb = ceil(total / 64) + batch
    # blocks per kv head of d x 64 fp16 values, then one flag byte per block and
    # kv head, then the tile queue's counter, each part rounded up to 256 bytes.
    a = _pargs(total_tokens=1000, h_q=8, h_kv=2)
    nvb = 16 + 1
    assert B.gqa_prefill_workspace_bytes(a) == 2 * nvb * 128 * 64 * 2 + 256 + 256
    assert B.gqa_prefill_workspace_bytes(_pargs(total_tokens=129, d_head=64, batch=3)) == (3 + 3) * 64 * 64 * 2 + 256 + 256
    assert B.gqa_prefill_workspace_bytes(_pargs(total_tokens=1000, split_pv=1)) == 0
    assert B.gqa_prefill_workspace_bytes(_pargs(total_tokens=0)) == 0
    assert B.gqa_prefill_workspace_bytes(
        _pargs(total_tokens=1000, in_dtype=B.GQA_DTYPE_F16, out_dtype=B.GQA_DTYPE_F16)) == 17 * 128 * 64 * 2 + 256 + 256
    # The V copy's grid (nvb x h_kv workgroups) must stay below 2^31.
    assert _pvalidate(total_tokens=1 << 36, h_q=8, h_kv=2) == B.GQA_ERR_ARG and "2^31" in B.last_error_message()
    assert _pvalidate(total_tokens=1 << 36, h_q=8, h_kv=1) == B.GQA_OK
    assert _pvalidate(total_tokens=1 << 36, h_q=8, h_kv=2, split_pv=1) == B.GQA_OK
    need = B.gqa_prefill_workspace_bytes(a)
    assert _pvalidate(total_tokens=1000, h_q=8, h_kv=2, workspace=0x100000, workspace_bytes=need) == B.GQA_OK
    assert _pvalidate(total_tokens=1000, h_q=8, h_kv=2, workspace=0x100000,
                      workspace_bytes=need - 1) == B.GQA_ERR_WORKSPACE
    assert _pvalidate(total_tokens=1000, h_q=8, h_kv=2, workspace=0x100080,
                      workspace_bytes=need) == B.GQA_ERR_WORKSPACE and "aligned" in B.last_error_message()
    # A workspace is not checked where the call uses none.
    assert _pvalidate(total_tokens=1000, split_pv=1, workspace=0x100080, workspace_bytes=1) == B.GQA_OK
    # The size query skips the caller workspace's own checks.
    assert B.gqa_prefill_workspace_bytes(_pargs(total_tokens=1000, h_q=8, h_kv=2, workspace=0x100080,
                                                workspace_bytes=1)) == need


def test_workspace_bytes_reports_a_status(lib):
    """gqa_decode_workspace_bytes returns a status and writes the size through its
    pointer: NULL is GQA_ERR_NULL, invalid arguments give their validation status,
    and neither writes the output.  (num_chunks is explicit, so no device is asked.)"""
    L = lib
    a = _args(num_chunks=64)
    assert L.gqa_decode_workspace_bytes(ctypes.byref(a), None) == B.GQA_ERR_NULL
    n = ctypes.c_size_t(12345)
    bad = _args(num_chunks=64, h_q=30)
    assert L.gqa_decode_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == B.GQA_ERR_SHAPE
    assert n.value == 12345
    assert L.gqa_decode_workspace_bytes(None, ctypes.byref(n)) == B.GQA_ERR_NULL
    assert L.gqa_decode_workspace_bytes(ctypes.byref(a), ctypes.byref(n)) == B.GQA_OK
    st, plan = B.gqa_decode_make_plan(a, 256, 4)
    assert st == B.GQA_OK and n.value == plan.workspace_bytes


def test_noalloc_argument_checks_on_the_host(lib):
    """gqa_decode_noalloc refuses a NULL argument block, a caller workspace and
    invalid arguments before touching any device."""
    assert lib.gqa_decode_noalloc(None) == B.GQA_ERR_NULL
    a = _args(workspace=0x100000, workspace_bytes=1 << 20)
    assert lib.gqa_decode_noalloc(ctypes.byref(a)) == B.GQA_ERR_ARG
    assert "workspace" in B.last_error_message()
    a = _args(workspace_bytes=256)
    assert lib.gqa_decode_noalloc(ctypes.byref(a)) == B.GQA_ERR_ARG
    for kw, st in [(dict(batch=0), B.GQA_ERR_SHAPE), (dict(d_head=96), B.GQA_ERR_UNSUPPORTED),
                   (dict(q=0x10008), B.GQA_ERR_ALIGN), (dict(scale=math.nan), B.GQA_ERR_SCALE),
                   (dict(num_chunks=-1), B.GQA_ERR_ARG), (dict(q=0), B.GQA_ERR_NULL)]:
        a = _args(**kw)
        assert lib.gqa_decode_noalloc(ctypes.byref(a)) == st, kw


def test_fused_merge_plan(lib):
    """The fused merge: chosen automatically for at most 16 (sequence, kv head)
    units; whole workgroups of 4 ranges of one kv head (num_chunks a multiple of
    4 h_kv); fan-in from the fold volume (K R d 4 bytes <= 64 KiB, 2..64); tree
    levels from the range groups; the counters' reserve bounds its size."""
    # automatic: fused only with a max_seq_len hint within 4 x min_chunk (64) keys
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=32, h_kv=8), 256, 4)      # 8 units, no hint
    assert st == B.GQA_OK and p.fused == 0 and p.min_chunk == 64
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=32, h_kv=8, max_seq_len=257), 256, 4)
    assert st == B.GQA_OK and p.fused == 0
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=32, h_kv=8, max_seq_len=256), 256, 4)
    assert st == B.GQA_OK and p.fused == 1 and p.num_chunks == 1024 and p.split_blocks == 256
    assert (p.merge_blocks, p.merge_threads) == (0, 0)
    assert p.fold_fanin == 32 and p.fold_levels == 1                            # R 4: 2 KiB triples; 32 groups
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=32, h_kv=8, max_seq_len=1000, min_chunk=250), 256, 4)
    assert p.fused
    assert _validate(max_seq_len=-1) == B.GQA_ERR_ARG
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=8, h_kv=1, merge=B.GQA_MERGE_FUSED), 256, 4)   # R 8
    assert p.fused and p.fold_fanin == 16 and p.fold_levels == 2
    st, p = B.gqa_decode_make_plan(_args(batch=4, h_q=32, h_kv=8, max_seq_len=100), 256, 4)   # 32 units
    assert st == B.GQA_OK and p.fused == 0 and p.merge_blocks > 0
    st, p = B.gqa_decode_make_plan(_args(batch=4, h_q=32, h_kv=8, merge=B.GQA_MERGE_FUSED), 256, 4)
    assert st == B.GQA_OK and p.fused == 1
    F = B.GQA_MERGE_FUSED
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=64, h_kv=1, t_q=1, d_head=128, merge=F), 256, 4)   # R 64
    assert p.fused and p.fold_fanin == 2 and p.fold_levels == 8
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=1, h_kv=1, d_head=64, merge=F), 256, 4)            # R 1, d 64
    assert p.fused and p.fold_fanin == 64
    for nc, want in [(1, 32), (33, 32), (100, 96), (4096, 4096)]:               # multiples of 4 h_kv = 32
        st, p = B.gqa_decode_make_plan(_args(batch=1, num_chunks=nc, merge=F), 256, 4)
        assert st == B.GQA_OK and p.fused and p.num_chunks == want, (nc, p.num_chunks)
    # counters: levels x 2 x num_chunks / 4 within 64 KiB / 4 words
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=8, h_kv=1, num_chunks=1 << 15, max_seq_len=100), 256, 4)
    assert st == B.GQA_OK and p.fused == 0 and p.num_chunks == 1 << 15   # automatic: too many counters
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=8, h_kv=1, num_chunks=1 << 15, merge=B.GQA_MERGE_FUSED), 256, 4)
    assert st == B.GQA_OK and p.fused == 1 and p.num_chunks < 1 << 15            # forced: fewer wavefronts
    assert p.fold_levels * 2 * (p.num_chunks // 4) <= B.GQA_DECODE_COUNTER_BYTES // 4
    assert p.fold_levels * 2 * (2 * p.num_chunks // 4) > B.GQA_DECODE_COUNTER_BYTES // 4 - 4 * 2 * 16
    st, p = B.gqa_decode_make_plan(_args(batch=1, h_q=8192, h_kv=8192, merge=B.GQA_MERGE_FUSED), 256, 4)
    assert st == B.GQA_OK and p.fused and p.num_chunks == 4 * 8192 and p.fold_levels == 1   # 16384 counters
    a = _args(batch=1, h_q=8200, h_kv=8200, num_chunks=0, merge=B.GQA_MERGE_FUSED)   # 2 x 8200 counters
    st, _ = B.gqa_decode_make_plan(a, 256, 4)
    assert st == B.GQA_ERR_ARG and "counters" in B.last_error_message()
    a.num_chunks = 64
    assert B.gqa_decode_validate(a) == B.GQA_ERR_ARG
    assert _validate(merge=3) == B.GQA_ERR_ARG and _validate(merge=-1) == B.GQA_ERR_ARG
    # workspace: the counter reserve, then the wavefront slots, then (fused) the workgroup slots
    st, pk = B.gqa_decode_make_plan(_args(batch=1, num_chunks=256, merge=B.GQA_MERGE_KERNEL), 256, 4)
    st, pf = B.gqa_decode_make_plan(_args(batch=1, num_chunks=256, merge=B.GQA_MERGE_FUSED), 256, 4)
    slots = 256 * 2 * 4 * (128 + 2) * 4
    assert pk.workspace_bytes == B.GQA_DECODE_COUNTER_BYTES + slots
    assert pf.workspace_bytes == B.GQA_DECODE_COUNTER_BYTES + slots + slots // 4


def test_args_struct_layout(lib):
    assert ctypes.sizeof(B.GqaArgs) == 136 and B.GqaArgs.t_q.offset == 120 and B.GqaArgs.merge.offset == 124
    assert B.GqaArgs.max_seq_len.offset == 128
    assert ctypes.sizeof(B.GqaPlan) == 48 and B.GqaPlan.fused.offset == 32
