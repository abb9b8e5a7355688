// api.cpp -- the extern "C" entry points of libgqa_decode.so (declared in
// include/gqa_decode.h and include/gqa_prefill.h): validation, planning, the
// library-owned workspace cache, and the launches.  No C++ exception leaves this file.
#include <hip/hip_runtime.h>

#include <cmath>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "host.h"
#include "kernels.h"

namespace gqa {
const char *last_error();
}

namespace {

struct OwnedWorkspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<int, int> g_num_cus;                                   // device -> compute units
std::map<std::pair<int, int>, int> g_waves_per_cu;               // (device, variant) -> waves
// Library-owned workspaces per (device, stream, kind): decode and prefill keep
// separate buffers, since the prefill's V copy would overwrite the decode's
// counters (which must stay zero between calls).
enum WorkspaceKind { kDecodeWorkspace = 0, kPrefillWorkspace = 1 };
std::map<std::tuple<int, uintptr_t, int>, OwnedWorkspace> g_workspaces;

int variant_id(int in_dtype, int out_dtype, int D) { return (in_dtype << 3) | (out_dtype << 1) | (D == 128); }

int device_shape(int dev, int in_dtype, int out_dtype, int D, int *num_cus, int *waves_per_cu) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_num_cus.find(dev);
    if (it == g_num_cus.end()) {
        int n = 0;
        hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || n <= 0)
            return gqa::fail(GQA_ERR_HIP, "hipDeviceGetAttribute(compute units) failed: %s",
                             hipGetErrorString(e));
        it = g_num_cus.emplace(dev, n).first;
    }
    *num_cus = it->second;
    const auto key = std::make_pair(dev, variant_id(in_dtype, out_dtype, D));
    auto wt = g_waves_per_cu.find(key);
    if (wt == g_waves_per_cu.end()) {
        int blocks = 0;
        hipError_t e = gqa::sweep_occupancy(in_dtype, out_dtype, D, &blocks);
        if (e != hipSuccess || blocks <= 0)
            return gqa::fail(GQA_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
        wt = g_waves_per_cu.emplace(key, blocks * gqa::kWavesPerBlock).first;
    }
    *waves_per_cu = wt->second;
    return GQA_OK;
}

int owned_workspace(int dev, hipStream_t stream, int kind, size_t need, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    OwnedWorkspace &w = g_workspaces[std::make_tuple(dev, reinterpret_cast<uintptr_t>(stream), kind)];
    if (w.bytes < need) {
        if (w.ptr) {
            // Work already enqueued on this stream may still read the old buffer.
            hipError_t e = hipStreamSynchronize(stream);
            if (e != hipSuccess)
                return gqa::fail(GQA_ERR_HIP, "hipStreamSynchronize failed: %s", hipGetErrorString(e));
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        const size_t grow = ((need + need / 4) + (1u << 20) - 1) & ~static_cast<size_t>((1u << 20) - 1);
        hipError_t e = hipMalloc(&w.ptr, grow);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return gqa::fail(GQA_ERR_HIP, "hipMalloc(%zu) for the workspace failed: %s", grow,
                             hipGetErrorString(e));
        }
        w.bytes = grow;
        // The decode's fused merge counters must read zero before a call (every call
        // leaves them so); a new buffer starts zeroed, ordered before the call.
        if (kind == kDecodeWorkspace) {
            e = hipMemsetAsync(w.ptr, 0, gqa::kCounterBytes, stream);
            if (e != hipSuccess)
                return gqa::fail(GQA_ERR_HIP, "clearing the workspace counters failed: %s", hipGetErrorString(e));
        }
    }
    *out = w.ptr;
    return GQA_OK;
}

// Validation and plan of a decode call on the current device.
int decode_plan(const gqa_decode_args *a, int *dev, gqa_decode_plan *plan) {
    int st = gqa::validate(a);
    if (st != GQA_OK) return st;
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return gqa::fail(GQA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    int num_cus = 0, waves_per_cu = 0;
    st = device_shape(*dev, a->in_dtype, a->out_dtype, a->d_head, &num_cus, &waves_per_cu);
    if (st != GQA_OK) return st;
    return gqa::make_plan(a, num_cus, waves_per_cu, plan);
}

// Enqueues the sweep and merge kernels of a planned call with its workspace `ws`.
int decode_launch(const gqa_decode_args *a, const gqa_decode_plan &plan, void *ws) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(a->stream);
    const int G = a->h_q / a->h_kv;
    const gqa::WorkspaceLayout L =
        gqa::workspace_layout(plan.num_chunks, G * (a->t_q > 0 ? a->t_q : 1), a->d_head, plan.fused != 0);
    gqa::DecodeParams P;
    P.q = static_cast<const uint8_t *>(a->q);
    P.k = static_cast<const uint8_t *>(a->k);
    P.v = static_cast<const uint8_t *>(a->v);
    P.o = static_cast<uint8_t *>(a->o);
    P.seq_lens = a->seq_lens;
    P.ws_o = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + L.o_offset);
    P.ws_ml = reinterpret_cast<float2 *>(static_cast<uint8_t *>(ws) + L.ml_offset);
    P.ws2_o = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + L.o2_offset);
    P.ws2_ml = reinterpret_cast<float2 *>(static_cast<uint8_t *>(ws) + L.ml2_offset);
    P.counters = reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(ws) + L.counter_offset);
    P.fold_k_log2 = 0;
    while ((1 << P.fold_k_log2) < plan.fold_fanin) ++P.fold_k_log2;
    P.batch = a->batch;
    P.h_q = a->h_q;
    P.h_kv = a->h_kv;
    P.G = G;
    P.t_q = a->t_q > 0 ? a->t_q : 1;
    P.R = G * P.t_q;
    P.num_chunks = plan.num_chunks;
    P.min_chunk = plan.min_chunk;
    P.expect_len = a->batch == 1 && a->max_seq_len > 0 ? a->max_seq_len : 0;
    P.scale_log2 = static_cast<float>(static_cast<double>(a->scale) * 1.4426950408889634074);
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (a->sweep_events[0] && a->sweep_events[1]) {
        ev0 = reinterpret_cast<hipEvent_t>(a->sweep_events[0]);
        ev1 = reinterpret_cast<hipEvent_t>(a->sweep_events[1]);
    }
    hipError_t e;
    if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess)
        return gqa::fail(GQA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
    e = gqa::launch_sweep(P, a->in_dtype, a->out_dtype, a->d_head, plan.split_blocks, plan.fused != 0, stream);
    if (e != hipSuccess) return gqa::fail(GQA_ERR_HIP, "sweep kernel launch failed: %s", hipGetErrorString(e));
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess)
        return gqa::fail(GQA_ERR_HIP, "hipEventRecord failed: %s", hipGetErrorString(e));
    if (plan.fused) return GQA_OK;   // the merge ran inside the sweep
    e = gqa::launch_merge(P, a->out_dtype, a->d_head, plan.merge_blocks, plan.merge_threads,
                          plan.merge_slices, stream);
    if (e != hipSuccess) return gqa::fail(GQA_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
    return GQA_OK;
}

int decode_ex(const gqa_decode_args *a) {
    gqa::clear_error();
    int dev = 0;
    gqa_decode_plan plan;
    int st = decode_plan(a, &dev, &plan);
    if (st != GQA_OK) return st;
    void *ws = a->workspace;
    if (!ws) {
        st = owned_workspace(dev, reinterpret_cast<hipStream_t>(a->stream), kDecodeWorkspace, plan.workspace_bytes,
                             &ws);
        if (st != GQA_OK) return st;
    }
    return decode_launch(a, plan, ws);
}

// ------------------------------------------------------------------ no-allocation entry point
//
// Scratch of gqa_decode_noalloc: the partial triples of a call live in this
// file-scope device array instead of a workspace, so the call allocates nothing.
// Every device the library runs it on holds its own copy until the process ends;
// the array starts zeroed (as every device variable does), which is what its
// leading counter reserve needs, and every call leaves those counters zero; the
// rest needs no initialisation.  Host code never passes the array's name to
// a kernel (that would be the host-side stand-in, not a device address): it
// takes the device address once per device with hipGetSymbolAddress and uses
// that pointer.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

std::map<int, void *> g_scratch;   // device -> address of its `scratch`

int scratch_address(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return gqa::fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                             hipGetErrorString(e));
        it = g_scratch.emplace(dev, ptr).first;
    }
    *out = it->second;
    return GQA_OK;
}

int decode_noalloc(const gqa_decode_args *a) {
    gqa::clear_error();
    if (!a) return gqa::fail(GQA_ERR_NULL, "args is NULL");
    if (a->workspace || a->workspace_bytes)
        return gqa::fail(GQA_ERR_ARG, "gqa_decode_noalloc uses its own scratch: workspace must be NULL and "
                         "workspace_bytes 0");
    int st = gqa::validate(a);
    if (st != GQA_OK) return st;
    int dev = 0;
    gqa_decode_plan plan;
    st = decode_plan(a, &dev, &plan);
    if (st != GQA_OK) return st;
    if (plan.workspace_bytes > static_cast<size_t>(GQA_NOALLOC_SCRATCH_BYTES))
        return gqa::fail(GQA_ERR_WORKSPACE,
                         "the call needs %zu bytes of scratch (%d wavefronts x %d rows x d_head %d), above the "
                         "%d bytes gqa_decode_noalloc holds; pass a smaller num_chunks or use gqa_decode_ex",
                         plan.workspace_bytes, plan.num_chunks, (a->h_q / a->h_kv) * (a->t_q > 0 ? a->t_q : 1),
                         a->d_head, GQA_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    st = scratch_address(dev, &ws);
    if (st != GQA_OK) return st;
    return decode_launch(a, plan, ws);
}

// Resident prefill workgroups per compute unit, cached per (device, variant).
std::map<std::pair<int, int>, int> g_prefill_blocks_per_cu;

int prefill_ex(const gqa_prefill_args *a) {
    gqa::clear_error();
    int st = gqa::validate_prefill(a);
    if (st != GQA_OK) return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return gqa::fail(GQA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    int blocks = a->num_blocks;
    if (blocks == 0) {
        int num_cus = 0, waves = 0;
        st = device_shape(dev, GQA_DTYPE_BF16, GQA_DTYPE_BF16, a->d_head, &num_cus, &waves);
        if (st != GQA_OK) return st;
        std::lock_guard<std::mutex> lock(g_mu);
        const auto key = std::make_pair(dev, variant_id(a->in_dtype, a->out_dtype, a->d_head));
        auto it = g_prefill_blocks_per_cu.find(key);
        if (it == g_prefill_blocks_per_cu.end()) {
            int per_cu = 0;
            e = gqa::prefill_occupancy(a->in_dtype, a->out_dtype, a->d_head, &per_cu);
            if (e != hipSuccess || per_cu <= 0)
                return gqa::fail(GQA_ERR_HIP, "prefill occupancy query failed: %s", hipGetErrorString(e));
            it = g_prefill_blocks_per_cu.emplace(key, per_cu).first;
        }
        blocks = num_cus * it->second;
    }
    gqa::PrefillParams P;
    P.q = static_cast<const uint8_t *>(a->q);
    P.k = static_cast<const uint8_t *>(a->k);
    P.v = static_cast<const uint8_t *>(a->v);
    P.o = static_cast<uint8_t *>(a->o);
    P.seq_lens = a->seq_lens;
    P.batch = a->batch;
    P.h_q = a->h_q;
    P.h_kv = a->h_kv;
    P.G = a->h_q / a->h_kv;
    P.scale_log2 = static_cast<float>(static_cast<double>(a->scale) * 1.4426950408889634074);
    P.split_pv = a->split_pv;
    hipStream_t stream = reinterpret_cast<hipStream_t>(a->stream);
    const gqa::PrefillWorkspace W = gqa::prefill_workspace(a);
    P.vt = nullptr;
    P.vflags = nullptr;
    P.nvb = 0;
    P.queue = nullptr;
    if (W.bytes > 0) {
        void *ws = a->workspace;
        if (!ws) {
            st = owned_workspace(dev, stream, kPrefillWorkspace, W.bytes, &ws);
            if (st != GQA_OK) return st;
        }
        gqa::VprepParams V;
        V.v = P.v;
        V.vt = static_cast<uint8_t *>(ws);
        V.flags = static_cast<uint8_t *>(ws) + W.flags_offset;
        V.seq_lens = a->seq_lens;
        V.batch = a->batch;
        V.h_kv = a->h_kv;
        V.nvb = W.nvb;
        V.queue = reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(ws) + W.queue_offset);
        e = gqa::launch_vprep(V, a->in_dtype, a->d_head, stream);
        if (e != hipSuccess) return gqa::fail(GQA_ERR_HIP, "V copy kernel launch failed: %s", hipGetErrorString(e));
        P.vt = V.vt;
        P.vflags = V.flags;
        P.nvb = W.nvb;
        P.queue = V.queue;
    }
    e = gqa::launch_prefill(P, a->in_dtype, a->out_dtype, a->d_head, blocks, stream);
    if (e != hipSuccess) return gqa::fail(GQA_ERR_HIP, "prefill kernel launch failed: %s", hipGetErrorString(e));
    return GQA_OK;
}

gqa_prefill_args make_prefill_args(const void *q, const void *k, const void *v, void *o,
                                   const int32_t *seq_lens, int32_t batch, int64_t total_tokens, int32_t h_q,
                                   int32_t h_kv, int32_t d_head, float scale, void *stream, int dtype) {
    gqa_prefill_args a = {};
    a.total_tokens = total_tokens;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.seq_lens = seq_lens;
    a.batch = batch;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.d_head = d_head;
    a.scale = scale;
    a.in_dtype = dtype;
    a.out_dtype = dtype;
    a.stream = stream;
    return a;
}

gqa_decode_args make_args(const void *q, const void *k, const void *v, void *o,
                          const int32_t *seq_lens, int32_t batch, int32_t h_q, int32_t h_kv,
                          int32_t d_head, float scale, void *stream, int dtype) {
    gqa_decode_args a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.seq_lens = seq_lens;
    a.batch = batch;
    a.h_q = h_q;
    a.h_kv = h_kv;
    a.d_head = d_head;
    a.scale = scale;
    a.in_dtype = dtype;
    a.out_dtype = dtype;
    a.stream = stream;
    return a;
}

}  // namespace

extern "C" {

int gqa_decode_ex(const gqa_decode_args *args) {
    try {
        return decode_ex(args);
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_decode_noalloc(const gqa_decode_args *args) {
    try {
        return decode_noalloc(args);
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_decode(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
               int32_t batch, int32_t h_q, int32_t h_kv, int32_t d_head, float scale, void *stream) {
    const gqa_decode_args a =
        make_args(q, k, v, o, seq_lens, batch, h_q, h_kv, d_head, scale, stream, GQA_DTYPE_BF16);
    return gqa_decode_ex(&a);
}

int gqa_decode_f32(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
                   int32_t batch, int32_t h_q, int32_t h_kv, int32_t d_head, float scale,
                   void *stream) {
    const gqa_decode_args a =
        make_args(q, k, v, o, seq_lens, batch, h_q, h_kv, d_head, scale, stream, GQA_DTYPE_F32);
    return gqa_decode_ex(&a);
}

int gqa_decode_f16(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
                   int32_t batch, int32_t h_q, int32_t h_kv, int32_t d_head, float scale,
                   void *stream) {
    const gqa_decode_args a =
        make_args(q, k, v, o, seq_lens, batch, h_q, h_kv, d_head, scale, stream, GQA_DTYPE_F16);
    return gqa_decode_ex(&a);
}

int gqa_prefill_ex(const gqa_prefill_args *args) {
    try {
        return prefill_ex(args);
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_prefill(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens, int32_t batch,
                int64_t total_tokens, int32_t h_q, int32_t h_kv, int32_t d_head, float scale, void *stream) {
    const gqa_prefill_args a = make_prefill_args(q, k, v, o, seq_lens, batch, total_tokens, h_q, h_kv, d_head,
                                                 scale, stream, GQA_DTYPE_BF16);
    return gqa_prefill_ex(&a);
}

int gqa_prefill_f16(const void *q, const void *k, const void *v, void *o, const int32_t *seq_lens,
                    int32_t batch, int64_t total_tokens, int32_t h_q, int32_t h_kv, int32_t d_head, float scale,
                    void *stream) {
    const gqa_prefill_args a = make_prefill_args(q, k, v, o, seq_lens, batch, total_tokens, h_q, h_kv, d_head,
                                                 scale, stream, GQA_DTYPE_F16);
    return gqa_prefill_ex(&a);
}

int gqa_prefill_validate(const gqa_prefill_args *args) {
    try {
        gqa::clear_error();
        return gqa::validate_prefill(args);
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_prefill_workspace_bytes(const gqa_prefill_args *args, size_t *bytes) {
    try {
        gqa::clear_error();
        if (!bytes) return gqa::fail(GQA_ERR_NULL, "bytes is NULL");
        int st = gqa::validate_prefill(args, false);
        if (st != GQA_OK) return st;
        *bytes = gqa::prefill_workspace(args).bytes;
        return GQA_OK;
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_decode_validate(const gqa_decode_args *args) {
    try {
        gqa::clear_error();
        return gqa::validate(args);
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_decode_make_plan(const gqa_decode_args *args, int32_t num_cus, int32_t waves_per_cu,
                         gqa_decode_plan *plan) {
    try {
        gqa::clear_error();
        return gqa::make_plan(args, num_cus, waves_per_cu, plan);
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

int gqa_decode_workspace_bytes(const gqa_decode_args *args, size_t *bytes) {
    try {
        gqa::clear_error();
        if (!bytes) return gqa::fail(GQA_ERR_NULL, "bytes is NULL");
        int st = gqa::validate(args);
        if (st != GQA_OK) return st;
        int num_cus = 1, waves_per_cu = 1;
        if (args->num_chunks == 0) {
            int dev = 0;
            hipError_t e = hipGetDevice(&dev);
            if (e != hipSuccess)
                return gqa::fail(GQA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
            st = device_shape(dev, args->in_dtype, args->out_dtype, args->d_head, &num_cus, &waves_per_cu);
            if (st != GQA_OK) return st;
        }
        gqa_decode_plan plan;
        st = gqa::make_plan(args, num_cus, waves_per_cu, &plan);
        if (st != GQA_OK) return st;
        *bytes = plan.workspace_bytes;
        return GQA_OK;
    } catch (...) {
        return gqa::fail(GQA_ERR_HIP, "internal error");
    }
}

const char *gqa_status_str(int status) {
    switch (status) {
        case GQA_OK: return "GQA_OK";
        case GQA_ERR_NULL: return "GQA_ERR_NULL";
        case GQA_ERR_SHAPE: return "GQA_ERR_SHAPE";
        case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
        case GQA_ERR_ALIGN: return "GQA_ERR_ALIGN";
        case GQA_ERR_SCALE: return "GQA_ERR_SCALE";
        case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE";
        case GQA_ERR_HIP: return "GQA_ERR_HIP";
        case GQA_ERR_ARG: return "GQA_ERR_ARG";
        default: return "GQA_ERR_UNKNOWN";
    }
}

const char *gqa_last_error_message(void) { return gqa::last_error(); }

void gqa_release(void) {
    try {
        std::lock_guard<std::mutex> lock(g_mu);
        int cur = 0;
        const bool have_cur = hipGetDevice(&cur) == hipSuccess;
        for (auto &kv : g_workspaces) {
            if (!kv.second.ptr) continue;
            if (hipSetDevice(std::get<0>(kv.first)) == hipSuccess) {
                (void)hipDeviceSynchronize();
                (void)hipFree(kv.second.ptr);
            }
        }
        g_workspaces.clear();
        if (have_cur) (void)hipSetDevice(cur);
    } catch (...) {
    }
}

}  // extern "C"
