// rag_api.hip -- the extern "C" entry points of librag.so, the graph-captured
// pipeline and the host dispatch measurement.
//
// Host path ("Dispatch-Aware Ragged Attention for Pruned Vision Transformers",
// abstract: at post-pruning lengths the host-side dispatch of each attention
// call costs more than the GPU work, so the dispatch floor is what must come
// down): every entry point checks its arguments on the host, enqueues exactly
// one kernel on the caller's stream and returns; nothing is read back, nothing
// waits, nothing is allocated.  The pipeline captures the pass once into a
// HIP graph (the three launches, or the one gathered launch) so that a whole
// pack -> attend -> unpack pass is one hipGraphLaunch; it also enqueues the
// same pass from one host call as direct launches, which on ROCm 7.2 is the
// faster of the two (rag_measure_dispatch times a graph of one empty kernel
// beside them).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <new>
#include <vector>

#include "rag_internal.h"

using rag::set_error;

namespace {

rag_status hip_status(int err, const char* what)
{
    if (err == (int)hipSuccess) return RAG_OK;
    return set_error(RAG_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

__global__ void empty_kernel() {}
__global__ void empty_kernel_arg(const void*) {}

}  // namespace

extern "C" RAG_API rag_status rag_pack(const uint8_t* keep, int32_t B, int32_t N, const void* src,
                                       int64_t src_row_stride, int32_t row_bytes, void* packed,
                                       int64_t packed_row_stride, int32_t* cu_seqlens,
                                       int32_t* gather_idx, int32_t* max_seqlen_dev, void* stream)
{
    rag_status s = rag::validate_pack(keep, B, N, src, src_row_stride, row_bytes, packed,
                                      packed_row_stride, cu_seqlens, gather_idx);
    if (s != RAG_OK) return s;
    return hip_status(rag::launch_pack(keep, B, N, src, src_row_stride, row_bytes, packed,
                                       packed_row_stride, cu_seqlens, gather_idx, max_seqlen_dev,
                                       stream),
                      "rag_pack launch");
}

extern "C" RAG_API rag_status rag_attn(const void* q, const void* k, const void* v,
                                       int64_t q_row_stride, int64_t k_row_stride,
                                       int64_t v_row_stride, rag_dtype in_dtype,
                                       const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                       int32_t total_rows, int32_t H, int32_t head_dim,
                                       float scale, void* o, int64_t o_row_stride,
                                       rag_dtype out_dtype, void* stream)
{
    rag_status s = rag::validate_attn(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                      cu_seqlens, B, max_seqlen, total_rows, H, head_dim, scale, o,
                                      o_row_stride, out_dtype);
    if (s != RAG_OK) return s;
    return hip_status(rag::launch_attn(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                       cu_seqlens, nullptr, B, 0, max_seqlen, total_rows, H, scale,
                                       o, o_row_stride, out_dtype, rag::kLayoutRagged, 0u, stream),
                      "rag_attn launch");
}

extern "C" RAG_API rag_status rag_attn_tiled(const void* q, const void* k, const void* v,
                                             int64_t q_row_stride, int64_t k_row_stride,
                                             int64_t v_row_stride, rag_dtype in_dtype,
                                             const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                             int32_t total_rows, int32_t H, int32_t head_dim,
                                             float scale, void* o, int64_t o_row_stride,
                                             rag_dtype out_dtype, void* stream)
{
    rag_status s = rag::validate_attn(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                      cu_seqlens, B, max_seqlen, total_rows, H, head_dim, scale, o,
                                      o_row_stride, out_dtype);
    if (s != RAG_OK) return s;
    if ((s = rag::validate_tile_list(B, H, max_seqlen)) != RAG_OK) return s;
    return hip_status(rag::launch_attn(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                       cu_seqlens, nullptr, B, 0, max_seqlen, total_rows, H, scale,
                                       o, o_row_stride, out_dtype, rag::kLayoutRagged,
                                       rag::kAttnTileList, stream),
                      "rag_attn_tiled launch");
}

extern "C" RAG_API rag_status rag_unpack(const void* packed, int64_t packed_row_stride,
                                         int32_t row_bytes, const int32_t* cu_seqlens,
                                         const int32_t* gather_idx, int32_t B, int32_t N,
                                         void* dst, int64_t dst_row_stride, uint32_t flags,
                                         void* stream)
{
    rag_status s = rag::validate_unpack(packed, packed_row_stride, row_bytes, cu_seqlens,
                                        gather_idx, B, N, dst, dst_row_stride, flags);
    if (s != RAG_OK) return s;
    return hip_status(rag::launch_unpack(packed, packed_row_stride, row_bytes, cu_seqlens,
                                         gather_idx, B, N, dst, dst_row_stride, flags, stream),
                      "rag_unpack launch");
}

extern "C" RAG_API rag_status rag_repack(const uint8_t* keep_packed, const int32_t* cu_in,
                                         const int32_t* gather_in, int32_t B, int32_t max_rows_in,
                                         int32_t total_rows, const void* src,
                                         int64_t src_row_stride, int32_t row_bytes, void* dst,
                                         int64_t dst_row_stride, int32_t* cu_out,
                                         int32_t* gather_out, void* stream)
{
    rag_status s = rag::validate_repack(keep_packed, cu_in, gather_in, B, max_rows_in, total_rows,
                                        src, src_row_stride, row_bytes, dst, dst_row_stride,
                                        cu_out, gather_out);
    if (s != RAG_OK) return s;
    return hip_status(rag::launch_repack(keep_packed, cu_in, gather_in, B, max_rows_in, total_rows,
                                         src, src_row_stride, row_bytes, dst, dst_row_stride,
                                         cu_out, gather_out, stream),
                      "rag_repack launch");
}

extern "C" RAG_API rag_status rag_attn_padded(const void* q, const void* k, const void* v,
                                              int64_t q_row_stride, int64_t k_row_stride,
                                              int64_t v_row_stride, rag_dtype in_dtype,
                                              const uint8_t* keep, int32_t B, int32_t N,
                                              int32_t H, int32_t head_dim, float scale, void* o,
                                              int64_t o_row_stride, rag_dtype out_dtype,
                                              void* stream)
{
    rag_status s = rag::validate_attn_padded(q, k, v, q_row_stride, k_row_stride, v_row_stride,
                                             in_dtype, keep, B, N, H, head_dim, scale, o,
                                             o_row_stride, out_dtype);
    if (s != RAG_OK) return s;
    return hip_status(rag::launch_attn(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                       nullptr, keep, B, N, N, B * N, H, scale, o, o_row_stride,
                                       out_dtype, rag::kLayoutPadded, 0u, stream),
                      "rag_attn_padded launch");
}

extern "C" RAG_API rag_status rag_attn_gathered(const uint8_t* keep, int32_t B, int32_t N,
                                                int32_t max_seqlen, const void* q, const void* k, const void* v,
                                                int64_t q_row_stride, int64_t k_row_stride,
                                                int64_t v_row_stride, rag_dtype in_dtype,
                                                int32_t H, int32_t head_dim, float scale, void* o,
                                                int64_t o_row_stride, rag_dtype out_dtype,
                                                uint32_t flags, void* stream)
{
    rag_status s = rag::validate_attn_gathered(keep, B, N, max_seqlen, q, k, v, q_row_stride, k_row_stride,
                                               v_row_stride, in_dtype, H, head_dim, scale, o,
                                               o_row_stride, out_dtype, flags);
    if (s != RAG_OK) return s;
    return hip_status(rag::launch_attn(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                       nullptr, keep, B, N, max_seqlen ? max_seqlen : N, B * N, H,
                                       scale, o, o_row_stride, out_dtype, rag::kLayoutGathered,
                                       flags, stream),
                      "rag_attn_gathered launch");
}

// ---------------------------------------------------------------- pipeline
struct rag_pipeline {
    rag_pipeline_desc d;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

namespace {

// The three launches of one pass, in order, on `stream`.
rag_status enqueue_pass(const rag_pipeline_desc& d, void* stream)
{
    const int64_t C = (int64_t)d.H * d.head_dim;
    const int in_es = rag::dtype_bytes(d.in_dtype), out_es = rag::dtype_bytes(d.out_dtype);
    const int32_t in_row = (int32_t)(3 * C * in_es), out_row = (int32_t)(C * out_es);
    int e = rag::launch_pack(d.keep, d.B, d.N, d.src, d.src_row_stride, in_row, d.packed,
                             d.packed_row_stride, d.cu_seqlens, d.gather_idx, d.max_seqlen_dev,
                             stream);
    if (e != (int)hipSuccess) return hip_status(e, "pipeline pack");
    const char* base = static_cast<const char*>(d.packed);
    const int64_t ps = d.packed_row_stride / in_es;
    e = rag::launch_attn(base, base + C * in_es, base + 2 * C * in_es, ps, ps, ps, d.in_dtype,
                         d.cu_seqlens, nullptr, d.B, 0, d.max_seqlen ? d.max_seqlen : d.N,
                         d.B * d.N, d.H, d.scale, d.o_packed, d.o_packed_row_stride / out_es,
                         d.out_dtype, rag::kLayoutRagged, 0u, stream);
    if (e != (int)hipSuccess) return hip_status(e, "pipeline attn");
    e = rag::launch_unpack(d.o_packed, d.o_packed_row_stride, out_row, d.cu_seqlens, d.gather_idx,
                           d.B, d.N, d.dst, d.dst_row_stride, d.unpack_flags, stream);
    return hip_status(e, "pipeline unpack");
}

// The same pass as one launch: attention on the kept rows of src, output
// written to their rows of dst (no packed buffers, no offsets).
rag_status enqueue_fused(const rag_pipeline_desc& d, void* stream)
{
    const int64_t C = (int64_t)d.H * d.head_dim;
    const int in_es = rag::dtype_bytes(d.in_dtype), out_es = rag::dtype_bytes(d.out_dtype);
    const char* sr = static_cast<const char*>(d.src);
    const int64_t ss = d.src_row_stride / in_es;
    const int e = rag::launch_attn(sr, sr + C * in_es, sr + 2 * C * in_es, ss, ss, ss, d.in_dtype,
                                   nullptr, d.keep, d.B, d.N, d.max_seqlen ? d.max_seqlen : d.N,
                                   d.B * d.N, d.H, d.scale, d.dst,
                                   d.dst_row_stride / out_es, d.out_dtype, rag::kLayoutGathered,
                                   d.unpack_flags, stream);
    return hip_status(e, "pipeline fused attn");
}

}  // namespace

extern "C" RAG_API rag_status rag_pipeline_create(const rag_pipeline_desc* desc, rag_pipeline** out)
{
    if (!out) return set_error(RAG_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    rag_status s = rag::validate_pipeline(desc);
    if (s != RAG_OK) return s;
    rag_pipeline* p = new (std::nothrow) rag_pipeline;
    if (!p) return set_error(RAG_ERR_NO_MEMORY, "out of host memory");
    p->d = *desc;
    if (p->d.flags & RAG_PIPELINE_DIRECT) {  // direct launches: nothing to capture
        *out = p;
        return RAG_OK;
    }
    hipStream_t cs = nullptr;
    s = hip_status((int)hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "capture stream");
    if (s == RAG_OK) {
        s = hip_status((int)hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal),
                       "begin capture");
        if (s == RAG_OK) {
            rag_status es = (p->d.flags & RAG_PIPELINE_FUSED) ? enqueue_fused(p->d, cs) : enqueue_pass(p->d, cs);
            rag_status cs_end = hip_status((int)hipStreamEndCapture(cs, &p->graph), "end capture");
            s = es != RAG_OK ? es : cs_end;
        }
        if (s == RAG_OK)
            s = hip_status((int)hipGraphInstantiate(&p->exec, p->graph, nullptr, nullptr, 0),
                           "graph instantiate");
        (void)hipStreamDestroy(cs);
    }
    if (s != RAG_OK) {
        rag_pipeline_destroy(p);
        return s;
    }
    *out = p;
    return RAG_OK;
}

extern "C" RAG_API rag_status rag_pipeline_launch(rag_pipeline* p, void* stream)
{
    if (!p) return set_error(RAG_ERR_INVALID_ARG, "pipeline is NULL");
    if (p->d.flags & RAG_PIPELINE_DIRECT)
        return (p->d.flags & RAG_PIPELINE_FUSED) ? enqueue_fused(p->d, stream) : enqueue_pass(p->d, stream);
    if (!p->exec) return set_error(RAG_ERR_INVALID_ARG, "pipeline has no graph");
    return hip_status((int)hipGraphLaunch(p->exec, static_cast<hipStream_t>(stream)),
                      "hipGraphLaunch");
}

extern "C" RAG_API rag_status rag_pipeline_launch_eager(rag_pipeline* p, void* stream)
{
    if (!p) return set_error(RAG_ERR_INVALID_ARG, "pipeline is NULL");
    return enqueue_pass(p->d, stream);
}

extern "C" RAG_API rag_status rag_pipeline_launch_fused(rag_pipeline* p, void* stream)
{
    if (!p) return set_error(RAG_ERR_INVALID_ARG, "pipeline is NULL");
    return enqueue_fused(p->d, stream);
}

extern "C" RAG_API void rag_pipeline_destroy(rag_pipeline* p)
{
    if (!p) return;
    if (p->exec) (void)hipGraphExecDestroy(p->exec);
    if (p->graph) (void)hipGraphDestroy(p->graph);
    delete p;
}

// ------------------------------------------------------- dispatch measurement
namespace {

typedef std::chrono::steady_clock Clock;

void percentiles(std::vector<double>& v, double* out3)
{
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    const double qs[3] = {0.10, 0.50, 0.90};
    for (int i = 0; i < 3; ++i) out3[i] = n ? v[std::min(n - 1, (size_t)(qs[i] * (n - 1) + 0.5))] : 0.0;
}

double us_since(Clock::time_point t0, Clock::time_point t1)
{
    return std::chrono::duration<double, std::micro>(t1 - t0).count();
}

// Times `launch` (returning a rag_status) `iters` times: round trip with
// hipStreamSynchronize into rt[3], host enqueue time into enq[3] (if non-NULL).
template <typename F>
rag_status time_calls(F launch, hipStream_t st, int warmup, int iters, double* rt, double* enq)
{
    std::vector<double> a, b;
    try {  // (no exception crosses the C ABI; push_back below never reallocates)
        a.reserve(iters);
        b.reserve(iters);
    } catch (const std::bad_alloc&) {
        return set_error(RAG_ERR_NO_MEMORY, "out of host memory");
    }
    for (int i = 0; i < warmup + iters; ++i) {
        const Clock::time_point t0 = Clock::now();
        rag_status s = launch();
        const Clock::time_point t1 = Clock::now();
        if (s != RAG_OK) return s;
        rag_status ss = hip_status((int)hipStreamSynchronize(st), "hipStreamSynchronize");
        const Clock::time_point t2 = Clock::now();
        if (ss != RAG_OK) return ss;
        if (i >= warmup) {
            a.push_back(us_since(t0, t2));
            b.push_back(us_since(t0, t1));
        }
    }
    percentiles(a, rt);
    if (enq) percentiles(b, enq);
    return RAG_OK;
}

}  // namespace

extern "C" RAG_API rag_status rag_measure_dispatch(rag_pipeline* p, int32_t warmup, int32_t iters,
                                                   double* out_us, void* stream)
{
    if (!p || !out_us || warmup < 0 || iters < 1)
        return set_error(RAG_ERR_INVALID_ARG, "bad arguments to rag_measure_dispatch");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const rag_pipeline_desc& d = p->d;
    const int64_t C = (int64_t)d.H * d.head_dim;
    const int in_es = rag::dtype_bytes(d.in_dtype), out_es = rag::dtype_bytes(d.out_dtype);
    const char* pk = static_cast<const char*>(d.packed);
    const int64_t ps = d.packed_row_stride / in_es;
    const char* sr = static_cast<const char*>(d.src);
    const int64_t ss = d.src_row_stride / in_es;
    const int32_t maxlen = d.max_seqlen ? d.max_seqlen : d.N;

    auto empty = [&]() {
        hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, st);
        return hip_status((int)hipGetLastError(), "empty kernel");
    };
    auto attn = [&]() {
        return rag_attn(pk, pk + C * in_es, pk + 2 * C * in_es, ps, ps, ps, d.in_dtype,
                        d.cu_seqlens, d.B, maxlen, d.B * d.N, d.H, d.head_dim, d.scale, d.o_packed,
                        d.o_packed_row_stride / out_es, d.out_dtype, st);
    };
    auto eager = [&]() { return enqueue_pass(d, st); };
    auto graph = [&]() { return rag_pipeline_launch(p, st); };
    auto padded = [&]() {
        return rag_attn_padded(sr, sr + C * in_es, sr + 2 * C * in_es, ss, ss, ss, d.in_dtype,
                               d.keep, d.B, d.N, d.H, d.head_dim, d.scale, d.dst,
                               d.dst_row_stride / out_es, d.out_dtype, st);
    };
    auto fused = [&]() {
        return rag_attn_gathered(d.keep, d.B, d.N, d.max_seqlen, sr, sr + C * in_es, sr + 2 * C * in_es, ss, ss,
                                 ss, d.in_dtype, d.H, d.head_dim, d.scale, d.dst,
                                 d.dst_row_stride / out_es, d.out_dtype, d.unpack_flags, st);
    };
    rag_status s;
    if ((s = time_calls(empty, st, warmup, iters, out_us + 0, out_us + 3)) != RAG_OK) return s;
    if ((s = time_calls(attn, st, warmup, iters, out_us + 6, out_us + 9)) != RAG_OK) return s;
    if ((s = time_calls(eager, st, warmup, iters, out_us + 12, nullptr)) != RAG_OK) return s;
    if ((s = time_calls(graph, st, warmup, iters, out_us + 15, nullptr)) != RAG_OK) return s;
    if ((s = time_calls(padded, st, warmup, iters, out_us + 18, nullptr)) != RAG_OK) return s;
    if ((s = time_calls(fused, st, warmup, iters, out_us + 21, out_us + 24)) != RAG_OK) return s;
    auto empty_arg = [&]() {
        hipLaunchKernelGGL(empty_kernel_arg, dim3(1), dim3(64), 0, st, static_cast<const void*>(d.keep));
        return hip_status((int)hipGetLastError(), "empty kernel with an argument");
    };
    double unused_rt[3];
    if ((s = time_calls(empty_arg, st, warmup, iters, unused_rt, out_us + 27)) != RAG_OK) return s;
    // a graph of one empty kernel: what launching through a graph costs by itself
    hipGraph_t g1 = nullptr;
    hipGraphExec_t g1x = nullptr;
    hipStream_t cs = nullptr;
    s = hip_status((int)hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "capture stream");
    if (s == RAG_OK) {
        s = hip_status((int)hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal), "begin capture");
        if (s == RAG_OK) {
            hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, cs);
            const rag_status ls = hip_status((int)hipGetLastError(), "empty kernel capture");
            const rag_status es = hip_status((int)hipStreamEndCapture(cs, &g1), "end capture");
            s = ls != RAG_OK ? ls : es;
        }
        if (s == RAG_OK)
            s = hip_status((int)hipGraphInstantiate(&g1x, g1, nullptr, nullptr, 0), "graph instantiate");
        (void)hipStreamDestroy(cs);
    }
    auto graph1 = [&]() { return hip_status((int)hipGraphLaunch(g1x, st), "hipGraphLaunch"); };
    if (s == RAG_OK) s = time_calls(graph1, st, warmup, iters, out_us + 30, out_us + 33);
    if (g1x) (void)hipGraphExecDestroy(g1x);
    if (g1) (void)hipGraphDestroy(g1);
    return s;
}

extern "C" RAG_API rag_status rag_measure_stages(rag_pipeline* p, int32_t iters, double* out_us,
                                                 void* stream)
{
    if (!p || !out_us || iters < 1)
        return set_error(RAG_ERR_INVALID_ARG, "bad arguments to rag_measure_stages");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const rag_pipeline_desc& d = p->d;
    const int64_t C = (int64_t)d.H * d.head_dim;
    const int in_es = rag::dtype_bytes(d.in_dtype), out_es = rag::dtype_bytes(d.out_dtype);
    const int32_t in_row = (int32_t)(3 * C * in_es), out_row = (int32_t)(C * out_es);
    const char* pk = static_cast<const char*>(d.packed);
    const int64_t ps = d.packed_row_stride / in_es;
    const char* sr = static_cast<const char*>(d.src);
    const int64_t ss = d.src_row_stride / in_es;
    const int32_t maxlen = d.max_seqlen ? d.max_seqlen : d.N;
    auto pack = [&]() {
        return hip_status(rag::launch_pack(d.keep, d.B, d.N, d.src, d.src_row_stride, in_row,
                                           d.packed, d.packed_row_stride, d.cu_seqlens,
                                           d.gather_idx, d.max_seqlen_dev, st),
                          "pack");
    };
    auto attn = [&]() {
        return hip_status(rag::launch_attn(pk, pk + C * in_es, pk + 2 * C * in_es, ps, ps, ps,
                                           d.in_dtype, d.cu_seqlens, nullptr, d.B, 0, maxlen,
                                           d.B * d.N, d.H, d.scale, d.o_packed,
                                           d.o_packed_row_stride / out_es, d.out_dtype,
                                           rag::kLayoutRagged, 0u, st),
                          "attn");
    };
    auto unpack = [&]() {
        return hip_status(rag::launch_unpack(d.o_packed, d.o_packed_row_stride, out_row,
                                             d.cu_seqlens, d.gather_idx, d.B, d.N, d.dst,
                                             d.dst_row_stride, d.unpack_flags, st),
                          "unpack");
    };
    auto padded = [&]() {
        return hip_status(rag::launch_attn(sr, sr + C * in_es, sr + 2 * C * in_es, ss, ss, ss,
                                           d.in_dtype, nullptr, d.keep, d.B, d.N, d.N, d.B * d.N,
                                           d.H, d.scale, d.dst, d.dst_row_stride / out_es,
                                           d.out_dtype, rag::kLayoutPadded, 0u, st),
                          "padded");
    };
    auto eager = [&]() { return enqueue_pass(d, st); };
    auto graph = [&]() { return rag_pipeline_launch(p, st); };
    auto fused = [&]() { return enqueue_fused(d, st); };
    hipEvent_t e0 = nullptr, e1 = nullptr;
    rag_status s = hip_status((int)hipEventCreate(&e0), "hipEventCreate");
    if (s == RAG_OK) s = hip_status((int)hipEventCreate(&e1), "hipEventCreate");
    auto timed = [&](auto fn, double* out) -> rag_status {
        const int warm = std::max(1, iters / 10);
        for (int i = 0; i < warm; ++i)
            if (rag_status r = fn(); r != RAG_OK) return r;
        if (rag_status r = hip_status((int)hipEventRecord(e0, st), "hipEventRecord"); r != RAG_OK)
            return r;
        for (int i = 0; i < iters; ++i)
            if (rag_status r = fn(); r != RAG_OK) return r;
        if (rag_status r = hip_status((int)hipEventRecord(e1, st), "hipEventRecord"); r != RAG_OK)
            return r;
        if (rag_status r = hip_status((int)hipEventSynchronize(e1), "hipEventSynchronize");
            r != RAG_OK)
            return r;
        float ms = 0.f;
        if (rag_status r = hip_status((int)hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime");
            r != RAG_OK)
            return r;
        *out = (double)ms * 1e3 / iters;
        return RAG_OK;
    };
    if (s == RAG_OK) s = timed(pack, out_us + 0);
    if (s == RAG_OK) s = timed(attn, out_us + 1);
    if (s == RAG_OK) s = timed(unpack, out_us + 2);
    if (s == RAG_OK) s = timed(padded, out_us + 3);
    if (s == RAG_OK) s = timed(eager, out_us + 4);
    if (s == RAG_OK) s = timed(graph, out_us + 5);
    if (s == RAG_OK) s = timed(fused, out_us + 6);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return s;
}
