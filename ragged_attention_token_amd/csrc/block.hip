// block.hip -- one ViT encoder block on packed token rows, and the same block
// on the padded [B, N] rows, for timing the pipeline end to end.
//
// "Dispatch-Aware Ragged Attention for Pruned Vision Transformers" (abstract)
// measures end-to-end throughput of pruned DeiT models whose blocks run on the
// packed tokens; the pages fix the attention step (the ragged kernel) and the
// packing, not the rest of the block.  The block here is the standard
// pre-norm encoder block of DeiT (ViT) with random weights:
//     h  = LayerNorm1(x)
//     qkv = h Wqkv + bqkv                  (columns q | k | v, head-major)
//     a  = attention(qkv)                  (ragged, or padded with masked keys)
//     x1 = x + a Wproj + bproj
//     h2 = LayerNorm2(x1)
//     m  = GELU(h2 W1 + b1)
//     y  = x1 + m W2 + b2
// Row-wise steps (LayerNorm) are HIP kernels here; the four matrix products
// are plain library GEMMs (hipBLASLt, bf16 inputs, fp32 accumulation, bias /
// GELU / residual in its epilogue); the attention is this library's kernel.
// Every intermediate row is stored as bf16.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <map>
#include <new>
#include <utility>

#include "rag_device.h"
#include "rag_internal.h"

using rag::set_error;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
using rag::dev::u32x4;

constexpr int kLnRowsPerWave = 2;

// LayerNorm over rows of C bf16 values (C a multiple of 8, at most 2048):
// y = (x - mean) / sqrt(var + eps) * gamma + beta, mean and (biased) variance
// in fp32 over the row, y rounded to bf16.  Each wave normalises
// kLnRowsPerWave rows, 4 waves per workgroup; a lane holds NCH 16-byte chunks
// of each row (NCH = ceil(C / 512)), and every row's loads are issued before
// the first reduction.
template <int NCH>
__global__ __launch_bounds__(256) void layernorm_kernel(const __bf16* x, __bf16* y, int rows, int C,
                                                        const float* gamma, const float* beta,
                                                        float eps)
{
    constexpr int R = kLnRowsPerWave;
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    if (row0 >= rows) return;
    const int nchunk = C / 8;
    float v[R][NCH][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        // rows past the end read zeros (and are not written)
        const auto rx = rag::dev::make_rsrc(x + (int64_t)(row0 + r) * C,
                                            row0 + r < rows ? (uint32_t)C * 2u : 0u);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int ch = lane + 64 * j;
            const bf16x8 w = __builtin_bit_cast(bf16x8, rag::dev::ld16(rx, 16u * (uint32_t)ch));
#pragma unroll
            for (int e = 0; e < 8; ++e) v[r][j][e] = ch < nchunk ? static_cast<float>(w[e]) : 0.f;
        }
    }
    float mean[R], rstd[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += v[r][j][e];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        mean[r] = sum / (float)C;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const bool in = lane + 64 * j < nchunk;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = v[r][j][e] - mean[r];
                sq += in ? d * d : 0.f;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
        rstd[r] = 1.f / sqrtf(sq / (float)C + eps);
    }
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int ch = lane + 64 * j;
        if (ch >= nchunk) continue;
        const auto* g4 = reinterpret_cast<const f32x4*>(gamma + 8 * ch);
        const auto* b4 = reinterpret_cast<const f32x4*>(beta + 8 * ch);
        const f32x4 ga = g4[0], gb = g4[1], ba = b4[0], bb = b4[1];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (row0 + r >= rows) continue;
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float gm = e < 4 ? ga[e] : gb[e - 4], bt = e < 4 ? ba[e] : bb[e - 4];
                o[e] = static_cast<__bf16>((v[r][j][e] - mean[r]) * rstd[r] * gm + bt);
            }
            const auto ry = rag::dev::make_rsrc(y + (int64_t)(row0 + r) * C, (uint32_t)C * 2u);
            rag::dev::st16(__builtin_bit_cast(u32x4, o), ry, 16u * (uint32_t)ch);
        }
    }
}

// One GEMM of the block: D[M, N] = act(X[M, K] W[K, N] + bias) + R (row-major
// bf16 X, W, D, R; fp32 bias).  hipBLASLt is column-major, so the product is
// run as D^T = W^T X^T: m = N, n = M, k = K with W, X, D as stored.
struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    hipblasLtMatmulAlgo_t algo;
    bool residual = false;
};

enum GemmKind { kQkv = 0, kProj = 1, kFc1 = 2, kFc2 = 3 };

}  // namespace

struct rag_block {
    rag_block_desc d;
    int32_t C = 0, hidden = 0;
    hipblasLtHandle_t lt = nullptr;
    std::map<std::pair<int, int>, GemmPlan> plans;  // (kind, rows)
};

namespace {

void destroy_plan(GemmPlan& g)
{
    if (g.a) hipblasLtMatrixLayoutDestroy(g.a);
    if (g.b) hipblasLtMatrixLayoutDestroy(g.b);
    if (g.c) hipblasLtMatrixLayoutDestroy(g.c);
    if (g.desc) hipblasLtMatmulDescDestroy(g.desc);
    g = GemmPlan();
}

rag_status lt_status(hipblasStatus_t s, const char* what)
{
    if (s == HIPBLAS_STATUS_SUCCESS) return RAG_OK;
    return set_error(RAG_ERR_HIP, "%s: hipBLASLt status %d", what, (int)s);
}

// The plan of GEMM `kind` at M rows, built on first use and kept.
rag_status get_plan(rag_block* blk, int kind, int M, GemmPlan** out)
{
    auto it = blk->plans.find({kind, M});
    if (it != blk->plans.end()) {
        *out = &it->second;
        return RAG_OK;
    }
    const int C = blk->C, Hd = blk->hidden;
    int K = C, N = C;
    const void* bias = nullptr;
    hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
    bool residual = false;
    switch (kind) {
    case kQkv: K = C; N = 3 * C; bias = blk->d.b_qkv; break;
    case kProj: K = C; N = C; bias = blk->d.b_proj; residual = true; break;
    case kFc1: K = C; N = Hd; bias = blk->d.b_fc1; epi = HIPBLASLT_EPILOGUE_GELU_BIAS; break;
    default: K = Hd; N = C; bias = blk->d.b_fc2; residual = true; break;
    }
    GemmPlan g;
    g.residual = residual;
    rag_status s;
    if ((s = lt_status(hipblasLtMatmulDescCreate(&g.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F), "desc")) != RAG_OK)
        return s;
    const hipblasOperation_t op = HIPBLAS_OP_N;
    const hipDataType bias_type = HIP_R_32F;
    s = lt_status(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof op), "transa");
    if (s == RAG_OK)
        s = lt_status(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof op), "transb");
    if (s == RAG_OK)
        s = lt_status(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof epi), "epilogue");
    if (s == RAG_OK)
        s = lt_status(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof bias), "bias");
    if (s == RAG_OK)
        s = lt_status(hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                                      sizeof bias_type), "bias type");
    if (s == RAG_OK) s = lt_status(hipblasLtMatrixLayoutCreate(&g.a, HIP_R_16BF, N, K, N), "layout W");
    if (s == RAG_OK) s = lt_status(hipblasLtMatrixLayoutCreate(&g.b, HIP_R_16BF, K, M, K), "layout X");
    if (s == RAG_OK) s = lt_status(hipblasLtMatrixLayoutCreate(&g.c, HIP_R_16BF, N, M, N), "layout D");
    if (s == RAG_OK) {
        hipblasLtMatmulPreference_t pref = nullptr;
        s = lt_status(hipblasLtMatmulPreferenceCreate(&pref), "preference");
        if (s == RAG_OK) {
            const uint64_t ws = blk->d.workspace_bytes;
            s = lt_status(hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                                                sizeof ws), "workspace");
            hipblasLtMatmulHeuristicResult_t res[1];
            int found = 0;
            if (s == RAG_OK)
                s = lt_status(hipblasLtMatmulAlgoGetHeuristic(blk->lt, g.desc, g.a, g.b, g.c, g.c, pref, 1, res,
                                                              &found), "heuristic");
            if (s == RAG_OK && found < 1) s = set_error(RAG_ERR_UNSUPPORTED, "no GEMM algorithm for M=%d", M);
            if (s == RAG_OK) g.algo = res[0].algo;
            hipblasLtMatmulPreferenceDestroy(pref);
        }
    }
    if (s != RAG_OK) {
        destroy_plan(g);
        return s;
    }
    try {
        auto ins = blk->plans.emplace(std::make_pair(kind, M), g);
        *out = &ins.first->second;
    } catch (...) {
        destroy_plan(g);
        return set_error(RAG_ERR_NO_MEMORY, "out of host memory");
    }
    return RAG_OK;
}

rag_status run_gemm(rag_block* blk, int kind, int M, const void* W, const void* X, const void* R,
                    void* D, hipStream_t st)
{
    GemmPlan* g = nullptr;
    rag_status s = get_plan(blk, kind, M, &g);
    if (s != RAG_OK) return s;
    const float alpha = 1.f, beta = g->residual ? 1.f : 0.f;
    return lt_status(hipblasLtMatmul(blk->lt, g->desc, &alpha, W, g->a, X, g->b, &beta, g->residual ? R : D,
                                     g->c, D, g->c, &g->algo, blk->d.workspace, blk->d.workspace_bytes, st),
                     "matmul");
}

rag_status run_layernorm(const void* x, void* y, int rows, int C, const void* gamma, const void* beta, float eps,
                         hipStream_t st)
{
    if (rows == 0) return RAG_OK;
    const int per_group = 4 * kLnRowsPerWave;
    const dim3 grid((rows + per_group - 1) / per_group), block(256);
    const auto* xb = static_cast<const __bf16*>(x);
    auto* yb = static_cast<__bf16*>(y);
    const auto* gm = static_cast<const float*>(gamma);
    const auto* bt = static_cast<const float*>(beta);
    if (C <= 512)
        hipLaunchKernelGGL(layernorm_kernel<1>, grid, block, 0, st, xb, yb, rows, C, gm, bt, eps);
    else if (C <= 1024)
        hipLaunchKernelGGL(layernorm_kernel<2>, grid, block, 0, st, xb, yb, rows, C, gm, bt, eps);
    else
        hipLaunchKernelGGL(layernorm_kernel<4>, grid, block, 0, st, xb, yb, rows, C, gm, bt, eps);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? RAG_OK : set_error(RAG_ERR_HIP, "layernorm launch: %s", hipGetErrorString(e));
}

// Scratch layout (bf16 rows): h [rows, C] | qkv [rows, 3C] | a [rows, C] |
// x1 [rows, C] | m [rows, hidden]; h is reused for LayerNorm2's output.
size_t scratch_bytes(int64_t rows, int64_t C, int64_t hidden)
{
    return (size_t)rows * (size_t)(6 * C + hidden) * 2u;
}

rag_status forward(rag_block* blk, const void* x, void* y, int32_t rows, const int32_t* cu, const uint8_t* keep,
                   int32_t B, int32_t N, int32_t max_seqlen, void* scratch, int layout, hipStream_t st)
{
    const int C = blk->C;
    char* base = static_cast<char*>(scratch);
    char* h = base;
    char* qkv = h + (size_t)rows * C * 2;
    char* a = qkv + (size_t)rows * 3 * C * 2;
    char* x1 = a + (size_t)rows * C * 2;
    char* m = x1 + (size_t)rows * C * 2;
    const rag_block_desc& d = blk->d;
    rag_status s;
    if ((s = run_layernorm(x, h, rows, C, d.ln1_gamma, d.ln1_beta, d.eps, st)) != RAG_OK) return s;
    if ((s = run_gemm(blk, kQkv, rows, d.w_qkv, h, nullptr, qkv, st)) != RAG_OK) return s;
    const int e = rag::launch_attn(qkv, qkv + C * 2, qkv + 2 * C * 2, 3 * C, 3 * C, 3 * C, RAG_DTYPE_BF16, cu, keep,
                                   B, N, max_seqlen, rows, d.H, d.scale, a, C, RAG_DTYPE_BF16, layout, 0u, st);
    if (e != (int)hipSuccess) return set_error(RAG_ERR_HIP, "block attention: %s", hipGetErrorString((hipError_t)e));
    if ((s = run_gemm(blk, kProj, rows, d.w_proj, a, x, x1, st)) != RAG_OK) return s;
    if ((s = run_layernorm(x1, h, rows, C, d.ln2_gamma, d.ln2_beta, d.eps, st)) != RAG_OK) return s;
    if ((s = run_gemm(blk, kFc1, rows, d.w_fc1, h, nullptr, m, st)) != RAG_OK) return s;
    return run_gemm(blk, kFc2, rows, d.w_fc2, m, x1, y, st);
}

}  // namespace

extern "C" RAG_API size_t rag_block_scratch_bytes(int32_t rows, int32_t H, int32_t mlp_ratio)
{
    if (rows < 0 || H < 1 || mlp_ratio < 1) return 0;
    const int64_t C = (int64_t)H * RAG_HEAD_DIM;
    return scratch_bytes(rows, C, C * mlp_ratio);
}

extern "C" RAG_API rag_status rag_block_create(const rag_block_desc* desc, rag_block** out)
{
    if (!out) return set_error(RAG_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    rag_status s = rag::validate_block_desc(desc);
    if (s != RAG_OK) return s;
    rag_block* blk = new (std::nothrow) rag_block();
    if (!blk) return set_error(RAG_ERR_NO_MEMORY, "out of host memory");
    blk->d = *desc;
    blk->C = desc->H * RAG_HEAD_DIM;
    blk->hidden = blk->C * desc->mlp_ratio;
    s = lt_status(hipblasLtCreate(&blk->lt), "hipblasLtCreate");
    if (s != RAG_OK) {
        delete blk;
        return s;
    }
    *out = blk;
    return RAG_OK;
}

extern "C" RAG_API rag_status rag_block_forward(rag_block* blk, const void* x, void* y, int32_t rows,
                                                const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                                void* scratch, size_t scratch_bytes_given, void* stream)
{
    if (!blk) return set_error(RAG_ERR_INVALID_ARG, "block is NULL");
    rag_status s = rag::validate_block_call(x, y, rows, blk->C, scratch, scratch_bytes_given,
                                            scratch_bytes(rows, blk->C, blk->hidden));
    if (s != RAG_OK) return s;
    if (!cu_seqlens) return set_error(RAG_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (B < 1 || B > RAG_MAX_B) return set_error(RAG_ERR_INVALID_ARG, "B=%d out of range", B);
    if (max_seqlen < 1 || max_seqlen > 65535 * 64)
        return set_error(RAG_ERR_INVALID_ARG, "max_seqlen=%d out of range", max_seqlen);
    if (rows == 0) return RAG_OK;
    return forward(blk, x, y, rows, cu_seqlens, nullptr, B, 0, max_seqlen, scratch, rag::kLayoutRagged,
                   static_cast<hipStream_t>(stream));
}

extern "C" RAG_API rag_status rag_block_forward_padded(rag_block* blk, const void* x, void* y,
                                                       const uint8_t* keep, int32_t B, int32_t N,
                                                       void* scratch, size_t scratch_bytes_given,
                                                       void* stream)
{
    if (!blk) return set_error(RAG_ERR_INVALID_ARG, "block is NULL");
    if (!keep) return set_error(RAG_ERR_INVALID_ARG, "keep is NULL");
    if (B < 1 || N < 1 || B > RAG_MAX_B || N > RAG_MAX_N || (int64_t)B * N > INT32_MAX)
        return set_error(RAG_ERR_INVALID_ARG, "B=%d N=%d out of range", B, N);
    const int32_t rows = B * N;
    rag_status s = rag::validate_block_call(x, y, rows, blk->C, scratch, scratch_bytes_given,
                                            scratch_bytes(rows, blk->C, blk->hidden));
    if (s != RAG_OK) return s;
    return forward(blk, x, y, rows, nullptr, keep, B, N, N, scratch, rag::kLayoutPadded,
                   static_cast<hipStream_t>(stream));
}

extern "C" RAG_API void rag_block_destroy(rag_block* blk)
{
    if (!blk) return;
    for (auto& kv : blk->plans) destroy_plan(kv.second);
    if (blk->lt) hipblasLtDestroy(blk->lt);
    delete blk;
}
