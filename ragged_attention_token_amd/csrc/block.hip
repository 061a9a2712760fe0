// block.hip -- one ViT encoder block on packed token rows, and the same block
// on the padded [B, N] rows, for timing the pipeline end to end.
//
// "Dispatch-Aware Ragged Attention for Pruned Vision Transformers" (abstract)
// measures end-to-end throughput of pruned DeiT models whose blocks run on the
// packed tokens; the pages fix the attention step (the ragged kernel) and the
// packing, not the rest of the block.  The block here is the standard
// pre-norm encoder block of DeiT (ViT) with the caller's (e.g. random) weights:
//     h  = LayerNorm1(x)
//     qkv = h Wqkv^T + bqkv                (columns q | k | v, head-major)
//     a  = attention(qkv)                  (ragged, or padded with masked keys)
//     x1 = x + a Wproj^T + bproj
//     h2 = LayerNorm2(x1)
//     m  = GELU(h2 W1^T + b1)              (the exact GELU, x * Phi(x))
//     y  = x1 + m W2^T + b2
// with weights in the [out, in] layout of a linear layer.  Every step is a
// kernel of this library: the LayerNorm below, the GEMM of gemm.hip (bias,
// GELU and residual fused into its epilogue) and the attention of attn.hip.
// Every intermediate row is stored as bf16.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <new>

#include "rag_device.h"
#include "rag_internal.h"

using rag::set_error;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
using rag::dev::u32x4;

constexpr int kLnRowsPerWave = 2;

// Sum over the wave of one value per lane, as a butterfly over lane distances
// 32, 16, 8, 4, 2, 1: each step adds the value of the lane whose index differs
// in that bit (own + partner; the adds are commutative, so both lanes of a
// pair hold the same bits).  Distances 32 and 16 take the gfx950 permlane
// swaps; 8 is a rotation by 8 within each 16-lane row; 4 is a rotation by 4,
// which reads lane i^4's value because lanes i and i^8 already agree; 2 and 1
// are quad permutations.  No LDS round trips.
__device__ __forceinline__ float wave_sum(float x)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad 1,0,3,2
    return x;
}

// LayerNorm over rows of C bf16 values (C a multiple of 8, at most 2048):
// y = (x - mean) / sqrt(var + eps) * gamma + beta, mean and (biased) variance
// in fp32 over the row (two passes: the mean, then the squared deviations),
// y rounded to bf16.  Each wave normalises kLnRowsPerWave rows, 4 waves per
// workgroup; a lane holds NCH 16-byte chunks of each row (NCH = ceil(C / 512)).
// The wave index is made uniform so that the row addresses are scalar: every
// row's loads and the lane's gamma and beta are in flight together before the
// first reduction.  Chunks past the row read zeros, and their stores fall
// outside the row's buffer resource, which drops them.
template <int NCH>
__global__ __launch_bounds__(256) void layernorm_kernel(const __bf16* x, __bf16* y, int rows, int C,
                                                        const float* gamma, const float* beta,
                                                        float eps)
{
    constexpr int R = kLnRowsPerWave;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int row0 = (blockIdx.x * 4 + wave) * R;
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
            const bf16x8 w = __builtin_bit_cast(bf16x8, rag::dev::ld16(rx, 16u * (uint32_t)(lane + 64 * j)));
#pragma unroll
            for (int e = 0; e < 8; ++e) v[r][j][e] = static_cast<float>(w[e]);
        }
    }
    const auto rg = rag::dev::make_rsrc(gamma, (uint32_t)C * 4u);
    const auto rb = rag::dev::make_rsrc(beta, (uint32_t)C * 4u);
    f32x4 ga[NCH], gb[NCH], ba[NCH], bb[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const uint32_t off = 32u * (uint32_t)(lane + 64 * j);
        ga[j] = __builtin_bit_cast(f32x4, rag::dev::ld16(rg, off));
        gb[j] = __builtin_bit_cast(f32x4, rag::dev::ld16(rg, off + 16u));
        ba[j] = __builtin_bit_cast(f32x4, rag::dev::ld16(rb, off));
        bb[j] = __builtin_bit_cast(f32x4, rag::dev::ld16(rb, off + 16u));
    }
    float mean[R], rstd[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) sum += v[r][j][e];
        mean[r] = wave_sum(sum) / (float)C;
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
        rstd[r] = 1.f / sqrtf(wave_sum(sq) / (float)C + eps);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (row0 + r >= rows) continue;
        const auto ry = rag::dev::make_rsrc(y + (int64_t)(row0 + r) * C, (uint32_t)C * 2u);
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float gm = e < 4 ? ga[j][e] : gb[j][e - 4], bt = e < 4 ? ba[j][e] : bb[j][e - 4];
                o[e] = static_cast<__bf16>((v[r][j][e] - mean[r]) * rstd[r] * gm + bt);
            }
            rag::dev::st16(__builtin_bit_cast(u32x4, o), ry, 16u * (uint32_t)(lane + 64 * j));
        }
    }
}

}  // namespace

struct rag_block {
    rag_block_desc d;
    int32_t C = 0, hidden = 0;
};

namespace {

rag_status run_gemm(const void* X, const void* W, const void* bias, const void* R, void* D, int M, int N,
                    int K, int epi, hipStream_t st)
{
    const int e = rag::launch_gemm(X, W, static_cast<const float*>(bias), R, D, M, N, K, epi, st);
    return e == (int)hipSuccess ? RAG_OK : set_error(RAG_ERR_HIP, "GEMM launch: %s", hipGetErrorString((hipError_t)e));
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
                   int32_t B, int32_t N, int32_t max_seqlen, void* work, int layout, hipStream_t st)
{
    const int C = blk->C;
    char* base = static_cast<char*>(work);
    char* h = base;
    char* qkv = h + (size_t)rows * C * 2;
    char* a = qkv + (size_t)rows * 3 * C * 2;
    char* x1 = a + (size_t)rows * C * 2;
    char* m = x1 + (size_t)rows * C * 2;
    const rag_block_desc& d = blk->d;
    rag_status s;
    const int Hd = blk->hidden;
    if ((s = run_layernorm(x, h, rows, C, d.ln1_gamma, d.ln1_beta, d.eps, st)) != RAG_OK) return s;
    if ((s = run_gemm(h, d.w_qkv, d.b_qkv, nullptr, qkv, rows, 3 * C, C, rag::kGemmBias, st)) != RAG_OK) return s;
    const int e = rag::launch_attn(qkv, qkv + C * 2, qkv + 2 * C * 2, 3 * C, 3 * C, 3 * C, RAG_DTYPE_BF16, cu, keep,
                                   B, N, max_seqlen, rows, d.H, d.scale, a, C, RAG_DTYPE_BF16, layout, 0u, st);
    if (e != (int)hipSuccess) return set_error(RAG_ERR_HIP, "block attention: %s", hipGetErrorString((hipError_t)e));
    if ((s = run_gemm(a, d.w_proj, d.b_proj, x, x1, rows, C, C, rag::kGemmResidual, st)) != RAG_OK) return s;
    if ((s = run_layernorm(x1, h, rows, C, d.ln2_gamma, d.ln2_beta, d.eps, st)) != RAG_OK) return s;
    if ((s = run_gemm(h, d.w_fc1, d.b_fc1, nullptr, m, rows, Hd, C, rag::kGemmGelu, st)) != RAG_OK) return s;
    return run_gemm(m, d.w_fc2, d.b_fc2, x1, y, rows, C, Hd, rag::kGemmResidual, st);
}

}  // namespace

extern "C" RAG_API size_t rag_block_scratch_bytes(int32_t rows, int32_t H, int32_t mlp_ratio)
{
    if (rows < 0 || H < 1 || mlp_ratio < 1) return 0;
    const int64_t C = (int64_t)H * RAG_HEAD_DIM;
    return scratch_bytes(rows, C, C * mlp_ratio);
}

namespace {

// ---- the allocation-free forward (rag_block_forward_static) --------------
//
// Its intermediates live in this file-scope device array instead of a
// caller-provided buffer: each GPU the library runs on holds one copy for the
// life of the process, and every static call on that GPU shares it.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is handed to the kernels.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first use on that device and kept).  Returns RAG_OK and sets *ptr, or an
// error status.
rag_status static_scratch(void** ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(RAG_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(RAG_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(RAG_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_dev[dev].store(p, std::memory_order_release);  // the same value from any racing thread
    }
    *ptr = p;
    return RAG_OK;
}

}  // namespace

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
    // set-up of the allocation-free forward on the current device (a call on
    // another device looks its own copy up on first use)
    void* unused = nullptr;
    s = static_scratch(&unused);
    if (s != RAG_OK) {
        delete blk;
        return s;
    }
    *out = blk;
    return RAG_OK;
}

extern "C" RAG_API rag_status rag_block_forward(rag_block* blk, const void* x, void* y, int32_t rows,
                                                const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                                void* work, size_t work_bytes, void* stream)
{
    if (!blk) return set_error(RAG_ERR_INVALID_ARG, "block is NULL");
    rag_status s = rag::validate_block_call(x, y, rows, blk->C, work, work_bytes,
                                            scratch_bytes(rows, blk->C, blk->hidden));
    if (s != RAG_OK) return s;
    if (!cu_seqlens) return set_error(RAG_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (B < 1 || B > RAG_MAX_B) return set_error(RAG_ERR_INVALID_ARG, "B=%d out of range", B);
    if (max_seqlen < 1 || max_seqlen > 65535 * 64)
        return set_error(RAG_ERR_INVALID_ARG, "max_seqlen=%d out of range", max_seqlen);
    if (rows == 0) return RAG_OK;
    return forward(blk, x, y, rows, cu_seqlens, nullptr, B, 0, max_seqlen, work, rag::kLayoutRagged,
                   static_cast<hipStream_t>(stream));
}

extern "C" RAG_API rag_status rag_block_forward_static(rag_block* blk, const void* x, void* y, int32_t rows,
                                                       const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                                       void* stream)
{
    if (!blk) return set_error(RAG_ERR_INVALID_ARG, "block is NULL");
    if (rows < 0) return set_error(RAG_ERR_INVALID_ARG, "rows=%d must be >= 0", rows);
    const size_t need = scratch_bytes(rows, blk->C, blk->hidden);
    if (need > kStaticScratchBytes)
        return set_error(RAG_ERR_UNSUPPORTED,
                         "rows=%d needs %zu bytes of intermediates; the static scratch holds %zu "
                         "(at most %zu rows at C=%d)",
                         rows, need, kStaticScratchBytes,
                         kStaticScratchBytes / scratch_bytes(1, blk->C, blk->hidden), blk->C);
    void* ptr = nullptr;
    rag_status s = static_scratch(&ptr);
    if (s != RAG_OK) return s;
    return rag_block_forward(blk, x, y, rows, cu_seqlens, B, max_seqlen, ptr, kStaticScratchBytes, stream);
}

extern "C" RAG_API rag_status rag_block_forward_padded(rag_block* blk, const void* x, void* y,
                                                       const uint8_t* keep, int32_t B, int32_t N,
                                                       void* work, size_t work_bytes, void* stream)
{
    if (!blk) return set_error(RAG_ERR_INVALID_ARG, "block is NULL");
    if (!keep) return set_error(RAG_ERR_INVALID_ARG, "keep is NULL");
    if (B < 1 || N < 1 || B > RAG_MAX_B || N > RAG_MAX_N || (int64_t)B * N > INT32_MAX)
        return set_error(RAG_ERR_INVALID_ARG, "B=%d N=%d out of range", B, N);
    const int32_t rows = B * N;
    rag_status s = rag::validate_block_call(x, y, rows, blk->C, work, work_bytes,
                                            scratch_bytes(rows, blk->C, blk->hidden));
    if (s != RAG_OK) return s;
    return forward(blk, x, y, rows, nullptr, keep, B, N, N, work, rag::kLayoutPadded,
                   static_cast<hipStream_t>(stream));
}

extern "C" RAG_API void rag_block_destroy(rag_block* blk)
{
    delete blk;
}
