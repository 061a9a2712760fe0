// gemm.hip -- the matrix products of the ViT encoder block on gfx950.
//
// "Dispatch-Aware Ragged Attention for Pruned Vision Transformers" (abstract)
// measures pruned DeiT models end to end; around the attention, each encoder
// block runs four dense products on the kept token rows (qkv projection,
// output projection, the two MLP layers).  They are plain GEMMs with an
// element-wise epilogue, written here for CDNA4:
//
//     D[m, n] = epi( sum_k X[m, k] W[n, k] + bias[n] )  (+ R[m, n])
//
// X [M, K] bf16 row-major (token rows), W [N, K] bf16 row-major (the
// [out, in] layout of a linear layer's weight), bias fp32 [N], R / D [M, N]
// bf16 row-major; fp32 accumulation; epi = identity or the exact GELU
// x * Phi(x) (DeiT's MLP activation), with Phi from erfc by the Chebyshev
// formula of Numerical Recipes (Press et al., 2nd ed., section 6.2, "erfcc":
// relative error below 1.2e-7 for every argument, so both tails of x Phi(x)
// keep full relative accuracy before the one rounding to bf16).
//
// Design (ours):
//   * both operands are K-contiguous, so both MFMA operands come from LDS rows
//     with one 16-byte read per lane; the product is computed transposed,
//     D^T = W X^T, so that a lane's four accumulator values are four
//     consecutive output columns of one row;
//   * the epilogue stages each wave's 64 x 64 fp32 block in LDS and writes
//     rows back 16 bytes per lane, 128 contiguous bytes per 8 lanes (the
//     accumulator layout would store 16 rows x 32 bytes per instruction);
//   * workgroup tile 128 (m) x 128 (n), four wave64s in a 2 x 2 arrangement,
//     each owning 64 x 64 outputs (4 x 4 blocks of v_mfma_f32_16x16x32_bf16,
//     fp32 accumulators in VGPRs);
//   * k advances 64 at a time through two LDS buffers: while k-tile kt is
//     multiplied from one, k-tile kt + 1 is requested into the other by buffer
//     loads that write LDS (eight 16-byte loads per lane, no registers and no
//     LDS store instructions); one wait and one barrier per k-tile.  LDS rows are 128 bytes
//     (64 bf16) with the eight 16-byte chunks of row r permuted by XOR with
//     swz(r), so that 16 lanes reading chunk c of 16 consecutive rows hit
//     distinct banks;
//   * tiles are numbered so that each of the eight XCDs (workgroup w runs on
//     XCD w mod 8) owns a contiguous range of row tiles: the n-tiles that
//     share an X tile are fetched into one L2;
//   * rows past M read as zero and their stores are dropped (buffer resources
//     ending at row M); columns past N are skipped per lane (N is a multiple of
//     64, so a lane's four columns are all in or all out).
#include <hip/hip_runtime.h>

#include "rag_device.h"
#include "rag_internal.h"

namespace rag {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
using dev::i32x4;
using dev::ld16;
using dev::make_rsrc;
using dev::u32x4;

constexpr int kBM = 128;  // X rows per workgroup
constexpr int kBN = 128;  // W rows (output columns) per workgroup
constexpr int kBK = 64;   // k per LDS tile: one 128-byte LDS row per operand row
constexpr int kThreads = 256;
constexpr int kTileBytes = (kBM + kBN) * kBK * 2;  // one k-tile of both operands: 32 KiB
constexpr int kLoads = kTileBytes / 16 / kThreads;  // 16-byte loads per lane per k-tile: 8

struct GemmParams {
    const __bf16* x;
    const __bf16* w;
    const float* bias;
    const __bf16* r;
    __bf16* d;
    int32_t M, N, K;
    int32_t tiles_n;  // ceil(N / kBN)
    int32_t tiles;    // ceil(M / kBM) * tiles_n
    int32_t per_xcd;  // ceil(tiles / 8): tiles of each XCD
};

// Slot of chunk c of LDS row r is c ^ swz(r); swz depends on r mod 16 only.
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// erfc(z) for z >= 0, relative error < 1.2e-7 (the Numerical Recipes
// Chebyshev fit, in Horner form): t = 1 / (1 + z/2),
// erfc(z) = t exp(-z^2 + c0 + t (c1 + t (c2 + ... + t c9))).
__device__ __forceinline__ float erfc_nonneg(float z)
{
    const float t = __builtin_amdgcn_rcpf(1.f + 0.5f * z);
    float r = 0.17087277f;
    r = __builtin_fmaf(r, t, -0.82215223f);
    r = __builtin_fmaf(r, t, 1.48851587f);
    r = __builtin_fmaf(r, t, -1.13520398f);
    r = __builtin_fmaf(r, t, 0.27886807f);
    r = __builtin_fmaf(r, t, -0.18628806f);
    r = __builtin_fmaf(r, t, 0.09678418f);
    r = __builtin_fmaf(r, t, 0.37409196f);
    r = __builtin_fmaf(r, t, 1.00002368f);
    r = __builtin_fmaf(r, t, -1.26551223f);
    const float e = __builtin_fmaf(-z, z, r);  // the exponent, natural base
    return t * __builtin_amdgcn_exp2f(e * 1.44269504088896341f);
}

// The exact GELU, x * Phi(x), Phi(x) = erfc(-x / sqrt(2)) / 2: for x < 0
// Phi = erfc(|x|/sqrt(2)) / 2, else 1 - erfc(|x|/sqrt(2)) / 2.
__device__ __forceinline__ float gelu_exact(float x)
{
    const float h = 0.5f * erfc_nonneg(fabsf(x) * 0.70710678118654752f);
    return x * (x < 0.f ? h : 1.f - h);
}

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmParams p)
{
    // two k-tiles; in each, W rows [0, 16K) then X rows [16K, 32K)
    __shared__ __attribute__((aligned(16))) char lds[2 * kTileBytes];

    const int wg = blockIdx.x;
    const int t = (wg & 7) * p.per_xcd + (wg >> 3);
    if (t >= p.tiles) return;  // uniform over the workgroup
    const int tm = t / p.tiles_n;
    const int m0 = tm * kBM, n0 = (t - tm * p.tiles_n) * kBN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases and branches
    const int r16 = lane & 15, g = lane >> 4;
    const uint32_t rowb = (uint32_t)p.K * 2u;  // bytes per operand row

    // operand rows of this tile; rows past M (or N) read as zero
    const i32x4 rx = dev::rsrc_words(p.x + (int64_t)m0 * p.K, (uint32_t)min(kBM, p.M - m0) * rowb);
    const i32x4 rw = dev::rsrc_words(p.w + (int64_t)n0 * p.K, (uint32_t)min(kBN, p.N - n0) * rowb);

    // Staging: load j (0..7) of thread tid moves LDS bytes [16 (tid + 256 j), +16)
    // of the k-tile: LDS row tid / 8 + 32 j (W rows 0..127 for j < 4, then X
    // rows), slot tid % 8, which holds global chunk slot ^ swz(row) of that row
    // (swz depends on the row mod 16, the same for every j).  The loads write
    // LDS themselves (no registers, no LDS store instructions): wave w's load j
    // fills the 1 KiB at 16 (64 w + 256 j), 16 bytes per lane.
    uint32_t goff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 3) + 32 * j;
        goff[j] = (uint32_t)row * rowb + 16u * (uint32_t)((tid & 7) ^ swz(row));
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;  // (the low half of a flat LDS pointer)
    auto request = [&](int kt, int buf) {
        const uint32_t kb = (uint32_t)kt * (kBK * 2);
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const uint32_t base = lds0 + (uint32_t)(buf * kTileBytes) + 16u * (uint32_t)(64 * wave + kThreads * j);
            dev::ld_lds16_untracked(j < 4 ? rw : rx, base, goff[j & 3] + kb);
        }
    };

    // wave (wn, wm) owns W rows 64 wn .. and X rows 64 wm .. of the tile
    const int wn = wave & 1, wm = wave >> 1;
    const int sz = swz(r16);
    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = p.K / kBK;
    request(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        // k-tile kt + 1 goes to the other buffer, last read before the previous
        // barrier, while tile kt is multiplied
        if (kt + 1 < nk) request(kt + 1, (kt + 1) & 1);
        const char* st = lds + (kt & 1) * kTileBytes;
        const char* sW = st + 128 * (64 * wn + r16);
        const char* sX = st + kBN * 128 + 128 * (64 * wm + r16);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {  // k 0..31, 32..63 of the tile
            const int co = 16 * ((g + 4 * kk) ^ sz);
            bf16x8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = *reinterpret_cast<const bf16x8*>(sW + 2048 * i + co);
                b[i] = *reinterpret_cast<const bf16x8*>(sX + 2048 * i + co);
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma(a[nb], b[mb], acc[nb][mb]);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile kt + 1 has landed
        __syncthreads();  // ... and every wave is done with tile kt
    }

    // ---- epilogue: acc[nb][mb][i] = D[m0 + 64 wm + 16 mb + r16][n0 + 64 wn + 16 nb + 4 g + i].
    // Each wave stages its 64 x 64 fp32 block in LDS (free after the loop's
    // last barrier; 16 KiB per wave) and writes it back row-contiguously: a
    // lane takes 8 consecutive columns of one row (16 output bytes), 8 lanes a
    // whole 128-byte row segment, where the accumulator layout would give 16
    // rows x 32 bytes per store.  Rows are 256 bytes (16 chunks of 16 bytes);
    // chunk c of row r sits at chunk c ^ (r & 15), so that both the accumulator
    // writes (16 rows, one chunk each) and the row reads (two rows of 8 chunk
    // pairs per 16 lanes) hit distinct banks.  The arithmetic is the same
    // as element by element: (acc + bias), GELU, + residual, one rounding.
    const int n0w = n0 + 64 * wn;  // the wave's first column
    if (n0w >= p.N) return;        // (N is a multiple of 64: a wave's columns are all in or all out)
    char* so = lds + wave * (64 * 256);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int row = 16 * mb + r16, chunk = 4 * nb + g;
            *reinterpret_cast<f32x4*>(so + row * 256 + 16 * (chunk ^ r16)) = acc[nb][mb];
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const int mrows = min(kBM, p.M - m0);
    const auto rd = make_rsrc(p.d + (int64_t)m0 * p.N, (uint32_t)mrows * (uint32_t)p.N * 2u);
    const auto rr = make_rsrc(p.r ? p.r + (int64_t)m0 * p.N : p.d, p.r ? (uint32_t)mrows * (uint32_t)p.N * 2u : 0u);
    const int cl = lane & 7;  // the lane's 8 columns: 8 cl .. 8 cl + 7 of the wave's 64
    const f32x4 bias0 = *reinterpret_cast<const f32x4*>(p.bias + n0w + 8 * cl);
    const f32x4 bias1 = *reinterpret_cast<const f32x4*>(p.bias + n0w + 8 * cl + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 8 * j + (lane >> 3);  // row within the wave's block
        const char* src = so + row * 256;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(src + 16 * ((2 * cl) ^ (row & 15)));
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 16 * ((2 * cl + 1) ^ (row & 15)));
        const int m = 64 * wm + row;  // row within the tile
        const uint32_t off = ((uint32_t)m * (uint32_t)p.N + (uint32_t)(n0w + 8 * cl)) * 2u;
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a0[i] + bias0[i];
            v[4 + i] = a1[i] + bias1[i];
        }
        if constexpr (EPI == kGemmGelu) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = gelu_exact(v[i]);
        }
        if constexpr (EPI == kGemmResidual) {
            const bf16x8 r8 = __builtin_bit_cast(bf16x8, ld16(rr, off));
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += static_cast<float>(r8[i]);
        }
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = static_cast<__bf16>(v[i]);
        dev::st16(__builtin_bit_cast(u32x4, o), rd, off);
    }
}

}  // namespace

int launch_gemm(const void* x, const void* w, const float* bias, const void* r, void* d, int32_t M,
                int32_t N, int32_t K, int epi, void* stream)
{
    if (M <= 0) return (int)hipSuccess;
    GemmParams p;
    p.x = static_cast<const __bf16*>(x);
    p.w = static_cast<const __bf16*>(w);
    p.bias = bias;
    p.r = static_cast<const __bf16*>(r);
    p.d = static_cast<__bf16*>(d);
    p.M = M;
    p.N = N;
    p.K = K;
    p.tiles_n = (N + kBN - 1) / kBN;
    p.tiles = ((M + kBM - 1) / kBM) * p.tiles_n;
    p.per_xcd = (p.tiles + 7) / 8;
    const dim3 grid(8 * p.per_xcd), block(kThreads);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (epi == kGemmGelu) hipLaunchKernelGGL(gemm_kernel<kGemmGelu>, grid, block, 0, st, p);
    else if (epi == kGemmResidual) hipLaunchKernelGGL(gemm_kernel<kGemmResidual>, grid, block, 0, st, p);
    else hipLaunchKernelGGL(gemm_kernel<kGemmBias>, grid, block, 0, st, p);
    return (int)hipGetLastError();
}

}  // namespace rag
