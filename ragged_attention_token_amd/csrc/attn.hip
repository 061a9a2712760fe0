// attn.hip -- bidirectional multi-head attention on packed ragged sequences,
// and the padded comparator, for gfx950 (CDNA4).
//
// What is computed ("Dispatch-Aware Ragged Attention for Pruned Vision
// Transformers", abstract; agents-report.net "Triton Ragged Attention 與
// pack-attend-unpack", section 方法概覽, ragged attention kernel): for each image
// b (packed rows cu[b] .. cu[b+1]-1) and head h, O = softmax(scale Q K^T) V over
// that image's rows only, with no causal mask.  The padded form (same page,
// section 問題) runs the same attention over all N rows of every image with the
// dropped keys masked out.
//
// Kernel design (ours, for gfx950; the pages' Triton kernel is not followed):
//   * one workgroup = one (q-tile of 64 rows, head, image); 4 wave64s, each
//     owning 16 query rows.  A 1-D grid is remapped so that consecutive tiles
//     of one (image, head) land on the same XCD (shared K/V in that L2).
//     Tiles past an image's length exit at once (grid sized from max_seqlen).
//   * K and V are staged through LDS 64 keys at a time: K row-major, V
//     transposed (d-major), both zero-filled past the sequence end so that no
//     uninitialised value can reach an MFMA.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulate), so that each
//     lane holds the scores of ONE query row (lane & 15) for 4 keys per 16-key
//     block; the row max / row sum need only two cross-lane exchanges.
//   * online softmax in fp32 with exp2 (scale * log2 e folded into the scores);
//     the probabilities are split into bf16 high + low parts and
//     O^T += V^T P^T runs both through the same MFMA, so P is carried to about
//     16 mantissa bits.  fp32 inputs are split the same way (hi/lo for Q, K, V).
//   * the probabilities never leave registers: the MFMA result layout of S^T is
//     used directly as the B operand of the P.V product (keys are a summation
//     index, so the k-order only has to agree between the two operands).
#include <hip/hip_runtime.h>

#include "rag_internal.h"

namespace rag {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;        // head dimension
constexpr int kBM = 64;       // query rows per workgroup
constexpr int kBN = 64;       // keys per LDS tile
constexpr int kThreads = 256; // 4 waves x 16 query rows
constexpr int kKS = 72;       // LDS row stride of the K tile (bf16): 144 B
constexpr int kVS = 68;       // LDS row stride of the V^T tile (bf16): 136 B

struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t qs, ks, vs, os;  // row strides, elements
    const int32_t* cu;       // ragged
    const uint8_t* keep;     // padded
    int32_t B, N, H, total_rows, n_qtiles, total_wgs;
    float scale_log2;        // scale * log2(e)
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo)
{
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ uint32_t pack2(__bf16 a, __bf16 b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight consecutive input elements as bf16 (hi) and, for fp32 input, the bf16
// remainder (lo).  `ok` false gives zeros.
template <bool IN_F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, bool ok, bf16x8& hi,
                                      bf16x8& lo)
{
    if constexpr (!IN_F32) {
        if (ok) hi = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(base) + off);
        else hi = bf16x8{};
        lo = bf16x8{};
    } else {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (ok) {
            const float* f = static_cast<const float*>(base) + off;
            a = *reinterpret_cast<const float4*>(f);
            b = *reinterpret_cast<const float4*>(f + 4);
        }
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            __bf16 h, l;
            split_bf16(x[e], h, l);
            hi[e] = h;
            lo[e] = l;
        }
    }
}

template <bool IN_F32, bool OUT_F32, bool PADDED>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p)
{
    constexpr int NP = IN_F32 ? 2 : 1;  // bf16 planes: hi (and lo)
    __shared__ __attribute__((aligned(16))) __bf16 sK[NP][kBN * kKS];
    __shared__ __attribute__((aligned(16))) __bf16 sVt[NP][kD * kVS];
    __shared__ uint8_t sKeep[kBN];

    // ---- which (q-tile, head, image): XCD-aware remap of the 1-D grid -------
    // Workgroup ids are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of work items so one (image, head)'s tiles share an L2.
    const int id = blockIdx.x;
    const int total = p.total_wgs;
    const int xcd = id & 7, slot = id >> 3;
    const int per = total >> 3, extra = total & 7;
    const int w = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + slot;
    const int qt = w % p.n_qtiles;
    const int bh = w / p.n_qtiles;
    const int h = bh % p.H;
    const int b = bh / p.H;

    int64_t row0;
    int L;
    if constexpr (PADDED) {
        row0 = (int64_t)b * p.N;
        L = p.N;
    } else {
        const int s = min(max(p.cu[b], 0), p.total_rows);
        const int e = min(max(p.cu[b + 1], s), p.total_rows);
        row0 = s;
        L = e - s;
    }
    const int q0 = qt * kBM;
    if (q0 >= L) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int qrow = q0 + wave * 16 + r16;  // query row inside the image
    const bool wave_active = q0 + wave * 16 < L;
    const int64_t hoff = (int64_t)h * kD;

    // Q^T as the B operand: lane holds query row r16, d = 8g..8g+7 and 32+8g..
    bf16x8 qh0, qh1, ql0, ql1;
    {
        const int64_t off = (row0 + qrow) * p.qs + hoff + 8 * g;
        const bool ok = qrow < L;
        load8<IN_F32>(p.q, off, ok, qh0, ql0);
        load8<IN_F32>(p.q, off + 32, ok, qh1, ql1);
    }

    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int kt = 0; kt < L; kt += kBN) {
        const int nk = min(kBN, L - kt);
        __syncthreads();  // the previous tile is no longer read
        // ---- stage K (row-major) -------------------------------------------
#pragma unroll
        for (int j = 0; j < (kBN * kD / 8) / kThreads; ++j) {
            const int ci = tid + j * kThreads;
            const int key = ci >> 3, dg = ci & 7;
            bf16x8 hi, lo;
            load8<IN_F32>(p.k, (row0 + kt + key) * p.ks + hoff + 8 * dg, key < nk, hi, lo);
            *reinterpret_cast<bf16x8*>(&sK[0][key * kKS + 8 * dg]) = hi;
            if constexpr (IN_F32) *reinterpret_cast<bf16x8*>(&sK[NP - 1][key * kKS + 8 * dg]) = lo;
        }
        // ---- stage V transposed: thread owns keys 2kp, 2kp+1 and d 8dg..8dg+7
        {
            const int kp = tid >> 3, dg = tid & 7;
            const int k0 = 2 * kp, k1 = 2 * kp + 1;
            bf16x8 h0, l0, h1, l1;
            load8<IN_F32>(p.v, (row0 + kt + k0) * p.vs + hoff + 8 * dg, k0 < nk, h0, l0);
            load8<IN_F32>(p.v, (row0 + kt + k1) * p.vs + hoff + 8 * dg, k1 < nk, h1, l1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // keys k0, k1 side by side: one 32-bit LDS store per (d, key pair)
                const int off = (8 * dg + i) * kVS + k0;
                *reinterpret_cast<uint32_t*>(&sVt[0][off]) = pack2(h0[i], h1[i]);
                if constexpr (IN_F32)
                    *reinterpret_cast<uint32_t*>(&sVt[NP - 1][off]) = pack2(l0[i], l1[i]);
            }
        }
        if constexpr (PADDED) {
            if (tid < kBN) sKeep[tid] = (tid < nk) ? p.keep[row0 + kt + tid] : 0;
        }
        __syncthreads();
        if (!wave_active) continue;

        // ---- S^T = K Q^T: block kb holds keys kt+16kb+4g+i (i<4), query r16 --
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb * 16 < nk) {
                const __bf16* kr = &sK[0][(kb * 16 + r16) * kKS + 8 * g];
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kr);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kr + 32);
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
                t = mfma(a0, qh0, t);
                t = mfma(a1, qh1, t);
                if constexpr (IN_F32) {
                    const __bf16* kl = &sK[NP - 1][(kb * 16 + r16) * kKS + 8 * g];
                    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(kl);
                    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(kl + 32);
                    t = mfma(b0, qh0, t);
                    t = mfma(b1, qh1, t);
                    t = mfma(a0, ql0, t);
                    t = mfma(a1, ql1, t);
                }
                s[kb] = t;
            } else {
                s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }

        // ---- online softmax (fp32, base 2) ----------------------------------
        float mloc = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kb * 16 + 4 * g + i;
                bool ok = key < nk;
                if constexpr (PADDED) ok = ok && sKeep[key] != 0;
                const float x = ok ? s[kb][i] * p.scale_log2 : -INFINITY;
                s[kb][i] = x;
                mloc = fmaxf(mloc, x);
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = fast_exp2(s[kb][i] - m_use);
                s[kb][i] = e;
                psum += e;
            }
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;

        // ---- O^T += V^T P^T, 32 keys per MFMA ---------------------------------
        // k-slot e of lane group g: e<4 -> key 32c+4g+e, e>=4 -> key 32c+16+4g+e-4;
        // these are exactly the keys of s[2c][e] and s[2c+1][e-4].
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (c * 32 < nk) {
                bf16x8 ph, pl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    __bf16 hh, ll;
                    split_bf16(s[2 * c][e], hh, ll);
                    ph[e] = hh;
                    pl[e] = ll;
                    split_bf16(s[2 * c + 1][e], hh, ll);
                    ph[e + 4] = hh;
                    pl[e + 4] = ll;
                }
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int vo = (db * 16 + r16) * kVS + 32 * c + 4 * g;
                    const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(&sVt[0][vo]);
                    const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(&sVt[0][vo + 16]);
                    const bf16x8 av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[db] = mfma(av, ph, acc[db]);
                    acc[db] = mfma(av, pl, acc[db]);
                    if constexpr (IN_F32) {
                        const bf16x4 w0 = *reinterpret_cast<const bf16x4*>(&sVt[NP - 1][vo]);
                        const bf16x4 w1 = *reinterpret_cast<const bf16x4*>(&sVt[NP - 1][vo + 16]);
                        const bf16x8 al = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
                        acc[db] = mfma(al, ph, acc[db]);
                    }
                }
            }
        }
    }

    if (!wave_active) return;
    // ---- epilogue: O = acc / l; lane holds O[r16][16db + 4g + i] --------------
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qrow >= L) return;
    const int64_t ooff = (row0 + qrow) * p.os + hoff + 4 * g;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const f32x4 r = acc[db] * inv;
        if constexpr (OUT_F32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.o) + ooff + 16 * db) =
                make_float4(r[0], r[1], r[2], r[3]);
        } else {
            bf16x4 o4;
            o4[0] = static_cast<__bf16>(r[0]);
            o4[1] = static_cast<__bf16>(r[1]);
            o4[2] = static_cast<__bf16>(r[2]);
            o4[3] = static_cast<__bf16>(r[3]);
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.o) + ooff + 16 * db) = o4;
        }
    }
}

template <bool IN_F32, bool OUT_F32>
void launch_variant(const AttnParams& p, bool padded, hipStream_t st)
{
    const dim3 grid(p.total_wgs), block(kThreads);
    if (padded)
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, true>), grid, block, 0, st, p);
    else
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, false>), grid, block, 0, st, p);
}

}  // namespace

int launch_attn(const void* q, const void* k, const void* v, int64_t q_row_stride,
                int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                const int32_t* cu_seqlens, const uint8_t* keep, int32_t B, int32_t N,
                int32_t max_seqlen, int32_t total_rows, int32_t H, float scale, void* o,
                int64_t o_row_stride, int32_t out_dtype, bool padded, void* stream)
{
    AttnParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.qs = q_row_stride;
    p.ks = k_row_stride;
    p.vs = v_row_stride;
    p.os = o_row_stride;
    p.cu = cu_seqlens;
    p.keep = keep;
    p.B = B;
    p.N = N;
    p.H = H;
    p.total_rows = total_rows;
    p.n_qtiles = ((padded ? N : max_seqlen) + kBM - 1) / kBM;
    p.total_wgs = p.n_qtiles * H * B;
    p.scale_log2 = scale * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool in_f32 = in_dtype == RAG_DTYPE_F32, out_f32 = out_dtype == RAG_DTYPE_F32;
    if (in_f32 && out_f32) launch_variant<true, true>(p, padded, st);
    else if (in_f32) launch_variant<true, false>(p, padded, st);
    else if (out_f32) launch_variant<false, true>(p, padded, st);
    else launch_variant<false, false>(p, padded, st);
    return (int)hipGetLastError();
}

}  // namespace rag
