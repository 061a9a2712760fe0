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
//   * one workgroup = one (head, image, q-tile of 64 rows); 4 wave64s, each
//     owning 16 query rows.  The q-tile is the slowest grid dimension, so the
//     first tile of every (image, head) is dispatched before the later tiles,
//     most of which exit at once for pruned sequences (the grid is sized from
//     the host-side max_seqlen, never from device data).
//   * all global traffic goes through buffer resources whose range ends at the
//     image's last row: loads past the sequence end return zeros and stores
//     past it are dropped by the hardware, so no per-lane predicate is needed
//     and no uninitialised value can reach an MFMA.
//   * K and V are staged through LDS 64 keys at a time: K row-major, V
//     transposed (d-major) so that each lane's MFMA operand is contiguous.  The
//     next tile's loads are issued into registers before the current tile is
//     computed, so a long sequence costs one memory round trip, not one per tile.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulate): each lane
//     holds the scores of ONE query row (lane & 15) for 4 keys per 16-key
//     block, so the row max / row sum take two v_permlane{16,32}_swap steps.
//   * online softmax in fp32 with exp2; masking only in a sequence's last,
//     partial tile; no rescale on the first tile.  The probabilities are split
//     into bf16 high + low parts and O^T += V^T P^T runs both through the same
//     MFMA, so P is carried to about 16 mantissa bits.  fp32 inputs are split
//     the same way (hi/lo for Q, K, V).
//   * the probabilities never leave registers: the MFMA result layout of S^T is
//     used directly as the B operand of the P.V product (keys are a summation
//     index, so the k-order only has to agree between the two operands).
//   * the output goes through LDS so that each row segment is written by
//     consecutive lanes with 16-byte stores.
#include <hip/hip_runtime.h>

#include "rag_device.h"
#include "rag_internal.h"

namespace rag {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
using dev::u32x4;

constexpr int kD = 64;         // head dimension
constexpr int kBM = 64;        // query rows per workgroup
constexpr int kBN = 64;        // keys per LDS tile
constexpr int kThreads = 256;  // 4 waves x 16 query rows
constexpr int kKS = 72;        // LDS row stride of the K tile (bf16): 144 B
constexpr int kVS = 68;        // LDS row stride of the V^T tile (bf16): 136 B

// Where the rows of one image live.
enum Layout : int {
    kRagged = 0,    // packed rows cu[b] .. cu[b+1]-1
    kPadded = 1,    // all N rows b*N .. b*N+N-1, dropped keys masked
    kGathered = 2,  // the kept rows of b*N .. b*N+N-1, found from the keep row
};

struct AttnParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t qs, ks, vs, os;  // row strides, elements
    const int32_t* cu;       // ragged
    const uint8_t* keep;     // padded and gathered
    int32_t B, N, H, total_rows, max_len, n_qtiles, zero_dropped;
    float scale_log2;        // scale * log2(e)
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-lane value over the four 16-lane rows of the wave (lanes l,
// l^16, l^32, l^48), which hold the same query row.
__device__ __forceinline__ float row_max(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_sum(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t bits(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats as packed bf16 high parts (round to nearest even, one
// v_cvt_pk_bf16_f32) and packed bf16 remainders x - hi (exact in fp32, then
// rounded the same way): together they carry about 16 significant bits.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo)
{
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
    const float h0 = __uint_as_float(hi << 16);
    const float h1 = __uint_as_float(hi & 0xFFFF0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0 - h0, x1 - h1}, bf16x2));
}

using dev::kDropOffset;
using dev::ld16;
using dev::make_rsrc;

// Eight consecutive input elements at byte offset `off` as bf16 (hi) and, for
// fp32 input, the bf16 remainder x - hi (lo).
template <bool IN_F32>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16x8& hi, bf16x8& lo)
{
    if constexpr (!IN_F32) {
        hi = __builtin_bit_cast(bf16x8, ld16(r, off));
    } else {
        const f32x4 a = __builtin_bit_cast(f32x4, ld16(r, off));
        const f32x4 b = __builtin_bit_cast(f32x4, ld16(r, off + 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = e < 4 ? a[e] : b[e - 4];
            const __bf16 h = static_cast<__bf16>(x);
            hi[e] = h;
            lo[e] = static_cast<__bf16>(x - static_cast<float>(h));
        }
    }
}

// Gathered layout with RAG_UNPACK_ZERO_DROPPED: head h of every dropped row of
// the image is set to zero (one workgroup per (image, head) does it).
template <bool OUT_F32>
__device__ void zero_dropped_head(const AttnParams& p, int64_t row0, int h)
{
    constexpr int OES = OUT_F32 ? 4 : 2;
    constexpr int CHUNKS = kD * OES / 16;
    const uint32_t osb = (uint32_t)(p.os * OES);
    const auto ro = make_rsrc(static_cast<char*>(p.o) + (row0 * p.os + (int64_t)h * kD) * OES,
                              (uint32_t)(p.N - 1) * osb + kD * OES);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < p.N * CHUNKS; i += kThreads) {
        const int n = i / CHUNKS, cix = i - n * CHUNKS;
        if (p.keep[row0 + n] == 0) dev::st16(zero, ro, (uint32_t)n * osb + 16 * cix);
    }
}

template <bool IN_F32, bool OUT_F32, int LAYOUT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p)
{
    constexpr bool PADDED = LAYOUT == kPadded;
    constexpr bool GATHERED = LAYOUT == kGathered;
    constexpr int NP = IN_F32 ? 2 : 1;  // bf16 planes: hi (and lo)
    constexpr int ES = IN_F32 ? 4 : 2;  // input element bytes
    constexpr int OES = OUT_F32 ? 4 : 2;
    constexpr int K_PLANE = kBN * kKS;   // bf16 elements
    constexpr int V_PLANE = kD * kVS;
    constexpr int OUT_ROW = kD * OES + 16;                   // bytes, padded
    constexpr int SMEM = 2 * (NP * K_PLANE + NP * V_PLANE);  // bytes
    static_assert(4 * 16 * OUT_ROW <= SMEM, "output staging must fit the tile buffers");
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    __bf16* sK = reinterpret_cast<__bf16*>(smem);
    __bf16* sVt = sK + NP * K_PLANE;
    __shared__ uint8_t sKeep[kBN];
    extern __shared__ int s_pos[];  // gathered: the image's kept positions by rank (N ints)
    __shared__ int s_wsum[4];

    // ---- which (head, image, q-tile): a 3-D grid with the q-tile slowest, so
    // that the first q-tile of every (image, head) -- the only one most pruned
    // sequences have -- is dispatched before any tile that will exit at once.
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int qt = blockIdx.z;

    int64_t row0;
    int L;
    if constexpr (PADDED) {
        row0 = (int64_t)b * p.N;
        L = p.N;
    } else if constexpr (GATHERED) {
        row0 = (int64_t)b * p.N;
        L = dev::rank_kept(p.keep + row0, p.N, s_pos, s_wsum);
        if (p.zero_dropped && qt == 0) zero_dropped_head<OUT_F32>(p, row0, h);
    } else {
        const int s = min(max(p.cu[b], 0), p.total_rows);
        const int e = min(max(p.cu[b + 1], s), p.total_rows);
        row0 = s;
        L = min(e - s, p.max_len);
    }
    const int q0 = qt * kBM;
    if (q0 >= L) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const bool wave_active = q0 + wave * 16 < L;
    const int64_t hoff = (int64_t)h * kD;

    // Buffer resources covering this head's rows of the image: rows row0 ..
    // row0+span-1 (the L packed rows, or all N batch rows when gathered).
    const int span = GATHERED ? p.N : L;
    const uint32_t qsb = (uint32_t)(p.qs * ES), ksb = (uint32_t)(p.ks * ES),
                   vsb = (uint32_t)(p.vs * ES), osb = (uint32_t)(p.os * OES);
    const auto rq = make_rsrc(static_cast<const char*>(p.q) + (row0 * p.qs + hoff) * ES,
                              (uint32_t)(span - 1) * qsb + kD * ES);
    const auto rk = make_rsrc(static_cast<const char*>(p.k) + (row0 * p.ks + hoff) * ES,
                              (uint32_t)(span - 1) * ksb + kD * ES);
    const auto rv = make_rsrc(static_cast<const char*>(p.v) + (row0 * p.vs + hoff) * ES,
                              (uint32_t)(span - 1) * vsb + kD * ES);
    // Byte offset of the row of rank `r` (the r-th row of the sequence); rows
    // past the sequence fall outside the resource (zeros in, stores dropped).
    auto row_off = [&](int r, uint32_t stride) -> uint32_t {
        if constexpr (GATHERED) return r < L ? (uint32_t)s_pos[r] * stride : kDropOffset;
        else return (uint32_t)r * stride;
    };

    // Q^T as the B operand: lane holds query row r16, d = 8g..8g+7 and 32+8g..
    bf16x8 qh0, qh1, ql0, ql1;
    {
        const uint32_t off = row_off(q0 + wave * 16 + r16, qsb) + 8 * g * ES;
        load8<IN_F32>(rq, off, qh0, ql0);
        load8<IN_F32>(rq, off + 32 * ES, qh1, ql1);
    }

    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.scale_log2;

    // Registers carrying one K/V tile from global memory to LDS: this thread's
    // two 16-byte K pieces and its V key pair (hi and, for fp32 input, lo).
    bf16x8 kh0, kl0, kh1, kl1, vh0, vl0, vh1, vl1;
    const int k_key0 = tid >> 3, k_key1 = (tid + kThreads) >> 3, k_dg = tid & 7;
    const int v_kp = tid >> 3, v_dg = tid & 7;
    auto fetch = [&](int kt) {
        load8<IN_F32>(rk, row_off(kt + k_key0, ksb) + 8 * k_dg * ES, kh0, kl0);
        load8<IN_F32>(rk, row_off(kt + k_key1, ksb) + 8 * k_dg * ES, kh1, kl1);
        load8<IN_F32>(rv, row_off(kt + 2 * v_kp, vsb) + 8 * v_dg * ES, vh0, vl0);
        load8<IN_F32>(rv, row_off(kt + 2 * v_kp + 1, vsb) + 8 * v_dg * ES, vh1, vl1);
    };
    auto stash = [&]() {
        // K row-major; V transposed with keys 2kp, 2kp+1 side by side (one
        // 32-bit LDS store per (d, key pair))
        *reinterpret_cast<bf16x8*>(&sK[k_key0 * kKS + 8 * k_dg]) = kh0;
        *reinterpret_cast<bf16x8*>(&sK[k_key1 * kKS + 8 * k_dg]) = kh1;
        if constexpr (IN_F32) {
            *reinterpret_cast<bf16x8*>(&sK[K_PLANE + k_key0 * kKS + 8 * k_dg]) = kl0;
            *reinterpret_cast<bf16x8*>(&sK[K_PLANE + k_key1 * kKS + 8 * k_dg]) = kl1;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int o = (8 * v_dg + i) * kVS + 2 * v_kp;
            *reinterpret_cast<uint32_t*>(&sVt[o]) = bits(vh0[i]) | (bits(vh1[i]) << 16);
            if constexpr (IN_F32)
                *reinterpret_cast<uint32_t*>(&sVt[V_PLANE + o]) = bits(vl0[i]) | (bits(vl1[i]) << 16);
        }
    };
    fetch(0);

    for (int kt = 0; kt < L; kt += kBN) {
        const int nk = min(kBN, L - kt);
        if (kt > 0) __syncthreads();  // the previous tile is no longer read
        stash();
        if (kt + kBN < L) fetch(kt + kBN);  // in flight while this tile is computed
        if constexpr (PADDED) {
            if (tid < kBN) sKeep[tid] = (tid < nk) ? p.keep[row0 + kt + tid] : 0;
        }
        __syncthreads();
        if (!wave_active) continue;

        // ---- S^T = K Q^T: block kb holds keys kt+16kb+4g+i (i<4), query r16 --
        // All four blocks are computed: K rows past the sequence are zero in LDS.
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const __bf16* kr = &sK[(kb * 16 + r16) * kKS + 8 * g];
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kr);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kr + 32);
            s[kb] = mfma(a0, qh0, f32x4{0.f, 0.f, 0.f, 0.f});
            s[kb] = mfma(a1, qh1, s[kb]);
            if constexpr (IN_F32) {
                const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(kr + K_PLANE);
                const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(kr + K_PLANE + 32);
                s[kb] = mfma(b0, qh0, s[kb]);
                s[kb] = mfma(b1, qh1, s[kb]);
                s[kb] = mfma(a0, ql0, s[kb]);
                s[kb] = mfma(a1, ql1, s[kb]);
            }
        }

        // ---- online softmax (fp32, base 2) ----------------------------------
        // The exponent is c*s - m with c = scale*log2(e).  For c > 0 the max is
        // taken on the raw scores and the scale folds into one FMA per score;
        // otherwise the scores are scaled first (a rare, uniform branch).  Keys
        // past the tile (or dropped, padded form) become -inf.
        float cm = c;
        if (!(c > 0.f)) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[kb] *= c;
            cm = 1.f;
        }
        if (PADDED || nk < kBN) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = kb * 16 + 4 * g + i;
                    bool ok = key < nk;
                    if constexpr (PADDED) ok = ok && sKeep[key] != 0;
                    s[kb][i] = ok ? s[kb][i] : -INFINITY;
                }
            }
        }
        float mloc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]), fmaxf(fmaxf(s[0][3], s[1][0]), s[1][1]));
        mloc = fmaxf(mloc, fmaxf(fmaxf(fmaxf(s[1][2], s[1][3]), s[2][0]), fmaxf(fmaxf(s[2][1], s[2][2]), s[2][3])));
        mloc = fmaxf(mloc, fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3])));
        mloc = row_max(mloc) * cm;
        const float m_new = fmaxf(m_run, mloc);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        if (kt > 0) {
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) acc[db] *= alpha;
        }
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = fast_exp2(__builtin_fmaf(s[kb][i], cm, -m_use));
                s[kb][i] = e;
                psum += e;
            }
        }
        l_run += psum;

        // ---- O^T += V^T P^T, 32 keys per MFMA ---------------------------------
        // k-slot e of lane group g: e<4 -> key 32c+4g+e, e>=4 -> key 32c+16+4g+e-4;
        // these are exactly the keys of s[2c][e] and s[2c+1][e-4].
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            if (cc * 32 < nk) {
                u32x4 phw, plw;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = e < 2 ? s[2 * cc][2 * e] : s[2 * cc + 1][2 * e - 4];
                    const float x1 = e < 2 ? s[2 * cc][2 * e + 1] : s[2 * cc + 1][2 * e - 3];
                    uint32_t hw, lw;
                    split_pair(x0, x1, hw, lw);
                    phw[e] = hw;
                    plw[e] = lw;
                }
                const bf16x8 ph = __builtin_bit_cast(bf16x8, phw);
                const bf16x8 pl = __builtin_bit_cast(bf16x8, plw);
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int vo = (db * 16 + r16) * kVS + 32 * cc + 4 * g;
                    const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(&sVt[vo]);
                    const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(&sVt[vo + 16]);
                    const bf16x8 av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[db] = mfma(av, ph, acc[db]);
                    acc[db] = mfma(av, pl, acc[db]);
                    if constexpr (IN_F32) {
                        const bf16x4 w0 = *reinterpret_cast<const bf16x4*>(&sVt[V_PLANE + vo]);
                        const bf16x4 w1 = *reinterpret_cast<const bf16x4*>(&sVt[V_PLANE + vo + 16]);
                        const bf16x8 al = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
                        acc[db] = mfma(al, ph, acc[db]);
                    }
                }
            }
        }
    }

    // ---- epilogue: O = acc / l, staged through LDS for row-contiguous stores --
    __syncthreads();  // every wave is done with the K / V tiles
    if (!wave_active) return;
    const float lt = row_sum(l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    char* so = smem + wave * 16 * OUT_ROW;
    // lane holds O[r16][16db + 4g + i]
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const f32x4 r = acc[db] * inv;
        char* dst = so + r16 * OUT_ROW + (16 * db + 4 * g) * OES;
        if constexpr (OUT_F32) {
            *reinterpret_cast<f32x4*>(dst) = r;
        } else {
            bf16x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) o4[i] = static_cast<__bf16>(r[i]);
            *reinterpret_cast<bf16x4*>(dst) = o4;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const auto ro = make_rsrc(static_cast<char*>(p.o) + (row0 * p.os + hoff) * OES,
                              (uint32_t)(span - 1) * osb + kD * OES);
    constexpr int CHUNKS = kD * OES / 16;  // 16-byte pieces per row: 8 (bf16) or 16 (fp32)
#pragma unroll
    for (int j = 0; j < 16 * CHUNKS / 64; ++j) {
        const int piece = lane + 64 * j;
        const int r = piece / CHUNKS, cix = piece % CHUNKS;
        const u32x4 val = *reinterpret_cast<const u32x4*>(so + r * OUT_ROW + 16 * cix);
        __builtin_amdgcn_raw_buffer_store_b128(val, ro, row_off(q0 + wave * 16 + r, osb) + 16 * cix, 0, 0);
    }
}

template <bool IN_F32, bool OUT_F32>
void launch_variant(const AttnParams& p, int layout, hipStream_t st)
{
    const dim3 grid(p.H, p.B, p.n_qtiles), block(kThreads);
    if (layout == kPadded)
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kPadded>), grid, block, 0, st, p);
    else if (layout == kGathered)
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kGathered>), grid, block,
                           sizeof(int) * (size_t)p.N, st, p);
    else
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kRagged>), grid, block, 0, st, p);
}

}  // namespace

int launch_attn(const void* q, const void* k, const void* v, int64_t q_row_stride,
                int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                const int32_t* cu_seqlens, const uint8_t* keep, int32_t B, int32_t N,
                int32_t max_seqlen, int32_t total_rows, int32_t H, float scale, void* o,
                int64_t o_row_stride, int32_t out_dtype, int layout, uint32_t flags,
                void* stream)
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
    p.max_len = layout == kRagged ? max_seqlen : N;
    p.n_qtiles = (p.max_len + kBM - 1) / kBM;
    p.zero_dropped = (flags & RAG_UNPACK_ZERO_DROPPED) ? 1 : 0;
    p.scale_log2 = scale * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool in_f32 = in_dtype == RAG_DTYPE_F32, out_f32 = out_dtype == RAG_DTYPE_F32;
    if (in_f32 && out_f32) launch_variant<true, true>(p, layout, st);
    else if (in_f32) launch_variant<true, false>(p, layout, st);
    else if (out_f32) launch_variant<false, true>(p, layout, st);
    else launch_variant<false, false>(p, layout, st);
    return (int)hipGetLastError();
}

}  // namespace rag
