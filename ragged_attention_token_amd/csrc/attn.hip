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
// Kernel design (ours, for gfx950; the pages' Triton kernel is not followed).
// Two kernels compute it with the same arithmetic in the same order, so the
// one the host picks (by input dtype and max_seqlen) never changes a bit:
//   * attn_lds_kernel (bf16 input, up to 256 keys): an image's whole K and V
//     for one head are copied straight into LDS by buffer loads that write
//     LDS, one barrier, then every wave runs its 16-row query blocks over all
//     keys with no further synchronisation (see the comment at the kernel);
//   * attn_kernel (fp32 input, or longer sequences): one workgroup = one
//     (head, image, q-tile of 64 rows), 4 wave64s of 16 query rows, K / V
//     staged through LDS 64 keys at a time (row-major, as above), the
//     next tile's loads in registers while the current tile computes.
// Both:
//   * all global traffic goes through buffer resources whose range ends at
//     the image's last row: loads past the sequence end return zeros and
//     stores past it are dropped by the hardware, so no per-lane predicate is
//     needed and no uninitialised value can reach an MFMA;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp32 accumulate): each lane
//     holds the scores of ONE query row (lane & 15) for 4 keys per 16-key
//     block, so the row max takes two v_permlane{16,32}_swap steps;
//   * online softmax in fp32 with exp2, a lazily moved reference maximum and
//     row sums from the MFMA unit (see "online softmax shared by both
//     kernels"); masking only in a sequence's last, partial tile;
//   * the probabilities are split into bf16 high + low parts and O^T += V^T P^T
//     runs both through the same MFMA, so P is carried to about 16 mantissa
//     bits; fp32 inputs are split the same way (hi/lo for Q, K, V);
//   * the probabilities never leave registers: the MFMA result layout of S^T
//     is used directly as the B operand of the P.V product (keys are a
//     summation index, so the k-order only has to agree between the two
//     operands).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

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
// Tile kernel, grid launches: an XCD takes its (head, image) pairs kPairBlock
// at a time, every q-tile of the block before the next block.  1 puts a
// pair's q-tiles back to back (they then read the same K / V lines at the
// same moment); all of the XCD's pairs at once is a q-tile-slowest order,
// whose reuse distance lets Q and O streams evict the pairs' K / V from L2
// (N = 577: 1.33x the algorithmic bytes fetched).  4 fetches the algorithmic
// bytes and measured fastest of 1, 4, 16 and all.
constexpr int kPairBlock = 4;  // a power of two
constexpr int kMaxGridY = 65535;

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
    int32_t lds_rows;        // LDS-resident kernel: K / V rows held, max_len rounded up to 32
    int32_t out_stage;       // LDS-resident kernel: byte offset of the per-wave output slots (0: none)
    int32_t tl_kt;           // tile-list launch: key tiles of the longest image (else 0)
    float scale_log2;        // scale * log2(e)
    int32_t natural_first;   // gathered layout: request K/V in natural order beside the keep bytes
    uint32_t h_magic;        // floor(2^32 / H) + 1 (H >= 2): pair / H by a multiply-high
};

// (pair / H, pair % H) for pair < 2^32: the multiply-high by h_magic
// over-estimates the quotient by at most one, corrected once.
__device__ __forceinline__ void split_pair(uint32_t pair, int H, uint32_t h_magic, int& h, int& b)
{
    uint32_t q = pair;
    if (H > 1) {
        q = __umulhi(pair, h_magic);
        q -= (q * (uint32_t)H > pair) ? 1u : 0u;
    }
    b = (int)q;
    h = (int)(pair - q * (uint32_t)H);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of a per-lane value over the four 16-lane rows of the wave (lanes
// l, l^16, l^32, l^48), which hold the same query row.
__device__ __forceinline__ float row_max(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

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

// ---- online softmax shared by both kernels --------------------------------
//
// Exponents are taken in base 2 with c = scale * log2(e) folded into one FMA
// per score, c * s - m, where m is the row's running reference maximum (of
// c * s).  c must be positive: fold_scale negates Q for a negative scale and
// turns a zero scale into a tiny positive one (every product then rounds to
// an exponent of 0: uniform weights), so no tile pays for the other signs.
//
// Lazy rescaling: the reference m only moves when some row of the wave sees
// a tile maximum more than kLazyLog2 above it.  Otherwise the stale m is kept
// and the tile's probabilities are at most 2^kLazyLog2 (no overflow risk in
// fp32), which skips the accumulator rescale on almost every tile; O = acc / l
// does not depend on the reference.
//
// Row sums come from the MFMA unit: the same P.V product with an all-ones A
// operand gives, in every element of the lane's result, the sum of the
// probabilities of the lane's query row (the same bf16 hi + lo values that
// weight V, so numerator and denominator use identical P).
constexpr float kLazyLog2 = 8.f;

struct Online {
    float m;        // reference maximum of c * s for the lane's query row
    float neg_m;    // the exponent offset: -m, or 0 while m is -inf (no key yet)
    f32x4 acc[4];   // O^T: acc[db][i] = O[query r16][16 db + 4 g + i] (unnormalised)
    f32x4 lsum;     // row sums of P (all four elements equal)
};

__device__ __forceinline__ void online_init(Online& st)
{
    st.m = -INFINITY;
    st.neg_m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.lsum = f32x4{0.f, 0.f, 0.f, 0.f};
}

__device__ __forceinline__ bf16x8 negate_bf16(bf16x8 x)
{
    return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x) ^ 0x80008000u);
}

// Returns the positive exponent scale to use; negates the Q operand registers
// when c < 0 (c s = (-c)(-s)).
__device__ __forceinline__ float fold_scale(float c, bf16x8& q0, bf16x8& q1, bf16x8& q2, bf16x8& q3)
{
    if (c < 0.f) {
        q0 = negate_bf16(q0);
        q1 = negate_bf16(q1);
        q2 = negate_bf16(q2);
        q3 = negate_bf16(q3);
        c = -c;
    }
    return c > 0.f ? c : 1e-30f;
}

// Scores -> probabilities for one 64-key tile, in place.  s[kb][i] is the raw
// score of the lane's query and key 16 kb + 4 g + i of the tile.  FULL: all 64
// keys are present; otherwise keys >= nk are absent (their blocks need not be
// computed) and get probability 0.  PADDED: keys with keep byte 0 (keep_tile,
// indexed by key within the tile) are masked too.  `first`: the first tile of
// the row (the reference is set, nothing to rescale).
template <bool FULL, bool PADDED>
__device__ __forceinline__ void online_probs(f32x4 (&s)[4], int nk, const uint8_t* keep_tile,
                                             int g, float c, bool first, Online& st)
{
    if constexpr (!FULL || PADDED) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kb * 16 + 4 * g + i;
                bool ok = FULL || key < nk;
                if constexpr (PADDED) ok = ok && keep_tile[key] != 0;
                s[kb][i] = ok ? s[kb][i] : -INFINITY;
            }
        }
    }
    // this lane's maximum; the row's (over the four lanes of the query row) is
    // only formed when the reference is set or moved: some lane exceeds
    // m + kLazyLog2 exactly when the row maximum does (c > 0 keeps the order)
    float mloc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]), fmaxf(fmaxf(s[0][3], s[1][0]), s[1][1]));
    mloc = fmaxf(mloc, fmaxf(fmaxf(fmaxf(s[1][2], s[1][3]), s[2][0]), fmaxf(fmaxf(s[2][1], s[2][2]), s[2][3])));
    mloc = fmaxf(mloc, fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3])));
    if (first) {
        st.m = row_max(mloc) * c;
        st.neg_m = (st.m == -INFINITY) ? 0.f : -st.m;
    } else if (__ballot(mloc * c > st.m + kLazyLog2)) {  // uniform over the wave
        const float m_new = fmaxf(st.m, row_max(mloc) * c);
        const float alpha = fast_exp2(st.m - m_new);
#pragma unroll
        for (int db = 0; db < 4; ++db) st.acc[db] *= alpha;
        st.lsum *= alpha;
        st.m = m_new;
        st.neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (FULL || 16 * kb < nk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s[kb][i] = fast_exp2(__builtin_fmaf(s[kb][i], c, st.neg_m));
        } else {
            s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

// The P operand (B of O^T += V^T P^T) for keys 32 cc .. 32 cc + 31 of the
// tile, as bf16 hi + lo: k-slot e of lane group g is key 32cc + 4g + e (e < 4)
// or 32cc + 16 + 4g + e - 4 (e >= 4), the keys of s[2cc][e] and s[2cc+1][e-4].
// Also adds the chunk's row sums to st.lsum.
__device__ __forceinline__ void p_operand(const f32x4 (&s)[4], int cc, bf16x8& ph, bf16x8& pl,
                                          Online& st)
{
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
    ph = __builtin_bit_cast(bf16x8, phw);
    pl = __builtin_bit_cast(bf16x8, plw);
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    st.lsum = mfma(ones, ph, st.lsum);
    st.lsum = mfma(ones, pl, st.lsum);
}

// 1 / l for the lane's query row (0 for a row without keys).
__device__ __forceinline__ float online_inv(const Online& st)
{
    const float l = st.lsum[0];
    return l > 0.f ? 1.f / l : 0.f;
}

// ---- tile list of the ragged layout ---------------------------------------
//
// A tile-list launch covers the work items of a ragged batch with a 1-D grid
// in which no slot belongs to a query tile that a short image lacks, and in
// which the longest images come first ("Dispatch-Aware Ragged Attention for
// Pruned Vision Transformers", abstract: the kernel runs on ragged
// post-pruning lengths).  An item is one (image, head) pair, whole, or one
// 64-row query tile of it (four 16-row blocks).  Each workgroup derives its
// item from cu_seqlens alone (wave 0 does, and hands it to the other waves
// through LDS; no atomics, nothing written by an earlier launch):
//   * an image of L rows has nkt = ceil(L / 64) key tiles (0 when empty) and
//     n = 1 item (whole pairs) or n = nkt items (query tiles);
//   * items are ordered by nkt, largest first;
//   * the pairs of one nkt class are dealt round-robin to the eight XCDs
//     (workgroup w runs on XCD w mod 8) and all items of a pair go to its XCD,
//     so the pair's K and V rows are fetched into one L2.
// The grid is an upper bound the host computes from B, H and max_seqlen;
// workgroups past the items of their XCD return at once (they come last).
// Limits (checked by the host): B <= 1024 (lane l holds the key-tile counts of
// images 64 i + l, 4 bits each, i < 16), max_seqlen <= 960 (nkt <= 15) and
// H <= 64 (every item index stays below 2^17, see udiv_small).
struct Item {
    int b, h, q0, q1, L;  // query blocks [q0, q1)
    int64_t row0;
};

// a / d and a % d for 0 <= a < 2^20 and d >= 1 (wave-uniform values): the
// float estimate a * rcp(d) is within a * 2^-22 < 1/4 of a / d, so after
// truncation one correction step each way gives the exact quotient.
__device__ __forceinline__ int udiv_small(int a, int d, int& rem)
{
    int q = (int)((float)a * __builtin_amdgcn_rcpf((float)d));
    int r = a - q * d;
    if (r < 0) { --q; r += d; }
    if (r >= d) { ++q; r -= d; }
    rem = r;
    return q;
}

template <bool WHOLE>
__device__ __forceinline__ bool tile_item(const AttnParams& p, Item& it)
{
    const int lane = threadIdx.x & 63;
    const int nch = (p.B + 63) >> 6;
    const auto rc = make_rsrc(p.cu, (uint32_t)(p.B + 1) * 4u);  // cu[b], b > B reads 0
    auto seq_len = [&](int s, int e) {
        s = min(max(s, 0), p.total_rows);
        e = min(max(e, s), p.total_rows);
        return min(e - s, p.max_len);
    };
    // the chunks' offsets are requested at once (straight-line code: no load
    // waits for another): 4 chunks when B <= 256, else 16; chunks past B read
    // zeros, i.e. empty images
    int cs[16], ce[16];
    auto load_chunks = [&](auto nc_tag) {
        constexpr int NC = decltype(nc_tag)::value;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t off = 4u * (uint32_t)(64 * i + lane);
            cs[i] = i < NC ? (int)__builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0) : 0;
            ce[i] = i < NC ? (int)__builtin_amdgcn_raw_buffer_load_b32(rc, off + 4u, 0, 0) : 0;
        }
    };
    if (nch <= 4) load_chunks(std::integral_constant<int, 4>{});
    else load_chunks(std::integral_constant<int, 16>{});
    uint64_t kt4 = 0;  // key-tile count of image 64 i + lane in bits [4i, 4i + 4)
#pragma unroll
    for (int i = 0; i < 16; ++i) kt4 |= (uint64_t)((seq_len(cs[i], ce[i]) + 63) >> 6) << (4 * i);
    auto class_mask = [&](int i, int k) -> uint64_t {
        return __ballot((int)((kt4 >> (4 * i)) & 15u) == k);
    };

    // the nkt class of this workgroup's item, and its place among the XCD's
    // items of that class
    const int x = blockIdx.x & 7;
    int pos = blockIdx.x >> 3;
    int k = p.tl_kt, G = 0;
    for (; k >= 1; --k) {
        G = 0;
        for (int i = 0; i < nch; ++i) G += __popcll(class_mask(i, k));
        const int pairs = G * p.H;
        const int mine = pairs > x ? (pairs - x + 7) >> 3 : 0;  // pairs x, x + 8, ...
        const int items = WHOLE ? mine : mine * k;
        if (pos < items) break;
        pos -= items;
    }
    if (k < 1) return false;
    int part = 0, r;
    const int pi = WHOLE ? pos : udiv_small(pos, k, part);
    it.h = udiv_small(x + 8 * pi, G, r);  // pair x + 8 pi = h G + r: the r-th image of the class
    int b = 0, s = 0, e = 0;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // (constant i: the offsets stay in registers)
        if (i < nch && !found) {
            const uint64_t msk = class_mask(i, k);
            const int c = __popcll(msk);
            if (r < c) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0u));
                const int l = __builtin_ctzll(__ballot(((msk >> lane) & 1u) && below == (uint32_t)r));
                b = 64 * i + l;
                s = __builtin_amdgcn_readlane(cs[i], l);  // the image's offsets, already loaded
                e = __builtin_amdgcn_readlane(ce[i], l);
                found = true;
            }
            r -= c;
        }
    }
    it.b = b;
    it.row0 = min(max(s, 0), p.total_rows);
    it.L = seq_len(s, e);
    const int nqb = (it.L + 15) >> 4;
    it.q0 = WHOLE ? 0 : 4 * part;
    it.q1 = WHOLE ? nqb : min(4 * part + 4, nqb);
    return true;
}

// The workgroup's item: wave 0 derives it, the others read it from LDS (the
// decode's loads and scalar steps are paid once per workgroup).  Returns false
// for a workgroup past its XCD's items (uniform over the workgroup).
template <bool WHOLE>
__device__ __forceinline__ bool workgroup_item(const AttnParams& p, Item& it)
{
    __shared__ int s_item[6];
    if (threadIdx.x < 64) {
        Item w{};
        const bool ok = tile_item<WHOLE>(p, w);
        if (threadIdx.x == 0) {
            s_item[0] = ok ? w.b : -1;
            s_item[1] = w.h;
            s_item[2] = w.q0;
            s_item[3] = w.q1;
            s_item[4] = w.L;
            s_item[5] = (int)w.row0;  // row0 <= total_rows < 2^31
        }
    }
    __syncthreads();
    // equal in every lane; read from lane 0 they are scalars for the compiler
    it.b = __builtin_amdgcn_readfirstlane(s_item[0]);
    it.h = __builtin_amdgcn_readfirstlane(s_item[1]);
    it.q0 = __builtin_amdgcn_readfirstlane(s_item[2]);
    it.q1 = __builtin_amdgcn_readfirstlane(s_item[3]);
    it.L = __builtin_amdgcn_readfirstlane(s_item[4]);
    it.row0 = __builtin_amdgcn_readfirstlane(s_item[5]);
    return it.b >= 0;
}

// Grid of a tile-list launch: on each XCD at most ceil(B H n_max / 8) + sum_k n_k
// items (n_k = 1 for whole pairs, k for query tiles; n_max = n_kt_max).
int tile_list_grid(int B, int H, int kt_max, bool whole)
{
    const int64_t n_max = whole ? 1 : kt_max;
    int64_t per_xcd = ((int64_t)B * H * n_max + 7) / 8;
    per_xcd += whole ? kt_max : kt_max * (kt_max + 1) / 2;
    return (int)(8 * per_xcd);
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
    for (int i = threadIdx.x; i < p.N * CHUNKS; i += blockDim.x) {
        const int n = i / CHUNKS, cix = i - n * CHUNKS;
        if (p.keep[row0 + n] == 0) dev::st16(zero, ro, (uint32_t)n * osb + 16 * cix);
    }
}

// ---- LDS operand layout shared by both kernels ------------------------------
//
// K and V rows are held in LDS as 128-byte rows (64 bf16) in natural row-major
// order, with the eight 16-byte chunks of row r permuted by XOR with swz(r).
// The permutation makes both operand reads conflict-free across 16
// consecutive rows: the K reads (ds_read_b128, lane = row) and the V reads
// with gfx950's transposing read ds_read_b64_tr_b16, which delivers V^T's MFMA
// operand from row-major V.
constexpr int kRowBytes = kD * 2;     // one head's bf16 row

// Slot of chunk c of row r is c ^ swz(r); swz depends on r mod 16 only.
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Four bf16 of one LDS column: lane j of each 16-lane group receives element
// (k, j) of the 4 x 16 block whose row segments the group's lanes address.
__device__ __forceinline__ bf16x4 ld_tr4(const char* lds_addr)
{
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)lds_addr));
}

// Per-lane LDS offsets inside a 16-row block.
//  K (A operand of S^T): row r16, chunks g and g + 4 of the row (the second
//  is this one XOR 64).
__device__ __forceinline__ uint32_t k_operand_offset(int r16, int g)
{
    return 128u * r16 + 16u * (uint32_t)(g ^ swz(r16));
}
//  V (A operand of O^T += V^T P^T, transposing read) for 16-column block db:
//  lane i of group g addresses row 4g + i/4, columns 16 db + 4 (i % 4) .. + 3;
//  it receives V[4g + k][16 db + i] for k = 0..3 -- keys 4g..4g+3 of d-row i,
//  the k-slots that match the probabilities' layout (p_operand).
__device__ __forceinline__ uint32_t v_operand_offset(int r16, int g, int db)
{
    const int vrow = 4 * g + (r16 >> 2);
    return 128u * vrow + 16u * (uint32_t)((2 * db + ((r16 & 3) >> 1)) ^ swz(vrow)) + 8u * (r16 & 1);
}

// ---- loads the compiler does not track ------------------------------------
//
// The tile kernel's K/V loads into LDS (dev::ld_lds16_untracked) and the
// gathered layout's speculative loads are inline assembly, waited for with
// explicit counts: the compiler cannot tell that LDS-writing loads and the
// LDS words read meanwhile (the current K/V tile, the keep ranking's words) do
// not overlap, and its own waits would serialise them.  A wave's loads
// complete in issue order, which the count-based wait for the keep bytes
// (issued first) relies on.
using dev::i32x4;
using dev::ld_lds16_untracked;
using dev::rsrc_words;

// One byte at offset off of the resource, zero-extended.  The result register
// is written when the load completes: read it only after a wait_vm() that
// covers the load and a vm_done() on it.
__device__ __forceinline__ uint32_t ld_u8_untracked(i32x4 r, uint32_t off)
{
    uint32_t x;
    asm volatile("buffer_load_ubyte %0, %1, %2, 0 offen" : "=v"(x) : "v"(off), "s"(r));
    return x;
}

// Waits until at most n (wave-uniform, even, >= 0) of this wave's
// vector-memory operations are outstanding; an n above 14 waits for 14.
__device__ __forceinline__ void wait_vm(int n)
{
    const int u = __builtin_amdgcn_readfirstlane(n);
    asm volatile(
        "s_cmp_lt_u32 %0, 2\n\ts_cbranch_scc1 0f\n\t"
        "s_cmp_lt_u32 %0, 4\n\ts_cbranch_scc1 2f\n\t"
        "s_cmp_lt_u32 %0, 6\n\ts_cbranch_scc1 4f\n\t"
        "s_cmp_lt_u32 %0, 8\n\ts_cbranch_scc1 6f\n\t"
        "s_cmp_lt_u32 %0, 10\n\ts_cbranch_scc1 8f\n\t"
        "s_cmp_lt_u32 %0, 12\n\ts_cbranch_scc1 10f\n\t"
        "s_cmp_lt_u32 %0, 14\n\ts_cbranch_scc1 12f\n\t"
        "s_waitcnt vmcnt(14)\n\ts_branch 1f\n"
        "12:\n\ts_waitcnt vmcnt(12)\n\ts_branch 1f\n"
        "10:\n\ts_waitcnt vmcnt(10)\n\ts_branch 1f\n"
        "8:\n\ts_waitcnt vmcnt(8)\n\ts_branch 1f\n"
        "6:\n\ts_waitcnt vmcnt(6)\n\ts_branch 1f\n"
        "4:\n\ts_waitcnt vmcnt(4)\n\ts_branch 1f\n"
        "2:\n\ts_waitcnt vmcnt(2)\n\ts_branch 1f\n"
        "0:\n\ts_waitcnt vmcnt(0)\n"
        "1:"
        :
        : "s"(u)
        : "memory", "scc");
}

// Marks x as produced after the preceding volatile statements (a wait_vm), so
// that no read of it is scheduled before them.
__device__ __forceinline__ void vm_done(uint32_t& x) { asm volatile("" : "+v"(x)); }

template <bool IN_F32, bool OUT_F32, int LAYOUT, bool TILES>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p)
{
    constexpr bool PADDED = LAYOUT == kPadded;
    constexpr bool GATHERED = LAYOUT == kGathered;
    constexpr int NP = IN_F32 ? 2 : 1;  // bf16 planes: hi (and lo)
    constexpr int ES = IN_F32 ? 4 : 2;  // input element bytes
    constexpr int OES = OUT_F32 ? 4 : 2;
    constexpr int PLANE = kBN * kRowBytes;        // one bf16 plane of a 64-key K or V tile
    constexpr int OUT_ROW = kD * OES + 16;        // bytes, padded
    // fp32 input: K planes, then V planes, staged through registers; bf16
    // input: two K/V tile buffers filled by LDS-writing loads.  The output is
    // staged in the same bytes afterwards.
    constexpr int KV_BYTES = IN_F32 ? 2 * NP * PLANE : 4 * PLANE;
    constexpr int SMEM = KV_BYTES > 4 * 16 * OUT_ROW ? KV_BYTES : 4 * 16 * OUT_ROW;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    char* sK = smem;
    char* sV = smem + NP * PLANE;
    __shared__ uint8_t sKeep[2][kBN];  // padded: keep bytes of the tile in each buffer
    extern __shared__ int s_pos[];  // gathered: the image's kept positions by rank (N ints)
    __shared__ int s_wsum[16];  // keep ranking: up to 4 planes x 4 waves

    // ---- which (head, image, query blocks): TILES, the tile list's item (four
    // query blocks at most); otherwise a grid of (pair, q-tile of four blocks)
    // slots, pair = (head, image), laid out for the XCDs: workgroup i runs on
    // XCD i % 8 as that XCD's (i / 8)-th; pairs are dealt round-robin to the
    // XCDs and each XCD runs the q-tiles of kPairBlock of its pairs before the
    // next kPairBlock, so every q-tile after a pair's first finds the pair's
    // K and V in that XCD's L2 instead of fetching them again.  Slots past the
    // last pair exit at once.
    // The grid is (8 * kPairBlock * q-tiles, blocks of pairs), the second
    // folded into (Y, Z) beyond kMaxGridY: x = XCD + 8 * (pair in the block +
    // kPairBlock * q-tile), so the dispatch order is the linear id and x % 8
    // the XCD, and the decode is shifts and masks.
    int h, b, qt;
    if constexpr (!TILES) {
        const uint32_t x = blockIdx.x;
        const uint32_t blk = blockIdx.y + gridDim.y * blockIdx.z;
        qt = (int)(x / (8u * kPairBlock));
        const uint32_t pair = (x & 7u) + 8u * (blk * kPairBlock + ((x >> 3) & (kPairBlock - 1)));
        if (pair >= (uint32_t)p.H * (uint32_t)p.B) return;  // uniform over the workgroup
        split_pair(pair, p.H, p.h_magic, h, b);
    }

    int64_t row0;
    int L, qlo, qhi;
    if constexpr (TILES) {
        static_assert(LAYOUT == kRagged, "the tile list is built from cu_seqlens");
        Item it;
        if (!workgroup_item<false>(p, it)) return;  // uniform over the workgroup
        h = it.h;
        b = it.b;
        row0 = it.row0;
        L = it.L;
        qlo = it.q0;
        qhi = it.q1;
    } else if constexpr (PADDED) {
        row0 = (int64_t)b * p.N;
        L = p.N;
    } else if constexpr (GATHERED) {
        row0 = (int64_t)b * p.N;
        L = p.N <= 4 * kThreads ? dev::rank_kept_planes<4>(p.keep + row0, p.N, s_pos, s_wsum, 4)
                                : dev::rank_kept(p.keep + row0, p.N, s_pos, s_wsum);
        L = min(__builtin_amdgcn_readfirstlane(L), p.max_len);  // (a workgroup reduction: uniform)
        if (p.zero_dropped && qt == 0) zero_dropped_head<OUT_F32>(p, row0, h);
    } else {
        const int s = min(max(p.cu[b], 0), p.total_rows);
        const int e = min(max(p.cu[b + 1], s), p.total_rows);
        row0 = s;
        L = min(e - s, p.max_len);
    }
    if constexpr (!TILES) {
        qlo = qt * (kBM / 16);
        qhi = (L + 15) >> 4;
    }
    if (qlo >= qhi) return;
    const int qrow = 16 * qlo;  // first query row of the workgroup

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loops and addresses
    const int r16 = lane & 15, g = lane >> 4;
    const bool wave_active = qlo + wave < qhi;
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
    bf16x8 qh0, qh1, ql0 = {}, ql1 = {};
    {
        const uint32_t off = row_off(qrow + wave * 16 + r16, qsb) + 8 * g * ES;
        load8<IN_F32>(rq, off, qh0, ql0);
        load8<IN_F32>(rq, off + 32 * ES, qh1, ql1);
    }
    // (bf16 input: formed once the first K/V tile has landed, below)
    float c = 0.f;
    if constexpr (IN_F32) c = fold_scale(p.scale_log2, qh0, qh1, ql0, ql1);
    Online st;
    online_init(st);

    const uint32_t koff0 = k_operand_offset(r16, g);
    const uint32_t koff1 = koff0 ^ 64u;
    uint32_t voff[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] = v_operand_offset(r16, g, db);

    // One 64-key tile at key kt from K / V rows at kbase / vbase in LDS (the
    // operand layout above; fp32 input: the lo planes PLANE bytes after) and
    // keep_tile (padded); FULL: all 64 keys present (no key-range masking).
    auto compute = [&](auto full_tag, const int kt, const char* kbase, const char* vbase,
                       const uint8_t* keep_tile) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int nk = min(kBN, L - kt);
        // ---- S^T = K Q^T: block kb holds keys kt+16kb+4g+i (i<4), query r16
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (FULL || kb == 0 || 16 * kb < nk) {
                const char* kr = kbase + 2048 * kb;
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kr + koff0);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kr + koff1);
                s[kb] = mfma(a0, qh0, f32x4{0.f, 0.f, 0.f, 0.f});
                s[kb] = mfma(a1, qh1, s[kb]);
                if constexpr (IN_F32) {
                    const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(kr + PLANE + koff0);
                    const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(kr + PLANE + koff1);
                    s[kb] = mfma(b0, qh0, s[kb]);
                    s[kb] = mfma(b1, qh1, s[kb]);
                    s[kb] = mfma(a0, ql0, s[kb]);
                    s[kb] = mfma(a1, ql1, s[kb]);
                }
            } else {
                s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};  // absent keys, masked below
            }
        }
        online_probs<FULL, PADDED>(s, nk, keep_tile, g, c, kt == 0, st);
        // ---- O^T += V^T P^T, 32 keys per MFMA ----------------------------
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            if (FULL || cc * 32 < nk) {
                bf16x8 ph, pl;
                p_operand(s, cc, ph, pl, st);
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const char* vr = vbase + 4096 * cc + voff[db];
                    const bf16x4 v0 = ld_tr4(vr);
                    const bf16x4 v1 = ld_tr4(vr + 2048);
                    const bf16x8 av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    st.acc[db] = mfma(av, ph, st.acc[db]);
                    st.acc[db] = mfma(av, pl, st.acc[db]);
                    if constexpr (IN_F32) {
                        const bf16x4 w0 = ld_tr4(vr + PLANE);
                        const bf16x4 w1 = ld_tr4(vr + PLANE + 2048);
                        const bf16x8 al = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
                        st.acc[db] = mfma(al, ph, st.acc[db]);
                    }
                }
            }
        }
    };

    if constexpr (IN_F32) {
        // Registers carrying one K/V tile from global memory to LDS: this
        // thread's 16-byte chunk k_dg of key rows k_row0 and k_row1, of K and
        // of V (hi and lo).  Eight consecutive lanes store one 128-byte LDS
        // row, in the permuted chunk order of the operand layout.
        bf16x8 kh0, kl0, kh1, kl1, vh0, vl0, vh1, vl1;
        const int k_row0 = tid >> 3, k_row1 = (tid + kThreads) >> 3, k_dg = tid & 7;
        const uint32_t so0 = 128u * k_row0 + 16u * (uint32_t)(k_dg ^ swz(k_row0));
        const uint32_t so1 = 128u * k_row1 + 16u * (uint32_t)(k_dg ^ swz(k_row1));
        auto fetch = [&](int kt) {
            load8<IN_F32>(rk, row_off(kt + k_row0, ksb) + 8 * k_dg * ES, kh0, kl0);
            load8<IN_F32>(rk, row_off(kt + k_row1, ksb) + 8 * k_dg * ES, kh1, kl1);
            load8<IN_F32>(rv, row_off(kt + k_row0, vsb) + 8 * k_dg * ES, vh0, vl0);
            load8<IN_F32>(rv, row_off(kt + k_row1, vsb) + 8 * k_dg * ES, vh1, vl1);
        };
        auto stash = [&]() {
            *reinterpret_cast<bf16x8*>(sK + so0) = kh0;
            *reinterpret_cast<bf16x8*>(sK + so1) = kh1;
            *reinterpret_cast<bf16x8*>(sV + so0) = vh0;
            *reinterpret_cast<bf16x8*>(sV + so1) = vh1;
            *reinterpret_cast<bf16x8*>(sK + PLANE + so0) = kl0;
            *reinterpret_cast<bf16x8*>(sK + PLANE + so1) = kl1;
            *reinterpret_cast<bf16x8*>(sV + PLANE + so0) = vl0;
            *reinterpret_cast<bf16x8*>(sV + PLANE + so1) = vl1;
        };
        fetch(0);
        // Stage the tile at key kt into LDS (the next one's loads go out
        // meanwhile), then compute it.  The full tiles run in one loop and the
        // partial last tile after it.
        auto tile = [&](auto full_tag, const int kt) {
            const int nk = min(kBN, L - kt);
            if (kt > 0) __syncthreads();  // the previous tile is no longer read
            stash();
            if (kt + kBN < L) fetch(kt + kBN);  // in flight while this tile is computed
            if constexpr (PADDED) {
                if (tid < kBN) sKeep[0][tid] = (tid < nk) ? p.keep[row0 + kt + tid] : 0;
            }
            __syncthreads();
            if (wave_active) compute(full_tag, kt, sK, sV, sKeep[0]);
        };
        int kt = 0;
        for (; kt + kBN <= L; kt += kBN) tile(std::true_type{}, kt);
        if (kt < L) tile(std::false_type{}, kt);
    } else {
        // bf16 input: K and V tiles go straight into LDS by LDS-writing loads
        // (no registers, no LDS store instructions), into two tile buffers:
        // tile t + 1 is requested into one while tile t is computed from the
        // other, and one barrier per tile separates them.  The loads are
        // untracked (see above) and waited for explicitly before the barrier.
        // Wave w moves 8-row blocks w and w + 4 of K and of V (1 KiB each);
        // lane l writes slot l & 7 of row l >> 3 of its block.
        const int lr = lane >> 3, slot = lane & 7;
        const uint32_t c16e = 16u * (uint32_t)(slot ^ swz(lr)), c16o = 16u * (uint32_t)(slot ^ swz(8 + lr));
        const i32x4 rkw = rsrc_words(static_cast<const char*>(p.k) + (row0 * p.ks + hoff) * ES,
                                     (uint32_t)(span - 1) * ksb + kD * ES);
        const i32x4 rvw = rsrc_words(static_cast<const char*>(p.v) + (row0 * p.vs + hoff) * ES,
                                     (uint32_t)(span - 1) * vsb + kD * ES);
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;  // (the low half of a flat LDS pointer)
        auto request = [&](int kt, int buf) {
            const uint32_t base = lds0 + (uint32_t)(buf * 2 * PLANE);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = wave + 4 * jj;
                const int row = kt + 8 * j + lr;
                const uint32_t c16 = (j & 1) ? c16o : c16e;
                ld_lds16_untracked(rkw, base + 1024u * (uint32_t)j, row_off(row, ksb) + c16);
                ld_lds16_untracked(rvw, base + PLANE + 1024u * (uint32_t)j, row_off(row, vsb) + c16);
            }
        };
        // padded: key kt + tid's keep byte (tid < 64; 0 past the sequence)
        auto keep_byte = [&](int kt) -> uint8_t {
            return (tid < kBN && kt + tid < L) ? p.keep[row0 + kt + tid] : (uint8_t)0;
        };
        const int nt = (L + kBN - 1) / kBN;
        uint8_t kbyte = 0;
        if constexpr (PADDED) kbyte = keep_byte(0);
        request(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // Q, requested before tile 0, has landed with it: a use of Q here puts
        // the compiler's own wait for it where it costs nothing (at the first
        // score product it would also wait for the next tile's loads).
        asm volatile("" : "+v"(qh0), "+v"(qh1));
        c = fold_scale(p.scale_log2, qh0, qh1, ql0, ql1);
        if constexpr (PADDED) {
            if (tid < kBN) sKeep[0][tid] = kbyte;
        }
        __syncthreads();
        auto step = [&](auto full_tag, int t) {
            const int kt = t * kBN, buf = t & 1;
            if (t + 1 < nt) {
                if constexpr (PADDED) kbyte = keep_byte(kt + kBN);
                request(kt + kBN, buf ^ 1);
            }
            if (wave_active) {
                const char* kbase = smem + buf * 2 * PLANE;
                compute(full_tag, kt, kbase, kbase + PLANE, sKeep[buf]);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the next tile has landed
            if constexpr (PADDED) {
                if (t + 1 < nt && tid < kBN) sKeep[buf ^ 1][tid] = kbyte;
            }
            __syncthreads();  // ... and every wave is done with this one
        };
        int t = 0;
        for (; (t + 1) * kBN <= L; ++t) step(std::true_type{}, t);
        if (t * kBN < L) step(std::false_type{}, t);
    }

    // ---- epilogue: O = acc / l, staged through LDS for row-contiguous stores --
    __syncthreads();  // every wave is done with the K / V tiles
    if (!wave_active) return;
    const float inv = online_inv(st);
    char* so = smem + wave * 16 * OUT_ROW;
    // lane holds O[r16][16db + 4g + i]
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        const f32x4 r = st.acc[db] * inv;
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
        __builtin_amdgcn_raw_buffer_store_b128(val, ro, row_off(qrow + wave * 16 + r, osb) + 16 * cix, 0, 0);
    }
}

// ---- LDS-resident kernel (bf16 input, sequences of up to kLdsMaxRows keys) --
//
// One workgroup = one (head, image, query split) with W = blockDim.x / 64
// waves, and every wave owns exactly one 16-row query block (block
// qs * W + wave).  The image's whole K and V for the head are copied from
// global memory straight into LDS by buffer loads that write LDS (gfx950
// buffer_load ... lds: no registers and no ALU work on the way), followed by
// ONE barrier; after it each wave runs its block over all keys with no
// further synchronisation, and waves without a block exit.  Compared with a
// tile loop this removes the per-tile barriers and register staging, reads K
// and V once per (image, head) and query split, and lets the last partial key
// tile skip its empty 16-key blocks.  K and V rows use the LDS operand layout
// above.
constexpr int kLdsRowAlign = 32;      // K / V rows in LDS: a multiple of the P.V k-depth
constexpr int kMaxWaves = 16;         // 16 query blocks: every block of kLdsMaxRows rows
constexpr int kLdsMaxRows = 256;      // 64 KiB of K + V: two workgroups per CU
constexpr size_t kLdsStageMax = 80 * 1024;  // K + V + keep data + output slots: two workgroups per CU

// TL: 0 = grid of (head, image, query split); tile list of 1 = whole pairs,
// 2 = 64-row query tiles.  NAT (gathered layout, few pairs): K and V are
// requested in natural order beside the keep bytes (see the gathered setup).
// STAGE (few pairs): the output goes out through per-wave LDS slots at byte
// p.out_stage as whole-row 16-byte chunks (see the epilogue).
template <bool OUT_F32, int LAYOUT, bool MULTI, int TL, bool NAT = false, bool STAGE = false>
__global__ __launch_bounds__(64 * kMaxWaves) void attn_lds_kernel(AttnParams p)
{
    constexpr bool PADDED = LAYOUT == kPadded;
    constexpr bool GATHERED = LAYOUT == kGathered;
    constexpr int OES = OUT_F32 ? 4 : 2;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ int s_wsum[4 * kMaxWaves];  // keep ranking: up to 4 planes x W waves

    constexpr bool TILES = TL != 0;
    static_assert(!TILES || LAYOUT == kRagged, "the tile list is built from cu_seqlens");
    int h = blockIdx.x, b = blockIdx.y;
    const int qs = blockIdx.z;
    const int nw = blockDim.x >> 6;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loops and addresses
    const int r16 = lane & 15, g = lane >> 4;

    // LDS: K rows [0, R), V rows [0, R), then the gathered layout's kept
    // positions (N ints) or the padded layout's keep bytes (N rounded up to 64).
    const int R = p.lds_rows;
    char* sK = lds;
    char* sV = lds + R * kRowBytes;
    int* s_pos = reinterpret_cast<int*>(lds + 2 * R * kRowBytes);
    uint8_t* s_keep = reinterpret_cast<uint8_t*>(lds + 2 * R * kRowBytes);

    int64_t row0;
    int L, qlo = qs * nw, qhi;  // this workgroup's query blocks: qlo + wave (+ k * qstride) < qhi
    bool natural = false;       // NAT: K, V and the wave's Q rows are already requested (every row kept)
    bf16x8 qa0 = {}, qa1 = {};  // the wave's Q^T operand (see load_q)
    if constexpr (TILES) {
        Item it;
        if (!workgroup_item<TL == 1>(p, it)) return;  // uniform over the workgroup
        h = it.h;
        b = it.b;
        row0 = it.row0;
        L = it.L;
        qlo = it.q0;
        qhi = it.q1;
    } else if constexpr (PADDED) {
        row0 = (int64_t)b * p.N;
        L = p.N;
        const int nkeep = (p.N + 63) & ~63;
        for (int n = tid; n < nkeep; n += blockDim.x) s_keep[n] = n < p.N ? p.keep[row0 + n] : 0;
    } else if constexpr (GATHERED) {
        row0 = (int64_t)b * p.N;
        // NAT (few pairs, and a bound max_seqlen >= N that admits an
        // unpruned image; the host checks N <= 4 * 64 * waves): the image's K
        // and V rows are requested in natural order beside its keep bytes,
        // and kept if every row is kept, one memory round trip instead of the
        // keep bytes' and then the gathered rows'.  Otherwise the gathered
        // loads below overwrite them.  With many pairs the extra traffic
        // costs more than the round trip saves.
        if constexpr (NAT) {
            const int nt = 64 * nw;
            const i32x4 rkeep = rsrc_words(p.keep + row0, (uint32_t)p.N);
            uint32_t kb[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) kb[k] = ld_u8_untracked(rkeep, (uint32_t)(tid + k * nt));
            const int64_t hoff0 = (int64_t)h * kD;
            const uint32_t ksb0 = (uint32_t)(p.ks * 2), vsb0 = (uint32_t)(p.vs * 2);
            const i32x4 rkw = rsrc_words(static_cast<const char*>(p.k) + (row0 * p.ks + hoff0) * 2,
                                         (uint32_t)(p.N - 1) * ksb0 + kRowBytes);
            const i32x4 rvw = rsrc_words(static_cast<const char*>(p.v) + (row0 * p.vs + hoff0) * 2,
                                         (uint32_t)(p.N - 1) * vsb0 + kRowBytes);
            const int nrb = ((p.N + kLdsRowAlign - 1) & ~(kLdsRowAlign - 1)) >> 3;
            const int lr = lane >> 3, slot = lane & 7;
            const uint32_t c16e = 16u * (uint32_t)(slot ^ swz(lr)), c16o = 16u * (uint32_t)(slot ^ swz(8 + lr));
            int issued = 0;
            for (int j = wave; j < nrb; j += nw) {
                const uint32_t c16 = (j & 1) ? c16o : c16e;
                const uint32_t row = (uint32_t)(8 * j + lr);
                ld_lds16_untracked(rkw, (uint32_t)(uintptr_t)(sK + 1024 * j), row * ksb0 + c16);
                ld_lds16_untracked(rvw, (uint32_t)(uintptr_t)(sV + 1024 * j), row * vsb0 + c16);
                issued += 2;
            }
            // the wave's first query block, as load_q would read it with every
            // row kept (rows past N read as zeros, as dropped rows do there)
            if (qlo + wave < (p.N + 15) >> 4) {
                const uint32_t qsb0 = (uint32_t)(p.qs * 2);
                const auto rq0 = make_rsrc(static_cast<const char*>(p.q) + (row0 * p.qs + hoff0) * 2,
                                           (uint32_t)(p.N - 1) * qsb0 + kRowBytes);
                const uint32_t off = (uint32_t)(16 * (qlo + wave) + r16) * qsb0 + 16 * g;
                qa0 = __builtin_bit_cast(bf16x8, ld16(rq0, off));
                qa1 = __builtin_bit_cast(bf16x8, ld16(rq0, off + 64));
                issued += 2;
            }
            wait_vm(issued);  // the keep bytes, issued first, have landed
            bool dropped = false;  // a position < N of this thread is dropped
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                vm_done(kb[k]);
                dropped = dropped || (tid + k * nt < p.N && kb[k] == 0u);
            }
            // every row kept: one barrier decides it, and no ranking is needed
            // (the rows are in natural order); else rank as below
            const bool wave_dropped = __ballot(dropped) != 0ull;  // (all lanes take part)
            if (lane == 0) s_wsum[wave] = wave_dropped;
            __syncthreads();
            natural = true;
            for (int w = 0; w < nw; ++w) natural = natural && s_wsum[w] == 0;
            natural = __builtin_amdgcn_readfirstlane((int)natural) != 0;  // uniform (read from LDS)
            if (!natural) {
                __syncthreads();  // every wave has read s_wsum before the ranking rewrites it
                L = dev::rank_kept_planes_loaded<4>(kb, s_pos, s_wsum, nw);
            } else {
                L = p.N;
            }
        } else {
            L = p.N <= 4 * 64 * nw ? dev::rank_kept_planes<4>(p.keep + row0, p.N, s_pos, s_wsum, nw)
                                   : dev::rank_kept_waves(p.keep + row0, p.N, s_pos, s_wsum, nw);
        }
        L = min(__builtin_amdgcn_readfirstlane(L), p.max_len);  // (a workgroup reduction: uniform)
        if (p.zero_dropped && qs == 0) zero_dropped_head<OUT_F32>(p, row0, h);
    } else {
        const int s = min(max(p.cu[b], 0), p.total_rows);
        const int e = min(max(p.cu[b + 1], s), p.total_rows);
        row0 = s;
        L = min(e - s, p.max_len);
    }
    if constexpr (!TILES) qhi = (L + 15) >> 4;  // 16-row query blocks
    if (qlo >= qhi) return;                      // uniform over the workgroup

    const int64_t hoff = (int64_t)h * kD;
    const int span = GATHERED ? p.N : L;
    const uint32_t qsb = (uint32_t)(p.qs * 2), ksb = (uint32_t)(p.ks * 2), vsb = (uint32_t)(p.vs * 2),
                   osb = (uint32_t)(p.os * OES);
    const auto rq = make_rsrc(static_cast<const char*>(p.q) + (row0 * p.qs + hoff) * 2,
                              (uint32_t)(span - 1) * qsb + kRowBytes);
    const auto rk = make_rsrc(static_cast<const char*>(p.k) + (row0 * p.ks + hoff) * 2,
                              (uint32_t)(span - 1) * ksb + kRowBytes);
    const auto rv = make_rsrc(static_cast<const char*>(p.v) + (row0 * p.vs + hoff) * 2,
                              (uint32_t)(span - 1) * vsb + kRowBytes);
    auto row_off = [&](int r, uint32_t stride) -> uint32_t {
        if constexpr (GATHERED) {
            if (NAT && natural) return r < L ? (uint32_t)r * stride : kDropOffset;  // rank r is row r
            return r < L ? (uint32_t)s_pos[r] * stride : kDropOffset;
        } else {
            return (uint32_t)r * stride;
        }
    };

    // ---- K, V -> LDS: one instruction moves 8 rows (1 KiB); lane l writes
    // LDS bytes [16 l, 16 l + 16) of the block, i.e. slot l & 7 of row l >> 3,
    // so it fetches the global chunk that the permutation puts in that slot
    // (the permutation repeats every 16 rows: one lane offset per row parity
    // of the 8-row block).  Rows past the sequence, up to the multiple of 32,
    // read as zeros.
    if (!NAT || !natural) {
        // (NAT: the natural-order loads into the same LDS rows have landed
        // first; by now they have, so the wait costs nothing)
        if constexpr (NAT) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const int nrb = ((L + kLdsRowAlign - 1) & ~(kLdsRowAlign - 1)) >> 3;
        const int lr = lane >> 3, slot = lane & 7;
        const uint32_t c16e = 16u * (uint32_t)(slot ^ swz(lr)), c16o = 16u * (uint32_t)(slot ^ swz(8 + lr));
        for (int j = wave; j < nrb; j += nw) {
            const int row = 8 * j + lr;
            const uint32_t c16 = (j & 1) ? c16o : c16e;
            // (offsets computed first: a lambda call inside the builtin's
            // argument list stops clang's host pass from emitting the stub)
            const uint32_t koff = row_off(row, ksb) + c16, voff = row_off(row, vsb) + c16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(sK + 1024 * j), 16, koff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(sV + 1024 * j), 16, voff, 0, 0, 0);
        }
    }

    // Q^T as the B operand of S^T = K Q^T: lane holds query row r16 of the
    // block, d = 8g..8g+7 and 32+8g..32+8g+7.  The wave's blocks are
    // qs * W + wave + k * gridDim.z * W: one of them, or (MULTI) one or more.
    int qb = qlo + wave;
    const int qstride = gridDim.z * nw;
    auto load_q = [&](int blk) {
        const uint32_t off = row_off(16 * blk + r16, qsb) + 16 * g;
        qa0 = __builtin_bit_cast(bf16x8, ld16(rq, off));
        qa1 = __builtin_bit_cast(bf16x8, ld16(rq, off + 64));
    };
    if (qb < qhi && !(NAT && natural)) load_q(qb);
    __builtin_amdgcn_s_waitcnt(0);  // every load of this wave has landed (LDS included)
    __syncthreads();
    if (qb >= qhi) return;

    // per-lane LDS offsets of the K and V operands inside a 16-row block
    const uint32_t koff0 = k_operand_offset(r16, g);
    const uint32_t koff1 = koff0 ^ 64u;
    uint32_t voff[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] = v_operand_offset(r16, g, db);

    const auto ro = make_rsrc(static_cast<char*>(p.o) + (row0 * p.os + hoff) * OES,
                              (uint32_t)(span - 1) * osb + kD * OES);
    for (;;) {  // the wave's query blocks
        bf16x8 unused0 = {}, unused1 = {};
        const float c = fold_scale(p.scale_log2, qa0, qa1, unused0, unused1);
        Online st;
        online_init(st);

        // One tile at key kt; FULL: all 64 keys present (no key-range masking).
        // The full tiles run in one loop and the partial last tile after it.
        auto tile = [&](auto full_tag, const int kt) {
            constexpr bool FULL = decltype(full_tag)::value;
            const int nk = min(kBN, L - kt);
            const char* kbase = sK + kt * kRowBytes;
            const char* vbase = sV + kt * kRowBytes;
            // ---- S^T = K Q^T over the 16-key blocks that hold keys ----------
            f32x4 s[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                if (FULL || kb == 0 || 16 * kb < nk) {
                    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kbase + 2048 * kb + koff0);
                    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kbase + 2048 * kb + koff1);
                    s[kb] = mfma(a0, qa0, f32x4{0.f, 0.f, 0.f, 0.f});
                    s[kb] = mfma(a1, qa1, s[kb]);
                } else {
                    s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};  // absent keys, masked below
                }
            }
            online_probs<FULL, PADDED>(s, nk, s_keep + kt, g, c, kt == 0, st);
            // ---- O^T += V^T P^T, 32 keys per MFMA ----------------------------
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                if (FULL || cc * 32 < nk) {
                    bf16x8 ph, pl;
                    p_operand(s, cc, ph, pl, st);
#pragma unroll
                    for (int db = 0; db < 4; ++db) {
                        const bf16x4 v0 = ld_tr4(vbase + 4096 * cc + voff[db]);
                        const bf16x4 v1 = ld_tr4(vbase + 4096 * cc + 2048 + voff[db]);
                        const bf16x8 av = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                        st.acc[db] = mfma(av, ph, st.acc[db]);
                        st.acc[db] = mfma(av, pl, st.acc[db]);
                    }
                }
            }
        };
        if constexpr (MULTI) {
            // long sequences: the full tiles unrolled (at most kLdsMaxRows / kBN
            // of them), so that every LDS offset is an immediate and no address
            // arithmetic runs per tile (fewer VALU instructions and registers;
            // the short-sequence launches keep the loop's smaller code)
#pragma unroll
            for (int t = 0; t < kLdsMaxRows / kBN; ++t)
                if ((t + 1) * kBN <= L) tile(std::true_type{}, t * kBN);
            const int kt = L & ~(kBN - 1);  // the partial last tile, if any
            if (kt < L) tile(std::false_type{}, kt);
        } else {
            int kt = 0;
            for (; kt + kBN <= L; kt += kBN) tile(std::true_type{}, kt);
            if (kt < L) tile(std::false_type{}, kt);
        }

        // ---- epilogue: O = acc / l; lane holds O[16 qb + r16][16 db + 4g + i] ----
        const float inv = online_inv(st);
        if constexpr (STAGE) {
            // The block's 16 output rows go through the wave's own LDS slot
            // and out as 16-byte chunks, 128 contiguous bytes per 8 lanes (the
            // accumulator layout alone stores 16 rows x 32 or 64 bytes per
            // instruction).  Chunk c of slot row r sits at c ^ (r mod NCH) so
            // that both the accumulator writes and the row reads spread over
            // the banks.  The slot is rewritten only after this wave's reads
            // of it (its next block), which LDS orders within a wave.
            constexpr int RB = kD * OES;  // bytes per output row: 128 (bf16) or 256 (fp32)
            constexpr int NCH = RB / 16;  // 16-byte chunks per row
            char* so = lds + p.out_stage + wave * 16 * RB;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const f32x4 r = st.acc[db] * inv;
                if constexpr (OUT_F32) {
                    *reinterpret_cast<f32x4*>(so + r16 * RB + 16 * ((4 * db + g) ^ (r16 & (NCH - 1)))) = r;
                } else {
                    bf16x4 o4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o4[i] = static_cast<__bf16>(r[i]);
                    *reinterpret_cast<bf16x4*>(so + r16 * RB + 16 * ((2 * db + (g >> 1)) ^ (r16 & (NCH - 1))) +
                                               8 * (g & 1)) = o4;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's slot writes are done
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < 16 * NCH / 64; ++k) {
                const int row = lane / NCH + k * (64 / NCH), ch = lane % NCH;
                const u32x4 val = *reinterpret_cast<const u32x4*>(so + row * RB + 16 * (ch ^ (row & (NCH - 1))));
                __builtin_amdgcn_raw_buffer_store_b128(val, ro, row_off(16 * qb + row, osb) + 16u * (uint32_t)ch, 0, 0);
            }
        } else if constexpr (!OUT_F32) {
            // bf16: lane (r16, g) holds columns 16 db + 4g .. + 3 of its row.  One
            // v_permlane16_swap per register pair exchanges between lanes l and
            // l ^ 16 (groups g and g ^ 1) so that an even-g lane ends with
            // columns 16 db + 4g .. + 7 of db = 0 and 2, an odd-g lane those of
            // db = 1 and 3 (from 16 db + 4 (g - 1)): two 16-byte stores per lane,
            // each instruction writing 64 contiguous bytes of 16 rows.
            uint32_t w[4][2];
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const f32x4 r = st.acc[db] * inv;
                bf16x4 o4;
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = static_cast<__bf16>(r[i]);
                const u32x2 u = __builtin_bit_cast(u32x2, o4);
                w[db][0] = u[0];
                w[db][1] = u[1];
            }
            u32x4 ch[2];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const auto s0 = __builtin_amdgcn_permlane16_swap(w[2 * pr][0], w[2 * pr + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(w[2 * pr][1], w[2 * pr + 1][1], false, false);
                ch[pr] = u32x4{s0[0], s1[0], s0[1], s1[1]};
            }
            const uint32_t orow = row_off(16 * qb + r16, osb);
            const uint32_t col = 16u * (uint32_t)(g & 1) + 4u * (uint32_t)(g & 2);
            __builtin_amdgcn_raw_buffer_store_b128(ch[0], ro, orow + col * 2u, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(ch[1], ro, orow + (32u + col) * 2u, 0, 0);
        } else {
            const uint32_t orow = row_off(16 * qb + r16, osb);  // fp32: 16 bytes per lane already
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const f32x4 r = st.acc[db] * inv;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r), ro,
                                                       orow + (uint32_t)(16 * db + 4 * g) * OES, 0, 0);
            }
        }
        if constexpr (!MULTI) break;  // (single-block launches: one block per wave)
        qb += qstride;
        if (qb >= qhi) break;
        load_q(qb);
    }
}

// LDS bytes of attn_lds_kernel for a launch, or 0 where it does not apply
// (fp32 input, or more than 64 KiB: K + V of up to kLdsMaxRows rows plus the
// layout's keep data, so that at least two workgroups share a CU).
size_t lds_kernel_bytes(const AttnParams& p, bool in_f32, int layout)
{
    if (in_f32) return 0;
    const int rows = (p.max_len + kLdsRowAlign - 1) & ~(kLdsRowAlign - 1);
    if (rows > kLdsMaxRows) return 0;
    size_t bytes = (size_t)2 * rows * kRowBytes;
    if (layout == kGathered) bytes += sizeof(int) * (size_t)p.N;
    if (layout == kPadded) bytes += (size_t)((p.N + 63) & ~63);
    return bytes <= 64 * 1024 ? bytes : 0;
}

template <bool OUT_F32, bool MULTI, bool STAGE = false>
void launch_lds_layout(const AttnParams& p, int layout, dim3 grid, dim3 block, size_t lds_bytes,
                       hipStream_t st)
{
    if (layout == kPadded)
        hipLaunchKernelGGL((attn_lds_kernel<OUT_F32, kPadded, MULTI, 0, false, STAGE>), grid, block, lds_bytes, st, p);
    else if (layout == kGathered && !MULTI && p.natural_first && p.N <= 4 * (int)block.x)
        hipLaunchKernelGGL((attn_lds_kernel<OUT_F32, kGathered, false, 0, true, STAGE>), grid, block, lds_bytes, st, p);
    else if (layout == kGathered)
        hipLaunchKernelGGL((attn_lds_kernel<OUT_F32, kGathered, MULTI, 0, false, STAGE>), grid, block, lds_bytes, st, p);
    else if (p.tl_kt == 0)
        hipLaunchKernelGGL((attn_lds_kernel<OUT_F32, kRagged, MULTI, 0, false, STAGE>), grid, block, lds_bytes, st, p);
    else if (grid.z == 1)  // tile list, many pairs (or few with one query split): whole (image, head) pairs
        hipLaunchKernelGGL((attn_lds_kernel<OUT_F32, kRagged, MULTI, 1, false, STAGE>),
                           dim3(tile_list_grid(p.B, p.H, p.tl_kt, true)), block, lds_bytes, st, p);
    else  // tile list, few pairs: the query splits are 64-row query tiles
        hipLaunchKernelGGL((attn_lds_kernel<OUT_F32, kRagged, false, 2, false, STAGE>),
                           dim3(tile_list_grid(p.B, p.H, p.tl_kt, false)), block, lds_bytes, st, p);
}

// Compute units of the current device (cached per device; 0 if the query fails).
int device_cus()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cached[dev] = n;
    return n;
}

template <bool OUT_F32>
void launch_lds_variant(AttnParams p, int layout, size_t lds_bytes, hipStream_t st)
{
    // With many (image, head) pairs a workgroup holds all of an image's 16-row
    // query blocks (K and V are read once): one block per wave up to 8 blocks,
    // two per wave beyond (so that two workgroups fit a CU and one's K / V load
    // overlaps the other's compute).  With few pairs the blocks are split over
    // gridDim.z workgroups of at most 4 waves, one block each, so that more CUs
    // share the work.  A tile-list launch (p.tl_kt > 0, ragged layout) keeps
    // these workgroup shapes, its items being the whole pairs, or the 64-row
    // query tiles (4 blocks on 4 waves) with few pairs.  Ragged launches with
    // fewer than four pairs per CU split images of more than 8 blocks in two
    // workgroups of one block per wave: the last long images then end sooner
    // (DeiT-B with ragged lengths in [20, 197]: 5% less time; more splits or
    // the gathered and padded layouts, which rank or mask the keep row in
    // every workgroup, measured slower).
    const int nqb = (p.max_len + 15) / 16;
    const int64_t npairs = (int64_t)p.B * p.H;
    const bool many = npairs >= 256;
    const bool halves = layout == kRagged && p.tl_kt == 0 && many && nqb > 8 && npairs < 4 * (int64_t)device_cus();
    int waves;
    if (halves)
        waves = (nqb + 1) / 2;
    else if (many)  // one block per wave up to 8, else two
        waves = nqb <= 8 ? nqb : (nqb + 1) / 2;
    else
        waves = min(nqb, 4);
    const int splits = halves ? 2 : many ? 1 : (nqb + waves - 1) / waves;
    p.lds_rows = (p.max_len + kLdsRowAlign - 1) & ~(kLdsRowAlign - 1);
    if (p.tl_kt > 0 && !many) waves = 4;
    // With few pairs (the latency-bound small batches, whose last stores end
    // the launch) the output goes through per-wave LDS slots (16 rows each)
    // after K, V and the layout's keep data: B = 1-4 attention and the
    // one-launch pass 4-5% sooner.  With many pairs the extra LDS traffic
    // cost more than the whole-row stores saved (the headline batch 1.5%
    // slower, the unpruned one-launch pass 17%).
    const size_t base = (lds_bytes + 15) & ~(size_t)15;
    const size_t staged = base + (size_t)waves * 16 * kD * (OUT_F32 ? 4 : 2);
    const dim3 grid(p.H, p.B, splits), block(64 * waves);
    if (!many && staged <= kLdsStageMax) {  // (few pairs: one block per wave)
        p.out_stage = (int32_t)base;
        launch_lds_layout<OUT_F32, false, true>(p, layout, grid, block, staged, st);
    } else if (waves * splits >= nqb) {
        launch_lds_layout<OUT_F32, false>(p, layout, grid, block, lds_bytes, st);
    } else {
        launch_lds_layout<OUT_F32, true>(p, layout, grid, block, lds_bytes, st);
    }
}

template <bool IN_F32, bool OUT_F32>
void launch_variant(const AttnParams& p, int layout, hipStream_t st)
{
    if (p.tl_kt > 0) {  // the tile list's items: one 64-row q-tile's worth of blocks
        const dim3 grid(tile_list_grid(p.B, p.H, p.tl_kt, false)), block(kThreads);
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kRagged, true>), grid, block, 0, st, p);
        return;
    }
    // one slot per (pair, q-tile); blocks of 8 * kPairBlock pairs
    const int64_t nblk = ((int64_t)p.H * p.B + 8 * kPairBlock - 1) / (8 * kPairBlock);
    const int64_t gy = std::min<int64_t>(nblk, kMaxGridY);
    const dim3 grid((unsigned)(8 * kPairBlock * p.n_qtiles), (unsigned)gy,
                    (unsigned)((nblk + gy - 1) / gy)), block(kThreads);
    if (layout == kPadded)
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kPadded, false>), grid, block, 0, st, p);
    else if (layout == kGathered)
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kGathered, false>), grid, block,
                           sizeof(int) * (size_t)p.N, st, p);
    else
        hipLaunchKernelGGL((attn_kernel<IN_F32, OUT_F32, kRagged, false>), grid, block, 0, st, p);
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
    p.max_len = layout == kPadded ? N : max_seqlen;
    p.n_qtiles = (p.max_len + kBM - 1) / kBM;
    p.zero_dropped = (flags & RAG_UNPACK_ZERO_DROPPED) ? 1 : 0;
    p.lds_rows = 0;
    p.out_stage = 0;
    p.tl_kt = (layout == kRagged && (flags & kAttnTileList)) ? (p.max_len + 63) / 64 : 0;
    p.natural_first = (layout == kGathered && max_seqlen >= N && (int64_t)B * H < 256) ? 1 : 0;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.h_magic = H > 1 ? (uint32_t)((1ull << 32) / (uint64_t)H + 1ull) : 0u;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool in_f32 = in_dtype == RAG_DTYPE_F32, out_f32 = out_dtype == RAG_DTYPE_F32;
    const size_t lds_bytes = lds_kernel_bytes(p, in_f32, layout);
    if (lds_bytes) {
        if (out_f32) launch_lds_variant<true>(p, layout, lds_bytes, st);
        else launch_lds_variant<false>(p, layout, lds_bytes, st);
    } else if (in_f32 && out_f32) launch_variant<true, true>(p, layout, st);
    else if (in_f32) launch_variant<true, false>(p, layout, st);
    else if (out_f32) launch_variant<false, true>(p, layout, st);
    else launch_variant<false, false>(p, layout, st);
    return (int)hipGetLastError();
}

}  // namespace rag
