// pack.hip -- token packing and write-back for ragged ViT attention on gfx950.
//
// Pack ("Triton Ragged Attention 與 pack-attend-unpack", agents-report.net,
// section 方法概覽, fused token packing): from the keep mask, build the per-image
// offsets cu_seqlens and the destination (gather) index, then copy the kept
// token rows into one flat buffer.  Unpack (same section, write-back): copy each
// packed row back to its batch position.
//
// One launch each.
//
// Pack: workgroup (b, s) copies column slice s (a contiguous range of 16-byte
// vectors, the same for every row) of ALL kept rows of image b, so every
// workgroup of an image with kept rows has work whatever the prune rate, and
// the grid (B x S, S chosen so that about 1024 workgroups cover the batch) is
// filled in one dispatch round.
//   1. ranks inside image b: the image's N keep bytes are read once; a 64-lane
//      ballot + popcount gives each kept position its rank, and the kept
//      positions are listed by rank in LDS;
//   2. the offset of image b (number of kept tokens in images 0..b-1) is
//      counted from 16-byte words of the keep mask; those loads are issued
//      right after the image's keep bytes, so they travel during the ranking
//      (each workgroup recounts the prefix, at most B*N bytes that stay in L2:
//      no atomics and no inter-workgroup waits, so the result is
//      deterministic);
//   3. the slice's source rows are requested (up to kUnroll 16-byte loads per
//      lane in flight), the prefix count is reduced, and the rows are stored.
// Unpack: workgroup (b, c) serves packed rows [c*R, c*R + R) of image b; the
// chunk index is the slowest grid dimension, so the first chunk of every image
// is dispatched before the later chunks, which pruned images mostly lack.
// All row traffic goes through buffer resources: a lane past the end gets an
// offset outside the resource, so its load reads zero and its store is dropped
// by the hardware; no predicated register arrays are needed.
// An extra workgroup row (b == B) computes max_b L_b when asked for.
#include <hip/hip_runtime.h>

#include "rag_device.h"
#include "rag_internal.h"

namespace rag {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;                           // unpack: 16-byte vectors per lane per batch
constexpr int kBatch = kThreads * kUnroll;           // vectors per workgroup per batch
constexpr int kPackUnroll = 4;                       // pack: 16-byte vectors per lane per batch
constexpr int kPrefixLoads = 8;                      // keep-mask words per lane per round
constexpr int kPackTargetGroups = 768;               // workgroups a pack launch aims for
using dev::kDropOffset;
using dev::ld16;
using dev::make_rsrc;
using dev::st16;
using dev::u32x4;

struct PackParams {
    const uint8_t* keep;
    const uint8_t* src;
    uint8_t* packed;
    int32_t* cu;
    int32_t* gather;
    int32_t* max_len;
    const int32_t* cu_in;      // re-pack: the input's images (packed rows)
    const int32_t* gather_in;  // re-pack: the input rows' original batch rows
    int64_t src_stride;
    int64_t packed_stride;
    // N: rows per image (pack) or the host bound of rows per input image (re-pack)
    int32_t B, N, row_vecs, slice_vecs;  // slice s: vectors [s*slice_vecs, ...) of a row
    int32_t total_rows;                  // re-pack: rows of the input (cu_in is clamped to it)
    uint32_t n_magic;                    // floor(2^32 / N) + 1
};

struct UnpackParams {
    const uint8_t* packed;
    uint8_t* dst;
    const int32_t* cu;
    const int32_t* gather;
    int64_t packed_stride;
    int64_t dst_stride;
    int32_t B, N, row_vecs, rows, zero_dropped;
};

// Number of nonzero bytes in a 32-bit word: bit 7 of each byte of
// ((w & 0x7f..) + 0x7f..) | w is set exactly when that byte is nonzero, and the
// addition cannot carry across bytes.
__device__ __forceinline__ int nonzero_bytes(uint32_t w)
{
    const uint32_t y = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w;
    return __popc(y & 0x80808080u);
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
    return v;
}

// Sum over the workgroup; every thread gets the total.  `red` holds kWaves ints.
__device__ __forceinline__ int block_sum(int v, int* red)
{
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    __syncthreads();
    return t;
}

// Kept tokens in keep[0, nbytes), counted by the workgroup from 16-byte words
// (kPrefixLoads per lane per round) through a buffer resource over the full
// words; words past it read as zero.  prefix_load issues a round, prefix_count
// adds up the loaded round, the further rounds and the tail bytes, and reduces
// over the workgroup (every thread gets the total).
struct Prefix {
    __amdgpu_buffer_rsrc_t rk;
    uint32_t nwords;
    u32x4 x[kPrefixLoads];
};

__device__ __forceinline__ void prefix_load(Prefix& pf, uint32_t w0)
{
#pragma unroll
    for (int j = 0; j < kPrefixLoads; ++j) pf.x[j] = ld16(pf.rk, (w0 + threadIdx.x + j * kThreads) << 4);
}

__device__ __forceinline__ int prefix_words(const Prefix& pf)
{
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kPrefixLoads; ++j)
        cnt += nonzero_bytes(pf.x[j][0]) + nonzero_bytes(pf.x[j][1]) + nonzero_bytes(pf.x[j][2]) +
               nonzero_bytes(pf.x[j][3]);
    return cnt;
}

__device__ __forceinline__ Prefix prefix_begin(const uint8_t* keep, int64_t nbytes)
{
    Prefix pf;
    pf.nwords = (uint32_t)(nbytes >> 4);
    pf.rk = make_rsrc(keep, pf.nwords << 4);
    prefix_load(pf, 0);
    return pf;
}

__device__ int prefix_count(Prefix& pf, const uint8_t* keep, int64_t nbytes, int* red)
{
    int cnt = prefix_words(pf);
    for (uint32_t w0 = kThreads * kPrefixLoads; w0 < pf.nwords; w0 += kThreads * kPrefixLoads) {
        prefix_load(pf, w0);
        cnt += prefix_words(pf);
    }
    const uint32_t tail0 = pf.nwords << 4;
    if ((int64_t)threadIdx.x < nbytes - tail0) cnt += keep[tail0 + threadIdx.x] != 0;
    return block_sum(cnt, red);
}

// max_b L_b, by the extra workgroup row.  Per-image counts are accumulated in
// LDS (cnt[], `window` ints) for windows of images at a time.
__device__ void max_length_pass(const PackParams& p, int* cnt, int window, int* red)
{
    const int tid = threadIdx.x;
    const uint32_t N = (uint32_t)p.N;
    int best = 0;
    for (int img0 = 0; img0 < p.B; img0 += window) {
        const int nimg = min(window, p.B - img0);
        for (int i = tid; i < nimg; i += kThreads) cnt[i] = 0;
        __syncthreads();
        const uint32_t lo = (uint32_t)img0 * N, hi = (uint32_t)(img0 + nimg) * N;
        const uint32_t wlo = (lo + 15u) >> 4, whi = hi >> 4;  // full 16-byte words
        if (N >= 16) {
            // kPrefixLoads words per lane in flight, then counted
            const uint4* kw = reinterpret_cast<const uint4*>(p.keep);
            for (uint32_t w0 = wlo; w0 < whi; w0 += kThreads * kPrefixLoads) {
                uint4 x[kPrefixLoads];
#pragma unroll
                for (int j = 0; j < kPrefixLoads; ++j) {
                    const uint32_t w = w0 + tid + j * kThreads;
                    x[j] = w < whi ? kw[w] : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int j = 0; j < kPrefixLoads; ++j) {
                    const uint32_t w = w0 + tid + j * kThreads;
                    if (w >= whi) continue;
                    const uint32_t P = w << 4;
                    // image of the word's first byte: P / N by a multiply-high
                    // with n_magic = floor(2^32 / N) + 1 (an over-estimate by
                    // less than one, corrected once)
                    uint32_t f = __umulhi(P, p.n_magic);
                    f -= (f * N > P) ? 1u : 0u;
                    // bytes of the word that belong to image f; the rest to f + 1
                    const int nfirst = (int)min((f + 1u) * N - P, 16u);
                    const uint32_t words[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
                    int first = 0, second = 0;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int fb = nfirst - 4 * k;  // bytes of dword k in image f
                        const uint32_t m = fb >= 4 ? 0xFFFFFFFFu : (fb <= 0 ? 0u : (1u << (8 * fb)) - 1u);
                        first += nonzero_bytes(words[k] & m);
                        second += nonzero_bytes(words[k] & ~m);
                    }
                    if (first) atomicAdd(&cnt[f - img0], first);
                    if (second) atomicAdd(&cnt[f + 1u - img0], second);
                }
            }
        } else {
            for (uint32_t i = (wlo << 4) + tid; i < (whi << 4); i += kThreads)
                if (p.keep[i]) atomicAdd(&cnt[i / N - img0], 1);
        }
        // bytes outside the full words: the head [lo, 16*wlo) and tail [16*whi, hi)
        const uint32_t head_end = min(wlo << 4, hi);
        for (uint32_t i = lo + tid; i < head_end; i += kThreads)
            if (p.keep[i]) atomicAdd(&cnt[i / N - img0], 1);
        const uint32_t tail_start = max(whi << 4, head_end);
        for (uint32_t i = tail_start + tid; i < hi; i += kThreads)
            if (p.keep[i]) atomicAdd(&cnt[i / N - img0], 1);
        __syncthreads();
        for (int i = tid; i < nimg; i += kThreads) best = max(best, cnt[i]);
        __syncthreads();
    }
    best = wave_max(best);
    if ((tid & 63) == 0) red[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        int m = 0;
        for (int w = 0; w < kWaves; ++w) m = max(m, red[w]);
        p.max_len[0] = m;
    }
}

// RAGGED_IN = false: pack.  Image b's source rows are b*N .. b*N+N-1 and its
// keep bytes keep[b*N ..]; gather entries are the source rows.
// RAGGED_IN = true: re-pack (a later pruning stage).  Image b's source rows
// are the packed rows cu_in[b] .. cu_in[b+1]-1 (at most N of them) with one
// keep byte per packed row; gather entries are gather_in of the kept rows.
// Either way the offset of image b counts the keep bytes before its first
// row, and the rest is the same compaction.
template <bool RAGGED_IN>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackParams p)
{
    extern __shared__ int s_pos[];  // max(N, 256) ints
    __shared__ int s_red[kWaves];
    const int tid = threadIdx.x;
    const int b = blockIdx.x, sl = blockIdx.y;
    if (!RAGGED_IN && b == p.B) {
        if (sl == 0) max_length_pass(p, s_pos, max(p.N, kThreads), s_red);
        return;
    }
    int64_t img_row0;
    int n_in;  // rows of the image in the input
    if constexpr (RAGGED_IN) {
        const int s = min(max(p.cu_in[b], 0), p.total_rows);
        const int e = min(max(p.cu_in[b + 1], s), p.total_rows);
        img_row0 = s;
        n_in = min(e - s, p.N);
    } else {
        img_row0 = (int64_t)b * p.N;
        n_in = p.N;
    }
    // The image's keep bytes are requested first and the prefix words after
    // them, so the ranking waits for the former only.
    int L;
    Prefix pf;
    if (p.N <= kThreads) {
        // (a buffer load: positions past the image read as zero, no branch)
        const uint32_t kbyte = __builtin_amdgcn_raw_buffer_load_b8(
            make_rsrc(p.keep + img_row0, (uint32_t)n_in), (uint32_t)tid, 0, 0);
        pf = prefix_begin(p.keep, img_row0);
        L = dev::rank_kept_preloaded(kbyte != 0u, s_pos, s_red, kWaves);
    } else {
        pf = prefix_begin(p.keep, img_row0);
        L = dev::rank_kept(p.keep + img_row0, n_in, s_pos, s_red);
    }
    // L and the offset below come out of workgroup reductions through LDS, so
    // they are equal in every lane, but the compiler cannot tell: read from
    // lane 0 they are scalars, and the destination's buffer resource built
    // from them stays in scalar registers (otherwise every row store runs in
    // a loop over the distinct resources of the wave's lanes).
    L = __builtin_amdgcn_readfirstlane(L);
    if (L == 0 && sl > 0) return;  // uniform; slice 0 still writes cu

    // this slice: vectors [c0, c0 + w) of every row.  Lane tid starts at
    // vector tid of the slice (row tid / w, column tid % w) and steps by
    // kThreads vectors at a time: a cursor (row, col) advanced by (dr, dc) with
    // a carry, so no per-vector division.  A vector on a row >= L re-reads
    // row 0 and its store gets an offset outside the destination.
    const int c0 = sl * p.slice_vecs;
    const int w = min(p.slice_vecs, p.row_vecs - c0);
    const int dr = kThreads / w, dc = kThreads - dr * w;
    const uint32_t sstride = (uint32_t)p.src_stride, pstride = (uint32_t)p.packed_stride;
    const auto rs = make_rsrc(p.src + img_row0 * p.src_stride, (uint32_t)(n_in * p.src_stride));
    auto advance = [&](int& r, int& col) {
        r += dr;
        col += dc;
        if (col >= w) {
            col -= w;
            r += 1;
        }
    };
    // Loads the batch starting at cursor (r, col): all LDS position reads
    // first, then all row loads (one LDS and one memory round trip).
    auto load_batch = [&](int r, int col, u32x4 (&dst)[kPackUnroll]) {
        int pos[kPackUnroll];
        uint32_t cb[kPackUnroll];
#pragma unroll
        for (int j = 0; j < kPackUnroll; ++j) {
            pos[j] = s_pos[r < L ? r : 0];
            cb[j] = 16u * (uint32_t)(c0 + col);
            advance(r, col);
        }
#pragma unroll
        for (int j = 0; j < kPackUnroll; ++j) dst[j] = ld16(rs, (uint32_t)pos[j] * sstride + cb[j]);
    };
    int r = tid / w, col = tid - (tid / w) * w;  // cursor of the current batch
    u32x4 x[kPackUnroll];
    load_batch(r, col, x);

    const int offset = __builtin_amdgcn_readfirstlane(prefix_count(pf, p.keep, img_row0, s_red));
    if (sl == 0) {
        if (tid == 0) {
            p.cu[b + 1] = offset + L;
            if (b == 0) p.cu[0] = 0;
        }
        for (int t = tid; t < L; t += kThreads) {
            if constexpr (RAGGED_IN) p.gather[offset + t] = p.gather_in[img_row0 + s_pos[t]];
            else p.gather[offset + t] = (int32_t)(img_row0 + s_pos[t]);
        }
    }
    if (L == 0) return;
    const auto rd = make_rsrc(p.packed + (int64_t)offset * p.packed_stride, (uint32_t)L * pstride);
    const int total = L * w;
    // A step requests the next batch into `nxt` and then stores the batch in
    // `cur`, with no branch between the two, so the compiler's waits before
    // the stores cover only `cur`'s loads.  The two register sets alternate
    // between steps (no copy of one into the other), and the last batch is
    // stored on its own.
    constexpr int kB = kPackUnroll * kThreads;
    auto store = [&](const u32x4 (&cur)[kPackUnroll]) {
#pragma unroll
        for (int j = 0; j < kPackUnroll; ++j) {
            st16(cur[j], rd, r < L ? (uint32_t)r * pstride + 16u * (uint32_t)(c0 + col) : kDropOffset);
            advance(r, col);
        }
    };
    auto step = [&](const u32x4 (&cur)[kPackUnroll], u32x4 (&nxt)[kPackUnroll]) {
        int rn = r, cn = col;
#pragma unroll
        for (int j = 0; j < kPackUnroll; ++j) advance(rn, cn);  // next batch's cursor
        load_batch(rn, cn, nxt);
        store(cur);
    };
    u32x4 y[kPackUnroll];
    for (int vb = 0;; vb += 2 * kB) {  // vb: the first vector of the batch in x (uniform)
        if (vb + kB >= total) {
            store(x);
            break;
        }
        step(x, y);
        if (vb + 2 * kB >= total) {
            store(y);
            break;
        }
        step(y, x);
    }
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackParams p)
{
    __shared__ uint32_t s_kept[RAG_MAX_N / 32];
    const int tid = threadIdx.x;
    const int b = blockIdx.x, c = blockIdx.y;  // chunk slowest: chunk 0 of every image first
    const int64_t cap = (int64_t)p.B * p.N;
    const int64_t start = min(max((int64_t)p.cu[b], (int64_t)0), cap);
    const int64_t end = min(max((int64_t)p.cu[b + 1], start), cap);
    const int L = (int)min(end - start, (int64_t)p.N);
    const int64_t img_row0 = (int64_t)b * p.N;
    const auto rdst = make_rsrc(p.dst + img_row0 * p.dst_stride, (uint32_t)(p.N * p.dst_stride));

    if (p.zero_dropped) {
        const int nwords = (p.N + 31) >> 5;
        for (int i = tid; i < nwords; i += kThreads) s_kept[i] = 0u;
        __syncthreads();
        for (int t = tid; t < L; t += kThreads) {
            const int64_t g = (int64_t)p.gather[start + t] - img_row0;
            if (g >= 0 && g < p.N) atomicOr(&s_kept[g >> 5], 1u << (g & 31));
        }
        __syncthreads();
        // this chunk zeroes the dropped positions in [c*rows, c*rows + rows)
        const int n0 = c * p.rows, n1 = min(n0 + p.rows, p.N);
        const int total = (n1 > n0 ? n1 - n0 : 0) * p.row_vecs;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (int v = tid; v < total; v += kThreads) {
            const int r = v / p.row_vecs;
            const int col = v - r * p.row_vecs;
            const int n = n0 + r;
            const bool dropped = !((s_kept[n >> 5] >> (n & 31)) & 1u);
            st16(zero, rdst, dropped ? (uint32_t)n * (uint32_t)p.dst_stride + 16u * col : kDropOffset);
        }
    }

    const int r0 = c * p.rows;
    const int nr = min(p.rows, L - r0);
    if (nr <= 0) return;
    const int total = nr * p.row_vecs;
    const auto rsrc = make_rsrc(p.packed + (start + r0) * p.packed_stride,
                                (uint32_t)(nr * p.packed_stride));
    const auto rg = make_rsrc(p.gather + start + r0, (uint32_t)nr * 4u);
    const uint32_t img0 = (uint32_t)img_row0;
    // vector v: its packed row r, column col; past the chunk, r >= nr and the
    // loads through rsrc / rg read zeros while the store gets a dropped offset
    for (int v = tid; v - tid < total; v += kBatch) {
        int r[kUnroll], col[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            r[j] = (v + j * kThreads) / p.row_vecs;
            col[j] = (v + j * kThreads) - r[j] * p.row_vecs;
        }
        // all loads first (gather indices, then rows), then the offsets
        const uint32_t g0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, 4u * r[0], 0, 0);
        const uint32_t g1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, 4u * r[1], 0, 0);
        const uint32_t g2 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, 4u * r[2], 0, 0);
        const uint32_t g3 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rg, 4u * r[3], 0, 0);
        const u32x4 x0 = ld16(rsrc, (uint32_t)r[0] * (uint32_t)p.packed_stride + 16u * col[0]);
        const u32x4 x1 = ld16(rsrc, (uint32_t)r[1] * (uint32_t)p.packed_stride + 16u * col[1]);
        const u32x4 x2 = ld16(rsrc, (uint32_t)r[2] * (uint32_t)p.packed_stride + 16u * col[2]);
        const u32x4 x3 = ld16(rsrc, (uint32_t)r[3] * (uint32_t)p.packed_stride + 16u * col[3]);
        const uint32_t gg[kUnroll] = {g0 - img0, g1 - img0, g2 - img0, g3 - img0};
        uint32_t d[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const bool ok = v + j * kThreads < total && gg[j] < (uint32_t)p.N;
            d[j] = ok ? gg[j] * (uint32_t)p.dst_stride + 16u * col[j] : kDropOffset;
        }
        st16(x0, rdst, d[0]);
        st16(x1, rdst, d[1]);
        st16(x2, rdst, d[2]);
        st16(x3, rdst, d[3]);
    }
}

}  // namespace

int launch_pack(const uint8_t* keep, int32_t B, int32_t N, const void* src,
                int64_t src_row_stride, int32_t row_bytes, void* packed,
                int64_t packed_row_stride, int32_t* cu_seqlens, int32_t* gather_idx,
                int32_t* max_seqlen_dev, void* stream)
{
    PackParams p;
    p.keep = keep;
    p.src = static_cast<const uint8_t*>(src);
    p.packed = static_cast<uint8_t*>(packed);
    p.cu = cu_seqlens;
    p.gather = gather_idx;
    p.max_len = max_seqlen_dev;
    p.cu_in = nullptr;
    p.gather_in = nullptr;
    p.total_rows = 0;
    p.src_stride = src_row_stride;
    p.packed_stride = packed_row_stride;
    p.B = B;
    p.N = N;
    p.row_vecs = row_bytes / 16;
    p.n_magic = (uint32_t)((1ull << 32) / (uint64_t)N + 1ull);
    // slices: enough for about kPackTargetGroups workgroups, each at least 16
    // vectors (256 bytes) of every row
    const int max_slices = max(1, p.row_vecs / 16);
    const int slices = min(max_slices, max(1, (kPackTargetGroups + B - 1) / B));
    p.slice_vecs = (p.row_vecs + slices - 1) / slices;
    const int used = (p.row_vecs + p.slice_vecs - 1) / p.slice_vecs;  // no empty slice
    const dim3 grid(B + (max_seqlen_dev ? 1 : 0), used);
    const size_t lds = sizeof(int) * (size_t)max(N, kThreads);
    hipLaunchKernelGGL(pack_kernel<false>, grid, dim3(kThreads), lds, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

int launch_repack(const uint8_t* keep_packed, const int32_t* cu_in, const int32_t* gather_in,
                  int32_t B, int32_t max_rows_in, int32_t total_rows, const void* src,
                  int64_t src_row_stride, int32_t row_bytes, void* dst, int64_t dst_row_stride,
                  int32_t* cu_out, int32_t* gather_out, void* stream)
{
    PackParams p;
    p.keep = keep_packed;
    p.src = static_cast<const uint8_t*>(src);
    p.packed = static_cast<uint8_t*>(dst);
    p.cu = cu_out;
    p.gather = gather_out;
    p.max_len = nullptr;
    p.cu_in = cu_in;
    p.gather_in = gather_in;
    p.src_stride = src_row_stride;
    p.packed_stride = dst_row_stride;
    p.B = B;
    p.N = max_rows_in;
    p.total_rows = total_rows;
    p.row_vecs = row_bytes / 16;
    p.n_magic = 0;  // no max-length pass
    const int max_slices = max(1, p.row_vecs / 16);
    const int slices = min(max_slices, max(1, (kPackTargetGroups + B - 1) / B));
    p.slice_vecs = (p.row_vecs + slices - 1) / slices;
    const int used = (p.row_vecs + p.slice_vecs - 1) / p.slice_vecs;
    const dim3 grid(B, used);
    const size_t lds = sizeof(int) * (size_t)max(max_rows_in, kThreads);
    hipLaunchKernelGGL(pack_kernel<true>, grid, dim3(kThreads), lds, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

int launch_unpack(const void* packed, int64_t packed_row_stride, int32_t row_bytes,
                  const int32_t* cu_seqlens, const int32_t* gather_idx, int32_t B, int32_t N,
                  void* dst, int64_t dst_row_stride, uint32_t flags, void* stream)
{
    UnpackParams p;
    p.packed = static_cast<const uint8_t*>(packed);
    p.dst = static_cast<uint8_t*>(dst);
    p.cu = cu_seqlens;
    p.gather = gather_idx;
    p.packed_stride = packed_row_stride;
    p.dst_stride = dst_row_stride;
    p.B = B;
    p.N = N;
    p.row_vecs = row_bytes / 16;
    p.rows = rows_per_chunk(row_bytes);
    p.zero_dropped = (flags & RAG_UNPACK_ZERO_DROPPED) ? 1 : 0;
    const dim3 grid(B, (N + p.rows - 1) / p.rows);
    hipLaunchKernelGGL(unpack_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace rag
