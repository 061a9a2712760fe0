// pack.hip -- token packing and write-back for ragged ViT attention on gfx950.
//
// Pack ("Triton Ragged Attention 與 pack-attend-unpack", agents-report.net,
// section 方法概覽, fused token packing): from the keep mask, build the per-image
// offsets cu_seqlens and the destination (gather) index, then copy the kept
// token rows into one flat buffer.  Unpack (same section, write-back): copy each
// packed row back to its batch position.
//
// One launch each.  Workgroup (c, b) serves rows [c*R, c*R + R) of image b:
//   1. ranks inside image b: the image's N keep bytes are read once; a 64-lane
//      ballot + popcount gives each kept position its rank, and the kept
//      positions are listed by rank in LDS;
//   2. offset of image b = number of kept tokens in images 0..b-1, counted from
//      16-byte words of the keep mask (each workgroup recounts the prefix, which
//      is at most B*N bytes and stays in L2; no atomics, no inter-workgroup
//      waits, so the result is deterministic);
//   3. copy: 16-byte vector loads and stores, several in flight per lane.
// An extra workgroup row (b == B) computes max_b L_b when asked for.
#include <hip/hip_runtime.h>

#include "rag_internal.h"

namespace rag {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;

struct PackParams {
    const uint8_t* keep;
    const uint8_t* src;
    uint8_t* packed;
    int32_t* cu;
    int32_t* gather;
    int32_t* max_len;
    int64_t src_stride;
    int64_t packed_stride;
    int32_t B, N, row_vecs, rows;
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

__device__ __forceinline__ int nonzero_bytes(uint4 x)
{
    return nonzero_bytes(x.x) + nonzero_bytes(x.y) + nonzero_bytes(x.z) + nonzero_bytes(x.w);
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

// Kept tokens in keep[0, nbytes): 16-byte words, kUnroll loads in flight per lane.
__device__ int count_kept_prefix(const uint8_t* keep, int64_t nbytes, int* red)
{
    const int tid = threadIdx.x;
    const int64_t nwords = nbytes >> 4;
    const uint4* kw = reinterpret_cast<const uint4*>(keep);
    int cnt = 0;
    for (int64_t w0 = tid; w0 < nwords; w0 += (int64_t)kThreads * kUnroll) {
        uint4 x[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int64_t w = w0 + (int64_t)j * kThreads;
            x[j] = (w < nwords) ? kw[w] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) cnt += nonzero_bytes(x[j]);
    }
    const int64_t tail0 = nwords << 4;
    if (tid < nbytes - tail0) cnt += keep[tail0 + tid] != 0;
    return block_sum(cnt, red);
}

// Lists image b's kept positions by rank into pos[] and returns L_b.
__device__ int rank_image(const uint8_t* krow, int N, int* pos, int* wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int L = 0;
    for (int base = 0; base < N; base += kThreads) {
        const int n = base + tid;
        const bool kept = n < N && krow[n] != 0;
        const uint64_t m = __ballot(kept);
        const int below = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[wave] = __popcll(m);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int x = wsum[w];
            before += (w < wave) ? x : 0;
            total += x;
        }
        if (kept) pos[L + before + below] = n;
        L += total;
        __syncthreads();
    }
    return L;
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
            const uint4* kw = reinterpret_cast<const uint4*>(p.keep);
            for (uint32_t w = wlo + tid; w < whi; w += kThreads) {
                const uint4 x = kw[w];
                const uint32_t P = w << 4;
                const uint32_t f = P / N;             // image of the word's first byte
                const uint32_t e = (f + 1u) * N;      // first byte of the next image
                const uint32_t words[4] = {x.x, x.y, x.z, x.w};
                int first = 0, second = 0;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const bool nz = ((words[j >> 2] >> (8 * (j & 3))) & 0xFFu) != 0u;
                    if (P + (uint32_t)j < e) first += nz; else second += nz;
                }
                if (first) atomicAdd(&cnt[f - img0], first);
                if (second) atomicAdd(&cnt[f + 1u - img0], second);
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

__global__ __launch_bounds__(kThreads) void pack_kernel(PackParams p)
{
    extern __shared__ int s_pos[];  // max(N, 256) ints
    __shared__ int s_red[kWaves];
    const int tid = threadIdx.x;
    const int b = blockIdx.y, c = blockIdx.x;
    if (b == p.B) {
        if (c == 0) max_length_pass(p, s_pos, max(p.N, kThreads), s_red);
        return;
    }
    const int L = rank_image(p.keep + (int64_t)b * p.N, p.N, s_pos, s_red);
    const int r0 = c * p.rows;
    if (c > 0 && r0 >= L) return;  // nothing to copy; chunk 0 still writes cu
    const int offset = count_kept_prefix(p.keep, (int64_t)b * p.N, s_red);
    if (c == 0 && tid == 0) {
        p.cu[b + 1] = offset + L;
        if (b == 0) p.cu[0] = 0;
    }
    const int nr = min(p.rows, L - r0);
    if (nr <= 0) return;
    const int64_t img_row0 = (int64_t)b * p.N;
    if (tid < nr) p.gather[offset + r0 + tid] = (int32_t)(img_row0 + s_pos[r0 + tid]);

    const int total = nr * p.row_vecs;
    const int64_t dst_row0 = (int64_t)offset + r0;
    for (int v0 = tid; v0 < total; v0 += kThreads * kUnroll) {
        uint4 x[kUnroll];
        int64_t dst_off[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int v = v0 + j * kThreads;
            if (v < total) {
                const int r = v / p.row_vecs;
                const int col = v - r * p.row_vecs;
                const int64_t srow = img_row0 + s_pos[r0 + r];
                x[j] = *reinterpret_cast<const uint4*>(p.src + srow * p.src_stride + col * 16);
                dst_off[j] = (dst_row0 + r) * p.packed_stride + col * 16;
            }
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            if (v0 + j * kThreads < total)
                *reinterpret_cast<uint4*>(p.packed + dst_off[j]) = x[j];
        }
    }
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackParams p)
{
    __shared__ uint32_t s_kept[RAG_MAX_N / 32];
    const int tid = threadIdx.x;
    const int b = blockIdx.y, c = blockIdx.x;
    const int64_t cap = (int64_t)p.B * p.N;
    const int64_t start = min(max((int64_t)p.cu[b], (int64_t)0), cap);
    const int64_t end = min(max((int64_t)p.cu[b + 1], start), cap);
    const int L = (int)min(end - start, (int64_t)p.N);
    const int64_t img_row0 = (int64_t)b * p.N;

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
        for (int v = tid; v < total; v += kThreads) {
            const int r = v / p.row_vecs;
            const int col = v - r * p.row_vecs;
            const int n = n0 + r;
            if (!((s_kept[n >> 5] >> (n & 31)) & 1u))
                *reinterpret_cast<uint4*>(p.dst + (img_row0 + n) * p.dst_stride + col * 16) =
                    make_uint4(0u, 0u, 0u, 0u);
        }
    }

    const int r0 = c * p.rows;
    const int nr = min(p.rows, L - r0);
    if (nr <= 0) return;
    const int total = nr * p.row_vecs;
    for (int v0 = tid; v0 < total; v0 += kThreads * kUnroll) {
        uint4 x[kUnroll];
        int64_t dst_off[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int v = v0 + j * kThreads;
            dst_off[j] = -1;
            if (v < total) {
                const int r = v / p.row_vecs;
                const int col = v - r * p.row_vecs;
                const int64_t t = start + r0 + r;
                const int64_t g = (int64_t)p.gather[t] - img_row0;
                x[j] = *reinterpret_cast<const uint4*>(p.packed + t * p.packed_stride + col * 16);
                if (g >= 0 && g < p.N) dst_off[j] = (img_row0 + g) * p.dst_stride + col * 16;
            }
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
            if (dst_off[j] >= 0) *reinterpret_cast<uint4*>(p.dst + dst_off[j]) = x[j];
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
    p.src_stride = src_row_stride;
    p.packed_stride = packed_row_stride;
    p.B = B;
    p.N = N;
    p.row_vecs = row_bytes / 16;
    p.rows = rows_per_chunk(row_bytes);
    const dim3 grid((N + p.rows - 1) / p.rows, B + (max_seqlen_dev ? 1 : 0));
    const size_t lds = sizeof(int) * (size_t)max(N, kThreads);
    hipLaunchKernelGGL(pack_kernel, grid, dim3(kThreads), lds, static_cast<hipStream_t>(stream), p);
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
    const dim3 grid((N + p.rows - 1) / p.rows, B);
    hipLaunchKernelGGL(unpack_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace rag
