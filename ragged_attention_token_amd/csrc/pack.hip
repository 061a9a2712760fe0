// pack.hip -- token packing and write-back for ragged ViT attention on gfx950.
//
// Pack ("Triton Ragged Attention 與 pack-attend-unpack", agents-report.net,
// section 方法概覽, fused token packing): from the keep mask, build the per-image
// offsets cu_seqlens and the destination (gather) index, then copy the kept
// token rows into one flat buffer.  Unpack (same section, write-back): copy each
// packed row back to its batch position.
//
// One launch each.  Workgroup (b, c) serves rows [c*R, c*R + R) of image b; the
// chunk index is the slowest grid dimension, so the first chunk of every image
// is dispatched before the later chunks, which pruned images mostly lack.
//   1. ranks inside image b: the image's N keep bytes are read once; a 64-lane
//      ballot + popcount gives each kept position its rank, and the kept
//      positions are listed by rank in LDS;
//   2. the chunk's source rows are requested (four 16-byte loads per lane in
//      flight), and while they travel:
//   3. offset of image b = number of kept tokens in images 0..b-1, counted from
//      16-byte words of the keep mask (each workgroup recounts the prefix, at
//      most B*N bytes that stay in L2; no atomics and no inter-workgroup waits,
//      so the result is deterministic);
//   4. the rows are stored.
// All row traffic goes through buffer resources: a lane past the chunk's end
// gets an offset outside the resource, so its load reads zero and its store is
// dropped by the hardware; no predicated register arrays are needed.
// An extra workgroup row (b == B) computes max_b L_b when asked for.
#include <hip/hip_runtime.h>

#include "rag_device.h"
#include "rag_internal.h"

namespace rag {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 4;                           // 16-byte vectors per lane per batch
constexpr int kBatch = kThreads * kUnroll;           // vectors per workgroup per batch
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

// Kept tokens in keep[0, nbytes): 16-byte words through a buffer resource
// (words past the range read as zero), eight loads in flight per lane.
__device__ int count_kept_prefix(const uint8_t* keep, int64_t nbytes, int* red)
{
    const int tid = threadIdx.x;
    const uint32_t nwords = (uint32_t)(nbytes >> 4);
    const auto rk = make_rsrc(keep, nwords << 4);
    int cnt = 0;
    for (uint32_t w0 = 0; w0 < nwords; w0 += kThreads * 8) {
        u32x4 x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = ld16(rk, (w0 + tid + j * kThreads) << 4);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            cnt += nonzero_bytes(x[j][0]) + nonzero_bytes(x[j][1]) + nonzero_bytes(x[j][2]) +
                   nonzero_bytes(x[j][3]);
    }
    const uint32_t tail0 = nwords << 4;
    if (tid < nbytes - tail0) cnt += keep[tail0 + tid] != 0;
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

// Byte offset, inside image b's source rows, of 16-byte vector v of the chunk;
// a vector past the chunk re-reads the chunk's first row (its store is dropped).
__device__ __forceinline__ uint32_t pack_src_off(const PackParams& p, const int* pos, int r0,
                                                 int total, int v)
{
    const int vv = v < total ? v : 0;
    const int r = vv / p.row_vecs;
    const int col = vv - r * p.row_vecs;
    return (uint32_t)pos[r0 + r] * (uint32_t)p.src_stride + 16u * col;
}

__device__ __forceinline__ uint32_t pack_dst_off(const PackParams& p, int total, int v)
{
    if (v >= total) return kDropOffset;
    const int r = v / p.row_vecs;
    const int col = v - r * p.row_vecs;
    return (uint32_t)r * (uint32_t)p.packed_stride + 16u * col;
}

__global__ __launch_bounds__(kThreads) void pack_kernel(PackParams p)
{
    extern __shared__ int s_pos[];  // max(N, 256) ints
    __shared__ int s_red[kWaves];
    const int tid = threadIdx.x;
    const int b = blockIdx.x, c = blockIdx.y;  // chunk slowest: chunk 0 of every image first
    if (b == p.B) {
        if (c == 0) max_length_pass(p, s_pos, max(p.N, kThreads), s_red);
        return;
    }
    const int64_t img_row0 = (int64_t)b * p.N;
    const int L = dev::rank_kept(p.keep + img_row0, p.N, s_pos, s_red);
    const int r0 = c * p.rows;
    if (c > 0 && r0 >= L) return;  // nothing to copy; chunk 0 still writes cu
    const int nr = max(0, min(p.rows, L - r0));
    const int total = nr * p.row_vecs;

    // source rows of image b; destination rows are placed once the offset is known
    const auto rs = make_rsrc(p.src + img_row0 * p.src_stride, (uint32_t)(p.N * p.src_stride));
    int v = tid;
    u32x4 x0 = ld16(rs, pack_src_off(p, s_pos, r0, total, v));
    u32x4 x1 = ld16(rs, pack_src_off(p, s_pos, r0, total, v + kThreads));
    u32x4 x2 = ld16(rs, pack_src_off(p, s_pos, r0, total, v + 2 * kThreads));
    u32x4 x3 = ld16(rs, pack_src_off(p, s_pos, r0, total, v + 3 * kThreads));

    const int offset = count_kept_prefix(p.keep, img_row0, s_red);
    if (c == 0 && tid == 0) {
        p.cu[b + 1] = offset + L;
        if (b == 0) p.cu[0] = 0;
    }
    if (tid < nr) p.gather[offset + r0 + tid] = (int32_t)(img_row0 + s_pos[r0 + tid]);
    const auto rd = make_rsrc(p.packed + ((int64_t)offset + r0) * p.packed_stride,
                              (uint32_t)(nr * p.packed_stride));
    for (;;) {
        st16(x0, rd, pack_dst_off(p, total, v));
        st16(x1, rd, pack_dst_off(p, total, v + kThreads));
        st16(x2, rd, pack_dst_off(p, total, v + 2 * kThreads));
        st16(x3, rd, pack_dst_off(p, total, v + 3 * kThreads));
        v += kBatch;
        if (v - tid >= total) break;  // uniform: every lane sees the same v - tid
        x0 = ld16(rs, pack_src_off(p, s_pos, r0, total, v));
        x1 = ld16(rs, pack_src_off(p, s_pos, r0, total, v + kThreads));
        x2 = ld16(rs, pack_src_off(p, s_pos, r0, total, v + 2 * kThreads));
        x3 = ld16(rs, pack_src_off(p, s_pos, r0, total, v + 3 * kThreads));
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
    p.src_stride = src_row_stride;
    p.packed_stride = packed_row_stride;
    p.B = B;
    p.N = N;
    p.row_vecs = row_bytes / 16;
    p.rows = rows_per_chunk(row_bytes);
    const dim3 grid(B + (max_seqlen_dev ? 1 : 0), (N + p.rows - 1) / p.rows);
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
    const dim3 grid(B, (N + p.rows - 1) / p.rows);
    hipLaunchKernelGGL(unpack_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace rag
