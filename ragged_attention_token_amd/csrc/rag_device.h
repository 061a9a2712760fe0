// rag_device.h -- device helpers shared by the kernels of librag.so (HIP only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rag {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw 32-bit buffer resource, gfx9 family
// Outside every resource the kernels build (all span < 2^31 bytes), with room
// for the column offsets (< 64 KiB) added to it without wrapping.
constexpr uint32_t kDropOffset = 0xFFFF0000u;

// A buffer resource over [base, base + bytes).  Loads outside it return zeros
// and stores outside it are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// The four words of the raw buffer resource over [base, base + bytes) that
// make_rsrc builds, for loads written in inline assembly.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, (int)kRsrcWord3};
}

// Sixteen bytes per lane at offset voff of the resource, written to LDS at
// lds_addr + 16 lane (lds_addr wave-uniform), by a buffer load that writes LDS
// (no registers).  The compiler does not track it: it cannot tell that such a
// load and the LDS words read meanwhile (another buffer) do not overlap, and
// its own waits would serialise them; every use waits with an explicit
// s_waitcnt vmcnt.  The LDS base goes in through M0 as an input operand; the
// s_nop gives the M0 write the wait state the load needs.
__device__ __forceinline__ void ld_lds16_untracked(i32x4 r, uint32_t lds_addr, uint32_t voff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r), "{m0}"(lds_addr));
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ void st16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// Lists the positions n < N with krow[n] != 0 in ascending order into pos[]
// (the rank of a kept position is its index in pos) and returns their number.
// A workgroup of nw wave64s reads the row once: a 64-lane ballot plus popcount
// gives each kept position its rank inside its wave, and an nw-entry LDS table
// (wsum) the ranks of the waves before it.  Every thread of the workgroup must
// call it; blockDim.x must be 64 * nw.
__device__ __forceinline__ int rank_kept_waves(const uint8_t* krow, int N, int* pos, int* wsum,
                                               int nw)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int L = 0;
    for (int base = 0; base < N; base += 64 * nw) {
        const int n = base + tid;
        const bool kept = n < N && krow[n] != 0;
        const uint64_t m = __ballot(kept);
        const int below = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[wave] = __popcll(m);
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < nw; ++w) {
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

// rank_kept_waves for rows of at most 64 * nw positions whose keep byte each
// thread has already loaded (kept = this thread's position is kept), so that
// the caller can issue other loads between the byte load and the ranking.
__device__ __forceinline__ int rank_kept_preloaded(bool kept, int* pos, int* wsum, int nw)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t m = __ballot(kept);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < nw; ++w) {
        const int x = wsum[w];
        before += (w < wave) ? x : 0;
        total += x;
    }
    if (kept) pos[before + below] = tid;
    __syncthreads();
    return total;
}

// rank_kept_waves for rows of at most KMAX * 64 * nw positions whose keep
// bytes are already in registers: thread t of the workgroup holds kb[k], the
// byte of position t + k * 64 nw (0 past N).  Positions are ranked plane by
// plane (plane k = [k 64 nw, (k+1) 64 nw)), which is ascending order.  wsum
// holds KMAX * nw ints.
template <int KMAX>
__device__ __forceinline__ int rank_kept_planes_loaded(const uint32_t (&kb)[KMAX], int* pos, int* wsum, int nw)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nt = 64 * nw;
    int below[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const uint64_t m = __ballot(kb[k] != 0u);
        below[k] = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[k * nw + wave] = __popcll(m);
    }
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        int before = 0, plane = 0;
        for (int w = 0; w < nw; ++w) {
            const int x = wsum[k * nw + w];
            before += (w < wave) ? x : 0;
            plane += x;
        }
        if (kb[k] != 0u) pos[total + before + below[k]] = tid + k * nt;
        total += plane;
    }
    __syncthreads();
    return total;
}

// rank_kept_planes_loaded with every keep byte requested before the first
// barrier (one memory round trip), read through a buffer resource over the
// row (positions past N read as zero).
template <int KMAX>
__device__ __forceinline__ int rank_kept_planes(const uint8_t* krow, int N, int* pos, int* wsum,
                                                int nw)
{
    const int tid = threadIdx.x, nt = 64 * nw;
    const auto rk = make_rsrc(krow, (uint32_t)N);
    uint32_t kb[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) kb[k] = __builtin_amdgcn_raw_buffer_load_b8(rk, (uint32_t)(tid + k * nt), 0, 0);
    return rank_kept_planes_loaded<KMAX>(kb, pos, wsum, nw);
}

// rank_kept_waves for a 256-thread workgroup (wsum holds 4 ints).
__device__ __forceinline__ int rank_kept(const uint8_t* krow, int N, int* pos, int* wsum)
{
    return rank_kept_waves(krow, N, pos, wsum, 4);
}

}  // namespace dev
}  // namespace rag
