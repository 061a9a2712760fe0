// rag_internal.h -- declarations shared by the translation units of librag.so.
// HIP-free on purpose: rag_validate.cpp includes it and builds with any C++17
// compiler, so argument checking can be tested without a GPU.
#pragma once

#include <cstdint>

#include "rag.h"

namespace rag {

// Record a message for rag_last_error() on this thread and return `s`.
rag_status set_error(rag_status s, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();

// ---- argument checks (host only, run before anything is enqueued) ----
rag_status validate_pack(const uint8_t* keep, int32_t B, int32_t N, const void* src,
                         int64_t src_row_stride, int32_t row_bytes, const void* packed,
                         int64_t packed_row_stride, const int32_t* cu_seqlens,
                         const int32_t* gather_idx);
rag_status validate_repack(const uint8_t* keep_packed, const int32_t* cu_in,
                           const int32_t* gather_in, int32_t B, int32_t max_rows_in,
                           int32_t total_rows, const void* src, int64_t src_row_stride,
                           int32_t row_bytes, const void* dst, int64_t dst_row_stride,
                           const int32_t* cu_out, const int32_t* gather_out);
rag_status validate_unpack(const void* packed, int64_t packed_row_stride, int32_t row_bytes,
                           const int32_t* cu_seqlens, const int32_t* gather_idx, int32_t B,
                           int32_t N, const void* dst, int64_t dst_row_stride, uint32_t flags);
rag_status validate_attn(const void* q, const void* k, const void* v, int64_t q_row_stride,
                         int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                         const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                         int32_t total_rows, int32_t H, int32_t head_dim, float scale,
                         const void* o, int64_t o_row_stride, int32_t out_dtype);
// rag_attn_tiled's extra limits (B, H, max_seqlen of the tile list).
rag_status validate_tile_list(int32_t B, int32_t H, int32_t max_seqlen);
rag_status validate_attn_padded(const void* q, const void* k, const void* v,
                                int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                                int32_t in_dtype, const uint8_t* keep, int32_t B, int32_t N,
                                int32_t H, int32_t head_dim, float scale, const void* o,
                                int64_t o_row_stride, int32_t out_dtype);
rag_status validate_attn_gathered(const uint8_t* keep, int32_t B, int32_t N, int32_t max_seqlen,
                                  const void* q,
                                  const void* k, const void* v, int64_t q_row_stride,
                                  int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                                  int32_t H, int32_t head_dim, float scale, const void* o,
                                  int64_t o_row_stride, int32_t out_dtype, uint32_t flags);
rag_status validate_pipeline(const rag_pipeline_desc* d);
rag_status validate_block_desc(const rag_block_desc* d);
rag_status validate_block_call(const void* x, const void* y, int32_t rows, int32_t C,
                               const void* scratch, size_t scratch_given, size_t scratch_needed);

inline int dtype_bytes(int32_t dt) { return dt == RAG_DTYPE_F32 ? 4 : 2; }

// ---- work split of the row-copy kernels (pack / unpack) ----
// Rows of one image handled by one workgroup, chosen so that a workgroup moves
// a few tens of KiB; the grid is ceil(N / rows) x B.
int rows_per_chunk(int32_t row_bytes);

// ---- launchers (defined in the .hip files; return a hipError_t value) ----
int launch_pack(const uint8_t* keep, int32_t B, int32_t N, const void* src,
                int64_t src_row_stride, int32_t row_bytes, void* packed,
                int64_t packed_row_stride, int32_t* cu_seqlens, int32_t* gather_idx,
                int32_t* max_seqlen_dev, void* stream);
int launch_repack(const uint8_t* keep_packed, const int32_t* cu_in, const int32_t* gather_in,
                  int32_t B, int32_t max_rows_in, int32_t total_rows, const void* src,
                  int64_t src_row_stride, int32_t row_bytes, void* dst, int64_t dst_row_stride,
                  int32_t* cu_out, int32_t* gather_out, void* stream);
int launch_unpack(const void* packed, int64_t packed_row_stride, int32_t row_bytes,
                  const int32_t* cu_seqlens, const int32_t* gather_idx, int32_t B, int32_t N,
                  void* dst, int64_t dst_row_stride, uint32_t flags, void* stream);
// layout: 0 = packed ragged rows (cu_seqlens), 1 = padded [B, N] rows with
// dropped keys masked, 2 = gathered: the kept rows of the [B, N] layout, found
// from the keep row, output written to those rows (flags: zero-dropped).
// max_seqlen bounds the rows per image for layouts 0 and 2 (ignored for 1).
enum { kLayoutRagged = 0, kLayoutPadded = 1, kLayoutGathered = 2 };
// flags bit (library-internal, ragged layout): launch over the device-built
// tile list (B <= kTileListMaxB, H <= kTileListMaxH, max_seqlen <=
// kTileListMaxLen: the decode's item indices stay below 2^17).
constexpr uint32_t kAttnTileList = 1u << 16;
constexpr int kTileListMaxB = 1024;
constexpr int kTileListMaxH = 64;
constexpr int kTileListMaxLen = 960;
int launch_attn(const void* q, const void* k, const void* v, int64_t q_row_stride,
                int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                const int32_t* cu_seqlens, const uint8_t* keep, int32_t B, int32_t N,
                int32_t max_seqlen, int32_t total_rows, int32_t H, float scale, void* o,
                int64_t o_row_stride, int32_t out_dtype, int layout, uint32_t flags,
                void* stream);

// ---- the encoder block's matrix products (gemm.hip) ----
// D[M, N] = epi(X[M, K] W[N, K]^T + bias) (+ R): X, W, R, D bf16 row-major,
// bias fp32; K a multiple of 64, N a multiple of 64; 16-byte aligned bases.
enum { kGemmBias = 0, kGemmResidual = 1, kGemmGelu = 2 };
int launch_gemm(const void* x, const void* w, const float* bias, const void* r, void* d, int32_t M,
                int32_t N, int32_t K, int epi, void* stream);

}  // namespace rag
