// rag_validate.cpp -- host-side argument checks and the per-thread error text.
// No HIP call lives here: every check runs before anything is enqueued, and the
// unit tests exercise each error path on a machine without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "rag_internal.h"

namespace rag {

namespace {
thread_local char g_error[512] = "";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int32_t dt) { return dt == RAG_DTYPE_F32 || dt == RAG_DTYPE_BF16; }
}  // namespace

rag_status set_error(rag_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_error[0] = '\0'; }

int rows_per_chunk(int32_t row_bytes)
{
    // one batch of four 16-byte vectors per lane of a 256-lane workgroup
    int r = 16384 / (row_bytes > 0 ? row_bytes : 1);
    if (r < 1) r = 1;
    if (r > 64) r = 64;
    return r;
}

// The copy kernels address one image's rows (and one chunk of packed rows)
// through 32-bit byte offsets.
static rag_status check_image_span(const char* what, int32_t N, int64_t stride)
{
    if ((int64_t)std::max(N, 64) * stride >= ((int64_t)1 << 31))
        return set_error(RAG_ERR_UNSUPPORTED, "%s: max(N, 64) rows x %lld-byte stride >= 2^31 bytes",
                         what, (long long)stride);
    return RAG_OK;
}

static rag_status check_rows(const char* what, const void* base, int64_t stride, int32_t row_bytes)
{
    if (!base) return set_error(RAG_ERR_INVALID_ARG, "%s is NULL", what);
    if (stride < row_bytes)
        return set_error(RAG_ERR_INVALID_ARG, "%s row stride %lld is smaller than row_bytes %d",
                         what, (long long)stride, row_bytes);
    if (!aligned16(base) || (stride & 15))
        return set_error(RAG_ERR_ALIGNMENT, "%s base and row stride must be multiples of 16 bytes",
                         what);
    return RAG_OK;
}

static rag_status check_batch(int32_t B, int32_t N)
{
    if (B < 1 || N < 1) return set_error(RAG_ERR_INVALID_ARG, "B=%d and N=%d must be >= 1", B, N);
    if (B > RAG_MAX_B || N > RAG_MAX_N)
        return set_error(RAG_ERR_UNSUPPORTED, "B=%d N=%d exceed the limits B<=%d N<=%d", B, N,
                         RAG_MAX_B, RAG_MAX_N);
    if ((int64_t)B * N > INT32_MAX)
        return set_error(RAG_ERR_UNSUPPORTED, "B*N must fit in int32");
    return RAG_OK;
}

rag_status validate_pack(const uint8_t* keep, int32_t B, int32_t N, const void* src,
                         int64_t src_row_stride, int32_t row_bytes, const void* packed,
                         int64_t packed_row_stride, const int32_t* cu_seqlens,
                         const int32_t* gather_idx)
{
    rag_status s = check_batch(B, N);
    if (s != RAG_OK) return s;
    if (!keep) return set_error(RAG_ERR_INVALID_ARG, "keep is NULL");
    if (!aligned16(keep)) return set_error(RAG_ERR_ALIGNMENT, "keep must be 16-byte aligned");
    if (row_bytes < 16) return set_error(RAG_ERR_INVALID_ARG, "row_bytes=%d must be >= 16", row_bytes);
    if (row_bytes & 15) return set_error(RAG_ERR_ALIGNMENT, "row_bytes=%d must be a multiple of 16", row_bytes);
    if ((s = check_rows("src", src, src_row_stride, row_bytes)) != RAG_OK) return s;
    if ((s = check_rows("packed", packed, packed_row_stride, row_bytes)) != RAG_OK) return s;
    if (!cu_seqlens || !gather_idx)
        return set_error(RAG_ERR_INVALID_ARG, "cu_seqlens and gather_idx must not be NULL");
    if ((s = check_image_span("src", N, src_row_stride)) != RAG_OK) return s;
    return check_image_span("packed", N, packed_row_stride);
}

rag_status validate_repack(const uint8_t* keep_packed, const int32_t* cu_in,
                           const int32_t* gather_in, int32_t B, int32_t max_rows_in,
                           int32_t total_rows, const void* src, int64_t src_row_stride,
                           int32_t row_bytes, const void* dst, int64_t dst_row_stride,
                           const int32_t* cu_out, const int32_t* gather_out)
{
    rag_status s = check_batch(B, max_rows_in);
    if (s != RAG_OK) return s;
    if (total_rows < 0) return set_error(RAG_ERR_INVALID_ARG, "total_rows=%d must be >= 0", total_rows);
    if (!keep_packed) return set_error(RAG_ERR_INVALID_ARG, "keep_packed is NULL");
    if (!aligned16(keep_packed))
        return set_error(RAG_ERR_ALIGNMENT, "keep_packed must be 16-byte aligned");
    if (!cu_in || !gather_in || !cu_out || !gather_out)
        return set_error(RAG_ERR_INVALID_ARG, "cu_in, gather_in, cu_out and gather_out must not be NULL");
    if (row_bytes < 16) return set_error(RAG_ERR_INVALID_ARG, "row_bytes=%d must be >= 16", row_bytes);
    if (row_bytes & 15) return set_error(RAG_ERR_ALIGNMENT, "row_bytes=%d must be a multiple of 16", row_bytes);
    if ((s = check_rows("src", src, src_row_stride, row_bytes)) != RAG_OK) return s;
    if ((s = check_rows("dst", dst, dst_row_stride, row_bytes)) != RAG_OK) return s;
    if (src == dst) return set_error(RAG_ERR_INVALID_ARG, "src and dst must not overlap");
    if ((s = check_image_span("src", max_rows_in, src_row_stride)) != RAG_OK) return s;
    return check_image_span("dst", max_rows_in, dst_row_stride);
}

rag_status validate_unpack(const void* packed, int64_t packed_row_stride, int32_t row_bytes,
                           const int32_t* cu_seqlens, const int32_t* gather_idx, int32_t B,
                           int32_t N, const void* dst, int64_t dst_row_stride, uint32_t flags)
{
    rag_status s = check_batch(B, N);
    if (s != RAG_OK) return s;
    if (flags & ~RAG_UNPACK_ZERO_DROPPED)
        return set_error(RAG_ERR_UNSUPPORTED, "unknown unpack flags 0x%x", flags);
    if (row_bytes < 16) return set_error(RAG_ERR_INVALID_ARG, "row_bytes=%d must be >= 16", row_bytes);
    if (row_bytes & 15) return set_error(RAG_ERR_ALIGNMENT, "row_bytes=%d must be a multiple of 16", row_bytes);
    if ((s = check_rows("packed", packed, packed_row_stride, row_bytes)) != RAG_OK) return s;
    if ((s = check_rows("dst", dst, dst_row_stride, row_bytes)) != RAG_OK) return s;
    if (!cu_seqlens || !gather_idx)
        return set_error(RAG_ERR_INVALID_ARG, "cu_seqlens and gather_idx must not be NULL");
    if ((s = check_image_span("dst", N, dst_row_stride)) != RAG_OK) return s;
    return check_image_span("packed", N, packed_row_stride);
}

static rag_status check_attn_common(const void* q, const void* k, const void* v, int64_t qs,
                                    int64_t ks, int64_t vs, int32_t in_dtype, int32_t B,
                                    int32_t H, int32_t head_dim, float scale, const void* o,
                                    int64_t os, int32_t out_dtype)
{
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
        return set_error(RAG_ERR_UNSUPPORTED, "dtype must be RAG_DTYPE_F32 or RAG_DTYPE_BF16");
    if (head_dim != RAG_HEAD_DIM)
        return set_error(RAG_ERR_UNSUPPORTED, "head_dim=%d; only %d is built", head_dim,
                         RAG_HEAD_DIM);
    if (H < 1) return set_error(RAG_ERR_INVALID_ARG, "H=%d must be >= 1", H);
    // (the kernels number the (head, image) pairs with 32-bit integers)
    if ((int64_t)B * H > INT32_MAX)
        return set_error(RAG_ERR_UNSUPPORTED, "B*H=%lld (head, image) pairs exceed 2^31-1",
                         (long long)B * H);
    if (!std::isfinite(scale)) return set_error(RAG_ERR_INVALID_ARG, "scale must be finite");
    const int64_t C = (int64_t)H * head_dim;
    const void* ptrs[4] = {q, k, v, o};
    const int64_t strides[4] = {qs, ks, vs, os};
    const int32_t dts[4] = {in_dtype, in_dtype, in_dtype, out_dtype};
    const char* names[4] = {"q", "k", "v", "o"};
    for (int i = 0; i < 4; ++i) {
        if (!ptrs[i]) return set_error(RAG_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (strides[i] < C)
            return set_error(RAG_ERR_INVALID_ARG, "%s row stride %lld < H*head_dim %lld", names[i],
                             (long long)strides[i], (long long)C);
        if (!aligned16(ptrs[i]) || ((strides[i] * dtype_bytes(dts[i])) & 15))
            return set_error(RAG_ERR_ALIGNMENT,
                             "%s base and row stride must be multiples of 16 bytes", names[i]);
    }
    return RAG_OK;
}

// The kernels address one image's rows through 32-bit byte offsets: the span
// of `rows` rows must stay below 2^31 bytes for every operand.
static rag_status check_span(int64_t rows, int64_t qs, int64_t ks, int64_t vs, int32_t in_dtype,
                             int64_t os, int32_t out_dtype)
{
    const int64_t ie = dtype_bytes(in_dtype), oe = dtype_bytes(out_dtype);
    const int64_t widest = std::max(std::max(qs, ks) * ie, std::max(vs * ie, os * oe));
    if (rows * widest >= ((int64_t)1 << 31))
        return set_error(RAG_ERR_UNSUPPORTED,
                         "one image spans >= 2^31 bytes (%lld rows x %lld-byte stride)",
                         (long long)rows, (long long)widest);
    return RAG_OK;
}

rag_status validate_attn(const void* q, const void* k, const void* v, int64_t q_row_stride,
                         int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                         const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                         int32_t total_rows, int32_t H, int32_t head_dim, float scale,
                         const void* o, int64_t o_row_stride, int32_t out_dtype)
{
    if (B < 1 || B > RAG_MAX_B) return set_error(RAG_ERR_INVALID_ARG, "B=%d out of [1, %d]", B, RAG_MAX_B);
    if (max_seqlen < 1) return set_error(RAG_ERR_INVALID_ARG, "max_seqlen=%d must be >= 1", max_seqlen);
    if (max_seqlen > 65535 * 64)
        return set_error(RAG_ERR_UNSUPPORTED, "max_seqlen=%d exceeds %d", max_seqlen, 65535 * 64);
    if (total_rows < 0) return set_error(RAG_ERR_INVALID_ARG, "total_rows=%d must be >= 0", total_rows);
    if (!cu_seqlens) return set_error(RAG_ERR_INVALID_ARG, "cu_seqlens is NULL");
    rag_status s = check_attn_common(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype,
                                     B, H, head_dim, scale, o, o_row_stride, out_dtype);
    if (s != RAG_OK) return s;
    return check_span(max_seqlen, q_row_stride, k_row_stride, v_row_stride, in_dtype, o_row_stride,
                      out_dtype);
}

rag_status validate_tile_list(int32_t B, int32_t H, int32_t max_seqlen)
{
    if (H > kTileListMaxH)
        return set_error(RAG_ERR_UNSUPPORTED, "tile list: H=%d exceeds %d", H, kTileListMaxH);
    if (B > kTileListMaxB)
        return set_error(RAG_ERR_UNSUPPORTED, "tile list: B=%d exceeds %d", B, kTileListMaxB);
    if (max_seqlen > kTileListMaxLen)
        return set_error(RAG_ERR_UNSUPPORTED, "tile list: max_seqlen=%d exceeds %d", max_seqlen,
                         kTileListMaxLen);
    return RAG_OK;
}

rag_status validate_attn_padded(const void* q, const void* k, const void* v,
                                int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                                int32_t in_dtype, const uint8_t* keep, int32_t B, int32_t N,
                                int32_t H, int32_t head_dim, float scale, const void* o,
                                int64_t o_row_stride, int32_t out_dtype)
{
    rag_status s = check_batch(B, N);
    if (s != RAG_OK) return s;
    if (!keep) return set_error(RAG_ERR_INVALID_ARG, "keep is NULL");
    s = check_attn_common(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype, B, H, head_dim,
                          scale, o, o_row_stride, out_dtype);
    if (s != RAG_OK) return s;
    return check_span(N, q_row_stride, k_row_stride, v_row_stride, in_dtype, o_row_stride,
                      out_dtype);
}

rag_status validate_attn_gathered(const uint8_t* keep, int32_t B, int32_t N, int32_t max_seqlen,
                                  const void* q, const void* k, const void* v, int64_t q_row_stride,
                                  int64_t k_row_stride, int64_t v_row_stride, int32_t in_dtype,
                                  int32_t H, int32_t head_dim, float scale, const void* o,
                                  int64_t o_row_stride, int32_t out_dtype, uint32_t flags)
{
    if (flags & ~RAG_UNPACK_ZERO_DROPPED)
        return set_error(RAG_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    if (max_seqlen < 0 || max_seqlen > N)
        return set_error(RAG_ERR_INVALID_ARG, "max_seqlen=%d must lie in [0, N=%d]", max_seqlen, N);
    return validate_attn_padded(q, k, v, q_row_stride, k_row_stride, v_row_stride, in_dtype, keep,
                                B, N, H, head_dim, scale, o, o_row_stride, out_dtype);
}

rag_status validate_pipeline(const rag_pipeline_desc* d)
{
    if (!d) return set_error(RAG_ERR_INVALID_ARG, "desc is NULL");
    if (d->head_dim != RAG_HEAD_DIM)
        return set_error(RAG_ERR_UNSUPPORTED, "head_dim=%d; only %d is built", d->head_dim,
                         RAG_HEAD_DIM);
    if (!valid_dtype(d->in_dtype) || !valid_dtype(d->out_dtype))
        return set_error(RAG_ERR_UNSUPPORTED, "dtype must be RAG_DTYPE_F32 or RAG_DTYPE_BF16");
    if (d->H < 1) return set_error(RAG_ERR_INVALID_ARG, "H=%d must be >= 1", d->H);
    if (d->max_seqlen < 0 || d->max_seqlen > d->N)
        return set_error(RAG_ERR_INVALID_ARG, "max_seqlen=%d must lie in [0, N]", d->max_seqlen);
    if (d->flags & ~(RAG_PIPELINE_FUSED | RAG_PIPELINE_DIRECT))
        return set_error(RAG_ERR_UNSUPPORTED, "unknown pipeline flags 0x%x", d->flags);
    const int64_t C = (int64_t)d->H * d->head_dim;
    const int64_t in_row = 3 * C * dtype_bytes(d->in_dtype);
    const int64_t out_row = C * dtype_bytes(d->out_dtype);
    if (in_row > INT32_MAX || out_row > INT32_MAX)
        return set_error(RAG_ERR_UNSUPPORTED, "row too large");
    rag_status s = validate_pack(d->keep, d->B, d->N, d->src, d->src_row_stride, (int32_t)in_row,
                                 d->packed, d->packed_row_stride, d->cu_seqlens, d->gather_idx);
    if (s != RAG_OK) return s;
    const int64_t in_es = dtype_bytes(d->in_dtype), out_es = dtype_bytes(d->out_dtype);
    if (d->packed_row_stride % in_es || d->o_packed_row_stride % out_es)
        return set_error(RAG_ERR_ALIGNMENT, "row strides must be whole elements");
    s = validate_attn(d->packed, d->packed, d->packed, d->packed_row_stride / in_es,
                      d->packed_row_stride / in_es, d->packed_row_stride / in_es, d->in_dtype,
                      d->cu_seqlens, d->B, d->max_seqlen ? d->max_seqlen : d->N, d->B * d->N,
                      d->H, d->head_dim, d->scale, d->o_packed, d->o_packed_row_stride / out_es,
                      d->out_dtype);
    if (s != RAG_OK) return s;
    s = validate_unpack(d->o_packed, d->o_packed_row_stride, (int32_t)out_row, d->cu_seqlens,
                        d->gather_idx, d->B, d->N, d->dst, d->dst_row_stride, d->unpack_flags);
    if (s != RAG_OK) return s;
    if (d->src_row_stride % in_es || d->dst_row_stride % out_es)
        return set_error(RAG_ERR_ALIGNMENT, "row strides must be whole elements");
    return validate_attn_gathered(d->keep, d->B, d->N, d->max_seqlen, d->src, d->src, d->src,
                                  d->src_row_stride / in_es, d->src_row_stride / in_es,
                                  d->src_row_stride / in_es, d->in_dtype, d->H, d->head_dim,
                                  d->scale, d->dst, d->dst_row_stride / out_es, d->out_dtype,
                                  d->unpack_flags);
}

extern "C" RAG_API const char* rag_last_error(void) { return rag::g_error; }

extern "C" RAG_API const char* rag_status_string(rag_status s)
{
    switch (s) {
    case RAG_OK: return "RAG_OK";
    case RAG_ERR_INVALID_ARG: return "RAG_ERR_INVALID_ARG";
    case RAG_ERR_UNSUPPORTED: return "RAG_ERR_UNSUPPORTED";
    case RAG_ERR_ALIGNMENT: return "RAG_ERR_ALIGNMENT";
    case RAG_ERR_HIP: return "RAG_ERR_HIP";
    case RAG_ERR_NO_MEMORY: return "RAG_ERR_NO_MEMORY";
    }
    return "RAG_ERR_UNKNOWN";
}

extern "C" RAG_API int32_t rag_version(void) { return 100; }

rag_status validate_block_desc(const rag_block_desc* d)
{
    if (!d) return set_error(RAG_ERR_INVALID_ARG, "desc is NULL");
    if (d->H < 1 || d->H > 32) return set_error(RAG_ERR_UNSUPPORTED, "H=%d must lie in [1, 32]", d->H);
    if (d->mlp_ratio < 1 || d->mlp_ratio > 8)
        return set_error(RAG_ERR_UNSUPPORTED, "mlp_ratio=%d must lie in [1, 8]", d->mlp_ratio);
    if (!(d->eps > 0.f) || !std::isfinite(d->eps))
        return set_error(RAG_ERR_INVALID_ARG, "eps must be positive and finite");
    if (!std::isfinite(d->scale)) return set_error(RAG_ERR_INVALID_ARG, "scale must be finite");
    const void* ptrs[] = {d->ln1_gamma, d->ln1_beta, d->w_qkv, d->b_qkv, d->w_proj, d->b_proj,
                          d->ln2_gamma, d->ln2_beta, d->w_fc1, d->b_fc1, d->w_fc2, d->b_fc2};
    const char* names[] = {"ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_proj", "b_proj",
                           "ln2_gamma", "ln2_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2"};
    for (int i = 0; i < 12; ++i) {
        if (!ptrs[i]) return set_error(RAG_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ptrs[i])) return set_error(RAG_ERR_ALIGNMENT, "%s must be 16-byte aligned", names[i]);
    }
    return RAG_OK;
}

rag_status validate_block_call(const void* x, const void* y, int32_t rows, int32_t C,
                               const void* scratch, size_t scratch_given, size_t scratch_needed)
{
    if (rows < 0) return set_error(RAG_ERR_INVALID_ARG, "rows=%d must be >= 0", rows);
    if ((int64_t)rows * 9 * C >= ((int64_t)1 << 31))
        return set_error(RAG_ERR_UNSUPPORTED, "rows=%d too large for 32-bit row offsets", rows);
    if (!x || !y || !scratch) return set_error(RAG_ERR_INVALID_ARG, "x, y and scratch must not be NULL");
    if (!aligned16(x) || !aligned16(y) || !aligned16(scratch))
        return set_error(RAG_ERR_ALIGNMENT, "x, y and scratch must be 16-byte aligned");
    if (scratch_given < scratch_needed)
        return set_error(RAG_ERR_INVALID_ARG, "scratch of %zu bytes is smaller than the %zu needed",
                         scratch_given, scratch_needed);
    return RAG_OK;
}

}  // namespace rag
