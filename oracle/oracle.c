/*
 * oracle.c -- plain, slow, fp64 CPU reference for the pack -> attend -> unpack
 * path of "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
 * (arXiv 2604.15408).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no code, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * Sources (page titles and sections):
 *   [abstract]  "Dispatch-Aware Ragged Attention for Pruned Vision Transformers",
 *               English abstract (paperdance.org card and the info.umar.mx
 *               record): a bidirectional attention kernel that runs on ragged,
 *               token-pruned ViT sequences inside a pack-attend-unpack pipeline;
 *               its outputs agree with padded attention (tiny logit gap,
 *               identical top-1).
 *   [blog-method] agents-report.net, "Triton Ragged Attention 與
 *               pack-attend-unpack", section "方法概覽" (method overview):
 *               pack = per-image offset vector cu_seqlens + destination
 *               indices, then a copy of the surviving tokens into one flat
 *               buffer; ragged attention on that buffer; unpack = write the
 *               results back to their original batch positions via cu_seqlens.
 *   [blog-problem] same page, section "問題：填充與派遣的瓶頸" (problem): the
 *               padded form pads every image to one length and masks.
 *   [abstract-v1] the same paper's earlier abstract (fugumt.com summary
 *               page): the four pruning methods it evaluates.
 *
 * Every routine below is the plain definition written out, with no blocking,
 * fusion or reordering: loops in the order the definition reads.
 *
 * Readings taken where the pages are silent:
 *   - tokens keep their original order inside a packed sequence (a stable
 *     compaction), so gather indices rise within an image;
 *   - a keep byte that is nonzero means "keep";
 *   - "bidirectional" means no mask inside an image: every kept token attends
 *     to every kept token of its own image, itself included, and to nothing
 *     outside it;
 *   - the inputs are taken exactly as stored (bf16 or fp32 bit patterns,
 *     decoded exactly to fp64); all arithmetic is fp64;
 *   - an image with no kept token contributes no packed rows; in the padded
 *     form its rows (all keys masked) are defined as zero.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_DTYPE_F32 0
#define ORACLE_DTYPE_BF16 1

/* bfloat16 is the upper half of an IEEE binary32 pattern, so the exact value
 * is that binary32 number with a zero lower half. */
double oracle_bf16_to_f64(uint16_t bits)
{
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Element i of a row, decoded exactly to fp64. */
static double load_elem(const void* base, int dtype, int64_t index)
{
    if (dtype == ORACLE_DTYPE_BF16)
        return oracle_bf16_to_f64(((const uint16_t*)base)[index]);
    return (double)((const float*)base)[index];
}

/*
 * Pack ([blog-method], fused token packing).
 *   For each image b in order, idx_b is the ascending list of positions n with
 *   keep[b][n] != 0.  cu[0] = 0, cu[b+1] = cu[b] + |idx_b|.
 *   gather[cu[b] + i] = b*N + idx_b[i] (the token's row in the [B,N] batch).
 *   packed row cu[b] + i is a byte copy of source row b*N + idx_b[i].
 * Row strides are in bytes.  Returns the total T = cu[B].
 */
int64_t oracle_pack(const uint8_t* keep, int32_t B, int32_t N,
                    const uint8_t* src, int64_t src_row_stride, int32_t row_bytes,
                    uint8_t* packed, int64_t packed_row_stride,
                    int32_t* cu_seqlens, int32_t* gather_idx)
{
    int64_t t = 0;
    cu_seqlens[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t n = 0; n < N; ++n) {
            if (keep[(int64_t)b * N + n] != 0) {
                int64_t row = (int64_t)b * N + n;
                gather_idx[t] = (int32_t)row;
                memcpy(packed + t * packed_row_stride, src + row * src_row_stride,
                       (size_t)row_bytes);
                ++t;
            }
        }
        cu_seqlens[b + 1] = (int32_t)t;
    }
    return t;
}

/*
 * Re-pack: a later pruning stage on tokens that are already packed.  The
 * pages' pruning methods ([abstract-v1]: Threshold-L2, DynamicViT, EViT, ATS)
 * drop tokens at more than one depth of the network; the plainest reading of
 * the pack step ([blog-method]) for a later stage is the same compaction
 * applied to the packed rows, with each surviving row remembering its place
 * in the original [B, N] batch.
 *   Image b of the input is packed rows cu_in[b] .. cu_in[b+1]-1.  For each
 *   image b in order, idx_b is the ascending list of those rows t with
 *   keep[t] != 0 (one keep byte per packed row).  cu_out[0] = 0,
 *   cu_out[b+1] = cu_out[b] + |idx_b|.  gather_out[cu_out[b] + i] =
 *   gather_in[idx_b[i]] (the original batch row, not the packed row), and
 *   output row cu_out[b] + i is a byte copy of input row idx_b[i].
 * Row strides are in bytes.  Returns the total T' = cu_out[B].
 */
int64_t oracle_repack(const uint8_t* keep, const int32_t* cu_in, const int32_t* gather_in,
                      int32_t B, const uint8_t* src, int64_t src_row_stride, int32_t row_bytes,
                      uint8_t* out, int64_t out_row_stride, int32_t* cu_out, int32_t* gather_out)
{
    int64_t t_out = 0;
    cu_out[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        for (int64_t t = cu_in[b]; t < cu_in[b + 1]; ++t) {
            if (keep[t] != 0) {
                gather_out[t_out] = gather_in[t];
                memcpy(out + t_out * out_row_stride, src + t * src_row_stride, (size_t)row_bytes);
                ++t_out;
            }
        }
        cu_out[b + 1] = (int32_t)t_out;
    }
    return t_out;
}

/*
 * Unpack ([blog-method], write-back).  dst row gather[t] receives packed row t
 * for every t < cu[B]; no other dst row is touched.  Row strides in bytes.
 */
void oracle_unpack(const uint8_t* packed, int64_t packed_row_stride, int32_t row_bytes,
                   const int32_t* cu_seqlens, const int32_t* gather_idx, int32_t B,
                   uint8_t* dst, int64_t dst_row_stride)
{
    int64_t T = cu_seqlens[B];
    for (int64_t t = 0; t < T; ++t)
        memcpy(dst + (int64_t)gather_idx[t] * dst_row_stride, packed + t * packed_row_stride,
               (size_t)row_bytes);
}

/*
 * Attention of one query row against a set of key rows, fp64:
 *   s_j = scale * <q, k_j>,  p_j = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j),
 *   o   = sum_j p_j v_j.
 * key_ok[j] == 0 removes key j from the set (padded form only); NULL keeps all.
 * If the set is empty the output is zero.
 */
static void attend_one_row(const void* qb, const void* kb, const void* vb, int dtype,
                           int64_t q_row, const int64_t* key_rows, const uint8_t* key_ok,
                           int32_t nkeys, int64_t q_stride, int64_t k_stride, int64_t v_stride,
                           int32_t head_off, int32_t d, double scale, double* s_buf,
                           double* out)
{
    int any = 0;
    double mx = -INFINITY;
    for (int32_t j = 0; j < nkeys; ++j) {
        if (key_ok && !key_ok[j])
            continue;
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c)
            dot += load_elem(qb, dtype, q_row * q_stride + head_off + c) *
                   load_elem(kb, dtype, key_rows[j] * k_stride + head_off + c);
        s_buf[j] = scale * dot;
        if (!any || s_buf[j] > mx)
            mx = s_buf[j];
        any = 1;
    }
    for (int32_t c = 0; c < d; ++c)
        out[c] = 0.0;
    if (!any)
        return;
    double denom = 0.0;
    for (int32_t j = 0; j < nkeys; ++j) {
        if (key_ok && !key_ok[j])
            continue;
        s_buf[j] = exp(s_buf[j] - mx);
        denom += s_buf[j];
    }
    for (int32_t j = 0; j < nkeys; ++j) {
        if (key_ok && !key_ok[j])
            continue;
        double p = s_buf[j] / denom;
        for (int32_t c = 0; c < d; ++c)
            out[c] += p * load_elem(vb, dtype, key_rows[j] * v_stride + head_off + c);
    }
}

/*
 * Ragged attention ([abstract]; [blog-method], ragged attention kernel).
 *   Image b owns packed rows cu[b] .. cu[b+1]-1.  For every head h (columns
 *   h*d .. h*d+d-1 of a row) and every query row i of image b:
 *     O[i, h] = softmax_j(scale * Q[i,h] . K[j,h]) V[j,h],  j over image b only.
 *   q/k/v strides are in elements (row to row); o is fp64 with stride o_stride.
 *   s_buf must hold max_b L_b doubles; rows_buf must hold max_b L_b int64.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attn(const void* q, const void* k, const void* v, int64_t q_stride,
                int64_t k_stride, int64_t v_stride, int32_t dtype, const int32_t* cu_seqlens,
                int32_t B, int32_t H, int32_t d, double scale, double* o, int64_t o_stride,
                double* s_buf, int64_t* rows_buf)
{
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
    for (int32_t b = 0; b < B; ++b) {
        int64_t start = cu_seqlens[b];
        int32_t L = cu_seqlens[b + 1] - cu_seqlens[b];
        if (L < 0)
            return -1;
        for (int32_t j = 0; j < L; ++j)
            rows_buf[j] = start + j;
        for (int32_t h = 0; h < H; ++h)
            for (int32_t i = 0; i < L; ++i)
                attend_one_row(q, k, v, dtype, start + i, rows_buf, NULL, L, q_stride,
                               k_stride, v_stride, h * d, d, scale, s_buf,
                               o + (start + i) * o_stride + (int64_t)h * d);
    }
    return 0;
}

/*
 * The ragged attention of selected query rows only (the same definition as
 * oracle_attn, for the outputs of a batch too large to compute whole):
 * rows[r] is a packed row index; its image b is the one with cu[b] <= row <
 * cu[b+1] (cu non-decreasing).  o[r, h*d .. h*d+d-1] gets
 * O[row, h].  Returns 0, or -1 on a bad argument (a row outside [0, cu[B])).
 */
int oracle_attn_rows(const void* q, const void* k, const void* v, int64_t q_stride,
                     int64_t k_stride, int64_t v_stride, int32_t dtype, const int32_t* cu_seqlens,
                     int32_t B, int32_t H, int32_t d, double scale, const int64_t* rows,
                     int32_t nrows, double* o, int64_t o_stride, double* s_buf, int64_t* rows_buf)
{
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
    for (int32_t r = 0; r < nrows; ++r) {
        const int64_t row = rows[r];
        if (row < 0 || row >= cu_seqlens[B])
            return -1;
        int32_t b = 0;  /* the image holding the row */
        while (!(cu_seqlens[b] <= row && row < cu_seqlens[b + 1]))
            ++b;
        const int64_t first = cu_seqlens[b];
        const int32_t L = cu_seqlens[b + 1] - cu_seqlens[b];
        for (int32_t j = 0; j < L; ++j)
            rows_buf[j] = first + j;
        for (int32_t h = 0; h < H; ++h)
            attend_one_row(q, k, v, dtype, row, rows_buf, NULL, L, q_stride, k_stride, v_stride,
                           h * d, d, scale, s_buf, o + (int64_t)r * o_stride + (int64_t)h * d);
    }
    return 0;
}

/*
 * Padded attention ([blog-problem]): every image keeps all N positions; key n of
 * image b takes part only if keep[b][n] != 0; every query position n (kept or
 * not) gets an output row.  Rows are b*N + n.  Kept query rows equal the
 * ragged result; an image with no kept key gives zero rows.
 */
int oracle_attn_padded(const void* q, const void* k, const void* v, int64_t q_stride,
                       int64_t k_stride, int64_t v_stride, int32_t dtype,
                       const uint8_t* keep, int32_t B, int32_t N, int32_t H, int32_t d,
                       double scale, double* o, int64_t o_stride, double* s_buf,
                       int64_t* rows_buf)
{
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
    for (int32_t b = 0; b < B; ++b) {
        for (int32_t n = 0; n < N; ++n)
            rows_buf[n] = (int64_t)b * N + n;
        const uint8_t* ok = keep + (int64_t)b * N;
        for (int32_t h = 0; h < H; ++h)
            for (int32_t n = 0; n < N; ++n)
                attend_one_row(q, k, v, dtype, (int64_t)b * N + n, rows_buf, ok, N, q_stride,
                               k_stride, v_stride, h * d, d, scale, s_buf,
                               o + ((int64_t)b * N + n) * o_stride + (int64_t)h * d);
    }
    return 0;
}
