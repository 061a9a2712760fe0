/*
 * rag.h -- C ABI of librag.so: ragged pack -> attend -> unpack for token-pruned
 * Vision Transformers on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "Dispatch-Aware Ragged Attention for Pruned Vision
 * Transformers" (arXiv 2604.15408):
 *   [abstract]     the English abstract (paperdance.org card, info.umar.mx
 *                  record): after token pruning, ViT sequences are short (at
 *                  most 197 tokens at 224x224) and of different lengths per
 *                  image; a bidirectional attention kernel runs directly on
 *                  these ragged sequences, and the pruning savings only show in
 *                  wall-clock time if the host-side dispatch cost per call is
 *                  small.  The calls follow the variable-length attention
 *                  convention: packed tokens, cu_seqlens, max_seqlen.
 *   [blog-method]  agents-report.net, "Triton Ragged Attention 與
 *                  pack-attend-unpack", section 方法概覽 (method overview):
 *                  pack (cu_seqlens + destination indices from the pruning
 *                  decision, then a vectorised copy of the surviving tokens into
 *                  one flat buffer), ragged attention on that buffer, unpack
 *                  (write results back to their batch positions via cu_seqlens).
 *   [blog-problem] same page, section 問題 (problem): the padded form pads every
 *                  image to one length and masks, reading and writing the whole
 *                  padded tensor.
 *
 * Conventions for every call:
 *   - All tensors are device memory owned by the caller.  The library never
 *     allocates or frees on these paths; it owns only rag_pipeline objects.
 *   - Every call enqueues its kernel(s) on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream) and returns without synchronising.  No
 *     value travels back to the host: T = cu_seqlens[B] and the longest kept
 *     length stay on the device, and grids are sized from host-side upper
 *     bounds (B, N, max_seqlen).
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns an error status and enqueues nothing.  Device data
 *     (keep bytes, cu_seqlens, gather_idx) is the caller's contract; kernels
 *     clamp offsets and indices into the buffers they were given, so bad data
 *     gives wrong numbers, not out-of-bounds accesses.
 *   - Nothing throws across the ABI and nothing aborts.  After a non-OK status,
 *     rag_last_error() returns a message for the calling thread.
 *   - Buffers passed to one call must not overlap, except q/k/v, which may be
 *     views into one fused row.
 */
#ifndef RAG_H
#define RAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(RAG_BUILDING_LIBRARY)
#define RAG_API __attribute__((visibility("default")))
#else
#define RAG_API
#endif

/* Status of every call. */
typedef enum rag_status {
    RAG_OK = 0,
    RAG_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, stride too small, ... */
    RAG_ERR_UNSUPPORTED = 2, /* head_dim != 64, unknown dtype or flag, size over a limit */
    RAG_ERR_ALIGNMENT = 3,   /* pointer, stride or row size not a multiple of 16 bytes */
    RAG_ERR_HIP = 4,         /* the HIP runtime reported an error (text in rag_last_error) */
    RAG_ERR_NO_MEMORY = 5    /* a host-side allocation of the library failed */
} rag_status;

/* Element types. */
typedef enum rag_dtype {
    RAG_DTYPE_F32 = 0,  /* IEEE binary32 */
    RAG_DTYPE_BF16 = 1  /* bfloat16 (upper half of binary32) */
} rag_dtype;

/* The only head dimension the attention kernels are built for (DeiT: 64). */
#define RAG_HEAD_DIM 64
/* Largest N (tokens per image before pruning) pack/unpack/padded accept. */
#define RAG_MAX_N 8192
/* Largest B (images per call). */
#define RAG_MAX_B 65535

/* rag_unpack flag: also write zeros to the dst rows of dropped tokens. */
#define RAG_UNPACK_ZERO_DROPPED 1u

/*
 * rag_pack -- keep mask to cu_seqlens and gather index, then copy the kept
 * token rows into one flat buffer ([blog-method], fused token packing).
 *
 *   keep        [B, N] uint8, row-major (row stride N), 16-byte aligned base.
 *               A nonzero byte keeps the token.  Position n of image b is the
 *               source row b*N + n.
 *   src         token rows; row r starts at src + r*src_row_stride (bytes).
 *   row_bytes   bytes copied per token row (e.g. a fused q|k|v row of
 *               3*H*64 elements); multiple of 16.
 *   packed      output rows, capacity B*N rows (T is known only on the
 *               device); row t at packed + t*packed_row_stride (bytes).
 *               Rows t >= T are not written.
 *   cu_seqlens  out, int32[B+1]: cu[0] = 0, cu[b+1] = cu[b] + L_b, where L_b
 *               is the number of kept tokens of image b.
 *   gather_idx  out, int32, capacity B*N: gather_idx[cu[b] + i] = b*N + n_i
 *               where n_0 < n_1 < ... are image b's kept positions (tokens keep
 *               their original order).  Entries >= T are not written.
 *   max_seqlen_dev  out, int32[1], max_b L_b; may be NULL (then not computed).
 *
 * Every output is a plain function of keep and src: bit-exact and the same on
 * every run.  Pointers (keep, src, packed) and strides must be multiples of 16
 * bytes (RAG_ERR_ALIGNMENT); strides must be >= row_bytes, and max(N, 64) rows
 * of either stride must span less than 2^31 bytes.  1 <= B <= RAG_MAX_B,
 * 1 <= N <= RAG_MAX_N.
 */
RAG_API rag_status rag_pack(const uint8_t* keep, int32_t B, int32_t N, const void* src,
                            int64_t src_row_stride, int32_t row_bytes, void* packed,
                            int64_t packed_row_stride, int32_t* cu_seqlens,
                            int32_t* gather_idx, int32_t* max_seqlen_dev, void* stream);

/*
 * rag_repack -- a later pruning stage on already packed tokens: keep a subset
 * of each image's packed rows, with no round trip through the [B, N] layout.
 * The pages' pruning methods ([abstract-v1]: Threshold-L2, DynamicViT, EViT,
 * ATS) drop tokens at more than one depth; this is the pack step
 * ([blog-method]) applied to a packed buffer.
 *
 *   keep_packed  uint8, one byte per input packed row (nonzero keeps it), at
 *                least total_rows bytes, 16-byte aligned base.
 *   cu_in        int32[B+1], device: image b is input rows cu_in[b] ..
 *                cu_in[b+1]-1; cu_in[0] = 0, non-decreasing (values are
 *                clamped to [0, total_rows]).
 *   gather_in    int32, device: the original batch row of each input row
 *                (e.g. rag_pack's gather_idx).
 *   max_rows_in  host bound of rows per input image (e.g. the max_seqlen of
 *                the previous stage), 1 .. RAG_MAX_N.  Images must not be
 *                longer (a longer image is read as its first max_rows_in rows
 *                and the outputs are then unspecified, though every access
 *                stays inside the buffers).
 *   total_rows   rows of the input buffers (capacity).
 *   src          input packed rows (row t at src + t*src_row_stride bytes).
 *   dst          output rows, capacity total_rows; must not overlap src.
 *   cu_out       out, int32[B+1]: cu_out[0] = 0, cu_out[b+1] = cu_out[b] + the
 *                number of kept rows of image b.
 *   gather_out   out, int32, capacity total_rows: gather_out[cu_out[b] + i] =
 *                gather_in[t_i], t_0 < t_1 < ... the kept input rows of image
 *                b -- the original batch row, so rag_unpack with cu_out /
 *                gather_out writes straight back to the [B, N] layout.
 *
 * Bit-exact; same alignment and stride rules as rag_pack, with max_rows_in in
 * the role of N.
 */
RAG_API rag_status rag_repack(const uint8_t* keep_packed, const int32_t* cu_in,
                              const int32_t* gather_in, int32_t B, int32_t max_rows_in,
                              int32_t total_rows, const void* src, int64_t src_row_stride,
                              int32_t row_bytes, void* dst, int64_t dst_row_stride,
                              int32_t* cu_out, int32_t* gather_out, void* stream);

/*
 * rag_attn -- bidirectional multi-head attention on packed ragged sequences
 * ([abstract]; [blog-method], ragged attention kernel).
 *
 * Image b owns packed rows cu_seqlens[b] .. cu_seqlens[b+1]-1.  For every head
 * h and every row i of image b:
 *     O[i, h] = sum_j softmax_j(scale * Q[i, h] . K[j, h]) V[j, h]
 * with j over the rows of image b only (no causal mask, no cross-image terms).
 *
 *   q, k, v     packed rows; head h of row t is the `head_dim` elements at
 *               X + t*X_row_stride + h*head_dim (strides in ELEMENTS).  q, k, v
 *               may be views into one fused row (q | k | v).
 *   in_dtype    BF16, or F32 (each value is then split exactly enough into a
 *               bf16 high and low part that the result matches fp32 inputs).
 *   cu_seqlens  int32[B+1], device; non-decreasing, values in [0, total_rows].
 *   max_seqlen  host-side upper bound of max_b L_b (e.g. N).  Sizes the grid;
 *               an image longer than max_seqlen is treated as its first
 *               max_seqlen rows (later rows are neither attended nor written).
 *   total_rows  capacity of q/k/v/o in rows; cu values are clamped to it.
 *   H, head_dim heads; head_dim must be RAG_HEAD_DIM.
 *   scale       softmax scale (finite), e.g. 1/sqrt(64).
 *   o           output rows (same row indexing); out_dtype F32, or BF16
 *               (round to nearest even of the value the F32 mode stores).
 *
 * Arithmetic: bf16 MFMA products with fp32 accumulation and an fp32 online
 * softmax; the softmax weights are split into bf16 high + low parts for the
 * P.V product.  Deterministic (no atomics).  Max abs error vs exact fp64
 * attention on the same inputs: <= 2e-3 for F32 output (measured well below).
 * Pointers must be 16-byte aligned and row strides multiples of 16 bytes;
 * max_seqlen times the widest row stride must stay below 2^31 bytes, and B*H
 * must not exceed 2^31 - 1 (RAG_ERR_UNSUPPORTED otherwise; also for
 * rag_attn_padded and rag_attn_gathered).
 */
RAG_API rag_status rag_attn(const void* q, const void* k, const void* v, int64_t q_row_stride,
                            int64_t k_row_stride, int64_t v_row_stride, rag_dtype in_dtype,
                            const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                            int32_t total_rows, int32_t H, int32_t head_dim, float scale,
                            void* o, int64_t o_row_stride, rag_dtype out_dtype, void* stream);

/*
 * rag_attn_tiled -- rag_attn launched over a device-built tile list
 * ([abstract]: attention on ragged post-pruning lengths; the work list is this
 * library's design).
 *
 *   Same arguments, result and error behaviour as rag_attn, and the same
 *   values bit for bit.  Instead of a grid with one slot per (head, image,
 *   query tile) -- where every image gets as many slots as the longest one and
 *   a short image's extra slots exit at once -- the launch is a 1-D grid whose
 *   workgroups each derive one work item (an (image, head) pair, or one 64-row
 *   query tile of it) from cu_seqlens on the device: items of images with more
 *   64-key tiles come first, and all items of one pair run on one XCD.
 *   Limits: B <= 1024, H <= 64 and max_seqlen <= 960 (RAG_ERR_UNSUPPORTED
 *   otherwise, before any launch).
 */
RAG_API rag_status rag_attn_tiled(const void* q, const void* k, const void* v,
                                  int64_t q_row_stride, int64_t k_row_stride, int64_t v_row_stride,
                                  rag_dtype in_dtype, const int32_t* cu_seqlens, int32_t B,
                                  int32_t max_seqlen, int32_t total_rows, int32_t H,
                                  int32_t head_dim, float scale, void* o, int64_t o_row_stride,
                                  rag_dtype out_dtype, void* stream);

/*
 * rag_unpack -- scatter packed rows back to their batch positions
 * ([blog-method], write-back via cu_seqlens).
 *
 *   dst row gather_idx[t] = packed row t, for t < cu_seqlens[B].  Rows of
 *   dropped tokens are left untouched, unless flags has
 *   RAG_UNPACK_ZERO_DROPPED, in which case they are set to zero bytes.
 *   cu_seqlens / gather_idx as produced by rag_pack (gather values of image b
 *   lie in [b*N, (b+1)*N); others are skipped).  Same alignment and span
 *   rules as rag_pack.  Bit-exact.
 */
RAG_API rag_status rag_unpack(const void* packed, int64_t packed_row_stride, int32_t row_bytes,
                              const int32_t* cu_seqlens, const int32_t* gather_idx, int32_t B,
                              int32_t N, void* dst, int64_t dst_row_stride, uint32_t flags,
                              void* stream);

/*
 * rag_attn_padded -- the padded comparator ([blog-problem]): the same
 * attention on the unpacked [B, N] layout, every image padded to N rows, key n
 * of image b taking part only if keep[b*N + n] != 0.  Every query row (kept or
 * dropped) is written; kept rows equal rag_attn's result up to rounding.  An
 * image with no kept token gets zero rows.  Work is B*N*N per head whatever the
 * prune rate.  q/k/v/o rows are b*N + n; other arguments as in rag_attn.
 */
RAG_API rag_status rag_attn_padded(const void* q, const void* k, const void* v,
                                   int64_t q_row_stride, int64_t k_row_stride,
                                   int64_t v_row_stride, rag_dtype in_dtype, const uint8_t* keep,
                                   int32_t B, int32_t N, int32_t H, int32_t head_dim, float scale,
                                   void* o, int64_t o_row_stride, rag_dtype out_dtype,
                                   void* stream);

/*
 * rag_attn_gathered -- the whole pack -> attend -> unpack pass as ONE launch
 * ([blog-method]: the same three steps; [abstract]: per-call dispatch is what
 * hides the pruning savings, so fewer launches is the point).
 *
 * Same attention as rag_attn, but on the unpacked [B, N] layout: the rows of
 * image b are b*N + n_0, b*N + n_1, ... where n_0 < n_1 < ... are the positions
 * with keep[b*N + n] != 0, read straight from q/k/v (no packed copy), and O is
 * written straight to those rows of o (no unpack copy).  No cu_seqlens or
 * gather index is built: each workgroup ranks its image's keep row in LDS.
 * Bit-for-bit equal to rag_pack -> rag_attn -> rag_unpack on the kept rows
 * (same kernel arithmetic, same key order).  Rows of dropped tokens are left
 * untouched, or zeroed with RAG_UNPACK_ZERO_DROPPED.  keep [B, N] uint8 (any
 * alignment); other arguments as in rag_attn_padded.
 *   max_seqlen  host-side upper bound of the kept count per image, in [0, N];
 *               0 means N.  It sizes the launch (LDS and waves per workgroup),
 *               so a tight bound (e.g. the pruning method's kept count) is
 *               faster.  As in rag_attn, an image with more kept rows is
 *               treated as its first max_seqlen kept rows (later kept rows are
 *               neither attended nor written).
 */
RAG_API rag_status rag_attn_gathered(const uint8_t* keep, int32_t B, int32_t N,
                                     int32_t max_seqlen, const void* q,
                                     const void* k, const void* v, int64_t q_row_stride,
                                     int64_t k_row_stride, int64_t v_row_stride,
                                     rag_dtype in_dtype, int32_t H, int32_t head_dim, float scale,
                                     void* o, int64_t o_row_stride, rag_dtype out_dtype,
                                     uint32_t flags, void* stream);

/*
 * A whole pack -> attend -> unpack pass captured once into a HIP graph, so
 * that each later pass costs one host call ([abstract]: the per-call host
 * dispatch cost is what hides the pruning savings).  The same pass can also
 * be enqueued from one host call as direct launches (rag_pipeline_launch_eager:
 * three; rag_pipeline_launch_fused: one), which on ROCm 7.2 is the lower-latency
 * choice: one hipGraphLaunch costs more host time than three direct launches,
 * whatever the graph holds (rag_measure_dispatch reports both, and a graph of
 * one empty kernel beside them).
 *
 * The attention reads fused rows of the packed buffer: q at element 0, k at
 * element H*64, v at element 2*H*64 of each row (src rows are [3, H, 64]).
 * Buffers are fixed at creation; relaunching reads the current contents.
 */
/* rag_pipeline_desc.flags.
 * RAG_PIPELINE_FUSED: the pass is the one-launch pass (rag_attn_gathered,
 *   src -> dst) instead of the three stages.
 * RAG_PIPELINE_DIRECT: rag_pipeline_launch enqueues the pass as direct
 *   launches (three, or one with RAG_PIPELINE_FUSED) instead of replaying a
 *   graph; no graph is captured.  On ROCm 7.2 this is the lower-latency
 *   pipeline: with both flags, one rag_pipeline_launch is one kernel launch.
 *   Measured round trips (launch + stream sync) at B <= 4: 14.4-17.9 us with
 *   both flags, against ~31 us for the graph and 16.4 us for padded attention
 *   alone, whose latency the fused pass beats from 50% pruning on. */
#define RAG_PIPELINE_FUSED 1u
#define RAG_PIPELINE_DIRECT 2u
typedef struct rag_pipeline_desc {
    const uint8_t* keep;     /* [B, N] */
    int32_t B, N, H, head_dim;
    rag_dtype in_dtype;      /* element type of src / packed */
    rag_dtype out_dtype;     /* element type of o_packed / dst */
    float scale;
    int32_t max_seqlen;      /* host upper bound, <= N; 0 means N */
    const void* src;         /* [B*N] fused rows of 3*H*64 elements */
    int64_t src_row_stride;  /* bytes */
    void* packed;            /* capacity B*N fused rows */
    int64_t packed_row_stride; /* bytes */
    int32_t* cu_seqlens;     /* [B+1] */
    int32_t* gather_idx;     /* capacity B*N */
    int32_t* max_seqlen_dev; /* [1] or NULL */
    void* o_packed;          /* capacity B*N rows of H*64 out_dtype elements */
    int64_t o_packed_row_stride; /* bytes */
    void* dst;               /* [B*N] rows of H*64 out_dtype elements */
    int64_t dst_row_stride;  /* bytes */
    uint32_t unpack_flags;
    uint32_t flags;          /* 0, or RAG_PIPELINE_FUSED and / or RAG_PIPELINE_DIRECT */
} rag_pipeline_desc;

typedef struct rag_pipeline rag_pipeline;

/* Check the descriptor, capture the pass (the three calls, or with
 * RAG_PIPELINE_FUSED the one gathered launch) into a graph and instantiate it
 * (not with RAG_PIPELINE_DIRECT).  Runs nothing on the device.  *out is NULL
 * on error. */
RAG_API rag_status rag_pipeline_create(const rag_pipeline_desc* desc, rag_pipeline** out);
/* Enqueue one pass on `stream`: a single hipGraphLaunch of the captured pass,
 * or with RAG_PIPELINE_DIRECT the pass's direct launches. */
RAG_API rag_status rag_pipeline_launch(rag_pipeline* p, void* stream);
/* Enqueue the same pass as three plain launches (no graph) on `stream`. */
RAG_API rag_status rag_pipeline_launch_eager(rag_pipeline* p, void* stream);
/* Enqueue the same pass as one rag_attn_gathered launch on `stream`: src -> dst
 * directly (packed, o_packed, cu_seqlens and gather_idx are not touched). */
RAG_API rag_status rag_pipeline_launch_fused(rag_pipeline* p, void* stream);
/* Free the graph; the caller must make sure no launch is still pending. */
RAG_API void rag_pipeline_destroy(rag_pipeline* p);

/*
 * Host-side dispatch measurement (the quantity [abstract] is about), taken in
 * C++ with no Python in the loop.  Times, in microseconds, with
 * std::chrono::steady_clock over `iters` repetitions after `warmup`:
 *   [0..2]   empty kernel: launch + hipStreamSynchronize, p10 / p50 / p90
 *   [3..5]   empty kernel: host enqueue only (launch call return), p10/p50/p90
 *   [6..8]   rag_attn from the pipeline desc: launch + sync
 *   [9..11]  rag_attn: host enqueue only
 *   [12..14] pack + attn + unpack as three launches: launch + sync
 *   [15..17] the same pass as one hipGraphLaunch: launch + sync
 *   [18..20] rag_attn_padded on the desc's src/keep (output into dst): launch + sync
 *   [21..23] the pass as one rag_attn_gathered launch: launch + sync
 *   [24..26] rag_attn_gathered: host enqueue only
 *   [27..29] an empty kernel taking one pointer argument: host enqueue only
 *            (beside [3..5], the runtime's cost of passing kernel arguments)
 *   [30..32] a graph holding one empty kernel: hipGraphLaunch + sync
 *   [33..35] the same: the hipGraphLaunch call alone (beside [3..5], the
 *            runtime's cost of launching a graph rather than a kernel)
 * `out_us` must hold RAG_FLOOR_N doubles.  Runs work on `stream`.
 */
#define RAG_FLOOR_N 36
RAG_API rag_status rag_measure_dispatch(rag_pipeline* p, int32_t warmup, int32_t iters,
                                        double* out_us, void* stream);

/*
 * Device time per launch, in microseconds, of each stage of the pipeline's
 * workload: HIP events on `stream` around `iters` back-to-back launches (after
 * iters/10 unmeasured ones), divided by `iters`.  Launches come from C++, so the
 * figure is the kernel's duration plus the hardware's launch-to-launch gap,
 * with no host overhead when the kernel outlasts its own enqueue.
 *   [0] rag_pack  [1] rag_attn  [2] rag_unpack  [3] rag_attn_padded (on the
 *   desc's src / keep, output into dst)  [4] pack + attn + unpack as three
 *   launches  [5] the same pass as one hipGraphLaunch  [6] the same pass as one
 *   rag_attn_gathered launch
 * `out_us` must hold RAG_STAGES_N doubles.  Overwrites the desc's buffers.
 */
#define RAG_STAGES_N 7
RAG_API rag_status rag_measure_stages(rag_pipeline* p, int32_t iters, double* out_us, void* stream);

/*
 * ---- one ViT encoder block on packed rows (end-to-end timing) ----------------
 *
 * [abstract] reports end-to-end throughput of pruned DeiT models whose blocks
 * run on the packed tokens; the pages fix the attention and the packing, not
 * the rest of the block.  rag_block runs DeiT's pre-norm encoder block with
 * the caller's (e.g. random) weights on [rows, C] bf16 token rows, C = H * 64:
 *     h = LN1(x); qkv = h Wqkv^T + bqkv; a = attention(qkv);
 *     x1 = x + a Wproj^T + bproj; m = GELU(LN2(x1) W1^T + b1); y = x1 + m W2^T + b2
 * with GELU the exact x * Phi(x) (Phi the standard normal CDF) and every step
 * a kernel of this library: LayerNorm (biased variance, eps inside the root),
 * the matrix products (bf16 inputs, fp32 accumulation, bias / GELU / residual
 * applied before the one rounding to bf16), and the attention (ragged over
 * cu_seqlens, or the padded form over keep).  Every intermediate is stored as
 * bf16.
 *
 * Weights: bf16, row-major [out, in] -- the layout of a linear layer's weight
 * (y = x W^T) -- 16-byte aligned; Wqkv's output rows are q | k | v, each
 * head-major (head h = rows h*64 ..).  Biases and LayerNorm gamma / beta:
 * fp32, 16-byte aligned.  The descriptor's pointers must stay valid while the
 * block exists.
 */
typedef struct rag_block_desc {
    int32_t H;          /* heads; C = H * 64, at most 2048 */
    int32_t mlp_ratio;  /* MLP hidden width = mlp_ratio * C (DeiT: 4), 1 .. 8 */
    float eps;          /* LayerNorm epsilon (DeiT: 1e-6), > 0 */
    float scale;        /* attention scale (e.g. 1/sqrt(64)), finite */
    const void* ln1_gamma;
    const void* ln1_beta;
    const void* w_qkv;  /* [3C, C] */
    const void* b_qkv;  /* [3C] */
    const void* w_proj; /* [C, C] */
    const void* b_proj; /* [C] */
    const void* ln2_gamma;
    const void* ln2_beta;
    const void* w_fc1;  /* [mlp_ratio*C, C] */
    const void* b_fc1;  /* [mlp_ratio*C] */
    const void* w_fc2;  /* [C, mlp_ratio*C] */
    const void* b_fc2;  /* [C] */
} rag_block_desc;

typedef struct rag_block rag_block;

/* Device scratch a forward pass over `rows` rows needs (0 for bad arguments):
 * the bf16 intermediates, rows * (6C + mlp_ratio*C) * 2 bytes. */
RAG_API size_t rag_block_scratch_bytes(int32_t rows, int32_t H, int32_t mlp_ratio);
/* Checks the descriptor and keeps a copy; allocates only the small host-side
 * object, no device memory. */
RAG_API rag_status rag_block_create(const rag_block_desc* desc, rag_block** out);
/* y = block(x) over `rows` packed rows (a host value: e.g. B times the kept
 * count of a fixed-rate pruning stage); attention over cu_seqlens (int32[B+1],
 * device) with max_seqlen as in rag_attn.  x, y: bf16 [rows, C] contiguous,
 * 16-byte aligned, not overlapping.  scratch: caller-owned device memory of
 * >= rag_block_scratch_bytes(rows, ...) bytes, 16-byte aligned.  Seven kernel
 * launches on `stream`; nothing is allocated or synchronised. */
RAG_API rag_status rag_block_forward(rag_block* blk, const void* x, void* y, int32_t rows,
                                     const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                     void* scratch, size_t scratch_bytes, void* stream);
/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward as rag_block_forward, with the intermediates in a static device
 * array of the library instead of a caller-provided scratch buffer.
 *   - Limit: rows * (6C + mlp_ratio*C) * 2 bytes must fit its 128 MiB
 *     (e.g. 17476 rows of DeiT-S, C = 384; 8738 rows of DeiT-B, C = 768);
 *     larger calls return RAG_ERR_UNSUPPORTED and enqueue nothing.
 *   - Nothing is allocated or freed by this call (no hipMalloc / hipFree, no
 *     allocating library routine).  Each GPU the library runs on holds one
 *     copy of the array until the process ends; its device address is looked
 *     up once per device (rag_block_create does it for the current device).
 *   - Every static call on one GPU shares that GPU's array: calls that overlap
 *     on one GPU (two streams, two threads) race and give wrong results;
 *     serialise them.  Nothing in the array must start at zero: each forward
 *     writes every intermediate before reading it.
 * Arguments, result and other errors as rag_block_forward. */
RAG_API rag_status rag_block_forward_static(rag_block* blk, const void* x, void* y, int32_t rows,
                                            const int32_t* cu_seqlens, int32_t B, int32_t max_seqlen,
                                            void* stream);
/* The same block on all B*N rows of the [B, N] layout with the padded
 * attention (keys with keep == 0 masked): the comparator of the packed pass. */
RAG_API rag_status rag_block_forward_padded(rag_block* blk, const void* x, void* y,
                                            const uint8_t* keep, int32_t B, int32_t N,
                                            void* scratch, size_t scratch_bytes, void* stream);
RAG_API void rag_block_destroy(rag_block* blk);

/* Message for the last non-OK status returned on the calling thread. */
RAG_API const char* rag_last_error(void);
/* Static name of a status code. */
RAG_API const char* rag_status_string(rag_status s);
/* Library ABI version (major*10000 + minor*100 + patch). */
RAG_API int32_t rag_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RAG_H */
