// Host-only driver for the sanitizer leg of the CPU tests: every argument
// check of librag.so (csrc/rag_validate.cpp) run on the rejection cases of
// tests/test_abi.py plus accepted calls, in a build with AddressSanitizer and
// UndefinedBehaviorSanitizer.  No HIP: the checks run before any launch, so
// fake, aligned device addresses are never dereferenced.  Prints "OK <n>" and
// exits 0 when every case returns the expected status and message.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "rag_internal.h"

using namespace rag;

static int g_cases = 0, g_fail = 0;

static void expect(rag_status got, rag_status want, const char* needle, int line)
{
    ++g_cases;
    const char* msg = rag_last_error();
    if (got != want || (needle && !std::strstr(msg, needle))) {
        ++g_fail;
        std::printf("line %d: status %d (want %d), message '%s' (want '%s')\n", line, (int)got, (int)want, msg,
                    needle ? needle : "");
    }
}
#define EXPECT(call, want, needle) expect((call), (want), (needle), __LINE__)

static const rag_status OK = RAG_OK, INV = RAG_ERR_INVALID_ARG, UNS = RAG_ERR_UNSUPPORTED, ALI = RAG_ERR_ALIGNMENT;
static uint8_t* const A = reinterpret_cast<uint8_t*>(0x100000);
static int32_t* const I = reinterpret_cast<int32_t*>(0x100000);
static uint8_t* at(uintptr_t off) { return reinterpret_cast<uint8_t*>(0x100000 + off); }

int main()
{
    const float inf = INFINITY, nan = NAN;
    // ---- pack
    auto pack = [&](const uint8_t* keep, int B, int N, const void* src, int64_t ss, int rb, const void* p,
                    int64_t ps, const int32_t* cu, const int32_t* g) {
        return validate_pack(keep, B, N, src, ss, rb, p, ps, cu, g);
    };
    EXPECT(pack(A, 2, 197, A, 2304, 2304, A, 2304, I, I), OK, nullptr);
    EXPECT(pack(A, 0, 197, A, 2304, 2304, A, 2304, I, I), INV, "B=0");
    EXPECT(pack(A, 2, 0, A, 2304, 2304, A, 2304, I, I), INV, "N=0");
    EXPECT(pack(A, 70000, 197, A, 2304, 2304, A, 2304, I, I), UNS, "limits");
    EXPECT(pack(A, 2, 9000, A, 2304, 2304, A, 2304, I, I), UNS, "limits");
    EXPECT(pack(nullptr, 2, 197, A, 2304, 2304, A, 2304, I, I), INV, "keep");
    EXPECT(pack(at(3), 2, 197, A, 2304, 2304, A, 2304, I, I), ALI, "keep");
    EXPECT(pack(A, 2, 197, A, 2304, 8, A, 2304, I, I), INV, "row_bytes");
    EXPECT(pack(A, 2, 197, A, 2304, 2308, A, 2304, I, I), ALI, "row_bytes");
    EXPECT(pack(A, 2, 197, nullptr, 2304, 2304, A, 2304, I, I), INV, "src");
    EXPECT(pack(A, 2, 197, at(8), 2304, 2304, A, 2304, I, I), ALI, "src");
    EXPECT(pack(A, 2, 197, A, 2000, 2304, A, 2304, I, I), INV, "src row stride");
    EXPECT(pack(A, 2, 197, A, 2304, 2304, A, 2328, I, I), ALI, "packed");
    EXPECT(pack(A, 2, 197, A, 2304, 2304, A, 2304, nullptr, I), INV, "cu_seqlens");
    EXPECT(pack(A, 2, 197, A, 2304, 2304, A, 2304, I, nullptr), INV, "gather_idx");
    EXPECT(pack(A, 2, 8192, A, 1 << 20, 2304, A, 2304, I, I), UNS, "2^31");
    // ---- repack
    auto repack = [&](const uint8_t* keep, const int32_t* ci, const int32_t* gi, int B, int maxr, int total,
                      const void* src, int64_t ss, int rb, const void* dst, int64_t ds, const int32_t* co,
                      const int32_t* go) {
        return validate_repack(keep, ci, gi, B, maxr, total, src, ss, rb, dst, ds, co, go);
    };
    uint8_t* D = at(0x1000000);
    EXPECT(repack(A, I, I, 2, 40, 80, A, 2304, 2304, D, 2304, I, I), OK, nullptr);
    EXPECT(repack(A, I, I, 0, 40, 80, A, 2304, 2304, D, 2304, I, I), INV, "B=0");
    EXPECT(repack(A, I, I, 2, 9000, 80, A, 2304, 2304, D, 2304, I, I), UNS, "limits");
    EXPECT(repack(A, I, I, 2, 40, -1, A, 2304, 2304, D, 2304, I, I), INV, "total_rows");
    EXPECT(repack(nullptr, I, I, 2, 40, 80, A, 2304, 2304, D, 2304, I, I), INV, "keep_packed");
    EXPECT(repack(at(3), I, I, 2, 40, 80, A, 2304, 2304, D, 2304, I, I), ALI, "keep_packed");
    EXPECT(repack(A, nullptr, I, 2, 40, 80, A, 2304, 2304, D, 2304, I, I), INV, "cu_in");
    EXPECT(repack(A, I, I, 2, 40, 80, A, 2304, 2304, D, 2300, I, I), INV, "dst row stride");
    EXPECT(repack(A, I, I, 2, 40, 80, A, 2304, 2304, A, 2304, I, I), INV, "overlap");
    EXPECT(repack(A, I, I, 2, 8192, 80, A, 1 << 20, 2304, D, 2304, I, I), UNS, "2^31");
    // ---- attention (ragged) and the tile list's limits
    auto attn = [&](const void* q, int64_t qs, int64_t ks, int dt, const int32_t* cu, int B, int maxlen,
                    int tr, int H, int hd, float scale, const void* o, int64_t os, int odt) {
        return validate_attn(q, A, A, qs, ks, 1152, dt, cu, B, maxlen, tr, H, hd, scale, o, os, odt);
    };
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, 788, 6, 64, 0.125f, A, 384, 0), OK, nullptr);
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, 788, 6, 32, 0.125f, A, 384, 0), UNS, "head_dim");
    EXPECT(attn(A, 1152, 1152, 7, I, 4, 197, 788, 6, 64, 0.125f, A, 384, 0), UNS, "dtype");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, 788, 0, 64, 0.125f, A, 384, 0), INV, "H=0");
    EXPECT(attn(A, 1152, 1152, 1, I, 0, 197, 788, 6, 64, 0.125f, A, 384, 0), INV, "B=0");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 0, 788, 6, 64, 0.125f, A, 384, 0), INV, "max_seqlen");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, -1, 6, 64, 0.125f, A, 384, 0), INV, "total_rows");
    EXPECT(attn(A, 1152, 1152, 1, nullptr, 4, 197, 788, 6, 64, 0.125f, A, 384, 0), INV, "cu_seqlens");
    EXPECT(attn(nullptr, 1152, 1152, 1, I, 4, 197, 788, 6, 64, 0.125f, A, 384, 0), INV, "q is NULL");
    EXPECT(attn(A, 100, 1152, 1, I, 4, 197, 788, 6, 64, 0.125f, A, 384, 0), INV, "q row stride");
    EXPECT(attn(A, 1152, 388, 1, I, 4, 197, 788, 6, 64, 0.125f, A, 384, 0), ALI, "k base");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, 788, 6, 64, 0.125f, A, 386, 0), ALI, "o base");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, 788, 6, 64, inf, A, 384, 0), INV, "scale");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 197, 788, 6, 64, nan, A, 384, 0), INV, "scale");
    EXPECT(attn(A, 1152, 1152, 1, I, 4, 65535 * 64 + 1, 788, 6, 64, 0.125f, A, 384, 0), UNS, "max_seqlen");
    EXPECT(validate_tile_list(1025, 6, 197), UNS, "B=1025");
    EXPECT(validate_tile_list(4, 65, 197), UNS, "H=65");
    EXPECT(validate_tile_list(4, 6, 961), UNS, "max_seqlen=961");
    EXPECT(validate_tile_list(1024, 64, 960), OK, nullptr);
    // ---- unpack, padded, gathered
    EXPECT(validate_unpack(A, 768, 768, I, I, 4, 197, A, 768, 0), OK, nullptr);
    EXPECT(validate_unpack(A, 768, 768, I, I, 4, 197, A, 768, 2), UNS, "flags");
    EXPECT(validate_unpack(A, 768, 768, nullptr, I, 4, 197, A, 768, 0), INV, "cu_seqlens");
    EXPECT(validate_unpack(A, 768, 768, I, I, 4, 197, at(4), 768, 0), ALI, "dst");
    EXPECT(validate_attn_padded(A, A, A, 1152, 1152, 1152, 1, nullptr, 4, 197, 6, 64, 0.125f, A, 384, 0), INV, "keep");
    EXPECT(validate_attn_padded(A, A, A, 1152, 1152, 1152, 1, A, 4, 197, 6, 48, 0.125f, A, 384, 0), UNS, "head_dim");
    EXPECT(validate_attn_gathered(A, 4, 197, 0, A, A, A, 1152, 1152, 1152, 1, 6, 64, 0.125f, A, 384, 0, 2), UNS, "flags");
    EXPECT(validate_attn_gathered(A, 4, 197, 198, A, A, A, 1152, 1152, 1152, 1, 6, 64, 0.125f, A, 384, 0, 0), INV, "max_seqlen");
    EXPECT(validate_attn_gathered(A, 4, 197, 40, A, A, A, 1152, 1152, 1152, 1, 6, 64, 0.125f, A, 384, 0, 1), OK, nullptr);
    // ---- pipeline descriptor
    rag_pipeline_desc d;
    std::memset(&d, 0, sizeof d);
    d.keep = A; d.B = 4; d.N = 197; d.H = 6; d.head_dim = 64; d.in_dtype = RAG_DTYPE_BF16; d.out_dtype = RAG_DTYPE_BF16;
    d.scale = 0.125f; d.src = A; d.src_row_stride = 2304; d.packed = A; d.packed_row_stride = 2304;
    d.cu_seqlens = I; d.gather_idx = I; d.o_packed = A; d.o_packed_row_stride = 768; d.dst = A; d.dst_row_stride = 768;
    EXPECT(validate_pipeline(&d), OK, nullptr);
    EXPECT(validate_pipeline(nullptr), INV, "desc");
    rag_pipeline_desc e = d; e.head_dim = 80;
    EXPECT(validate_pipeline(&e), UNS, "head_dim");
    e = d; e.max_seqlen = 500;
    EXPECT(validate_pipeline(&e), INV, "max_seqlen");
    e = d; e.src_row_stride = 2000;
    EXPECT(validate_pipeline(&e), INV, "src row stride");
    e = d; e.dst = at(8);
    EXPECT(validate_pipeline(&e), ALI, "dst");
    e = d; e.unpack_flags = 4;
    EXPECT(validate_pipeline(&e), UNS, "flags");
    e = d; e.flags = 4;
    EXPECT(validate_pipeline(&e), UNS, "pipeline flags");
    e = d; e.flags = RAG_PIPELINE_FUSED;
    EXPECT(validate_pipeline(&e), OK, nullptr);
    e = d; e.flags = RAG_PIPELINE_DIRECT | RAG_PIPELINE_FUSED;
    EXPECT(validate_pipeline(&e), OK, nullptr);
    // ---- encoder block
    rag_block_desc b;
    std::memset(&b, 0, sizeof b);
    b.H = 6; b.mlp_ratio = 4; b.eps = 1e-6f; b.scale = 0.125f;
    const void** ptrs[] = {&b.ln1_gamma, &b.ln1_beta, &b.w_qkv, &b.b_qkv, &b.w_proj, &b.b_proj,
                           &b.ln2_gamma, &b.ln2_beta, &b.w_fc1, &b.b_fc1, &b.w_fc2, &b.b_fc2};
    for (int i = 0; i < 12; ++i) *ptrs[i] = at(0x1000 * i);
    EXPECT(validate_block_desc(&b), OK, nullptr);
    rag_block_desc c = b; c.H = 33;
    EXPECT(validate_block_desc(&c), UNS, "H=33");
    c = b; c.mlp_ratio = 9;
    EXPECT(validate_block_desc(&c), UNS, "mlp_ratio");
    c = b; c.eps = 0.f;
    EXPECT(validate_block_desc(&c), INV, "eps");
    c = b; c.w_qkv = nullptr;
    EXPECT(validate_block_desc(&c), INV, "w_qkv");
    c = b; c.b_fc2 = at(4);
    EXPECT(validate_block_desc(&c), ALI, "b_fc2");
    EXPECT(validate_block_call(A, A, 100, 384, A, 1 << 20, 1 << 19), OK, nullptr);
    EXPECT(validate_block_call(A, A, -1, 384, A, 1 << 20, 1 << 19), INV, "rows");
    EXPECT(validate_block_call(A, A, 100, 384, A, 1 << 18, 1 << 19), INV, "scratch");
    EXPECT(validate_block_call(A, at(8), 100, 384, A, 1 << 20, 1 << 19), ALI, "aligned");
    EXPECT(validate_block_call(A, A, 1 << 30, 384, A, 1 << 20, 1 << 19), UNS, "too large");
    // the error text survives a long message (truncated, not overrun)
    EXPECT(set_error(RAG_ERR_INVALID_ARG, "%0600d", 7), INV, "0000");
    if (g_fail) {
        std::printf("FAILED %d of %d\n", g_fail, g_cases);
        return 1;
    }
    std::printf("OK %d\n", g_cases);
    return 0;
}
