// C-ABI front end of libattn.so: argument checks (host only, before any HIP
// call), chunk-size choice and workspace sizing for split-KV decode, and the
// launches on the caller's stream.  The contract of every entry point is in
// include/attn.h.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.h"
#include "attn_kernels.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

// Clear a stale error left by an unrelated earlier call, launch, and map the result.
template <typename F>
int run(F &&launch)
{
    (void)hipGetLastError();
    const hipError_t e = launch();
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Workgroups the split kernel should have at full capacity when the caller
// leaves the chunk size to the library: enough to keep all 256 compute units
// busy several times over, so uneven sequence lengths still balance.
constexpr long long kDecodeTargetWorkgroups = 1024;
constexpr int kDecodeMinChunk = 256;   // one pass of a split workgroup (8 waves x 32 tokens)
constexpr int kDecodeMaxChunk = 2048;  // longer chunks unbalance mixed-length batches

// Resolved chunk size, or a negative status.
int resolve_chunk(int batch, int n_kv_heads, int page_size, int max_blocks, int chunk_tokens)
{
    if (batch < 0 || n_kv_heads <= 0 || page_size <= 0 || max_blocks <= 0 || chunk_tokens < 0)
        return ATTN_ERR_SHAPE;
    const long long cap = (long long)max_blocks * page_size;
    if (cap > INT_MAX) return ATTN_ERR_UNSUPPORTED;
    if (chunk_tokens > 0) {
        if (chunk_tokens % attn::kDecodeTokenQuantum != 0) return ATTN_ERR_UNSUPPORTED;
        return chunk_tokens;
    }
    const long long units = (long long)(batch > 0 ? batch : 1) * n_kv_heads;
    const long long splits = (kDecodeTargetWorkgroups + units - 1) / units;
    long long chunk = (cap + splits - 1) / splits;
    chunk = (chunk + kDecodeMinChunk - 1) / kDecodeMinChunk * kDecodeMinChunk;
    if (chunk < kDecodeMinChunk) chunk = kDecodeMinChunk;
    if (chunk > kDecodeMaxChunk) chunk = kDecodeMaxChunk;
    return (int)chunk;
}

// Balanced split: with automatic chunking and several sequences, the split kernel
// runs this many workgroups in all (one resident 8-wave workgroup on each of the
// 256 compute units; 512 and 1024 measured slower on a batch of 32 mixed lengths),
// each KV head's share taking an equal part of that head's tokens across sequence
// boundaries, so a batch of mixed lengths ends with every workgroup busy until
// about the same time.
constexpr int kDecodeBalancedWorkgroups = 256;

int balanced_gh(int batch, int n_kv_heads, int chunk_tokens, bool variant)
{
    if (chunk_tokens != 0 || batch < 2 || variant || n_kv_heads <= 0) return 0;
    return kDecodeBalancedWorkgroups / n_kv_heads > 1 ? kDecodeBalancedWorkgroups / n_kv_heads : 1;
}

// Partials one sequence can have in the balanced split: at most one per workgroup
// of its KV head, and at most one per unit (one workgroup pass) of its tokens.
long long balanced_splits(int gh, int head_dim, long long capacity)
{
    const long long unit = (long long)attn::decode_split_waves(head_dim) * attn::kDecodeStepTokens;
    const long long units = (capacity + unit - 1) / unit;
    return units < gh ? units : gh;
}

size_t partial_bytes(int batch, int n_q_heads, long long splits, int head_dim)
{
    return (size_t)batch * (size_t)n_q_heads * (size_t)splits * (size_t)(head_dim + 1) * 4u;
}

// Variant options: window -1 (none) or >= 0; softcap 0 (none) or finite > 0.
bool variant_ok(int window_left, float softcap)
{
    return window_left >= -1 && softcap >= 0.f && isfinite(softcap);
}

// Shared body of the prefill entry points: padded layout (seqlen = N,
// total_tokens unused) or, with `packed`, the packed layout described by
// cu_seqlens (seqlen = the longest sequence).
int prefill_impl(bool packed, const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu_seqlens,
                 int batch, int seqlen, int total_tokens, int n_q_heads, int n_kv_heads, int head_dim, int dtype,
                 int causal, float scale, int window_left, float softcap, void *stream)
{
    if (batch < 0 || seqlen < 0 || (packed && total_tokens < 0) || n_q_heads <= 0 || n_kv_heads <= 0 ||
        head_dim <= 0 || !variant_ok(window_left, softcap))
        return ATTN_ERR_SHAPE;
    if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_GQA;
    if (!head_dim_ok(head_dim) || (dtype != ATTN_F32 && dtype != ATTN_BF16))
        return ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || seqlen == 0 || (packed && total_tokens == 0)) return ATTN_OK;
    if (!q || !k || !v || !o || !lse || (packed && !cu_seqlens)) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return ATTN_ERR_ALIGN;
    // element offsets are formed in 64-bit; the grid is one dimension of query
    // tiles, and one head's rows of one sequence (seqlen rounded up to a tile)
    // are addressed through a descriptor with a 32-bit range
    const long long row_bytes =
        packed ? (long long)n_q_heads * head_dim * (dtype == ATTN_F32 ? 4 : 2) : (long long)head_dim * 2;
    if ((long long)batch * n_q_heads * ((seqlen + 63) / 64) > INT_MAX ||
        ((long long)seqlen + 255) * row_bytes > 0xffffffffLL)
        return ATTN_ERR_UNSUPPORTED;

    attn::PrefillParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.B = batch; p.N = seqlen; p.Hq = n_q_heads; p.Hkv = n_kv_heads; p.head_dim = head_dim;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.cu_seqlens = packed ? cu_seqlens : nullptr;
    p.total = packed ? total_tokens : 0;
    p.window = window_left;
    p.softcap = softcap;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ATTN_BF16) return run([&] { return attn::launch_prefill_bf16(p, s); });
    return run([&] { return attn::launch_prefill_f32(p, s); });
}

// Shared body of the decode entry points; `append` selects the in-place append
// (k_new and v_new are then both required).
int decode_impl(bool append, const void *q, const void *k_new, const void *v_new, const void *k_cache,
                const void *v_cache, const int32_t *block_table, const int32_t *seq_lens, void *o, float *lse_or_null, int batch,
                int n_q_heads, int n_kv_heads, int head_dim, int page_size, int max_blocks_per_seq, int dtype,
                float scale, int window_left, float softcap, int chunk_tokens, void *workspace,
                size_t workspace_bytes, void *stream, bool kv_e4m3 = false, const float *descale_k = nullptr,
                const float *descale_v = nullptr, bool static_scratch = false)
{
    if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || page_size <= 0 ||
        max_blocks_per_seq <= 0 || chunk_tokens < 0 || !variant_ok(window_left, softcap))
        return ATTN_ERR_SHAPE;
    if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_GQA;
    if (!head_dim_ok(head_dim) || dtype != ATTN_BF16 ||
        n_q_heads / n_kv_heads > attn::kDecodeMaxGroup || (kv_e4m3 && head_dim == 256))
        return ATTN_ERR_UNSUPPORTED;
    // paged blocks of 16 tokens must not straddle pages
    if (block_table && page_size % attn::kDecodeTokenQuantum != 0) return ATTN_ERR_UNSUPPORTED;
    const int chunk = resolve_chunk(batch, n_kv_heads, page_size, max_blocks_per_seq, chunk_tokens);
    if (chunk < 0) return chunk;
    if (batch == 0) return ATTN_OK;
    if (!q || !k_cache || !v_cache || !seq_lens || !o) return ATTN_ERR_NULL;
    if (append && (!k_new || !v_new)) return ATTN_ERR_NULL;
    const long long cap = (long long)max_blocks_per_seq * page_size;
    const long long max_chunks = (cap + chunk - 1) / chunk;
    int gh = balanced_gh(batch, n_kv_heads, chunk_tokens, window_left >= 0 || softcap > 0.f);
    const long long bal_splits = gh > 0 ? balanced_splits(gh, head_dim, cap) : 0;
    // the static scratch takes the per-chunk split when the balanced one's partials do not fit
    if (static_scratch && gh > 0 && partial_bytes(batch, n_q_heads, bal_splits, head_dim) > attn::kNoAllocScratchBytes)
        gh = 0;
    const long long splits = gh > 0 ? bal_splits : max_chunks;
    if (static_scratch) {
        if (partial_bytes(batch, n_q_heads, splits, head_dim) > attn::kNoAllocScratchBytes) return ATTN_ERR_SCRATCH;
    } else {
        const size_t need = attn_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, page_size,
                                                        max_blocks_per_seq, chunk_tokens);
        if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    }
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (!static_scratch && !aligned16(workspace)) || (lse_or_null && !aligned16(lse_or_null)) ||
        (append && (!aligned16(k_new) || !aligned16(v_new))) ||
        (reinterpret_cast<uintptr_t>(descale_k) & 3u) != 0 || (reinterpret_cast<uintptr_t>(descale_v) & 3u) != 0)
        return ATTN_ERR_ALIGN;
    if (max_chunks > attn::kMaxSplits || max_chunks * n_kv_heads > attn::kMaxSplitWorkgroups ||
        batch > 65535 || (long long)batch * n_q_heads > attn::kMaxCombineRows)
        return ATTN_ERR_UNSUPPORTED;
    // every host check has passed: only now look up this GPU's static scratch
    if (static_scratch && attn::decode_scratch(&workspace) != hipSuccess) return ATTN_ERR_HIP;

    attn::DecodeParams p;
    p.q = q; p.k_cache = k_cache; p.v_cache = v_cache;
    p.block_table = block_table; p.seq_lens = seq_lens;
    p.o = o; p.lse = lse_or_null;
    p.B = batch; p.Hq = n_q_heads; p.Hkv = n_kv_heads; p.head_dim = head_dim;
    p.page_size = page_size; p.max_blocks = max_blocks_per_seq; p.dtype = dtype;
    p.scale = scale;
    p.chunk = chunk;
    p.max_chunks = (int)splits;
    p.bal_gh = gh;
    const size_t rows = (size_t)batch * n_q_heads;
    p.k_new = k_new;
    p.v_new = v_new;
    p.window = window_left;
    p.softcap = softcap;
    p.kv_e4m3 = kv_e4m3;
    p.descale_k = descale_k;
    p.descale_v = descale_v;
    p.o_parts = static_cast<float *>(workspace);
    p.lse_parts = p.o_parts + rows * (size_t)splits * head_dim;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run([&] { return attn::launch_decode(p, s); });
}

}  // namespace

extern "C" {

int attn_decode_check_tables(const int32_t *block_table_or_null, const int32_t *seq_lens, int batch,
                             int page_size, int max_blocks_per_seq, int num_blocks, int appended, int32_t *bad_out,
                             void *stream)
{
    if (batch < 0 || page_size <= 0 || max_blocks_per_seq <= 0 || (block_table_or_null && num_blocks < 0) ||
        (appended != 0 && appended != 1))
        return ATTN_ERR_SHAPE;
    if ((!seq_lens && batch > 0) || !bad_out) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0 || (reinterpret_cast<uintptr_t>(bad_out) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(block_table_or_null) & 3u) != 0)
        return ATTN_ERR_ALIGN;
    attn::TableCheckParams p;
    p.block_table = block_table_or_null;
    p.seq_lens = seq_lens;
    p.B = batch;
    p.page_size = page_size;
    p.max_blocks = max_blocks_per_seq;
    p.num_blocks = num_blocks;
    p.appended = appended;
    p.bad_out = bad_out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run([&] { return attn::launch_check_tables(p, s); });
}

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid size argument";
    case ATTN_ERR_GQA: return "n_q_heads is not a multiple of n_kv_heads";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, group size, page size or chunk size";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_SCRATCH: return "the decode's partials exceed the static scratch of attn_decode_noalloc";
    default: return "unknown status";
    }
}

int attn_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                 int seqlen, int n_q_heads, int n_kv_heads, int head_dim, int dtype, int causal,
                 float scale, void *stream)
{
    return prefill_impl(false, q, k, v, o, lse, nullptr, batch, seqlen, 0, n_q_heads, n_kv_heads, head_dim, dtype,
                        causal, scale, -1, 0.f, stream);
}

int attn_prefill_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *cu_seqlens, int batch, int max_seqlen, int total_tokens,
                        int n_q_heads, int n_kv_heads, int head_dim, int dtype, int causal, float scale,
                        void *stream)
{
    return prefill_impl(true, q, k, v, o, lse, cu_seqlens, batch, max_seqlen, total_tokens, n_q_heads, n_kv_heads,
                        head_dim, dtype, causal, scale, -1, 0.f, stream);
}

int attn_prefill_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                     const int32_t *cu_seqlens_or_null, int batch, int seqlen, int total_tokens,
                     int n_q_heads, int n_kv_heads, int head_dim, int dtype, int causal, float scale,
                     int window_left, float softcap, void *stream)
{
    return prefill_impl(cu_seqlens_or_null != nullptr, q, k, v, o, lse, cu_seqlens_or_null, batch, seqlen,
                        total_tokens, n_q_heads, n_kv_heads, head_dim, dtype, causal, scale, window_left, softcap,
                        stream);
}

namespace {

// Shared body of the FP8 prefill entry points: padded layout (seqlen = N) or,
// with `packed`, the packed layout described by cu_seqlens (seqlen = the
// longest sequence).
int prefill_fp8_impl(bool packed, const void *q, const void *k, const void *v, void *o, float *lse,
                     const float *descale_q, const float *descale_k, const float *descale_v,
                     const int32_t *cu_seqlens, int batch, int seqlen, int total_tokens, int n_q_heads,
                     int n_kv_heads, int head_dim, int causal, float scale, int window_left, float softcap,
                     void *stream)
{
    if (batch < 0 || seqlen < 0 || (packed && total_tokens < 0) || n_q_heads <= 0 || n_kv_heads <= 0 ||
        head_dim <= 0 || !variant_ok(window_left, softcap))
        return ATTN_ERR_SHAPE;
    if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_GQA;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || seqlen == 0 || (packed && total_tokens == 0)) return ATTN_OK;
    if (!q || !k || !v || !o || !lse || (packed && !cu_seqlens)) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        (reinterpret_cast<uintptr_t>(descale_q) & 3u) != 0 || (reinterpret_cast<uintptr_t>(descale_k) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(descale_v) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0)
        return ATTN_ERR_ALIGN;
    // one head's rows of one sequence (seqlen rounded up to a 128-row tile) are
    // addressed with 32-bit offsets; a packed row holds every head
    const long long row_bytes = packed ? (long long)n_q_heads * head_dim : head_dim;
    if ((long long)batch * n_q_heads * ((seqlen + 127) / 128) > INT_MAX ||
        ((long long)seqlen + 127) * row_bytes > 0xffffffffLL)
        return ATTN_ERR_UNSUPPORTED;
    attn::PrefillFp8Params p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.descale_q = descale_q; p.descale_k = descale_k; p.descale_v = descale_v;
    p.cu_seqlens = packed ? cu_seqlens : nullptr;
    p.total = packed ? total_tokens : 0;
    p.B = batch; p.N = seqlen; p.Hq = n_q_heads; p.Hkv = n_kv_heads; p.head_dim = head_dim;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.window = window_left;
    p.softcap = softcap;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run([&] { return attn::launch_prefill_fp8(p, s); });
}

}  // namespace

int attn_prefill_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                     const float *descale_q_or_null, const float *descale_k_or_null,
                     const float *descale_v_or_null, int batch, int seqlen, int n_q_heads, int n_kv_heads,
                     int head_dim, int causal, float scale, void *stream)
{
    return prefill_fp8_impl(false, q, k, v, o, lse, descale_q_or_null, descale_k_or_null, descale_v_or_null,
                            nullptr, batch, seqlen, 0, n_q_heads, n_kv_heads, head_dim, causal, scale, -1, 0.f,
                            stream);
}

int attn_prefill_fp8_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                            const float *descale_q_or_null, const float *descale_k_or_null,
                            const float *descale_v_or_null, const int32_t *cu_seqlens, int batch,
                            int max_seqlen, int total_tokens, int n_q_heads, int n_kv_heads, int head_dim,
                            int causal, float scale, void *stream)
{
    return prefill_fp8_impl(true, q, k, v, o, lse, descale_q_or_null, descale_k_or_null, descale_v_or_null,
                            cu_seqlens, batch, max_seqlen, total_tokens, n_q_heads, n_kv_heads, head_dim, causal,
                            scale, -1, 0.f, stream);
}

int attn_prefill_fp8_ext(const void *q, const void *k, const void *v, void *o, float *lse,
                         const float *descale_q_or_null, const float *descale_k_or_null,
                         const float *descale_v_or_null, const int32_t *cu_seqlens_or_null, int batch, int seqlen,
                         int total_tokens, int n_q_heads, int n_kv_heads, int head_dim, int causal, float scale,
                         int window_left, float softcap, void *stream)
{
    return prefill_fp8_impl(cu_seqlens_or_null != nullptr, q, k, v, o, lse, descale_q_or_null, descale_k_or_null,
                            descale_v_or_null, cu_seqlens_or_null, batch, seqlen, total_tokens, n_q_heads,
                            n_kv_heads, head_dim, causal, scale, window_left, softcap, stream);
}

int attn_decode_chunk_tokens(int batch, int n_kv_heads, int page_size, int max_blocks_per_seq,
                             int chunk_tokens)
{
    return resolve_chunk(batch, n_kv_heads, page_size, max_blocks_per_seq, chunk_tokens);
}

size_t attn_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                   int page_size, int max_blocks_per_seq, int chunk_tokens)
{
    if (n_q_heads <= 0 || head_dim <= 0) return 0;
    const int chunk = resolve_chunk(batch, n_kv_heads, page_size, max_blocks_per_seq, chunk_tokens);
    if (chunk <= 0) return 0;
    const long long cap = (long long)max_blocks_per_seq * page_size;
    const long long max_chunks = (cap + chunk - 1) / chunk;
    // the larger of the per-chunk split's partials and (automatic chunking, several
    // sequences) the balanced split's, so the workspace serves the call with or
    // without a window or soft-cap
    const int gh = balanced_gh(batch, n_kv_heads, chunk_tokens, false);
    const long long splits = gh > 0 && balanced_splits(gh, head_dim, cap) > max_chunks
                                 ? balanced_splits(gh, head_dim, cap) : max_chunks;
    return partial_bytes(batch, n_q_heads, splits, head_dim);
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_table, const int32_t *seq_lens, void *o, float *lse_or_null,
                int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                int max_blocks_per_seq, int dtype, float scale, int chunk_tokens, void *workspace,
                size_t workspace_bytes, void *stream)
{
    return decode_impl(false, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, o, lse_or_null, batch,
                       n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, dtype, scale, -1, 0.f,
                       chunk_tokens, workspace, workspace_bytes, stream);
}

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_table,
                        const int32_t *seq_lens, void *o, float *lse_or_null, int batch, int n_q_heads,
                        int n_kv_heads, int head_dim, int page_size, int max_blocks_per_seq, int dtype, float scale,
                        int chunk_tokens, void *stream)
{
    return decode_impl(false, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, o, lse_or_null, batch,
                       n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, dtype, scale, -1, 0.f,
                       chunk_tokens, nullptr, 0, stream, false, nullptr, nullptr, true);
}

int attn_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                       const int32_t *block_table, const int32_t *cache_seqlens, void *o,
                       float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                       int page_size, int max_blocks_per_seq, int dtype, float scale, int chunk_tokens,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(true, q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, o, lse_or_null, batch,
                       n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, dtype, scale, -1, 0.f,
                       chunk_tokens, workspace, workspace_bytes, stream);
}

int attn_decode_ext(const void *q, const void *k_new_or_null, const void *v_new_or_null, void *k_cache,
                    void *v_cache, const int32_t *block_table, const int32_t *seq_lens, void *o,
                    float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                    int max_blocks_per_seq, int dtype, float scale, int window_left, float softcap,
                    int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(k_new_or_null || v_new_or_null, q, k_new_or_null, v_new_or_null, k_cache, v_cache,
                       block_table, seq_lens, o, lse_or_null, batch, n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, dtype, scale,
                       window_left, softcap, chunk_tokens, workspace, workspace_bytes, stream);
}

int attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache, const float *descale_k_or_null,
                    const float *descale_v_or_null, const int32_t *block_table, const int32_t *seq_lens, void *o,
                    float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                    int max_blocks_per_seq, float scale, int chunk_tokens, void *workspace, size_t workspace_bytes,
                    void *stream)
{
    return decode_impl(false, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, o, lse_or_null, batch,
                       n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, ATTN_BF16, scale, -1, 0.f,
                       chunk_tokens, workspace, workspace_bytes, stream, true, descale_k_or_null, descale_v_or_null);
}

int attn_decode_fp8_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                           const float *descale_k_or_null, const float *descale_v_or_null, const int32_t *block_table,
                           const int32_t *cache_seqlens, void *o, float *lse_or_null, int batch, int n_q_heads,
                           int n_kv_heads, int head_dim, int page_size, int max_blocks_per_seq, float scale,
                           int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(true, q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, o, lse_or_null, batch,
                       n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, ATTN_BF16, scale, -1, 0.f,
                       chunk_tokens, workspace, workspace_bytes, stream, true, descale_k_or_null, descale_v_or_null);
}

int attn_decode_fp8_ext(const void *q, const void *k_cache, const void *v_cache, const float *descale_k_or_null,
                        const float *descale_v_or_null, const int32_t *block_table, const int32_t *seq_lens, void *o,
                        float *lse_or_null, int batch, int n_q_heads, int n_kv_heads, int head_dim, int page_size,
                        int max_blocks_per_seq, float scale, int window_left, float softcap, int chunk_tokens,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(false, q, nullptr, nullptr, k_cache, v_cache, block_table, seq_lens, o, lse_or_null, batch,
                       n_q_heads, n_kv_heads, head_dim, page_size, max_blocks_per_seq, ATTN_BF16, scale, window_left,
                       softcap, chunk_tokens, workspace, workspace_bytes, stream, true, descale_k_or_null,
                       descale_v_or_null);
}

int attn_lse_combine(const float *o_parts, const float *lse_parts, const int32_t *n_splits_or_null,
                     int rows, int max_splits, int head_dim, void *o, int o_dtype,
                     float *lse_or_null, void *stream)
{
    if (rows < 0 || max_splits <= 0 || head_dim <= 0) return ATTN_ERR_SHAPE;
    if (!head_dim_ok(head_dim) || (o_dtype != ATTN_F32 && o_dtype != ATTN_BF16))
        return ATTN_ERR_UNSUPPORTED;
    if (max_splits > attn::kMaxSplits || rows > attn::kMaxCombineRows) return ATTN_ERR_UNSUPPORTED;
    if (rows == 0) return ATTN_OK;
    if (!o_parts || !lse_parts || !o) return ATTN_ERR_NULL;
    if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) ||
        (lse_or_null && !aligned16(lse_or_null)) ||
        (n_splits_or_null && !aligned16(n_splits_or_null)))
        return ATTN_ERR_ALIGN;
    attn::CombineParams p;
    p.o_parts = o_parts; p.lse_parts = lse_parts; p.n_splits = n_splits_or_null;
    p.rows = rows; p.max_splits = max_splits; p.head_dim = head_dim;
    p.o = o; p.o_bf16 = (o_dtype == ATTN_BF16); p.lse = lse_or_null;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run([&] { return attn::launch_lse_combine(p, s); });
}

}  // extern "C"
