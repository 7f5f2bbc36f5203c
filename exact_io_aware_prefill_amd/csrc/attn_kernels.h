// Internal launch interface between the C-ABI front end (attn_api.cpp) and the
// gfx950 kernels.  Not installed; callers use include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// Tiled prefill, bf16 inputs on matrix cores (prefill_bf16.hip).
struct PrefillParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, N, Hq, Hkv, head_dim, causal;
    float scale;
    // packed variable-length batch (NULL: padded [B, H, N, d]): sequence b is
    // tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of [total, H, d] tensors, lse is
    // [Hq, total], and N is the longest sequence
    const int32_t *cu_seqlens = nullptr;
    int total = 0;
    // sliding window (row i sees keys >= i - window; -1: none) and logit
    // soft-cap (scores s become softcap * tanh(s / softcap); 0: none)
    int window = -1;
    float softcap = 0.f;
};
hipError_t launch_prefill_bf16(const PrefillParams &p, hipStream_t stream);

// Tiled prefill, float32 arithmetic (prefill_f32.hip).
hipError_t launch_prefill_f32(const PrefillParams &p, hipStream_t stream);

// Tiled prefill on FP8 (E4M3) inputs, bf16 output (prefill_fp8.hip).
struct PrefillFp8Params {
    const void *q, *k, *v;  // E4M3 codes: [B, Hq | Hkv, N, head_dim], or packed [T, Hq | Hkv, head_dim]
    void *o;                // bf16, q's layout
    float *lse;             // [B, Hq, N], or packed [Hq, T]
    const float *descale_q, *descale_k, *descale_v;  // [B, Hkv] or NULL (1)
    const int32_t *cu_seqlens;  // packed layout (N = the longest sequence), or NULL
    int total;                  // packed: T
    int B, N, Hq, Hkv, head_dim, causal;
    float scale;
    int window = -1;       // as PrefillParams
    float softcap = 0.f;
};
hipError_t launch_prefill_fp8(const PrefillFp8Params &p, hipStream_t stream);

// Split-KV decode: per-chunk partials, then the combine (decode.hip).
struct DecodeParams {
    const void *q, *k_cache, *v_cache;
    const int32_t *block_table;  // NULL: contiguous cache
    const int32_t *seq_lens;
    void *o;
    float *lse;  // may be NULL
    int B, Hq, Hkv, head_dim, page_size, max_blocks, dtype;
    float scale;
    int chunk;        // resolved chunk size (tokens)
    int max_chunks;   // ceil(max_blocks * page_size / chunk), or the balanced split's bound
    // Balanced split (0: one workgroup per (sequence, KV head, chunk)): bal_gh
    // workgroups per KV head each take an equal share of the head's tokens, in units
    // of one workgroup pass; max_chunks then bounds the splits of one sequence
    int bal_gh = 0;
    float *o_parts;   // [B*Hq, max_chunks, head_dim]
    float *lse_parts; // [B*Hq, max_chunks]
    // in-place append (both NULL for plain decode): rows [B, Hkv, head_dim]
    // written into the cache at token seq_lens[b], which the query then attends
    const void *k_new = nullptr, *v_new = nullptr;
    // sliding window (the query, token L-1, sees tokens >= L-1-window; -1: none)
    // and logit soft-cap (0: none), as for prefill
    int window = -1;
    float softcap = 0.f;
    // E4M3 cache (k_cache, v_cache hold one byte per element), with per-(sequence,
    // KV head) descales [B, Hkv] (NULL: 1); plain decode only, head_dim 64 or 128
    bool kv_e4m3 = false;
    const float *descale_k = nullptr, *descale_v = nullptr;
};
hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);

// Stand-alone combine of partials (decode.hip).
struct CombineParams {
    const float *o_parts, *lse_parts;
    const int32_t *n_splits;  // may be NULL
    int rows, max_splits, head_dim;
    void *o;
    bool o_bf16;  // true: o is bfloat16, false: float32
    float *lse;   // may be NULL
};
hipError_t launch_lse_combine(const CombineParams &p, hipStream_t stream);

// Device-side check of a decode's block table and lengths (decode.hip).
struct TableCheckParams {
    const int32_t *block_table;  // [B, max_blocks], or NULL (contiguous cache: lengths only)
    const int32_t *seq_lens;     // [B]
    int B, page_size, max_blocks, num_blocks;
    int appended;                // 1: lengths exclude a token appended in place
    int32_t *bad_out;            // one int32, overwritten
};
hipError_t launch_check_tables(const TableCheckParams &p, hipStream_t stream);
// Device scratch of attn_decode_noalloc: the address of this GPU's static
// array (looked up once per device, with that device current).
constexpr size_t kNoAllocScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
hipError_t decode_scratch(void **out);

// Decode tiling constants the host front end needs for validation/sizing.
constexpr int kDecodeMaxGroup = 16;  // largest supported n_q_heads / n_kv_heads
constexpr int kDecodeTokenQuantum = 16;  // chunk sizes are multiples of this
constexpr int kDecodeStepTokens = 32;    // tokens of one wave step of the split kernel
// waves of one split workgroup: d = 256 runs 4, the others 8
constexpr int decode_split_waves(int head_dim) { return head_dim == 256 ? 4 : 8; }
// Largest number of partials per row: a row's partials (splits x head_dim x 4
// bytes) are addressed through one buffer descriptor with a 31-bit range.
constexpr long long kMaxSplits = (1LL << 22) - 1;
// Largest one-dimensional grid of the decode kernels (workgroups x threads < 2^32).
constexpr long long kMaxSplitWorkgroups = (1LL << 23) - 1;   // 512-thread split workgroups
constexpr long long kMaxCombineRows = (1LL << 24) - 1;       // 256-thread combine workgroups

}  // namespace attn
