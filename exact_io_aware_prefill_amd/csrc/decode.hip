// Split-KV decode and the log-sum-exp combine for gfx950 (CDNA4).
//
// Method (pofe.ai, "FlashAttention for inference: tiled prefill and split-KV
// decoding", section "Decode: a different bottleneck"): the cached keys of one
// sequence are cut into chunks, one workgroup per (sequence, KV head, chunk);
// the workgroup loads each key/value row once and applies it to all query heads
// that share the KV head (grouped-query attention), reads the cache through the
// block table of a paged layout, and writes the chunk's normalised output o_k
// with its log-sum-exp lambda_k = m_k + ln l_k.  A second, small kernel merges
// the chunks with the combine rule of section "The online softmax, with every
// symbol defined": Lambda = ln sum_k exp(lambda_k), o = sum_k exp(lambda_k -
// Lambda) o_k.
//
// gfx950 mapping of the split kernel
//   * 8 waves per workgroup (4 for head_dim 256); wave w takes 32-token steps
//     w, w+8, ... of the chunk with its own online-softmax state; the waves'
//     states are merged through LDS at the end (the same combine rule, inside
//     the workgroup).
//   * A step is two 16-token blocks.  A block never crosses a page (pages hold
//     a multiple of 16 tokens), so each block is addressed through one scalar
//     buffer descriptor: one block-table lookup per 16 tokens, and tokens past
//     the sequence get an out-of-range offset and read as zero.
//   * Scores use v_mfma_f32_16x16x32_bf16 on S^T = K Q^T: the A operand is
//     loaded straight into registers (lane = token, 16 bytes of its row), the
//     B operand holds the group's query rows (padded to 16 with zeros) for the
//     whole kernel.  A lane of the accumulator owns one query head and four
//     tokens, so the softmax is in-register plus two cross-lane exchanges.
//   * The output is accumulated as O^T += V^T P^T on the same instruction; the
//     score accumulator (rounded to bf16) is the B operand as it stands.  V
//     rows are loaded coalesced (16 lanes per 256-byte row), stored unchanged
//     into a wave-private LDS slab, and the V^T operand is read back with the
//     LDS transpose read ds_read_b64_tr_b16 (in each 16-lane group, lane 4r+q
//     reads 4 dims of token row r and lane j receives dim j of the 4 rows), so
//     no VALU work is spent on the transpose.  16-byte chunk c of slab row r
//     sits at slot c ^ 2(r & 7) (D = 128; c ^ 2((r >> 1) & 3) for D = 64),
//     which makes both the row stores and the transpose reads bank-conflict
//     free on the 64-bank LDS.
//   * Each wave keeps two steps in flight (two register sets), so a workgroup
//     has 512 tokens of keys and values in flight: a whole 512-token chunk is
//     requested at once.
//   * A separate instantiation adds a sliding window and logit soft-capping (two
//     of the variants the page's section "Interaction with post-trained models"
//     lists).  With a window the query (token L-1) sees tokens L-1-w .. L-1:
//     chunks wholly before the window exit at once (the combine starts at the
//     first live chunk), waves skip their steps that end before it, and the one
//     step that straddles its start is masked.  Soft-capping maps each score s to
//     cap * tanh(s / cap) before the masking.
//   * Another instantiation reads an E4M3 (8-bit float) cache: half the bytes per
//     token, the quantity decode is bound by.  The codes convert exactly to bf16
//     (K in registers, V on its way into the slab), and the per-(sequence, KV
//     head) descales fold into the score scale and the output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Waves per split workgroup: 8 (two per SIMD).  d = 256 holds twice the K/V
// registers per step, so its workgroups are 4 waves of one per SIMD, with the
// same bytes in flight per compute unit.
template <int D> constexpr int split_waves() { return decode_split_waves(D); }
constexpr int kStep = kDecodeStepTokens;  // tokens per wave step (two 16-token blocks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBufferFlags = 0x00020000;       // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;  // per-lane offset that reads as zero

struct SplitArgs {
    const uint16_t *q, *k, *v;
    const int32_t *bt, *seq_lens;
    float *o_parts, *lse_parts;
    // In-place append (both NULL otherwise): the new token's key/value rows
    // [B, Hkv, D]; seq_lens then counts the tokens cached before it.
    const uint16_t *k_new, *v_new;
    int Hq, Hkv, group, page, max_blocks, chunk, max_chunks;
    int B;
    // Balanced work split (0: one workgroup per (sequence, KV head, chunk)).  With
    // bal_gh > 0 the grid is Hkv * bal_gh workgroups, KV head fastest; each KV head's
    // sequences, cut into units of one workgroup pass (256 tokens; 128 at d = 256),
    // form one list in sequence order, and workgroup r of the head takes units r*R .. r*R + R - 1 of it (R =
    // ceil(units / bal_gh)), writing one partial per sequence it touches: split k of
    // sequence b is that of workgroup floor(U_b / R) + k, U_b the sequence's first unit.
    int bal_gh;
    long long seq_tokens;  // tokens per sequence of the contiguous layout (= capacity)
    float scale_log2;
    // variant only: window (-1: none); soft-cap as x = cap_log2 * tanh(raw * scale / cap)
    // in base-2 units, with cap_log2 = cap * log2(e) and cap_k = 2 log2(e) scale / cap
    int window;
    float cap_log2, cap_k;
    // FP8 cache only: descale factors [B, Hkv] of K and V (NULL: 1)
    const float *dk, *dv;
};

// Tokens the query attends for sequence b, and the index of the appended token
// (-1 without append).  Lengths are clamped so nothing is read or written past
// the sequence's capacity; with append, a full cache's new row goes to the last slot.
__device__ __forceinline__ int attended_tokens(const SplitArgs &a, int b, int &t_new)
{
    const long long cap = a.seq_tokens;
    const long long sl = a.seq_lens[b];
    if (a.k_new) {
        t_new = (int)max(0LL, min(sl, cap - 1));
        return t_new + 1;
    }
    t_new = -1;
    return (int)max(0LL, min(sl, cap));
}

// Balanced split: units (workgroup passes of `unit` tokens) of sequence b.
__device__ __forceinline__ int seq_units(const SplitArgs &a, int b, int unit)
{
    int t_new;
    return (attended_tokens(a, b, t_new) + unit - 1) / unit;
}

__device__ __forceinline__ int wave_sum_int(int x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Balanced split, per wave (the result is wave-uniform): the units of all sequences
// and, for the unit `s`, the sequence holding it and that sequence's first unit.
// Requires s < total (so such a sequence exists).
__device__ __forceinline__ int bal_total_units(const SplitArgs &a, int unit, int lane)
{
    int total = 0;
    for (int base = 0; base < a.B; base += 64) {
        const int bb = base + lane;
        total += wave_sum_int(bb < a.B ? seq_units(a, bb, unit) : 0);
    }
    return total;
}

__device__ __forceinline__ void bal_find(const SplitArgs &a, int unit, int lane, int s, int &b_out, int &u_first)
{
    int off = 0;  // units of the sequences before this block of 64
    for (int base = 0; base < a.B; base += 64) {
        const int bb = base + lane;
        const int u = bb < a.B ? seq_units(a, bb, unit) : 0;
        int incl = u;  // inclusive prefix within the block
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const uint64_t hit = __builtin_amdgcn_ballot_w64(bb < a.B && off + incl > s);
        if (hit) {
            const int j = __builtin_ctzll(hit);
            b_out = base + j;
            u_first = off + __shfl(incl - u, j);
            return;
        }
        off += __shfl(incl, 63);
    }
    b_out = a.B - 1;  // not reached when s < total
    u_first = off;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Index of token t of sequence b in units of one token's rows (all KV heads):
// paged: slot t % page of page block_table[b][t / page]; contiguous: b*capacity + t.
__device__ __forceinline__ long long token_index(const SplitArgs &a, int b, int t)
{
    if (a.bt) {
        const int page = a.bt[(size_t)b * a.max_blocks + t / a.page];
        return (long long)page * a.page + (t % a.page);
    }
    return (long long)b * a.seq_tokens + t;
}

// slot permutation of the V slab rows (see the header comment; D = 256 rows are
// two bank lines and use the D = 128 permutation).  The E4M3 cache stores each
// loaded 16-byte chunk as two bf16 chunks, one store instruction for the even
// slots and one for the odd; its permutation also flips the low slot bit on odd
// bank lines (row r for D = 128, row pair r / 2 for D = 64), so the two rows of
// bank lines a store pass writes land on disjoint banks.  The flip keeps the
// permutation's 8-row period, and the transpose reads stay conflict-free.
template <int D, bool KV8 = false>
__device__ __forceinline__ int slab_swz(int r)
{
    const int base = D >= 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
    return KV8 ? base + (D >= 128 ? (r & 1) : ((r >> 1) & 1)) : base;
}

// K slab: chunk c of key row r at slot c ^ kslab_swz(r), rows as stored in the
// cache (2D bytes for bf16, D bytes of E4M3 codes).  Rows of 256 bytes or more
// permute by r & 15, rows of 128 bytes (two per bank line) by (r >> 1) & 7.  Both
// the row stores (16 lanes = one row's 16 chunks, or two rows' 8) and the score
// operand reads (16 lanes = one chunk of 16 consecutive rows) then hit 16 distinct
// 16-byte bank groups.
template <int D, bool KV8 = false>
__device__ __forceinline__ int kslab_swz(int r)
{
    return (KV8 ? D : 2 * D) >= 256 ? (r & 15) : ((r >> 1) & 7);
}

template <int D>
struct Geo {
    static constexpr int RB = D * 2;          // bytes of one token row of one head
    static constexpr int NC = D / 8;          // 16-byte chunks per row
    static constexpr int RPI = 64 / NC;       // V rows covered by one load instruction
    static constexpr int VI = kStep / RPI;    // V load instructions per step
    static constexpr int VIB = VI / 2;        // ... per 16-token block
    static constexpr int SLAB = kStep * RB;   // bytes of one wave's slab
    // the slab permutation repeats every 8 rows: every VP load instructions
    static constexpr int VP = RPI >= 8 ? 1 : 8 / RPI;
    static_assert(VI % VP == 0, "whole permutation periods per step");
};

// Load geometry of the cache: bf16 rows of 2D bytes, or E4M3 rows of D bytes.
template <int D, bool KV8>
struct KvGeo {
    static constexpr int RB = KV8 ? D : 2 * D;    // bytes of one token row of one head
    static constexpr int NC = RB / 16;            // 16-byte chunks per row
    static constexpr int RPI = 64 / NC;           // V rows covered by one load instruction
    static constexpr int VI = kStep / RPI;        // V load instructions per step
    static constexpr int VIB = VI / 2;            // ... per 16-token block
    static constexpr int KL = KV8 ? D / 64 : D / 32;  // 16-byte K loads per lane per block
};

// Registers of one step: K as loaded [block][load], V rows as loaded.
template <int D, bool KV8>
struct StepRegs {
    uint4 k[2][KvGeo<D, KV8>::KL];
    uint4 v[KvGeo<D, KV8>::VI];
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Four E4M3 bytes -> four bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w)
{
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Per-lane constants of the loads.
struct LaneOffsets {
    uint32_t k;  // K: token l16 of a block, bytes 16G.. of each 64-byte piece
    uint32_t v;  // V: token vtok of a load's rows, chunk vchunk
    int l16, vtok;
};

template <int D, bool KV8, bool KSL = false>
__device__ __forceinline__ void issue_step(const SplitArgs &a, StepRegs<D, KV8> &s, const char *kbase,
                                           const char *vbase, int b, int tb, int t_end, uint32_t rstride,
                                           const LaneOffsets &lo)
{
    using Gm = KvGeo<D, KV8>;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int t0 = tb + 16 * blk;
        const bool live = t0 < t_end;  // uniform; a dead block reads nothing and loads no table entry
        const long long row0 = live ? token_index(a, b, t0) * a.Hkv : 0;
        const uint32_t nrec = live ? 16u * rstride : 0u;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + row0 * Gm::RB, nrec);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + row0 * Gm::RB, nrec);
        if constexpr (!KSL) {
            // each lane loads its own score operand's bytes (key row l16): 16 rows of
            // 64 bytes per instruction (bf16), or their E4M3 codes
            const uint32_t ko = (t0 + lo.l16 < t_end) ? lo.k : kOutOfRange;
#pragma unroll
            for (int st = 0; st < Gm::KL; ++st) s.k[blk][st] = bload16(rk, ko + 64u * st, 0);
        } else {
            // K rows read as V rows are (RPI whole rows per instruction), which streams
            // faster; the step moves them through the wave's K slab into the operand
            // layout
            static_assert(Gm::KL * Gm::RPI == 16, "one 16-token block of K rows per block's loads");
#pragma unroll
            for (int st = 0; st < Gm::KL; ++st) {
                const int tok = Gm::RPI * st + lo.vtok;  // token within the block
                const uint32_t ko = (t0 + tok < t_end) ? lo.v : kOutOfRange;
                s.k[blk][st] = bload16(rk, ko, (uint32_t)(Gm::RPI * st) * rstride);
            }
        }
#pragma unroll
        for (int i = 0; i < Gm::VIB; ++i) {
            const int tok = Gm::RPI * i + lo.vtok;  // token within the block
            const uint32_t vo = (t0 + tok < t_end) ? lo.v : kOutOfRange;
            s.v[Gm::VIB * blk + i] = bload16(rv, vo, (uint32_t)(Gm::RPI * i) * rstride);
        }
    }
}

// First token the query sees: L-1-window with a window (variant only), else 0.
template <bool EXT>
__device__ __forceinline__ int window_start(const SplitArgs &a, int L)
{
    return (EXT && a.window >= 0) ? max(0, L - 1 - a.window) : 0;
}

// tanh(y) = 1 - 2 / (e^{2y} + 1), exact at y -> +-inf (rcp(+inf) = 0, rcp(1) = 1);
// returns cap_log2 * tanh(raw * scale / cap) with cap_k = 2 log2(e) scale / cap.
__device__ __forceinline__ float soft_cap_log2(float raw, float cap_log2, float cap_k)
{
    const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(raw * cap_k) + 1.f);
    return fmaf(-2.f * cap_log2, r, cap_log2);
}

// KV8: the cache holds E4M3 codes.  A lane's K bytes 16G + 64j .. +15 (dims
// 64j + 16G ..) become the bf16 operands of k-steps 2j and 2j+1, so its query
// fragments take the same dims (see the kernel); V rows are converted to bf16 on
// their way into the slab, as two 16-byte chunks per loaded chunk.
template <int D, bool EXT, bool KV8, bool KSL = false>
__device__ __forceinline__ void consume_step(const SplitArgs &a, const StepRegs<D, KV8> &s, char *slab,
                                             const bf16x8_t *qf, f32x4_t *acc, float &m, float &l, int tb,
                                             int t_lo, int t_end, int G, const uint32_t *vstore, uint32_t vread,
                                             float scale_log2, float cap_k, char *kslab, uint32_t kstore,
                                             uint32_t kread)
{
    using Gm = Geo<D>;
    using Lg = KvGeo<D, KV8>;
    if constexpr (KSL) {
        // K rows into the wave's K slab (in order with this wave's other LDS accesses,
        // so after the previous step's operand reads).  Load i holds rows RPI i + vtok,
        // whose permutation is that of row vtok XOR that of row RPI i, so its offset is
        // the lane's row-vtok offset XOR a constant, plus RPI i rows.
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < Lg::KL; ++i)
                *reinterpret_cast<uint4 *>(kslab + (blk * 16 + Lg::RPI * i) * Lg::RB +
                                           (kstore ^ (16u * kslab_swz<D, KV8>(Lg::RPI * i)))) = s.k[blk][i];
    }
    // scores of the two 16-token blocks
    f32x4_t st[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[blk][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            bf16x8_t kf;
            if constexpr (KV8) {
                // E4M3 codes of dims 64 (ks >> 1) + 16G .. + 15 of key row 16 blk + l16: chunk
                // 4 (ks >> 1) + G, from the slab at slot (4 (ks >> 1) + G) ^ swz
                const uint4 w = KSL ? *reinterpret_cast<const uint4 *>(kslab + blk * 16 * Lg::RB +
                                                                      (kread ^ (64u * (ks >> 1))))
                                    : s.k[blk][ks >> 1];
                const uint2 a0 = e4m3x4_to_bf16((ks & 1) ? w.z : w.x);
                const uint2 a1 = e4m3x4_to_bf16((ks & 1) ? w.w : w.y);
                kf = as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
            } else if constexpr (KSL) {
                // key row 16 blk + l16, chunk 4 ks + G, at slot (4 ks + G) ^ swz = 4 ks ^ (G ^ swz)
                kf = *reinterpret_cast<const bf16x8_t *>(kslab + blk * 16 * Gm::RB + (kread ^ (64u * ks)));
            } else {
                kf = as_bf16x8(s.k[blk][ks]);
            }
            st[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], st[blk], 0, 0, 0);
        }
    }
    // V rows into the wave's slab.  LDS executes one wave's accesses in order, so
    // these stores land after the previous step's transpose reads of the slab.
    if constexpr (KV8) {
#pragma unroll
        for (int i = 0; i < Lg::VI; ++i) {
            const uint4 w = s.v[i];
            const uint2 b0 = e4m3x4_to_bf16(w.x), b1 = e4m3x4_to_bf16(w.y);
            const uint2 b2 = e4m3x4_to_bf16(w.z), b3 = e4m3x4_to_bf16(w.w);
            char *row = slab + i * Lg::RPI * Gm::RB;
            *reinterpret_cast<uint4 *>(row + vstore[0]) = make_uint4(b0.x, b0.y, b1.x, b1.y);
            *reinterpret_cast<uint4 *>(row + vstore[1]) = make_uint4(b2.x, b2.y, b3.x, b3.y);
        }
    } else {
#pragma unroll
        for (int i = 0; i < Gm::VI; ++i)
            *reinterpret_cast<uint4 *>(slab + vstore[i % Gm::VP] + (i - i % Gm::VP) * Gm::RPI * Gm::RB) = s.v[i];
    }

    // online softmax over this step (lane: query l16, tokens 4G+i of each block)
    const bool tail = tb + kStep > t_end || (EXT && tb < t_lo);
    const bool capped = EXT && a.cap_log2 > 0.f;
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float xv = capped ? soft_cap_log2(st[blk][i], a.cap_log2, cap_k) : st[blk][i] * scale_log2;
            const int tok = tb + 16 * blk + 4 * G + i;
            if (tail && (tok >= t_end || (EXT && tok < t_lo))) xv = -INFINITY;
            x[4 * blk + i] = xv;
            mx = fmaxf(mx, xv);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // finite: every step a wave runs holds a token in [t_lo, t_end)
    const float m_new = fmaxf(m, mx);
    const float c = __builtin_amdgcn_exp2f(m - m_new);
    float rs = 0.f;
    bf16x8_t pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(x[j] - m_new);
        rs += p;
        pf[j] = (__bf16)p;
    }
    l = l * c + rs;
    m = m_new;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] *= c;

    // O^T += V^T P^T; P's k index 8G+j is token 4G+j (j < 4) or 16+4G+(j-4)
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
        const char *p = slab + (vread ^ (32u * nb));
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p + 16 * Gm::RB));
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[nb], 0, 0, 0);
    }
}

// APPEND selects the in-place append variant, EXT the window / soft-cap variant,
// KV8 an E4M3 cache (separate instantiations, so the plain decode keeps its
// register budget).
template <int D, bool APPEND, bool EXT, bool KV8 = false, bool BAL = false>
__global__ __launch_bounds__(split_waves<D>() * 64, D == 64 ? 4 : 1) void decode_split_kernel(SplitArgs a)
{
    static_assert(!BAL || !EXT, "the balanced split has no window or cap variant");
    // K rows through a wave-private LDS slab (balanced split, d >= 128): whole-row
    // loads stream faster than loads in the score operand's layout, which pays off on
    // long shares; the per-chunk split's short chunks keep K in registers
    constexpr bool KSL = BAL && D >= 128;
    using Gm = Geo<D>;
    using Lg = KvGeo<D, KV8>;
    constexpr int kWaves = split_waves<D>();
    // one slab per wave; reused at the end for the eight waves' [16][D] float outputs
    static_assert(Gm::SLAB == 16 * D * 4, "slab must hold a wave's 16 x D float output");
    __shared__ __attribute__((aligned(1024))) char slabs[kWaves * Gm::SLAB];
    __shared__ __attribute__((aligned(1024))) char kslabs[KSL ? kWaves * Gm::SLAB : 16];
    __shared__ float ml[2][kWaves][16];

    const int tid = threadIdx.x, lane = tid & 63;
    // the KV heads of one chunk are adjacent workgroups, so the heads' rows of the
    // same tokens (adjacent in memory) are requested at about the same time
    const int hk = blockIdx.x % a.Hkv;
    constexpr int UNIT = kWaves * kStep;  // balanced split: tokens of one unit (one workgroup pass)
    // this workgroup's segment: tokens t_begin .. t_end - 1 of sequence b, partial `split`
    int b, split, L, t_new, t_begin, t_end;
    int R = 1, s_next = 0, s_stop = 0, u_b = 0;  // balanced split state (units)
    if constexpr (!BAL) {
        split = blockIdx.x / a.Hkv;
        b = blockIdx.y;
        // lengths outside [0, capacity] are clamped so no read leaves the sequence's cache
        L = attended_tokens(a, b, t_new);
        t_begin = split * a.chunk;
        if (t_begin >= L) return;  // whole workgroup exits together: this chunk is empty
        t_end = min(t_begin + a.chunk, L);
    } else {
        const int r = blockIdx.x / a.Hkv;
        int s0;
        if (a.B <= 64) {
            // one load per lane: lane j holds sequence j's length, units and their
            // inclusive prefix, which give the total, the first sequence of this
            // workgroup's share and its length without further loads
            int tn = -1;
            const int Lj = lane < a.B ? attended_tokens(a, lane, tn) : 0;
            const int u = (Lj + UNIT - 1) / UNIT;
            int incl = u;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
            R = (total + a.bal_gh - 1) / a.bal_gh;
            s0 = r * R;
            s_stop = min(total, s0 + R);
            if (s0 >= s_stop) return;  // whole workgroup: nothing left for it
            const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.B && incl > s0);
            const int j = __builtin_ctzll(hit);
            b = __builtin_amdgcn_readfirstlane(j);
            u_b = __builtin_amdgcn_readfirstlane(__shfl(incl - u, j));
            L = __builtin_amdgcn_readfirstlane(__shfl(Lj, j));
            t_new = __builtin_amdgcn_readfirstlane(__shfl(tn, j));
        } else {
            const int total = __builtin_amdgcn_readfirstlane(bal_total_units(a, UNIT, lane));
            R = (total + a.bal_gh - 1) / a.bal_gh;
            s0 = r * R;
            s_stop = min(total, s0 + R);
            if (s0 >= s_stop) return;  // whole workgroup: nothing left for it
            bal_find(a, UNIT, lane, s0, b, u_b);
            b = __builtin_amdgcn_readfirstlane(b);
            u_b = __builtin_amdgcn_readfirstlane(u_b);
            L = attended_tokens(a, b, t_new);
        }
        const int u_end = min(s_stop, u_b + (L + UNIT - 1) / UNIT);
        t_begin = (s0 - u_b) * UNIT;
        t_end = min(L, (u_end - u_b) * UNIT);
        split = r - u_b / R;
        s_next = u_end;
    }
    const int t_lo = EXT ? window_start<EXT>(a, L) : 0;
    if (EXT && t_end <= t_lo) return;  // the chunk ends before the window: the combine skips it

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, G = lane >> 4;
    const int g = a.group;
    const uint32_t rstride = (uint32_t)a.Hkv * Lg::RB;  // bytes between consecutive tokens of one head


    LaneOffsets lo;
    lo.l16 = l16;
    lo.vtok = lane / Lg::NC;
    const int vchunk = lane % Lg::NC;
    lo.k = (uint32_t)l16 * rstride + 16u * G;
    lo.v = (uint32_t)lo.vtok * rstride + 16u * vchunk;
    char *slab = slabs + wave * Gm::SLAB;
    // slab byte offsets of this lane's V row stores by load instruction modulo
    // VP (instruction i covers rows i*RPI..; the slot permutation repeats every
    // 8 rows, i.e. every two instructions for D = 128, four for D = 256)
    uint32_t vstore[Gm::VP > 2 ? Gm::VP : 2];
    if constexpr (KV8) {
        // a loaded chunk (16 dims) becomes bf16 chunks 2 vchunk and 2 vchunk + 1 of
        // slab row lo.vtok + RPI i; the permutation repeats every 8 rows and RPI is
        // a multiple of 8, so the offsets hold for every load instruction
        static_assert(Lg::RPI % 8 == 0, "one permutation period per load instruction");
#pragma unroll
        for (int e = 0; e < 2; ++e)
            vstore[e] = (uint32_t)(lo.vtok * Gm::RB + 16 * ((2 * vchunk + e) ^ slab_swz<D, true>(lo.vtok)));
    } else {
#pragma unroll
        for (int par = 0; par < Gm::VP; ++par) {
            const int r = Gm::RPI * par + lo.vtok;
            vstore[par] = (uint32_t)(r * Gm::RB + 16 * (vchunk ^ slab_swz<D>(r)));
        }
    }
    // transpose reads: group G, lane 4r+q reads 8 bytes of slab row 4G+r, dims
    // 16nb + 4q..4q+3, i.e. chunk 2nb + (q >> 1); the permutation's bits above its
    // lowest move whole 32-byte chunk pairs and its lowest bit (E4M3 cache) only
    // swaps the two chunks of a pair, so d-block nb is a XOR by 32nb
    const int vrow = 4 * G + (l16 >> 2), vq = l16 & 3;
    const uint32_t vread = (uint32_t)(vrow * Gm::RB + 16 * ((vq >> 1) ^ slab_swz<D, KV8>(vrow)) + 8 * (vq & 1));
    // K slab: this lane stores chunk vchunk of rows RPI i + vtok of each block (offset
    // of row vtok here) and reads chunk 4 ks + G of row l16 (both blocks' rows, 16
    // apart, share the permutation)
    char *kslab = KSL ? kslabs + wave * Gm::SLAB : kslabs;
    const uint32_t kstore = (uint32_t)(lo.vtok * Lg::RB + 16 * (vchunk ^ kslab_swz<D, KV8>(lo.vtok)));
    const uint32_t kread = (uint32_t)(l16 * Lg::RB + 16 * (G ^ kslab_swz<D, KV8>(l16)));

    const char *kbase = reinterpret_cast<const char *>(a.k) + (size_t)hk * Lg::RB;
    const char *vbase = reinterpret_cast<const char *>(a.v) + (size_t)hk * Lg::RB;

    for (;;) {  // segments: one in the per-chunk split, one or more in the balanced one
        // append: only the workgroup whose segment holds the new token touches it
        const bool has_new = APPEND && t_new >= t_begin && t_new < t_end;  // workgroup-uniform
        // query fragments (B operand of S^T = K Q^T); rows >= g are zero padding.
        // k-step s holds dims 32s + 8G .. +7, or with the E4M3 cache dims
        // 64(s >> 1) + 16G + 8(s & 1) .. +7, the dims of the lane's converted K bytes.
        bf16x8_t qf[D / 32];
        {
            const uint16_t *qrow = a.q + ((size_t)b * a.Hq + (size_t)hk * g + l16) * D;
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                uint4 u = make_uint4(0, 0, 0, 0);
                const int d0 = KV8 ? 64 * (s >> 1) + 16 * G + 8 * (s & 1) : 32 * s + 8 * G;
                if (l16 < g) u = *reinterpret_cast<const uint4 *>(qrow + d0);
                qf[s] = as_bf16x8(u);
            }
        }
        // effective scale (the E4M3 cache folds its K descale in) and the V descale
        const float dkv = (KV8 && a.dk) ? a.dk[(size_t)b * a.Hkv + hk] : 1.f;
        const float dvv = (KV8 && a.dv) ? a.dv[(size_t)b * a.Hkv + hk] : 1.f;
        const float sl2 = a.scale_log2 * dkv;
        const float cap_k = a.cap_k * dkv;  // the cap acts on the scaled score raw * scale * descale_k

        f32x4_t acc[D / 16];
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[nb][i] = 0.f;
        float m = -INFINITY, l = 0.f;

        // This wave's steps start at t_begin + (wave + 8j) * 32, two in flight.  Loads
        // are issued unconditionally (a step past the chunk has empty descriptors and
        // reads nothing), so the number of loads in flight is the same on every path
        // and each step waits only for its own loads.
        const int stride = kWaves * kStep;
        int tb = t_begin + wave * kStep;
        if (APPEND && has_new) {
            // Write the new rows into the cache slot first: this workgroup is the only
            // reader of that slot, and its loads below are issued after the barrier,
            // which orders them after these stores.  A row is Lg::RB bytes (bf16, or
            // the E4M3 codes of an 8-bit cache, which the caller quantised with that
            // cache's descales), copied as RB / 16 16-byte chunks.
            constexpr int NCH = Lg::RB / 16;
            const long long row = token_index(a, b, t_new) * a.Hkv + hk;
            const size_t src = ((size_t)b * a.Hkv + hk) * Lg::RB;
            if (tid < NCH)
                reinterpret_cast<uint4 *>(const_cast<char *>(reinterpret_cast<const char *>(a.k)) + row * Lg::RB)[tid] =
                    reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(a.k_new) + src)[tid];
            else if (tid < 2 * NCH)
                reinterpret_cast<uint4 *>(const_cast<char *>(reinterpret_cast<const char *>(a.v)) +
                                          row * Lg::RB)[tid - NCH] =
                    reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(a.v_new) + src)[tid - NCH];
            __syncthreads();
        }
        // with a window, skip this wave's steps that end before it starts
        if (EXT && tb + kStep <= t_lo) tb += ((t_lo - tb - kStep) / stride + 1) * stride;
        if constexpr (!KV8) {
            StepRegs<D, KV8> r0, r1;
            issue_step<D, KV8, KSL>(a, r0, kbase, vbase, b, tb, t_end, rstride, lo);
            while (tb < t_end) {
                issue_step<D, KV8, KSL>(a, r1, kbase, vbase, b, tb + stride, t_end, rstride, lo);
                consume_step<D, EXT, KV8, KSL>(a, r0, slab, qf, acc, m, l, tb, t_lo, t_end, G, vstore, vread, sl2, cap_k,
                                      kslab, kstore, kread);
                tb += stride;
                if (tb >= t_end) break;
                issue_step<D, KV8, KSL>(a, r0, kbase, vbase, b, tb + stride, t_end, rstride, lo);
                consume_step<D, EXT, KV8, KSL>(a, r1, slab, qf, acc, m, l, tb, t_lo, t_end, G, vstore, vread, sl2, cap_k,
                                      kslab, kstore, kread);
                tb += stride;
            }
        } else {
            // A ring of NS register sets, NS - 1 steps issued ahead.  An E4M3 step is
            // half the bytes of a bf16 one, yet three or four steps in flight measured
            // slower than two (32k cache: 13.9 -> 14.5 / 14.7 us), so NS stays 2.
            constexpr int NS = 2;
            StepRegs<D, KV8> r[NS];
#pragma unroll
            for (int j = 0; j < NS - 1; ++j)
                issue_step<D, KV8, KSL>(a, r[j], kbase, vbase, b, tb + j * stride, t_end, rstride, lo);
            bool more = tb < t_end;
            while (more) {
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    if (more) {
                        issue_step<D, KV8, KSL>(a, r[(j + NS - 1) % NS], kbase, vbase, b, tb + (NS - 1) * stride, t_end,
                                           rstride, lo);
                        consume_step<D, EXT, KV8, KSL>(a, r[j], slab, qf, acc, m, l, tb, t_lo, t_end, G, vstore, vread,
                                                  sl2, cap_k, kslab, kstore, kread);
                        tb += stride;
                        more = tb < t_end;
                    }
                }
            }
        }

        // ---- merge the eight wave states (combine rule) ------------------------------
        // row sum of query l16 over the four token groups of the lane's column
        float lt = l + __shfl_xor(l, 16);
        lt += __shfl_xor(lt, 32);
        if (G == 0) {
            ml[0][wave][l16] = m;  // -inf for a wave that saw no token
            ml[1][wave][l16] = lt;
        }
        // The wave's slab now holds its unscaled output as [query][D] floats, the
        // 16-byte column chunk c of query row r at chunk c ^ r: the 16 rows a store
        // or load instruction touches per pass then fall on distinct banks.
        float *wo = reinterpret_cast<float *>(slab);
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
            *reinterpret_cast<f32x4_t *>(&wo[l16 * D + 4 * ((4 * nb + G) ^ l16)]) = acc[nb];
        __syncthreads();
        // wave w merges d-blocks w, w + kWaves, ... of all waves and writes the chunk's partial
        if (wave < D / 16 && l16 < g) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml[0][w][l16]);
            float Lsum = 0.f, e[kWaves];
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                e[w] = __builtin_amdgcn_exp2f(ml[0][w][l16] - M);  // 0 for a wave that saw no token
                Lsum += e[w] * ml[1][w][l16];
            }
            const size_t row = (size_t)b * a.Hq + (size_t)hk * g + l16;
            const float inv = dvv / Lsum;  // Lsum >= 1: the row's largest term is exp2(0)
#pragma unroll
            for (int nb = wave; nb < D / 16; nb += kWaves) {
                f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < kWaves; ++w)
                    sum += e[w] * *reinterpret_cast<const f32x4_t *>(
                                      reinterpret_cast<const float *>(slabs + w * Gm::SLAB) + l16 * D +
                                      4 * ((4 * nb + G) ^ l16));
                *reinterpret_cast<f32x4_t *>(&a.o_parts[(row * a.max_chunks + split) * D + 16 * nb + 4 * G]) =
                    sum * inv;
            }
            if (wave == 0 && G == 0) a.lse_parts[row * a.max_chunks + split] = (M + log2f(Lsum)) * kLn2;
        }
        if (!BAL || s_next >= s_stop) break;
        // balanced split: the next sequence with tokens, from its first unit (sequences
        // in between with no tokens have no units and are passed over)
        u_b += (L + UNIT - 1) / UNIT;
        do {
            ++b;
            L = attended_tokens(a, b, t_new);
        } while (L == 0);
        b = __builtin_amdgcn_readfirstlane(b);
        const int u_end = min(s_stop, u_b + (L + UNIT - 1) / UNIT);
        t_begin = 0;
        t_end = min(L, (u_end - u_b) * UNIT);
        split = (blockIdx.x / a.Hkv) - u_b / R;
        s_next = u_end;
        __syncthreads();  // every wave is done with the slabs before the next segment's steps
    }
}

// ---------------------------------------------------------------------------
// Combine: workgroups of 256 threads, one per row (sequence x query head) after
// the balanced split, two per row otherwise (each taking half of the row's
// columns).  Thread (sg, c) accumulates float4 column c over splits sg, sg + SG, ...
// The first batch of loads (partials and log-sum-exps of 64 splits) is issued
// before the row's split count is known: the loads stay inside the row's
// max_splits slots, and splits outside [first, ns) get weight 0 once the count
// arrives, so the count's load and the partials' loads are in flight together.
// Each wave reduces the row's log-sum-exps itself (no barrier); the SG partial
// sums meet in LDS.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;

// Cross-lane moves within a row of 16 lanes (DPP): quad_perm [1,0,3,2] and
// [2,3,0,1], half-row mirror (lane i <-> 7 - i) and row mirror (i <-> 15 - i).
// Applied in that order to a commutative reduction, each leaves every lane of a
// group of 2, 4, 8, then 16 lanes holding the group's result.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op)
{
    x = op(x, dpp_move<0xB1>(x));
    x = op(x, dpp_move<0x4E>(x));
    x = op(x, dpp_move<0x141>(x));
    x = op(x, dpp_move<0x140>(x));
    // the four rows' results, read from lanes 0, 16, 32, 48
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return op(op(r0, r1), op(r2, r3));
}

__device__ __forceinline__ float wave_max(float x)
{
    return wave_reduce(x, [](float u, float v) { return fmaxf(u, v); });
}

__device__ __forceinline__ float wave_sum(float x)
{
    return wave_reduce(x, [](float u, float v) { return u + v; });
}

struct CombineArgs {
    const float *o_parts, *lse_parts;
    const int32_t *n_splits;  // explicit per-row split counts, or NULL
    const int32_t *seq_lens;  // decode: splits = ceil(tokens / chunk), or NULL
    int Hq, chunk, max_splits, capacity;
    int append;  // decode with append: tokens = min(seq_lens, capacity - 1) + 1
    int window;  // decode with a window (-1: none): splits before the window's chunk are skipped
    // decode with the balanced split (bal_gh > 0): sequence b's splits are the
    // workgroups floor(U_b / R) .. floor((U_b + u_b - 1) / R) of its KV head, with u_b
    // its units of `unit` tokens, U_b those of the sequences before it, R =
    // ceil(all units / bal_gh); B sequences
    int bal_gh, unit, B;
    void *o;
    int o_bf16;
    float *lse;
};

// CS > 1: each row's columns are split over CS workgroups (each reduces the row's
// log-sum-exps itself), so twice the compute units read a few rows' partials: the
// 32k decode's 28 rows run on 56 workgroups, 0.26 us faster per call.
template <int D, bool BAL = false, int CS = 1>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(CombineArgs a)
{
    constexpr int C4 = D / 4;                    // float4 columns of a row
    constexpr int C4L = C4 / CS;                 // this workgroup's float4 columns
    static_assert(C4L * CS == C4 && kCombineThreads % C4L == 0, "whole column slices");
    constexpr int SG = kCombineThreads / C4L;    // split groups
    constexpr int U = SG >= 64 ? 1 : 64 / SG;    // splits per thread per batch (64 per batch)
    __shared__ f32x4_t red[SG][C4L];

    const size_t row = blockIdx.x / CS;
    const int cs = blockIdx.x % CS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int lcol = tid % C4L, col = cs * C4L + lcol, sg = tid / C4L;
    // descriptors over the row's max_splits slots (loads past them return zero);
    // split k is slot k of the row
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(reinterpret_cast<const char *>(a.o_parts + row * a.max_splits * D),
                                                (uint32_t)a.max_splits * D * 4u);
    const __amdgpu_buffer_rsrc_t rl =
        make_rsrc(reinterpret_cast<const char *>(a.lse_parts + row * a.max_splits), (uint32_t)a.max_splits * 4u);
    auto load_lam = [&](int k) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4u * (uint32_t)k, 0, 0));
    };
    // first batch, issued ahead of the split count: U splits per thread, or one with
    // the balanced split, whose rows have few live splits among many slots
    constexpr int pre = BAL ? 1 : U;
    f32x4_t v[U];
    float lk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = sg + SG * u;
        v[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        lk[u] = -INFINITY;
        if (u < pre) {
            v[u] = __builtin_bit_cast(f32x4_t, bload16(ro, (uint32_t)k * (D * 4) + 16u * col, 0));
            lk[u] = load_lam(k);
        }
    }
    float x0 = load_lam(lane);  // the log-sum-exp pass's first 64 splits

    int ns, first = 0;
    if (BAL) {
        auto units = [&](int b) {
            const int sl = a.seq_lens[b];
            const int L = a.append ? max(0, min(sl, a.capacity - 1)) + 1 : max(0, min(sl, a.capacity));
            return (L + a.unit - 1) / a.unit;
        };
        const int bq = (int)(row / a.Hq);
        int before = 0, total = 0;  // units of the sequences before this row's, and of all
        for (int base = 0; base < a.B; base += 64) {
            const int bb = base + lane;
            const int u = bb < a.B ? units(bb) : 0;
            before += wave_sum_int(bb < bq ? u : 0);
            total += wave_sum_int(u);
        }
        const int R = max(1, (total + a.bal_gh - 1) / a.bal_gh);
        const int ub = units(bq);
        ns = ub > 0 ? (before + ub - 1) / R - before / R + 1 : 0;
    } else if (a.seq_lens) {
        const int sl = a.seq_lens[row / a.Hq];
        const int L = a.append ? max(0, min(sl, a.capacity - 1)) + 1 : max(0, min(sl, a.capacity));
        ns = (L + a.chunk - 1) / a.chunk;
        if (a.window >= 0) first = max(0, L - 1 - a.window) / a.chunk;  // the chunk holding the window's start
    } else if (a.n_splits) {
        ns = a.n_splits[row];
    } else {
        ns = a.max_splits;
    }
    ns = max(0, min(ns, a.max_splits));
    first = min(first, ns);
    auto live = [&](int k) { return k >= first && k < ns; };
#pragma unroll
    for (int u = 0; u < U; ++u) lk[u] = (u < pre && live(sg + SG * u)) ? lk[u] : -INFINITY;

    // Lambda = mx + ln z, z = sum_k exp(lambda_k - mx), mx the largest live lambda:
    // every wave reduces the row on its own, a max pass, then one exponential per
    // lane and pass and a sum (lane reductions in registers, no LDS round trips)
    const int npass = (ns + 63) / 64;
    float mx = -INFINITY;
    for (int p = 0; p < npass; ++p) {
        const int k = lane + 64 * p;
        const float x = p == 0 ? x0 : load_lam(k);
        if (live(k)) mx = fmaxf(mx, x);
    }
    mx = wave_max(mx);
    const bool empty = (mx == -INFINITY);
    float z = 0.f;
    if (!empty) {
        for (int p = 0; p < npass; ++p) {
            const int k = lane + 64 * p;
            const float x = p == 0 ? x0 : load_lam(k);
            if (live(k)) z += expf(x - mx);  // lambda = -inf adds 0
        }
        z = wave_sum(z);
    }
    const float Lam = empty ? -INFINITY : mx + logf(z);

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (!empty) {
        // a split with lambda = -inf (dead, or empty) has weight 0 and contributes
        // nothing; its partial, possibly stale, is never read into the sum
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = expf(lk[u] - Lam);
            if (w != 0.f) acc += w * v[u];
        }
        for (int k0 = sg + SG * pre; k0 < ns; k0 += SG * U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + SG * u;
                v[u] = __builtin_bit_cast(f32x4_t, bload16(ro, (uint32_t)k * (D * 4) + 16u * col, 0));
                lk[u] = load_lam(k);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float w = expf((live(k0 + SG * u) ? lk[u] : -INFINITY) - Lam);
                if (w != 0.f) acc += w * v[u];
            }
        }
    }
    red[sg][lcol] = acc;
    __syncthreads();
    if (sg == 0) {
        f32x4_t sum = red[0][lcol];
#pragma unroll
        for (int s = 1; s < SG; ++s) sum += red[s][lcol];
        if (a.o_bf16) {
            uint16_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, (__bf16)sum[e]);
            uint2 packed;
            packed.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            packed.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            reinterpret_cast<uint2 *>(a.o)[row * C4 + col] = packed;
        } else {
            reinterpret_cast<f32x4_t *>(a.o)[row * C4 + col] = sum;
        }
    }
    if (tid == 0 && cs == 0 && a.lse) a.lse[row] = Lam;
}

template <int D>
hipError_t launch_combine(const CombineArgs &c, int rows, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    if (c.bal_gh > 0 && c.seq_lens)
        hipLaunchKernelGGL((lse_combine_kernel<D, true>), dim3((unsigned)rows), dim3(kCombineThreads), 0, stream, c);
    else
        hipLaunchKernelGGL((lse_combine_kernel<D, false, 2>), dim3((unsigned)rows * 2u), dim3(kCombineThreads), 0, stream,
                           c);
    return hipGetLastError();
}

hipError_t launch_combine_d(int head_dim, const CombineArgs &c, int rows, hipStream_t stream)
{
    if (head_dim == 128) return launch_combine<128>(c, rows, stream);
    if (head_dim == 64) return launch_combine<64>(c, rows, stream);
    return launch_combine<256>(c, rows, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream)
{
    if (p.B == 0) return hipSuccess;
    SplitArgs a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k_cache);
    a.v = static_cast<const uint16_t *>(p.v_cache);
    a.bt = p.block_table;
    a.seq_lens = p.seq_lens;
    a.o_parts = p.o_parts;
    a.lse_parts = p.lse_parts;
    a.k_new = static_cast<const uint16_t *>(p.k_new);
    a.v_new = static_cast<const uint16_t *>(p.v_new);
    a.dk = p.descale_k;
    a.dv = p.descale_v;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.group = p.Hq / p.Hkv;
    a.page = p.page_size;
    a.max_blocks = p.max_blocks;
    a.chunk = p.chunk;
    a.max_chunks = p.max_chunks;
    a.B = p.B;
    a.seq_tokens = (long long)p.max_blocks * p.page_size;
    a.scale_log2 = p.scale * kLog2e;
    // a window that reaches back past the first slot limits nothing
    a.window = (p.window >= 0 && (long long)p.window < a.seq_tokens) ? p.window : -1;
    a.cap_log2 = p.softcap > 0.f ? p.softcap * kLog2e : 0.f;
    a.cap_k = p.softcap > 0.f ? 2.f * kLog2e * p.scale / p.softcap : 0.f;
    const bool ext = a.window >= 0 || p.softcap > 0.f;
    a.bal_gh = ext ? 0 : p.bal_gh;  // the window and cap variant keeps one workgroup per chunk
    const dim3 grid = a.bal_gh > 0 ? dim3((unsigned)((long long)a.bal_gh * p.Hkv), 1u)
                                   : dim3((unsigned)((long long)p.max_chunks * p.Hkv), (unsigned)p.B);
    const bool append = a.k_new != nullptr;
    auto kernel = [&](auto dconst) {
        constexpr int DD = decltype(dconst)::value;
        constexpr int kThreads = split_waves<DD>() * 64;
        if (a.bal_gh > 0) {  // (never with a window or soft-cap)
            if constexpr (DD != 256) {
                if (p.kv_e4m3) {
                    if (append)
                        hipLaunchKernelGGL((decode_split_kernel<DD, true, false, true, true>), grid, dim3(kThreads), 0,
                                           stream, a);
                    else
                        hipLaunchKernelGGL((decode_split_kernel<DD, false, false, true, true>), grid, dim3(kThreads), 0,
                                           stream, a);
                    return;
                }
            }
            if (append)
                hipLaunchKernelGGL((decode_split_kernel<DD, true, false, false, true>), grid, dim3(kThreads), 0,
                                   stream, a);
            else
                hipLaunchKernelGGL((decode_split_kernel<DD, false, false, false, true>), grid, dim3(kThreads), 0,
                                   stream, a);
            return;
        }
        if constexpr (DD != 256) {
            if (p.kv_e4m3) {
                if (append)  // (the host allows no window or soft-cap with the E4M3 append)
                    hipLaunchKernelGGL((decode_split_kernel<DD, true, false, true>), grid, dim3(kThreads), 0, stream, a);
                else if (ext)
                    hipLaunchKernelGGL((decode_split_kernel<DD, false, true, true>), grid, dim3(kThreads), 0, stream, a);
                else
                    hipLaunchKernelGGL((decode_split_kernel<DD, false, false, true>), grid, dim3(kThreads), 0, stream, a);
                return;
            }
        }
        if (append && ext)
            hipLaunchKernelGGL((decode_split_kernel<DD, true, true>), grid, dim3(kThreads), 0, stream, a);
        else if (append)
            hipLaunchKernelGGL((decode_split_kernel<DD, true, false>), grid, dim3(kThreads), 0, stream, a);
        else if (ext)
            hipLaunchKernelGGL((decode_split_kernel<DD, false, true>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_split_kernel<DD, false, false>), grid, dim3(kThreads), 0, stream, a);
    };
    if (p.head_dim == 128)
        kernel(std::integral_constant<int, 128>());
    else if (p.head_dim == 64)
        kernel(std::integral_constant<int, 64>());
    else
        kernel(std::integral_constant<int, 256>());
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    CombineArgs c;
    c.o_parts = p.o_parts;
    c.lse_parts = p.lse_parts;
    c.n_splits = nullptr;
    c.seq_lens = p.seq_lens;
    c.Hq = p.Hq;
    c.chunk = p.chunk;
    c.max_splits = p.max_chunks;
    c.capacity = p.max_blocks * p.page_size;
    c.append = p.k_new != nullptr;
    c.window = a.window;
    c.bal_gh = a.bal_gh;
    c.unit = (p.head_dim == 256 ? split_waves<256>() : split_waves<128>()) * kStep;
    c.B = p.B;
    c.o = p.o;
    c.o_bf16 = 1;
    c.lse = p.lse;
    const int rows = p.B * p.Hq;
    return launch_combine_d(p.head_dim, c, rows, stream);
}

namespace {

// Table check: one workgroup walks every sequence's length and every table slot a
// decode of that length reads, counting entries outside their valid range, and
// thread 0 stores the total.  One workgroup and one plain store: no atomics and
// no memory that must start at zero, so the result is deterministic.
constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(TableCheckParams p)
{
    __shared__ unsigned long long partial[kCheckThreads / 64];
    const long long cap = (long long)p.max_blocks * p.page_size;
    unsigned long long bad = 0;  // 64-bit: a table may hold more than 2^32 entries
    for (int b = threadIdx.x; b < p.B; b += kCheckThreads) {
        const long long need = (long long)p.seq_lens[b] + p.appended;
        if (p.seq_lens[b] < 0 || need > cap) ++bad;
    }
    if (p.block_table) {
        const long long slots = (long long)p.B * p.max_blocks;
        for (long long i = threadIdx.x; i < slots; i += kCheckThreads) {
            const int b = (int)(i / p.max_blocks), j = (int)(i % p.max_blocks);
            // tokens a decode reads from this sequence, clamped into [0, capacity]
            const long long used = min(max((long long)p.seq_lens[b] + p.appended, 0LL), cap);
            if ((long long)j * p.page_size < used) {
                const int e = p.block_table[i];
                if (e < 0 || e >= p.num_blocks) ++bad;
            }
        }
    }
    // wave sums by shuffles, then the waves' sums through LDS
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_down(bad, off, 64);
    if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long t = 0;
        for (int w = 0; w < kCheckThreads / 64; ++w) t += partial[w];
        *p.bad_out = (int32_t)min(t, (unsigned long long)INT32_MAX);
    }
}

}  // namespace

// Partials of attn_decode_noalloc: one static array per GPU, alive until the process
// ends.  Host code never passes its name to a kernel (on the host the name is only a
// stand-in); it passes the device address looked up below.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t decode_scratch(void **out)
{
    constexpr int kMaxDevices = 64;
    static std::once_flag once[kMaxDevices];
    static void *addr[kMaxDevices];
    static hipError_t status[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    // once per device, with that device current (each GPU holds its own copy)
    std::call_once(once[dev], [&] { status[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)); });
    if (status[dev] != hipSuccess) return status[dev];
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_check_tables(const TableCheckParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(kCheckThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_lse_combine(const CombineParams &p, hipStream_t stream)
{
    CombineArgs c;
    c.o_parts = p.o_parts;
    c.lse_parts = p.lse_parts;
    c.n_splits = p.n_splits;
    c.seq_lens = nullptr;
    c.Hq = 1;
    c.chunk = 1;
    c.max_splits = p.max_splits;
    c.capacity = 0;
    c.append = 0;
    c.window = -1;
    c.bal_gh = 0;
    c.unit = 1;
    c.B = 0;
    c.o = p.o;
    c.o_bf16 = p.o_bf16 ? 1 : 0;
    c.lse = p.lse;
    return launch_combine_d(p.head_dim, c, p.rows, stream);
}

}  // namespace attn
