// Tiled exact prefill attention for gfx950 (CDNA4), bf16 inputs, matrix cores.
//
// Method (pofe.ai, "FlashAttention for inference: tiled prefill and split-KV
// decoding", section "Prefill: tiles, loop order and the tensor cores", and the
// update rule of section "The online softmax, with every symbol defined"): one
// workgroup owns one (sequence, query head, query tile); it walks the key/value
// tiles up to the causal limit, keeps each row's running max m and running sum
// l, rescales the unnormalised output by c = exp(m_old - m_new) when the max
// grows, never writes scores to memory, and finally writes O = acc / l and the
// row log-sum-exp m + ln l.  Tiles strictly above the diagonal are skipped and
// the diagonal tile is masked.
//
// gfx950 mapping
//   * workgroup = 4 waves x 32 query rows (128 rows); key/value tile = 32 keys.
//     The kernel fits in 167 VGPRs (d = 128) so three workgroups (three waves
//     per SIMD) are resident per compute unit: the operand reads from LDS are
//     the limiter, and the other waves' matrix work covers each wave's LDS
//     latency.  d = 256 runs two waves per SIMD.
//     (kBlocks > 1 would give each wave several 32-row blocks sharing every K
//     and V operand read, at the cost of registers and hence resident waves.)
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = K rows read from LDS, B = the block's Q rows kept in registers for the
//     whole kernel.  In the 32x32 accumulator a lane holds one query (lane % 32)
//     and 16 of the 32 keys, so the row sums are in-register work and the row
//     max (needed only on the rare path below) one exchange with lane ^ 32.
//   * The output is accumulated transposed as well, O^T += V^T P^T: the score
//     accumulator, rounded to bf16, is already the B operand (the contraction
//     over keys is order-free, so both operands use the key order in which the
//     accumulator holds them).  V tiles sit in LDS row-major and the V^T operand
//     comes from ds_read_b64_tr_b16 (lane 4r+q of a 16-lane group reads 4 dims
//     of key row r; lane j receives dim j of the 4 rows).
//   * K and V tiles go from memory straight into LDS (buffer loads with the LDS
//     destination bit; no registers, no VALU), double-buffered: step t loads
//     K(t+2) and V(t) while computing.  16-byte chunks are permuted per row so
//     the operand reads are bank-conflict free on the 64-bank LDS.  Each load
//     instruction has its own descriptor whose range ends at row N, so rows
//     past N read as zero and nothing outside the head is touched.
//   * Step t: the matrix cores run PV(t-1) while the vector ALUs compute the
//     probabilities of tile t (the instruction order is pinned with scheduling
//     groups so the two overlap inside the wave), then QK(t+1) into the freed
//     score registers.
//   * The exponentials of tile t use the running max from before the tile, so
//     they do not wait for the tile's own row max.  If a lane's probability sum
//     for the tile exceeds 256 (so some probability may exceed 2^8), or (window
//     variant) the row has no reference yet, a rare path raises the max to the
//     true running max,
//     rescales l and O by c and recomputes the tile's probabilities.  Any
//     reference value gives the same O = acc/l and LSE = m + ln l; the bound
//     keeps every probability <= 256 in float32.  The plain kernel takes its
//     first reference from the first tile's true row max.  Exponentials run in
//     base 2 with scale*log2(e) folded into one FMA; the reference is kept in
//     those units.
//   * Work order: longest first.  Workgroup ids walk (query tile descending,
//     sequence, KV head, query head) with the query head fastest: every head's
//     last (longest, under the causal mask) tile is dispatched before any
//     shorter one, and the query heads that share a KV head run side by side
//     and read the same key/value tiles.  Greedy dispatch of a longest-first
//     list leaves the least idle time at the end of the launch; it measured
//     3-5% faster at 16k-30k prompts and 8-11% at 8k than walking each KV head's
//     tiles in turn in zig-zag order.  When the (sequence, KV head) pairs divide
//     the 8 XCDs, each pair also gets its own XCDs, so its K/V tiles stay in
//     their L2s: the same speed, and 10x less HBM traffic (0.33 against 3.1 GB
//     per launch at 16k).
//   * A second instantiation adds a sliding window (row i sees keys i - w .. i;
//     the tile loop starts at the first tile of row q0's window and tiles that
//     reach below a row's window are masked as the diagonal is) and logit
//     soft-capping (each raw score becomes cap * tanh(score / cap) before the
//     masking), two of the variants the same page's section "Interaction with
//     post-trained models" lists as ones a kernel must support.  A row can
//     then meet tiles with no visible key before its window starts; its state
//     stays empty until it does.
//
// This file is compiled with -fno-honor-nans (inputs must be finite): the row
// max then maps to v_max3_f32 without NaN-quieting copies.  Infinities, which
// the masking relies on, keep their IEEE meaning.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 4;      // waves per workgroup
constexpr int kBlocks = 1;     // 32-row query blocks per wave
constexpr int kWavesPerSimd = 3;  // resident waves per SIMD the register budget is sized for (d <= 128)
constexpr int kBM = kWaves * kBlocks * 32;  // query rows per workgroup
constexpr int kBlockN = 32;    // keys per tile
constexpr int kKB = kBlockN / 32;  // 32-key score blocks per tile
constexpr int kKS = kBlockN / 16;  // 16-key steps of the P*V product per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxLaneSum = 256.f;            // a lane's tile sum above this redoes the tile
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer, 32-bit data format

// Two layouts share the kernel.  Padded batch: q, o [B, Hq, N, d], k, v
// [B, Hkv, N, d], lse [B, Hq, N] (cu_seqlens NULL).  Packed variable-length
// batch: sequence b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, o
// [T, Hq, d], k, v [T, Hkv, d] and lse [Hq, T].  Row r of head h of sequence b
// sits at base + b_off + h * head + r * row (in elements) with the strides below.
struct Args {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    const int32_t *cu_seqlens;  // packed layout, or NULL
    int B, N, Hq, Hkv, group, causal, n_qtiles, n_items;
    int T;                      // packed: total tokens
    long long q_head, q_row;    // strides of q and o (elements)
    long long kv_head, kv_row;  // strides of k and v
    long long lse_head;         // stride of lse between heads (rows are adjacent)
    int negate_q;      // 1 when the caller's scale is negative
    float scale_log2;  // |scale| * log2(e)
    float scale;       // |scale|
    // Variant kernel only.  window >= 0: row i sees keys >= i - window (-1: no
    // limit).  cap_raw > 0: raw scores x become cap_raw * tanh(x / cap_raw), with
    // cap_raw = softcap / |scale|, so that x * |scale| is softcap * tanh(s / softcap);
    // cap_k = 2 log2(e) / cap_raw.
    int window;
    float cap_raw, cap_k;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufferFlags);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Resident waves per SIMD the register budget is sized for.  d = 256 keeps twice
// the Q fragments and accumulators in registers (about 330 live values), so it
// runs two waves per SIMD and spills the excess to scratch (216 bytes per lane,
// reloaded about three times per step in the loop): at 16/8 heads, 8k-16k
// prompts, 27-34% faster than one wave per SIMD with every value in (accumulation)
// registers, whose operand latency is then exposed.  Grids of at most 512
// workgroups take the one-wave instantiation (WPS = 1; 8 bytes of scratch) instead:
// 15-22% faster there (16/8 heads, 1k-4k prompts), as latency, not residency,
// sets their time.
template <int D> constexpr int waves_per_simd() { return D == 256 ? 2 : kWavesPerSimd; }

// Waves of one key group: the key split (KS = 2) runs two 2-wave groups over a
// 64-row query tile, the plain kernel one 4-wave group over 128 rows.
constexpr int split_group_waves(int ks) { return ks > 1 ? 2 : kWaves; }

// Chunk permutations of the LDS tiles (16-byte chunk c of key row r sits at
// slot c ^ swz(r)).  D = 128: a row is one 256-byte bank line; the K operand
// reads of 16 consecutive rows and the V transpose reads of 4 rows x 64 bytes
// land on distinct banks.  D = 256: a row is two bank lines, same permutation.
// D = 64: two rows share a bank line.
template <int D> __device__ __forceinline__ int k_swz(int r) { return D >= 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ __forceinline__ int v_swz(int r) { return D >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Memory -> LDS loader of one K or V tile (32 rows of D bf16).  A tile is
// 32*D/8 chunks = D/16 wave instructions of 64 chunks (1 KiB each); wave w issues
// instructions w, w + 4, ...  With that interleave the slot a lane fills has the
// same row permutation in all of its instructions (d <= 128), so one per-lane
// offset serves them all and the per-instruction part goes into the (scalar)
// buffer base.  D = 256: an instruction covers 2 rows, so a lane's rows are 8
// apart and the K permutation (r & 15) alternates; odd instructions flip bit 3 of
// the chunk slot (`odd_xor`), the V permutation (r & 3) does not change.
template <int D, int NW = kWaves>
struct TileLoader {
    static constexpr int RB = D * 2;                 // bytes per key row
    static constexpr int NC = D / 8;                 // 16-byte chunks per row
    static constexpr int RPI = 64 / NC;              // key rows per instruction
    static constexpr int INSTR = kBlockN * NC / 64;  // wave instructions per tile
    static constexpr int PER_WAVE = (INSTR + NW - 1) / NW;
    static_assert(INSTR % NW == 0 || INSTR < NW, "tile instructions split evenly over the waves");
    // a lane's instructions fill rows RPI * NW apart: with 4 loading waves (d <= 128)
    // those rows share their permutation; d = 256, and 2 loading waves at d = 128
    // (rows 8 apart), flip it on odd instructions
    static constexpr bool FLIP = D == 256 || NW != kWaves;
    static_assert(NW == kWaves || (NW == 2 && D <= 128), "4 loading waves, or 2 at d <= 128");
    static_assert(D != 256 || NW == 4, "the d = 256 odd-instruction flip assumes 4 waves");
    uint32_t voff;     // per-lane byte offset from the first row an instruction fills
    uint32_t rowb;     // bytes between consecutive key rows in memory
    uint32_t odd_xor;  // D = 256: offset flip of odd instructions (0 when the permutation repeats)

    template <typename Swz>
    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes, Swz swz)
    {
        const int u = wave * 64 + lane;  // LDS slot of this lane in its first instruction
        const int r = u / NC, pos = u % NC;
        rowb = row_bytes;
        voff = (uint32_t)(lane / NC) * row_bytes + 16u * (uint32_t)(pos ^ swz(r));
        // the lane's row in an odd instruction is r + RPI * NW
        odd_xor = 16u * (uint32_t)(swz(r) ^ swz(r + RPI * NW));
    }
    // Issue the loads of the tile starting at key k0 of one head (rows rowb apart,
    // n rows) into the LDS tile `dst`.  Each instruction's descriptor starts at its
    // own first row and ends at row n, so rows past n read as zero.
    __device__ __forceinline__ void load(const uint16_t *head, int n, int k0, int wave, uint16_t *dst) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int ins = wave + i * NW;
            if (INSTR < NW && ins >= INSTR) break;  // wave-uniform
            const int row0 = k0 + ins * RPI;
            // (n - row0) * rowb < 2^32: the launcher bounds a head's padded rows to
            // 32-bit byte offsets.  readfirstlane keeps the descriptor in scalar registers.
            const uint32_t rec = __builtin_amdgcn_readfirstlane((uint32_t)max(n - row0, 0) * rowb);
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(reinterpret_cast<const char *>(head) + (long long)row0 * rowb, rec);
            const uint32_t off = (FLIP && (i & 1)) ? (voff ^ odd_xor) : voff;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)((char *)dst + ins * 1024), 16, off, 0, 0, 0);
        }
    }
};

// vmcnt(0): this wave's loads (including those that write LDS) have landed
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// S^T = K Q^T of one tile for the wave's two query blocks.  `kad` is the lane's
// byte offset of the K fragment of d-step 0, key rows l32 (+32 for kb = 1):
// chunk 2s + hh of row r sits at slot (2s + hh) ^ swz = 2s ^ (hh ^ swz), i.e.
// d-step s is a XOR by 32s.
template <int D>
__device__ __forceinline__ void qk_tile(f32x16_t (&S)[kBlocks][kKB], const uint16_t *Ks,
                                        const bf16x8_t (&qf)[kBlocks][D / 16], uint32_t kad)
{
    const char *kb0 = reinterpret_cast<const char *>(Ks);
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) S[b][kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(kb0 + kb * 32 * 2 * D + (kad ^ (32u * s)));
#pragma unroll
            for (int b = 0; b < kBlocks; ++b)
                S[b][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[b][s], S[b][kb], 0, 0, 0);
        }
}

// O^T += V^T P^T of one tile for both query blocks.  `vad` is the lane's byte
// offset for 16-key step 0 and d-block 0: in 16-lane group G, lane 4r+q reads
// key row 4hh + r, dims 16(G&1) + 4q..+3; the lane's 8 key values are rows
// 16ks + 4hh + {0..3} and 16ks + 8 + 4hh + {0..3}, the score accumulator's order.
// d-block db is a XOR by 64db (the permutation moves whole 64-byte units).
template <int D>
__device__ __forceinline__ void pv_tile(f32x16_t (&acc)[kBlocks][D / 32], const uint16_t *Vs,
                                        const bf16x8_t (&pf)[kBlocks][kKS], uint32_t vad)
{
    const char *vb0 = reinterpret_cast<const char *>(Vs);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const char *p = vb0 + 16 * ks * 2 * D + (vad ^ (64u * db));
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p);
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p + 8 * 2 * D));
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int b = 0; b < kBlocks; ++b)
                acc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[b][ks], acc[b][db], 0, 0, 0);
        }
}

// Probabilities of one block's tile against reference mb (= m * scale * log2 e),
// rounded to bf16 in pairs straight into the B operands of the P*V product, and
// the lane's float32 sum of the unrounded probabilities.
__device__ __forceinline__ float softmax_tile(const f32x16_t (&S)[kKB], float sl2, float mb, bf16x8_t (&pf)[kKS])
{
    float rs0, rs1;
    uint32_t w[kKS][4];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(S[kb][i], sl2, -mb));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(S[kb][i + 1], sl2, -mb));
            const bf16x2_t pk = {(__bf16)p0, (__bf16)p1};
            w[2 * kb + (i >> 3)][(i & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
            rs0 = (kb == 0 && i == 0) ? p0 : rs0 + p0;  // the first term starts the sum (no 0 + p)
            rs1 = (kb == 0 && i == 0) ? p1 : rs1 + p1;
        }
#pragma unroll
    for (int j = 0; j < kKS; ++j) pf[j] = __builtin_bit_cast(bf16x8_t, make_uint4(w[j][0], w[j][1], w[j][2], w[j][3]));
    return rs0 + rs1;
}

// Logit soft-cap of one raw score: cap * tanh(x / cap), with tanh(y) = 1 - 2 / (e^{2y} + 1)
// (exact for y -> +-inf: the reciprocal of +inf is 0, of 1 is 1), cap_k = 2 log2(e) / cap.
__device__ __forceinline__ float soft_cap(float x, float cap, float cap_k)
{
    const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x * cap_k) + 1.f);
    return fmaf(-2.f * cap, r, cap);
}

// EXT selects the variant with a sliding window and logit soft-capping (a separate
// instantiation, so the plain kernel keeps its instruction schedule).  KS = 2
// selects the key-split variant for prompts too short to fill the GPU: the
// workgroup is two groups of 2 waves over the same 64 query rows, group g walks
// half g of the tile's key range with its own tile buffers and online-softmax
// state, and group 1 hands its (m, l, acc) to group 0 through LDS at the end,
// where the two are merged by the combine rule (split-KV inside one workgroup).
template <int D, bool EXT, int KS = 1, int WPS = waves_per_simd<D>()>
__global__ __launch_bounds__(split_group_waves(KS) * 64 * KS, KS > 1 ? 2 : WPS) void prefill_bf16_kernel(Args a)
{
    static_assert(KS == 1 || (KS == 2 && !EXT && D <= 128), "key split: plain kernel, d <= 128");
    // rows may meet tiles with no visible key before any reference exists (window,
    // or a key group whose range starts past the row): the reference is then taken
    // on the rare path instead of in the prologue
    constexpr bool REF = EXT || KS > 1;
    constexpr int NW = split_group_waves(KS);  // waves of one key group
    constexpr int NT = NW * 64;                // threads of one key group
    constexpr int BM = NW * kBlocks * 32;      // query rows per workgroup
    constexpr int TE = kBlockN * D;  // elements per K or V tile
    // separate LDS objects, so in-flight loads into one buffer do not make the
    // compiler wait before reading another; one set per key group
    __shared__ __attribute__((aligned(1024))) uint16_t KB0s[KS][TE];
    __shared__ __attribute__((aligned(1024))) uint16_t KB1s[KS][TE];
    __shared__ __attribute__((aligned(1024))) uint16_t VB0s[KS][TE];
    __shared__ __attribute__((aligned(1024))) uint16_t VB1s[KS][TE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_wg = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
    const int grp = KS > 1 ? wave_wg / NW : 0;  // key group
    const int wave = KS > 1 ? wave_wg % NW : wave_wg;  // query block and loader slot in the group
    const int gtid = KS > 1 ? tid % NT : tid;
    uint16_t *const KB0 = KB0s[grp];
    uint16_t *const KB1 = KB1s[grp];
    uint16_t *const VB0 = VB0s[grp];
    uint16_t *const VB1 = VB1s[grp];
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- work item: (q tile descending, b, kv head, q head), query head fastest ----
    const int item = blockIdx.x;
    const int G = a.B * a.Hkv;
    int bg, j, r;
    if (G <= 8 && (8 % G) == 0 && (a.n_items % 8) == 0) {
        // workgroup i runs on XCD i % 8 (each XCD has its own L2): give each (sequence,
        // KV head) its own 8 / G XCDs, which take its (query tile descending, query
        // head) list in turn, so that XCD's L2 holds one KV head's tiles
        const int per = 8 / G, xcd = item & 7, slot = item >> 3;
        bg = xcd / per;
        const int p = slot * per + (xcd % per);
        j = p % a.group;
        r = p / a.group;
    } else {
        j = item % a.group;
        bg = (item / a.group) % G;
        r = item / (a.group * G);
    }
    const int b = bg / a.Hkv, hk = bg % a.Hkv;
    const int h = hk * a.group + j;
    const int qtile = a.n_qtiles - 1 - r;
    const int q0 = qtile * BM;
    // this sequence's first token and length
    long long tok0;
    int N;
    if (a.cu_seqlens) {
        // offsets outside [0, T] or a length above the launch's maximum are
        // clamped, so nothing outside the packed tensors is touched
        const int s0 = min(max(a.cu_seqlens[b], 0), a.T);
        const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.T);
        tok0 = s0;
        N = min(s1 - s0, a.N);
    } else {
        tok0 = (long long)b * a.N;
        N = a.N;
    }
    if (q0 >= N) return;  // whole workgroup: no query row of this tile exists
    // element offsets of this (sequence, head): packed rows are token-major
    const long long qo = a.cu_seqlens ? tok0 * a.Hq * D + (long long)h * a.q_head
                                      : ((long long)b * a.Hq + h) * a.q_head;
    const long long kvo = a.cu_seqlens ? tok0 * a.Hkv * D + (long long)hk * a.kv_head
                                       : ((long long)b * a.Hkv + hk) * a.kv_head;
    const long long lse_off = a.cu_seqlens ? (long long)h * a.lse_head + tok0 : ((long long)b * a.Hq + h) * a.lse_head;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(a.q + qo, (uint32_t)min((long long)N * a.q_row * 2, 0xFFFFFFFFLL));
    const uint16_t *const kh = a.k + kvo;
    const uint16_t *const vh = a.v + kvo;

    const int wrow0 = q0 + wave * (kBlocks * 32);  // first query row of this wave
    // Q fragments (B operand of S^T = K Q^T), resident for the whole kernel;
    // rows past N read as zero.
    bf16x8_t qf[kBlocks][D / 16];
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint4 u = bload16(rq, (uint32_t)(((long long)(wrow0 + 32 * bb + l32) * a.q_row + 16 * s + 8 * hh) * 2), 0);
            if (a.negate_q) {  // scale < 0: s*scale = (-s)*|scale|, so the max stays on raw scores
                u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
            }
            qf[bb][s] = as_bf16x8(u);
        }

    f32x16_t acc[kBlocks][D / 32];
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[bb][db][i] = 0.f;
    // mb: the reference max of the scores in base-2 units (raw max * scale * log2 e);
    // l: this lane's share of the row sum
    float mb[kBlocks], l[kBlocks];
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb) {
        mb[bb] = -INFINITY;
        l[bb] = 0.f;
    }
    const float sl2 = a.scale_log2;
    const int xlane = (lane ^ 32) << 2;  // ds_bpermute address of the other half-wave

    TileLoader<D, NW> kld, vld;
    kld.init(wave, lane, (uint32_t)(a.kv_row * 2), [](int rr) { return k_swz<D>(rr); });
    vld.init(wave, lane, (uint32_t)(a.kv_row * 2), [](int rr) { return v_swz<D>(rr); });
    // Operand reads address this group's buffers from group 0's, whose LDS addresses
    // are compile-time constants (they fold into the reads' immediate offsets, as in
    // the unsplit kernel, instead of costing an add per read and step), with the
    // group's offset in the per-lane offsets.  A tile is 2 TE bytes, a power of two,
    // and the reads' XOR terms stay below it, so they never reach the offset's bits.
    const uint16_t *const KR0 = KB0s[0], *const KR1 = KB1s[0], *const VR0 = VB0s[0], *const VR1 = VB1s[0];
    static_assert((2 * TE & (2 * TE - 1)) == 0, "tile bytes a power of two");
    const uint32_t goff = (uint32_t)grp * 2 * TE;
    const uint32_t kad = (uint32_t)(l32 * 2 * D + 16 * (hh ^ k_swz<D>(l32))) + goff;
    uint32_t vad;
    {
        const int j16 = lane & 15, h16 = (lane >> 4) & 1, rr = j16 >> 2, q = j16 & 3;
        const int row = 4 * hh + rr;
        const int c = 2 * h16 + (q >> 1);
        vad = (uint32_t)(row * 2 * D + 16 * (c ^ v_swz<D>(row)) + 8 * (q & 1)) + goff;
    }

    const int kend = a.causal ? min(N, q0 + BM) : N;  // keys this tile may see
    // with a window, the first tile that holds a key of row q0's window
    const int kbeg = (EXT && a.window >= 0) ? max(0, q0 - a.window) / kBlockN * kBlockN : 0;
    int ntiles = (kend - kbeg + kBlockN - 1) / kBlockN;  // >= 1: key q0 is visible to row q0
    int gbeg = kbeg;  // first key of this group's tiles
    if (KS > 1) {
        // group g takes tiles g*half .. g*half + half - 1; tiles past the range (the
        // second group's last one when the count is odd) lie past the diagonal or
        // past N, so the mask hides all their keys and they add nothing
        const int half = (ntiles + 1) / 2;
        gbeg = kbeg + grp * half * kBlockN;
        ntiles = half;
    }

    // ---- prologue ------------------------------------------------------------------
    // V buffers start as zeros: "tile -1" is multiplied by P = 0, and rows past N
    // of a ragged last tile must be finite whether or not the loads write them.
    for (int i = gtid; i < TE / 8; i += NT) {
        reinterpret_cast<uint4 *>(VB0)[i] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4 *>(VB1)[i] = make_uint4(0, 0, 0, 0);
    }
    kld.load(kh, N, gbeg, wave, KB0);
    if (ntiles > 1) kld.load(kh, N, gbeg + kBlockN, wave, KB1);
    wait_loads();
    __syncthreads();
    f32x16_t S[kBlocks][kKB];
    // diagonal / ragged tile: mask keys past the row (causal) or past N; with a
    // window also keys before row - window
    auto mask_tile = [&](int k0) {
        const bool win = EXT && a.window >= 0 && k0 < wrow0 + kBlocks * 32 - 1 - a.window;
        if ((a.causal && k0 + kBlockN - 1 > wrow0) || k0 + kBlockN > N || win) {
#pragma unroll
            for (int bb = 0; bb < kBlocks; ++bb) {
                const int qrow = wrow0 + 32 * bb + l32;
                const int lim = (a.causal ? min(qrow, N - 1) : N - 1) - (k0 + 4 * hh);
                const int low = win ? qrow - a.window - (k0 + 4 * hh) : INT_MIN;
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int e = 32 * kb + 8 * (i >> 2) + (i & 3);
                        if (e > lim || (EXT && e < low)) S[bb][kb][i] = -INFINITY;
                    }
            }
        }
    };
    // the row max of the visible keys of scores S, both half-waves combined
    auto row_max = [&](int bb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[bb][kb][i]);
        return fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, mx))));
    };
    qk_tile<D>(S, KR0, qf, kad);
    if (!REF) {
        // The plain kernel starts from the first tile's true max: every row sees key
        // 0 (causal) or all keys < N, so it is finite, and the steps need no check
        // for a missing reference.  (The variant's soft-cap and window act at the
        // start of each step, so it keeps the check.)
        mask_tile(kbeg);
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) mb[bb] = row_max(bb) * sl2;
    }
    bf16x8_t P0[kBlocks][kKS], P1[kBlocks][kKS];
#pragma unroll
    for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) P1[bb][ks][e] = (__bf16)0.f;  // "tile -1": P = 0 against zeroed VB1
    __syncthreads();  // every wave has read KB0 before step 0 refills it

    // One step.  S holds the scores of tile t; Pp the probabilities of tile t-1,
    // Pc receives tile t's.  K(t+1) is in Kn, V(t-1) in Vp; the step loads
    // K(t+2) into Kw and V(t) into Vw.
    auto step = [&](bf16x8_t (&Pp)[kBlocks][kKS], bf16x8_t (&Pc)[kBlocks][kKS], int t, const uint16_t *Kn,
                    const uint16_t *Vp, uint16_t *Kw, uint16_t *Vw) {
        const int k0 = gbeg + t * kBlockN;
        if (t + 2 < ntiles) kld.load(kh, N, k0 + 2 * kBlockN, wave, Kw);
        vld.load(vh, N, k0, wave, Vw);
        if (EXT && a.cap_raw > 0.f) {  // soft-cap before masking, so masked scores stay -inf
#pragma unroll
            for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) S[bb][kb][i] = soft_cap(S[bb][kb][i], a.cap_raw, a.cap_k);
        }
        mask_tile(k0);
        // ---- matrix cores: PV(t-1); vector ALUs: probabilities of tile t against
        // the reference max from before the tile (the variant's first tile, with no
        // reference yet, takes the rare path)
        // raised wave priority while this block issues: the arbiter then favours the
        // wave whose products and softmax interleave, over waves in their QK part
        __builtin_amdgcn_s_setprio(1);
        pv_tile<D>(acc, Vp, Pp, vad);
        float rs[kBlocks];
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) rs[bb] = softmax_tile(S[bb], sl2, mb[bb], Pc[bb]);
        // Instruction order of this block: the V operand reads run three products
        // ahead, and the softmax's VALU work is spread between the products so
        // the matrix cores and the vector ALUs overlap inside the wave.
        // (masks: 0x008 MFMA, 0x100 LDS read, 0x002 VALU)
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < kKS * (D / 32) * kBlocks; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // ---- rare: some probability may exceed 2^8 (or a row has no reference yet):
        // raise the reference to the true running max, rescale, redo the tile
        bool redo = REF && mb[0] == -INFINITY;
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) redo = redo || rs[bb] > kMaxLaneSum;
        if (__builtin_amdgcn_ballot_w64(redo)) {
            // an (empty) use of the first attempt on this path too, so the compiler
            // computes it above, between the products, instead of below the branch
#pragma unroll
            for (int bb = 0; bb < kBlocks; ++bb)
#pragma unroll
                for (int jj = 0; jj < kKS; ++jj) asm volatile("" ::"v"(Pc[bb][jj]));
#pragma unroll
            for (int bb = 0; bb < kBlocks; ++bb) {
                const float mb_new = fmaxf(mb[bb], row_max(bb) * sl2);
                // c = 0 while mb = -inf.  Only the variant can meet a row with no visible
                // key yet (mb_new = -inf); its state stays (mb, l, acc) = (-inf, 0, 0),
                // and a reference of 0 gives the masked scores probability 0.
                const bool none = REF && mb_new == -INFINITY;
                const float c = none ? 1.f : __builtin_amdgcn_exp2f(mb[bb] - mb_new);
                l[bb] *= c;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[bb][db][i] *= c;
                mb[bb] = mb_new;
                rs[bb] = softmax_tile(S[bb], sl2, none ? 0.f : mb[bb], Pc[bb]);
            }
        }
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) l[bb] += rs[bb];
        // ---- matrix cores: QK(t+1) into the freed score registers
        if (t + 1 < ntiles) {
            qk_tile<D>(S, Kn, qf, kad);
            // the first four K operand reads issue before the first product, so three
            // stay in flight behind the one each product consumes
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < (D / 16) * kKB * kBlocks; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        wait_loads();
        __syncthreads();
    };

    // step t reads K(t+1) from KB[(t+1)&1] and V(t-1) from VB[(t-1)&1];
    // it loads K(t+2) into KB[t&1] and V(t) into VB[t&1]
    for (int t = 0; t < ntiles; t += 2) {
        step(P1, P0, t, KR1, VR1, KB0, VB0);
        if (t + 1 < ntiles) step(P0, P1, t + 1, KR0, VR0, KB1, VB1);
    }
    // last product: P of tile ntiles-1 is in P0 (ntiles odd) or P1 (even), V in VB[(ntiles-1)&1]
    if (ntiles & 1)
        pv_tile<D>(acc, VR0, P0, vad);
    else
        pv_tile<D>(acc, VR1, P1, vad);

    if constexpr (KS > 1) {
        // group 1 hands its state to group 0 through LDS (the tile buffers are free
        // once every wave has finished its last product); group 0 merges it by the
        // combine rule: weights c_g = 2^(m_g - M) with M the larger reference (0 for
        // a group that saw no key of the row), l = sum c_g l_g, acc = sum c_g acc_g
        __shared__ float xml[NW][2][64];
        __syncthreads();
        // wave w of each group uses the w-th tile buffer array (KS * TE elements)
        static_assert(NW <= 4 && (D / 32) * 16 * 64 * 4 <= KS * TE * 2, "one exchange slab per wave");
        uint16_t *const xbuf = wave == 0 ? &KB0s[0][0] : wave == 1 ? &KB1s[0][0] : wave == 2 ? &VB0s[0][0] : &VB1s[0][0];
        f32x16_t *const slab = reinterpret_cast<f32x16_t *>(xbuf);
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    reinterpret_cast<float4 *>(slab)[(db * 4 + c) * 64 + lane] =
                        make_float4(acc[0][db][4 * c], acc[0][db][4 * c + 1], acc[0][db][4 * c + 2], acc[0][db][4 * c + 3]);
            xml[wave][0][lane] = mb[0];
            xml[wave][1][lane] = l[0];
        }
        __syncthreads();
        if (grp == 1) return;
        const float m1 = xml[wave][0][lane], l1 = xml[wave][1][lane];
        const float M = fmaxf(mb[0], m1);
        const float c0 = mb[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb[0] - M);
        const float c1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
        l[0] = c0 * l[0] + c1 * l1;
        mb[0] = M;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 o1 = reinterpret_cast<const float4 *>(slab)[(db * 4 + c) * 64 + lane];
                acc[0][db][4 * c] = c0 * acc[0][db][4 * c] + c1 * o1.x;
                acc[0][db][4 * c + 1] = c0 * acc[0][db][4 * c + 1] + c1 * o1.y;
                acc[0][db][4 * c + 2] = c0 * acc[0][db][4 * c + 2] + c1 * o1.z;
                acc[0][db][4 * c + 3] = c0 * acc[0][db][4 * c + 3] + c1 * o1.w;
            }
    }

    // ---- epilogue: O = acc / l, LSE = m * scale + ln l ---------------------------------
    if constexpr (KS > 1) {
        // key split (short prompts): O goes through the wave's own tile buffer in LDS, free
        // once the groups have merged, so the global stores write whole rows, 16 bytes per
        // lane (a store in accumulator order touches 32 rows per instruction, this one
        // 64 / (d / 8)): -0.6 us per workgroup, +4% at 2k prompts.  The plain kernel keeps
        // the direct stores: the staging's registers cost its main loop operand lookahead.
        static_assert(kBlocks == 1, "one 32-row query block per wave");
        char *const obuf = reinterpret_cast<char *>(wave == 0   ? &KB0s[0][0]
                                                    : wave == 1 ? &KB1s[0][0]
                                                    : wave == 2 ? &VB0s[0][0]
                                                                : &VB1s[0][0]);
        constexpr int RB = 2 * D;  // bytes per staged row
        constexpr int CH = D / 8;  // 16-byte chunks per row
        // chunk c of row r sits at slot c ^ oswz(r): the 32 rows a store instruction writes
        // and the rows a load instruction reads then spread over the banks
        auto oswz = [](int row) { return D == 64 ? ((row >> 1) & 7) : (row & 15); };
        {
            const int qrow = wrow0 + l32;
            const float lt =
                l[0] + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, l[0])));
            const float inv = 1.f / lt;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int ig = 0; ig < 4; ++ig) {
                    // dims 32 db + 8 ig + 4 hh .. + 3 of row l32: 16-byte chunk 4 db + ig, half hh
                    const bf16x2_t lo = {(__bf16)(acc[0][db][4 * ig + 0] * inv), (__bf16)(acc[0][db][4 * ig + 1] * inv)};
                    const bf16x2_t hi = {(__bf16)(acc[0][db][4 * ig + 2] * inv), (__bf16)(acc[0][db][4 * ig + 3] * inv)};
                    uint2 pk;
                    pk.x = __builtin_bit_cast(uint32_t, lo);
                    pk.y = __builtin_bit_cast(uint32_t, hi);
                    *reinterpret_cast<uint2 *>(obuf + l32 * RB + 16 * ((4 * db + ig) ^ oswz(l32)) + 8 * hh) = pk;
                }
            }
            if (qrow < N && hh == 0) a.lse[lse_off + qrow] = (mb[0] + log2f(lt)) * kLn2;  // mb * ln 2 = max * |scale|
        }
        {
            constexpr int LPR = CH;        // lanes per row
            constexpr int RPI = 64 / LPR;  // rows per instruction
            const int c = lane % LPR;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int rr = RPI * k + lane / LPR;  // the wave's own rows: no barrier needed
                const uint4 v = *reinterpret_cast<const uint4 *>(obuf + rr * RB + 16 * (c ^ oswz(rr)));
                const int qrow = wrow0 + rr;
                if (qrow < N) *reinterpret_cast<uint4 *>(a.o + qo + (long long)qrow * a.q_row + 8 * c) = v;
            }
        }
    } else {
#pragma unroll
        for (int bb = 0; bb < kBlocks; ++bb) {
            const int qrow = wrow0 + 32 * bb + l32;
            const float lt =
                l[bb] + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, l[bb])));
            if (qrow < N) {
                const float inv = 1.f / lt;
                uint16_t *orow = a.o + qo + (long long)qrow * a.q_row;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                    for (int ig = 0; ig < 4; ++ig) {
                        const int d0 = 32 * db + 8 * ig + 4 * hh;
                        const bf16x2_t lo = {(__bf16)(acc[bb][db][4 * ig + 0] * inv), (__bf16)(acc[bb][db][4 * ig + 1] * inv)};
                        const bf16x2_t hi = {(__bf16)(acc[bb][db][4 * ig + 2] * inv), (__bf16)(acc[bb][db][4 * ig + 3] * inv)};
                        uint2 pk;
                        pk.x = __builtin_bit_cast(uint32_t, lo);
                        pk.y = __builtin_bit_cast(uint32_t, hi);
                        *reinterpret_cast<uint2 *>(orow + d0) = pk;
                    }
                }
                if (hh == 0) a.lse[lse_off + qrow] = (mb[bb] + log2f(lt)) * kLn2;  // mb * ln 2 = max * |scale|
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams &p, hipStream_t stream)
{
    Args a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.o = static_cast<uint16_t *>(p.o);
    a.lse = p.lse;
    a.cu_seqlens = p.cu_seqlens;
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
    a.causal = p.causal;
    const long long D = p.head_dim;
    if (p.cu_seqlens) {  // packed [T, H, d]; lse [Hq, T]; N is the longest sequence
        a.T = p.total;
        a.q_head = D; a.q_row = (long long)p.Hq * D;
        a.kv_head = D; a.kv_row = (long long)p.Hkv * D;
        a.lse_head = p.total;
    } else {  // padded [B, H, N, d]; lse [B, Hq, N]
        a.T = p.B * p.N;
        a.q_head = (long long)p.N * D; a.q_row = D;
        a.kv_head = (long long)p.N * D; a.kv_row = D;
        a.lse_head = p.N;
    }
    a.n_qtiles = (p.N + kBM - 1) / kBM;
    a.negate_q = p.scale < 0.f ? 1 : 0;
    // |scale| below 1e-30 is raised to 1e-30: every probability still rounds to
    // exactly 1 (the scale-0 result), and the reference max stays finite.
    a.scale = fmaxf(fabsf(p.scale), 1e-30f);
    a.scale_log2 = a.scale * kLog2e;
    // a window reaching back past the first key limits nothing
    a.window = (p.window >= 0 && p.window < p.N) ? p.window : -1;
    a.cap_raw = p.softcap > 0.f ? p.softcap / a.scale : 0.f;
    a.cap_k = p.softcap > 0.f ? 2.f * kLog2e / a.cap_raw : 0.f;
    const bool ext = a.window >= 0 || p.softcap > 0.f;
    const long long items = (long long)a.n_qtiles * p.B * p.Hq;
    if (items == 0) return hipSuccess;
    if (items > 0x7fffffffLL) return hipErrorInvalidValue;
    // per-head byte ranges, including the padded last query tile, must fit 32 bits
    const long long rows = (long long)a.n_qtiles * kBM;
    if (rows * a.q_row * 2 > 0xffffffffLL || rows * a.kv_row * 2 > 0xffffffffLL) return hipErrorInvalidValue;
    a.n_items = (int)items;
    // Key split for grids that leave the GPU mostly idle: with at most
    // kSplitMaxItems 128-row tiles (two per compute unit on 256 compute units) the
    // longest query tiles' key walks set the time, and a second wave group that
    // takes half of each walk shortens them.  The split runs 64-row tiles (twice
    // the workgroups, 4 waves each, two per compute unit), which halves the
    // longest walk again and lets a compute unit hold two workgroups that need
    // not wait at each other's barriers.  Measured at 28/4 heads, d = 128: +6% at
    // N = 1024 and +3.5% at 2048 for the split with 128-row tiles over none, -14%
    // at 3072 (672 workgroups), hence the bound; 64-row tiles then +4 to +6% at
    // N = 1024-2048, +6 to +8% at d = 64, +0 to +3% at 480-512 tiles.  Needs at
    // least two query tiles.
    constexpr long long kSplitMaxItems = 2 * 256;
    const bool split = !ext && p.head_dim <= 128 && items <= kSplitMaxItems && a.n_qtiles >= 2;
    long long launched = items;
    if (split) {
        constexpr int rows_per_tile = split_group_waves(2) * kBlocks * 32;
        a.n_qtiles = (p.N + rows_per_tile - 1) / rows_per_tile;
        launched = (long long)a.n_qtiles * p.B * p.Hq;
        a.n_items = (int)launched;
    }
    // d = 256 on such grids: one wave per SIMD (see waves_per_simd)
    const bool one_wave = !ext && p.head_dim == 256 && items <= kSplitMaxItems;
    const dim3 grid((unsigned)launched), block(split ? split_group_waves(2) * 64 * 2 : kWaves * 64);
    auto launch = [&](auto dconst) {
        constexpr int DD = decltype(dconst)::value;
        if (ext)
            hipLaunchKernelGGL((prefill_bf16_kernel<DD, true>), grid, block, 0, stream, a);
        else if constexpr (DD <= 128) {
            if (split)
                hipLaunchKernelGGL((prefill_bf16_kernel<DD, false, 2>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((prefill_bf16_kernel<DD, false>), grid, block, 0, stream, a);
        } else {
            if (one_wave)
                hipLaunchKernelGGL((prefill_bf16_kernel<DD, false, 1, 1>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((prefill_bf16_kernel<DD, false>), grid, block, 0, stream, a);
        }
    };
    if (p.head_dim == 128)
        launch(std::integral_constant<int, 128>());
    else if (p.head_dim == 64)
        launch(std::integral_constant<int, 64>());
    else
        launch(std::integral_constant<int, 256>());
    return hipGetLastError();
}

}  // namespace attn
