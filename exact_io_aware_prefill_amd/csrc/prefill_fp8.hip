// Tiled exact prefill attention on FP8 (E4M3) inputs for gfx950 matrix cores.
//
// Method: the same tiled prefill with an online softmax as the bf16 kernel
// (pofe.ai, "FlashAttention for inference: tiled prefill and split-KV decoding",
// sections "Prefill: tiles, loop order and the tensor cores" and "The online
// softmax, with every symbol defined"), on 8-bit inputs, which the page names as
// the FlashAttention-3 direction (section "The bottleneck it attacks").  Scores
// are s = scale * dq * dk * <q8, k8> with per-(sequence, KV head) descale
// factors; the output is O = dv * sum_j p_j v8_j / l, written in bf16, and the
// row log-sum-exp over the scaled scores in float32.
//
// gfx950 mapping
//   * Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands,
//     unit block scales, float32 accumulation), transposed as in the bf16
//     kernel: S^T = K Q^T (A = K rows from LDS, B = the wave's 32 Q rows in
//     registers), O^T += V^T P^T (A = V^T from LDS, B = the probabilities).
//     The contraction depth is 64, so a key/value tile is 64 keys (two 32-key
//     score blocks) and one P*V product covers the whole tile.
//   * Operand slot s of A and slot s of B meet in the product (checked on the
//     GPU with an in-bounds probe).  A lane of the score accumulator holds
//     query l % 32 and, in block kb, keys 32 kb + 8 (r >> 2) + 4 (l >> 5) +
//     (r & 3) for register r; packed to E4M3 in register order these are the
//     lane's B slots 16 kb + r.  The V^T operand then needs, for slot 8t + k,
//     the value of key 16 t + 8 (k >> 2) + 4 (l >> 5) + (k & 3): one
//     ds_read_b64_tr_b8 per t, in which lanes 2k and 2k+1 of each 16-lane
//     group read the two halves of that key row's 16 bytes and lane j receives
//     byte j (dim j) of the 8 rows.
//   * Probabilities are exp2 of the scores against the running reference
//     (lazy max, as the bf16 kernel: a lane whose tile sum exceeds 256 redoes
//     the tile against the true max), so each is <= 256 < 448 and rounds to
//     E4M3 without saturating (round to nearest even).  The row sum l is kept
//     in float32 from the unrounded values, so the LSE does not see the
//     8-bit rounding; O does, by at most 2^-4 relative per term (and 2^-10
//     absolute below the normal range).
//   * Step t issues QK(t+1) into a second score buffer, then PV(t-1) with the
//     softmax of tile t; scheduling groups spread the softmax's vector work
//     over the four P*V products (after each, the four transpose reads of the
//     next product's V operand and twelve VALU instructions; two reads and ten
//     VALU measured 2% slower), so the matrix cores and the VALUs overlap
//     inside the wave.
//     The QK products stay in a block of their own (the guard on the last
//     step); pulling them into the interleave as well measured 0-1% slower.
//     Two waves per SIMD (about 205 VGPRs) cover each other's QK bursts; a
//     wave raises its priority over the P*V + softmax block (+2 to +3% at
//     8k-16k prompts, +8% at 4k), as the bf16 kernel does.
//   * K and V tiles go straight from memory into LDS (buffer loads with the LDS
//     destination bit), double-buffered.  16-byte chunk c of key row r sits at
//     slot c ^ swz(r); the permutations make the K operand reads (16 rows per
//     pass) and the transpose reads (8 rows x 2 chunks per 32 lanes) bank-
//     conflict free and are the same for every row a lane's load
//     instructions fill.
//   * Work order: longest first, as the bf16 kernel: every head's last query
//     tile before any shorter one, the query heads of a KV head side by side
//     (+9% at 16k prompts and +17% at 8k over per-KV-head zig-zag order).  When
//     the (sequence, KV head) pairs divide the 8 XCDs, each pair gets its own
//     XCDs so its 8-bit K/V tiles stay in their L2s (+2% more here; the bf16
//     kernel timed the same either way and keeps it for its traffic).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "attn_kernels.h"

namespace attn {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 4;                 // waves per workgroup, 32 query rows each
constexpr int kBM = kWaves * 32;          // query rows per workgroup
constexpr int kBlockN = 64;               // keys per tile (the product's depth)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxLaneSum = 256.f;      // a lane's tile sum above this redoes the tile
constexpr uint32_t kBufferFlags = 0x00020000u;
constexpr int kUnitScale = 127;           // E8M0 block scale 2^0

// Two layouts, as in the bf16 kernel.  Padded: q, o [B, Hq, N, D], k, v
// [B, Hkv, N, D], lse [B, Hq, N] (cu_seqlens NULL).  Packed: sequence b owns
// tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, o [T, Hq, D], k, v [T, Hkv, D]
// and lse [Hq, T].  Strides are in elements (bytes of the codes, bf16 of o).
struct Args {
    const uint8_t *q, *k, *v;  // E4M3 codes
    uint16_t *o;               // bf16
    float *lse;
    const float *dq, *dk, *dv; // [B, Hkv] descales, or NULL (1)
    const int32_t *cu_seqlens; // packed layout, or NULL
    int B, N, Hq, Hkv, group, causal, n_qtiles;
    int T;                     // packed: total tokens
    long long q_head, q_row;   // strides of q and o
    long long kv_head, kv_row; // strides of k and v
    long long lse_head;        // stride of lse between heads (rows are adjacent)
    float scale;
    // window / soft-cap instantiation only: row i sees keys >= i - window (-1: no
    // limit); softcap > 0 caps each scaled score s at softcap * tanh(s / softcap)
    int window;
    float softcap;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kBufferFlags);
}

// Chunk permutations (see the header).  D = 256: rows are 256 bytes (one bank
// line): the K operand reads (16 rows per pass, one chunk each) need 16 distinct
// slots, r & 15; the transpose reads (rows 0-3 and 8-11, or 4-7 and 12-15, two
// chunks each per 32 lanes) need those 8 rows' chunk pairs on distinct banks,
// 2 ((r & 3) | ((r >> 3) & 1) << 2).  D = 128: rows are 128 bytes (two per bank
// line).  D = 64: rows are 64 bytes (four per bank line).  Every permutation
// repeats within 16 rows, the spacing of a lane's rows in the loader.
template <int D> __device__ __forceinline__ int k_swz(int r)
{
    return D == 256 ? (r & 15) : D == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}
template <int D> __device__ __forceinline__ int v_swz(int r)
{
    return D == 256 ? 2 * ((r & 3) | (((r >> 3) & 1) << 2))
                    : D == 128 ? 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) : 2 * ((r >> 3) & 1);
}

// Memory -> LDS loader of one 64-row tile of D bytes per row: D/16 wave
// instructions of 64 16-byte chunks, wave w issuing instructions w, w + 4, ...
// A lane's rows in its instructions are 32 apart (16 for D = 256), which no
// permutation above distinguishes, so one per-lane offset serves them all.
template <int D>
struct TileLoader {
    static constexpr int NC = D / 16;           // chunks per row
    static constexpr int RPI = 64 / NC;         // rows per instruction
    static constexpr int INSTR = kBlockN * NC / 64;
    static constexpr int PER_WAVE = INSTR / kWaves;
    static_assert(INSTR % kWaves == 0, "tile instructions split evenly over the waves");
    static_assert(RPI * kWaves % 16 == 0 || PER_WAVE == 1, "a lane's rows are a multiple of 16 apart");
    uint32_t voff;  // per-lane byte offset from the first row an instruction fills
    uint32_t rowb;  // bytes between consecutive key rows in memory

    template <typename Swz>
    __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes, Swz swz)
    {
        const int u = wave * 64 + lane;
        const int r = u / NC, pos = u % NC;
        rowb = row_bytes;
        voff = (uint32_t)(lane / NC) * row_bytes + 16u * (uint32_t)(pos ^ swz(r));
    }
    // rows past n read as zero: each instruction's descriptor ends at row n
    // ((n - row0) * rowb < 2^32: the launcher bounds a head's padded rows)
    __device__ __forceinline__ void load(const uint8_t *head, int n, int k0, int wave, uint8_t *dst) const
    {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int ins = wave + i * kWaves;
            const int row0 = k0 + ins * RPI;
            const uint32_t rec = __builtin_amdgcn_readfirstlane((uint32_t)max(n - row0, 0) * rowb);
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(head + (long long)row0 * rowb, rec);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + ins * 1024), 16, voff, 0, 0, 0);
        }
    }
};

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ f32x16_t mfma8(i32x8_t a, i32x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0, kUnitScale);
}

// S^T = K Q^T for the tile's two 32-key blocks.  kad0/kad1: the lane's byte
// offsets of its two 16-byte K chunks for d-step 0 (d-step ds is a XOR by 64 ds).
template <int D>
__device__ __forceinline__ void qk_tile(f32x16_t (&S)[2], const uint8_t *Ks, const i32x8_t (&qf)[D / 64],
                                        uint32_t kad0, uint32_t kad1)
{
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 64; ++ds)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const uint8_t *base = Ks + kb * 32 * D;
            const uint4 lo = *reinterpret_cast<const uint4 *>(base + (kad0 ^ (64u * ds)));
            const uint4 hi = *reinterpret_cast<const uint4 *>(base + (kad1 ^ (64u * ds)));
            const i32x8_t kf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            S[kb] = mfma8(kf, qf[ds], S[kb]);
        }
}

// O^T += V^T P^T over the tile: one product per 32 dims, its A operand from four
// transpose reads (vad: the lane's address for t = 0, d-block 0; t adds 16 rows,
// d-block db is a XOR by 32 db).
template <int D>
__device__ __forceinline__ void pv_tile(f32x16_t (&acc)[D / 32], const uint8_t *Vs, i32x8_t pf, uint32_t vad)
{
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        i32x8_t vf;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const i32x2_t x =
                __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t *)(Vs + 16 * t * D + (vad ^ (32u * db))));
            vf[2 * t] = x[0];
            vf[2 * t + 1] = x[1];
        }
        acc[db] = mfma8(vf, pf, acc[db]);
    }
}

// Probabilities of one tile against reference mb (= m * sl2), packed to E4M3 in
// the order of the P*V operand's slots, and the lane's float32 sum of the
// unrounded values.
__device__ __forceinline__ float softmax_tile(const f32x16_t (&S)[2], float sl2, float mb, i32x8_t &pf)
{
    float rs0, rs1;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = 4 * (w & 3);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S[kb][r0], sl2, -mb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S[kb][r0 + 1], sl2, -mb));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(S[kb][r0 + 2], sl2, -mb));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(S[kb][r0 + 3], sl2, -mb));
        // the conversion keeps the other half of its destination: start from the
        // register's stale contents (replaced by the second conversion), not a zero
        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[w], false);
        packed = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, packed, true);
        pf[w] = packed;
        rs0 = w == 0 ? p0 + p2 : rs0 + (p0 + p2);  // the first terms start the sums (no 0 + p)
        rs1 = w == 0 ? p1 + p3 : rs1 + (p1 + p3);
    }
    return rs0 + rs1;
}

// PACKED selects the packed layout (a separate instantiation, so the padded one
// keeps its row strides as compile-time constants).
// Logit soft-cap of one raw score: cap * tanh(x / cap) with tanh(y) = 1 - 2 / (e^{2y} + 1)
// (exact for y -> +-inf), cap_k = 2 log2(e) / cap.
__device__ __forceinline__ float soft_cap(float x, float cap, float cap_k)
{
    const float r = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(x * cap_k) + 1.f);
    return fmaf(-2.f * cap, r, cap);
}

// EXT selects the sliding-window / soft-cap instantiation (the plain ones keep
// their instruction schedule).  D = 256 keeps twice the accumulators (128
// values) and Q fragments, about 280 live values, so it runs one wave per SIMD
// with the accumulation registers in use; D <= 128 runs two.
template <int D> constexpr int fp8_waves_per_simd() { return D == 256 ? 1 : 2; }

template <int D, bool PACKED, bool EXT>
__global__ __launch_bounds__(kWaves * 64, fp8_waves_per_simd<D>()) void prefill_fp8_kernel(Args a)
{
    constexpr int NT = kWaves * 64;
    constexpr int TB = kBlockN * D;  // bytes per K or V tile
    __shared__ __attribute__((aligned(1024))) uint8_t KB0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t KB1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t VB0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t VB1[TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- work item: (q tile descending, b, kv head, q head), query head fastest ----
    const int item = blockIdx.x;
    const int G = a.B * a.Hkv;
    const int n_items = a.n_qtiles * G * a.group;
    int bg, j, r;
    if (G <= 8 && (8 % G) == 0 && (n_items % 8) == 0) {
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
    const int q0 = qtile * kBM;
    // this sequence's first token and length
    long long tok0;
    int N;
    if (PACKED) {
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

    // effective scale of the raw 8-bit dot products, and the output factor
    const float dq = a.dq ? a.dq[b * a.Hkv + hk] : 1.f;
    const float dk = a.dk ? a.dk[b * a.Hkv + hk] : 1.f;
    const float dv = a.dv ? a.dv[b * a.Hkv + hk] : 1.f;
    const float eff = a.scale * dq * dk;
    const bool negate = eff < 0.f;  // s * eff = (-s) * |eff|: flip Q's sign bits
    const float aeff = fmaxf(fabsf(eff), 1e-30f);
    const float sl2 = aeff * kLog2e;
    // soft-cap on raw scores x: x * aeff becomes softcap * tanh(x * aeff / softcap)
    const float cap_raw = (EXT && a.softcap > 0.f) ? a.softcap / aeff : 0.f;
    const float cap_k = cap_raw > 0.f ? 2.f * kLog2e / cap_raw : 0.f;

    // element offsets of this (sequence, head): packed rows are token-major
    const long long qo = PACKED ? tok0 * a.Hq * D + (long long)h * a.q_head : ((long long)b * a.Hq + h) * a.q_head;
    const long long kvo = PACKED ? tok0 * a.Hkv * D + (long long)hk * a.kv_head : ((long long)b * a.Hkv + hk) * a.kv_head;
    const long long lse_off = PACKED ? (long long)h * a.lse_head + tok0 : ((long long)b * a.Hq + h) * a.lse_head;
    const long long q_row = PACKED ? a.q_row : D;        // elements between query rows
    const uint32_t kv_rowb = PACKED ? (uint32_t)a.kv_row : D;  // bytes between key rows
    const uint8_t *const kh = a.k + kvo;
    const uint8_t *const vh = a.v + kvo;
    const int wrow0 = q0 + wave * 32;

    // Q fragments: lane (query l32, half hh) holds dims 64 ds + 32 hh .. + 31
    i32x8_t qf[D / 64];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + qo, (uint32_t)min((long long)N * q_row, 0xFFFFFFFFLL));
        const uint32_t qrow_off = (uint32_t)((long long)(wrow0 + l32) * q_row) + 32u * hh;
        const int flip = negate ? (int)0x80808080u : 0;
#pragma unroll
        for (int ds = 0; ds < D / 64; ++ds) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              rq, qrow_off + 64u * ds + 16u * e, 0, 0));
                qf[ds][4 * e + 0] = (int)u.x ^ flip;
                qf[ds][4 * e + 1] = (int)u.y ^ flip;
                qf[ds][4 * e + 2] = (int)u.z ^ flip;
                qf[ds][4 * e + 3] = (int)u.w ^ flip;
            }
        }
    }

    f32x16_t acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int xlane = (lane ^ 32) << 2;

    TileLoader<D> kld, vld;
    kld.init(wave, lane, kv_rowb, [](int rr) { return k_swz<D>(rr); });
    vld.init(wave, lane, kv_rowb, [](int rr) { return v_swz<D>(rr); });
    const uint32_t kad0 = (uint32_t)(l32 * D + 16 * ((2 * hh) ^ k_swz<D>(l32)));
    const uint32_t kad1 = (uint32_t)(l32 * D + 16 * ((2 * hh + 1) ^ k_swz<D>(l32)));
    uint32_t vad;
    {
        const int g = lane >> 4, j16 = lane & 15, k = j16 >> 1, half8 = j16 & 1;
        const int r0 = 4 * hh + 8 * (k >> 2) + (k & 3);
        vad = (uint32_t)(r0 * D + 16 * ((g & 1) ^ v_swz<D>(r0)) + 8 * half8);
    }

    const int kend = a.causal ? min(N, q0 + kBM) : N;
    // with a window, the first tile holding a key of row q0's window
    const int kbeg = (EXT && a.window >= 0) ? max(0, q0 - a.window) / kBlockN * kBlockN : 0;
    const int ntiles = (kend - kbeg + kBlockN - 1) / kBlockN;  // >= 1: key q0 is visible to row q0

    // ---- prologue: V buffers start as zeros (tile -1 is multiplied by P = 0, and
    // rows past N must be finite)
    for (int i = tid; i < TB / 16; i += NT) {
        reinterpret_cast<uint4 *>(VB0)[i] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4 *>(VB1)[i] = make_uint4(0, 0, 0, 0);
    }
    kld.load(kh, N, kbeg, wave, KB0);
    if (ntiles > 1) kld.load(kh, N, kbeg + kBlockN, wave, KB1);
    wait_loads();
    __syncthreads();
    f32x16_t SA[2], SB[2];
    qk_tile<D>(SA, KB0, qf, kad0, kad1);
    i32x8_t P0, P1;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        P0[w] = 0;  // the packing reads each register's old contents (one half survives a step)
        P1[w] = 0;  // "tile -1": P = 0 against the zeroed VB1
    }
    __syncthreads();

    // step t: S holds tile t's scores, Sn receives tile t+1's (issued first, so
    // both products overlap the softmax of tile t)
    auto step = [&](f32x16_t (&S)[2], f32x16_t (&Sn)[2], i32x8_t &Pp, i32x8_t &Pc, int t, const uint8_t *Kn,
                    const uint8_t *Vp, uint8_t *Kw, uint8_t *Vw) {
        const int k0 = kbeg + t * kBlockN;
        if (t + 2 < ntiles) kld.load(kh, N, k0 + 2 * kBlockN, wave, Kw);
        vld.load(vh, N, k0, wave, Vw);
        if (EXT && cap_raw > 0.f) {  // soft-cap before masking, so masked scores stay -inf
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) S[kb][i] = soft_cap(S[kb][i], cap_raw, cap_k);
        }
        // a tile reaching below some row's window start (wrow0 + 31 - window for the wave's last row)
        const bool win = EXT && a.window >= 0 && k0 < wrow0 + 31 - a.window;
        if ((a.causal && k0 + kBlockN - 1 > wrow0) || k0 + kBlockN > N || win) {
            const int qrow = wrow0 + l32;
            const int lim = (a.causal ? min(qrow, N - 1) : N - 1) - (k0 + 4 * hh);
            const int low = win ? qrow - a.window - (k0 + 4 * hh) : INT_MIN;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int e = 32 * kb + 8 * (i >> 2) + (i & 3);
                    if (e > lim || (EXT && e < low)) S[kb][i] = -INFINITY;
                }
        }
        if (t + 1 < ntiles) qk_tile<D>(Sn, Kn, qf, kad0, kad1);
        // raised wave priority over the P*V products and the softmax: the SIMD's
        // other wave, in its QK products or at the barrier, yields the issue slots
        __builtin_amdgcn_s_setprio(1);
        pv_tile<D>(acc, Vp, Pp, vad);
        float rs = softmax_tile(S, sl2, m * sl2, Pc);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < (D / 64) * 2 + D / 32; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (__builtin_amdgcn_ballot_w64(m == -INFINITY || rs > kMaxLaneSum)) {
            asm volatile("" ::"v"(Pc));
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[kb][i]);
            mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, mx))));
            const float m_new = fmaxf(m, mx);
            // Only the window variant can meet a row with no visible key yet (m_new =
            // -inf): its state stays (m, l, acc) = (-inf, 0, 0), and a reference of 0
            // gives the masked scores probability 0.
            const bool none = EXT && m_new == -INFINITY;
            const float c = none ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * sl2);  // 0 while m = -inf
            l *= c;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] *= c;
            m = m_new;
            rs = softmax_tile(S, sl2, none ? 0.f : m * sl2, Pc);
        }
        l += rs;
        wait_loads();
        __syncthreads();
    };

    for (int t = 0; t < ntiles; t += 2) {
        step(SA, SB, P1, P0, t, KB1, VB1, KB0, VB0);
        if (t + 1 < ntiles) step(SB, SA, P0, P1, t + 1, KB0, VB0, KB1, VB1);
    }
    if (ntiles & 1)
        pv_tile<D>(acc, VB0, P0, vad);
    else
        pv_tile<D>(acc, VB1, P1, vad);

    // ---- epilogue: O = dv * acc / l (bf16), LSE = m * |eff| + ln l
    const int qrow = wrow0 + l32;
    const float lt = l + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, l)));
    if (qrow < N) {
        const float f = dv / lt;
        uint16_t *orow = a.o + qo + (long long)qrow * q_row;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                const int d0 = 32 * db + 8 * ig + 4 * hh;
                uint16_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) hv[e] = __builtin_bit_cast(uint16_t, (__bf16)(acc[db][4 * ig + e] * f));
                uint2 pk;
                pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
                pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = pk;
            }
        if (hh == 0) a.lse[lse_off + qrow] = m * aeff + log2f(lt) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_fp8(const PrefillFp8Params &p, hipStream_t stream)
{
    Args a;
    a.q = static_cast<const uint8_t *>(p.q);
    a.k = static_cast<const uint8_t *>(p.k);
    a.v = static_cast<const uint8_t *>(p.v);
    a.o = static_cast<uint16_t *>(p.o);
    a.lse = p.lse;
    a.dq = p.descale_q;
    a.dk = p.descale_k;
    a.dv = p.descale_v;
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
    a.causal = p.causal;
    a.scale = p.scale;
    a.cu_seqlens = p.cu_seqlens;
    a.T = p.total;
    const long long D = p.head_dim;
    if (p.cu_seqlens) {  // packed [T, H, D]
        a.q_head = D; a.q_row = (long long)p.Hq * D;
        a.kv_head = D; a.kv_row = (long long)p.Hkv * D;
        a.lse_head = p.total;
    } else {  // padded [B, H, N, D]
        a.q_head = (long long)p.N * D; a.q_row = D;
        a.kv_head = (long long)p.N * D; a.kv_row = D;
        a.lse_head = p.N;
    }
    a.n_qtiles = (p.N + kBM - 1) / kBM;
    const long long items = (long long)a.n_qtiles * p.B * p.Hq;
    if (items == 0) return hipSuccess;
    if (items > 0x7fffffffLL) return hipErrorInvalidValue;
    // one head's rows of one sequence, including the padded last query tile, are
    // addressed with 32-bit offsets (q rows are the widest)
    if ((long long)a.n_qtiles * kBM * a.q_row > 0xffffffffLL) return hipErrorInvalidValue;
    // a window reaching back past the first key limits nothing
    a.window = (p.window >= 0 && p.window < p.N) ? p.window : -1;
    a.softcap = p.softcap > 0.f ? p.softcap : 0.f;
    const bool ext = a.window >= 0 || a.softcap > 0.f;
    const dim3 grid((unsigned)items), block(kWaves * 64);
    auto launch = [&](auto dconst, auto packed, auto extc) {
        hipLaunchKernelGGL((prefill_fp8_kernel<decltype(dconst)::value, decltype(packed)::value, decltype(extc)::value>),
                           grid, block, 0, stream, a);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    auto by_ext = [&](auto dconst, auto packed) {
        if (ext)
            launch(dconst, packed, T_());
        else
            launch(dconst, packed, F_());
    };
    auto by_packed = [&](auto dconst) {
        if (p.cu_seqlens)
            by_ext(dconst, T_());
        else
            by_ext(dconst, F_());
    };
    if (p.head_dim == 128)
        by_packed(std::integral_constant<int, 128>());
    else if (p.head_dim == 256)
        by_packed(std::integral_constant<int, 256>());
    else
        by_packed(std::integral_constant<int, 64>());
    return hipGetLastError();
}

}  // namespace attn
