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
//   * workgroup = WAVES waves x 32 query rows; key/value tile = 64 keys.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = K rows read from LDS, B = the wave's Q rows kept in registers for the
//     whole kernel.  In the 32x32 accumulator a lane holds one query (lane % 32)
//     and 16 of the 32 keys, so the row max and row sum are in-register work
//     plus one exchange with the other half-wave (lane ^ 32).
//   * The output is accumulated transposed as well, O^T += V^T P^T: the score
//     accumulator, rounded to bf16, is already the B operand (the contraction
//     over keys is order-free, so both operands use the key order in which the
//     accumulator holds them) and every lane again owns one query, so the
//     rescale by c is per lane.  V is written to LDS transposed, in that key
//     order, so each A fragment is one 16-byte LDS read.
//   * Software pipeline: iteration t issues the P*V product of tile t-1 and the
//     scores of tile t+1 on the matrix cores while the vector ALUs compute the
//     softmax of tile t, all in one basic block, so the two units overlap
//     inside a wave.  K/V tiles are double-buffered in LDS and fetched one
//     iteration ahead with buffer loads (one descriptor per tile, rows past N
//     read as zero); one barrier per tile.
//   * The exponentials of tile t use the running max from before the tile,
//     so they do not wait for the tile's own row max.  Only if some row's new
//     scores exceed that max by more than 2^8 (in base-2 units) does a rare
//     fix-up path raise the max, rescale l and O by c, and recompute the tile's
//     probabilities.  Any reference value gives the same O = acc/l and
//     LSE = m + ln l; the bound keeps every probability <= 256 in float32.
//     Exponentials run in base 2 with scale*log2(e) folded into one FMA.
//   * Work order: consecutive workgroup ids are dispatched round-robin over the
//     8 XCDs, each with its own L2.  Ids are remapped so each XCD receives a
//     contiguous slice of a list ordered (sequence, KV head, query tile, query
//     head): the workgroups resident on one XCD share one KV head's keys and
//     values in L2.  Query tiles are listed in zig-zag order (last, first,
//     second last, second, ...) so every slice carries the same causal work
//     and the longest tiles start first.
//
// This file is compiled with -fno-honor-nans (inputs must be finite): the row
// max then maps to v_max3_f32 without NaN-quieting copies.  Infinities, which
// the masking relies on, keep their IEEE meaning.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBlockN = 64;  // keys per tile
constexpr int kXcds = 8;     // MI355X: workgroups are dispatched round-robin over 8 XCDs
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMaxLaneSum = 256.f;            // a lane's tile sum above this redoes the tile
constexpr uint32_t kBufferFlags = 0x00020000u;  // raw buffer, 32-bit data format

struct Args {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int B, N, Hq, Hkv, group, causal, n_qtiles, n_items;
    int negate_q;      // 1 when the caller's scale is negative
    float scale_log2;  // |scale| * log2(e)
    float scale;       // |scale|
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

// 64-byte unit permutation of the row-major V tile in LDS: unit u of key row r
// sits at u ^ vswz(r), so the transpose reads of 4 consecutive rows (64 bytes
// each) fall in distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? (r & 3) : ((r >> 1) & 1); }

// Global -> register -> LDS staging of one K tile and one V tile, both row-major
// (V is read back transposed by the LDS transpose read).  Each thread owns fixed
// 16-byte chunks; the tile's position is in the (scalar) descriptor, so a load is
// one buffer instruction with a per-lane offset fixed for the whole kernel.
template <int D, int NT>
struct Stage {
    static constexpr int KS = D + 8;        // K row stride in LDS (bf16): 16-byte aligned, bank-rotating
    static constexpr int KBUF = kBlockN * KS;
    static constexpr int VBUF = kBlockN * D;
    static constexpr int CHUNKS = kBlockN * D / 8;        // 16-byte chunks of a tile
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;    // per thread
    uint4 kr[CPT], vr[CPT];
    uint32_t goff[CPT], kls[CPT], vls[CPT];  // global byte offset in a tile / LDS element offsets

    __device__ __forceinline__ void init(int tid)
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int ch = tid + i * NT;
            const int r = ch / (D / 8), c = ch % (D / 8);
            goff[i] = (uint32_t)(r * D + 8 * c) * 2u;
            kls[i] = (uint32_t)(r * KS + 8 * c);
            vls[i] = (uint32_t)(r * D + 32 * ((c >> 2) ^ vswz<D>(r)) + 8 * (c & 3));
        }
    }

    __device__ __forceinline__ bool valid(int i, int tid) const { return CHUNKS % NT == 0 || tid + i * NT < CHUNKS; }

    // A tile's loads go through a descriptor based at the tile's first row whose
    // range ends at row N: rows past N read as zero and nothing past the head's
    // rows is touched.  (The range check applies to the per-lane offset, so the
    // tile offset is folded into the base rather than passed as a scalar offset.)
    __device__ __forceinline__ void load(uint4 (&dst)[CPT], const uint16_t *base, int N, int k0, int tid)
    {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (size_t)k0 * D, (uint32_t)max(N - k0, 0) * D * 2u);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if (valid(i, tid)) dst[i] = bload16(r, goff[i], 0);
    }
    __device__ __forceinline__ void load_k(const uint16_t *kh, int N, int k0, int tid) { load(kr, kh, N, k0, tid); }
    __device__ __forceinline__ void load_v(const uint16_t *vh, int N, int k0, int tid) { load(vr, vh, N, k0, tid); }
    __device__ __forceinline__ void store_k(uint16_t *Ks, int tid) const
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if (valid(i, tid)) *reinterpret_cast<uint4 *>(&Ks[kls[i]]) = kr[i];
    }
    __device__ __forceinline__ void store_v(uint16_t *Vs, int tid) const
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if (valid(i, tid)) *reinterpret_cast<uint4 *>(&Vs[vls[i]]) = vr[i];
    }
};

template <int D>
__device__ __forceinline__ void qk_tile(f32x16_t (&S)[2], const uint16_t *Ks, const bf16x8_t (&qf)[D / 16],
                                        int l32, int hh)
{
    constexpr int KS = D + 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(&Ks[(kb * 32 + l32) * KS + 16 * s + 8 * hh]);
            S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], S[kb], 0, 0, 0);
        }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// O^T += V^T P^T for one 64-key tile.  The A operand (V^T: 32 dims x 8 keys per
// lane) comes from the row-major V tile by two transpose reads: in 16-lane group
// G of the wave, lane 4r+q reads dims 16(G&1)+4q..+3 of key row kb+r, and lane j
// receives dim 16(G&1)+j of the 4 rows.  Keys follow the score accumulator's
// order: for 16-key step ks the lane's 8 values are keys 16ks + 4hh + {0..3} and
// 16ks + 8 + 4hh + {0..3}.  `vrd` is the lane's element offset for ks = 0, db = 0.
template <int D>
__device__ __forceinline__ void pv_tile(f32x16_t (&acc)[D / 32], const uint16_t *Vs, const bf16x8_t (&pf)[4],
                                        uint32_t vrd)
{
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            // rows 16ks.. keep the row's swizzle (16ks is a multiple of 4); unit db is a XOR
            const uint16_t *p = Vs + 16 * ks * D + (vrd ^ (32u * db));
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)p);
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(p + 8 * D));
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], acc[db], 0, 0, 0);
        }
}

// probabilities of one tile against reference mb (= m * scale * log2 e), their
// partial row sum, and the bf16 B operands of the P*V product
__device__ __forceinline__ float softmax_tile(const f32x16_t (&S)[2], float sl2, float mb, bf16x8_t (&pf)[4])
{
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(S[kb][i], sl2, -mb));
            if (i & 1) rs1 += p; else rs0 += p;
            pf[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
        }
    return rs0 + rs1;
}

template <int D, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 2) void prefill_bf16_kernel(Args a)
{
    constexpr int NT = WAVES * 64;
    constexpr int BM = WAVES * 32;
    using St = Stage<D, NT>;
    constexpr int KBUF = St::KBUF, VBUF = St::VBUF;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KBUF + 2 * VBUF];
    uint16_t *const KB0 = smem;
    uint16_t *const KB1 = smem + KBUF;
    uint16_t *const VB0 = smem + 2 * KBUF;
    uint16_t *const VB1 = smem + 2 * KBUF + VBUF;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- work item: XCD-contiguous slices of (b, kv head, zig-zag q tile, q head) ----
    int item;
    {
        const int x = blockIdx.x, xcd = x % kXcds, i = x / kXcds;
        const int base = a.n_items / kXcds, rem = a.n_items % kXcds;
        item = xcd * base + min(xcd, rem) + i;
    }
    const int j = item % a.group;
    const int r = (item / a.group) % a.n_qtiles;
    const int bg = item / (a.group * a.n_qtiles);
    const int b = bg / a.Hkv, hk = bg % a.Hkv;
    const int h = hk * a.group + j;
    const int qtile = (r & 1) ? (r >> 1) : a.n_qtiles - 1 - (r >> 1);
    const int bh = b * a.Hq + h;
    const int q0 = qtile * BM;
    const uint32_t head_bytes = (uint32_t)a.N * D * 2u;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + (size_t)bh * a.N * D, head_bytes);
    const uint16_t *const kh = a.k + (size_t)(b * a.Hkv + hk) * a.N * D;
    const uint16_t *const vh = a.v + (size_t)(b * a.Hkv + hk) * a.N * D;

    const int wrow0 = q0 + wave * 32;  // first query row of this wave
    const int qrow = wrow0 + l32;      // the query row this lane owns

    // Q fragments (B operand of S^T = K Q^T), resident for the whole kernel;
    // rows past N read as zero.
    bf16x8_t qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        uint4 u = bload16(rq, (uint32_t)(qrow * D + 16 * s + 8 * hh) * 2u, 0);
        if (a.negate_q) {  // scale < 0: s*scale = (-s)*|scale|, so the max stays on raw scores
            u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
        }
        qf[s] = as_bf16x8(u);
    }

    f32x16_t acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    float m = -INFINITY;  // reference max of raw scores for this lane's row
    float l = 0.f;        // this lane's share of the running sum (its 16 of every 32 keys)
    const float sl2 = a.scale_log2;
    const int xlane = (lane ^ 32) << 2;      // ds_bpermute address of the other half-wave
    // transpose-read offset of this lane into a V tile (see pv_tile)
    const uint32_t vrd = [&] {
        const int w = lane & 15, r = w >> 2, q = w & 3, g1 = (lane >> 4) & 1;
        return (uint32_t)((4 * hh + r) * D + 32 * vswz<D>(r) + 16 * g1 + 4 * q);
    }();

    const int kend = a.causal ? min(a.N, q0 + BM) : a.N;  // keys this tile may see
    const int ntiles = (kend + kBlockN - 1) / kBlockN;

    // ---- prologue: K(0) and K(1) staged, VB1 zeroed, S(0) formed, V(0) in flight ------
    St st;
    st.init(tid);
    st.load_k(kh, a.N, 0, tid);
    st.store_k(KB0, tid);
    st.load_k(kh, a.N, kBlockN, tid);  // tile 1 (zeros past N); never multiplied in if ntiles == 1
    st.store_k(KB1, tid);
    for (int i = tid; i < VBUF / 8; i += NT) reinterpret_cast<uint4 *>(VB1)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    f32x16_t S0[2], S1[2];
    qk_tile<D>(S0, KB0, qf, l32, hh);
    bf16x8_t P0[4], P1[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) P1[ks][e] = (__bf16)0.f;  // "tile -1": P = 0 against the zeroed VB1
    st.load_v(vh, a.N, 0, tid);
    __syncthreads();  // every wave has read KB0 before iteration 0 refills it

    // One pipeline step.  Sc = scores of tile t (formed last step), Sn receives
    // tile t+1; Pp = probabilities of tile t-1, Pc receives tile t's.
    auto step = [&](f32x16_t (&Sc)[2], f32x16_t (&Sn)[2], bf16x8_t (&Pp)[4], bf16x8_t (&Pc)[4], int t,
                    const uint16_t *Kn, const uint16_t *Vp, uint16_t *Kw, uint16_t *Vw) {
        const int k0 = t * kBlockN;
        if (t + 2 < ntiles) st.load_k(kh, a.N, k0 + 2 * kBlockN, tid);  // fetched during this step
        // diagonal / ragged tile: mask keys past the row (causal) or past N
        if ((a.causal && k0 + kBlockN - 1 > wrow0) || k0 + kBlockN > a.N) {
            const int lim = (a.causal ? min(qrow, a.N - 1) : a.N - 1) - (k0 + 4 * hh);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) Sc[kb][i] = -INFINITY;
        }
        // ---- hot block: matrix cores run PV(t-1) and S(t+1) while the ALUs do softmax(t)
        // against the reference max from before this tile (the first tile, with no
        // reference yet, always takes the branch below)
        pv_tile<D>(acc, Vp, Pp, vrd);
        qk_tile<D>(Sn, Kn, qf, l32, hh);
        float rs = softmax_tile(Sc, sl2, m * sl2, Pc);
        // ---- rare: some probability may exceed 2^8 (or the row has no reference
        // yet): raise the reference to the true running max, rescale, redo the tile
        if (__ballot(m == -INFINITY || rs > kMaxLaneSum)) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, Sc[kb][i]);
            mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, mx))));
            const float m_new = fmaxf(m, mx);
            const float c = __builtin_amdgcn_exp2f((m - m_new) * sl2);  // 0 while m = -inf
            l *= c;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] *= c;
            m = m_new;
            rs = softmax_tile(Sc, sl2, m * sl2, Pc);
        }
        l += rs;
        // ---- stage K(t+2) and V(t) for the next step ------------------------------------
        if (t + 2 < ntiles) st.store_k(Kw, tid);
        st.store_v(Vw, tid);
        if (t + 1 < ntiles) st.load_v(vh, a.N, k0 + kBlockN, tid);
        __syncthreads();
    };

    // iteration t reads K(t+1) from KB[(t+1)&1] and V(t-1) from VB[(t-1)&1];
    // it writes K(t+2) into KB[t&1] and V(t) into VB[t&1]
    for (int t = 0; t < ntiles; t += 2) {
        step(S0, S1, P1, P0, t, KB1, VB1, KB0, VB0);
        if (t + 1 < ntiles) step(S1, S0, P0, P1, t + 1, KB0, VB0, KB1, VB1);
    }
    // last product: P of tile ntiles-1 is in P0 (ntiles odd) or P1 (even), V in VB[(ntiles-1)&1]
    if (ntiles & 1)
        pv_tile<D>(acc, VB0, P0, vrd);
    else
        pv_tile<D>(acc, VB1, P1, vrd);

    // ---- epilogue: O = acc / l, LSE = m * scale + ln l ---------------------------------
    const float lt = l + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xlane, __builtin_bit_cast(int, l)));
    if (qrow < a.N) {
        const float inv = 1.f / lt;
        uint16_t *orow = a.o + ((size_t)bh * a.N + qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int ig = 0; ig < 4; ++ig) {
                const int d0 = 32 * db + 8 * ig + 4 * hh;
                __bf16 r0 = (__bf16)(acc[db][4 * ig + 0] * inv);
                __bf16 r1 = (__bf16)(acc[db][4 * ig + 1] * inv);
                __bf16 r2 = (__bf16)(acc[db][4 * ig + 2] * inv);
                __bf16 r3 = (__bf16)(acc[db][4 * ig + 3] * inv);
                uint2 pk;
                pk.x = (uint32_t)__builtin_bit_cast(uint16_t, r0) | ((uint32_t)__builtin_bit_cast(uint16_t, r1) << 16);
                pk.y = (uint32_t)__builtin_bit_cast(uint16_t, r2) | ((uint32_t)__builtin_bit_cast(uint16_t, r3) << 16);
                *reinterpret_cast<uint2 *>(orow + d0) = pk;
            }
        }
        if (hh == 0) a.lse[(size_t)bh * a.N + qrow] = m * a.scale + log2f(lt) * kLn2;
    }
}

template <int D, int WAVES>
hipError_t launch(const Args &a, hipStream_t stream)
{
    hipLaunchKernelGGL((prefill_bf16_kernel<D, WAVES>), dim3((unsigned)a.n_items), dim3(WAVES * 64), 0,
                       stream, a);
    return hipGetLastError();
}

#ifndef ATTN_PREFILL_WAVES
#define ATTN_PREFILL_WAVES 8
#endif

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams &p, hipStream_t stream)
{
    constexpr int W = ATTN_PREFILL_WAVES;
    Args a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.k = static_cast<const uint16_t *>(p.k);
    a.v = static_cast<const uint16_t *>(p.v);
    a.o = static_cast<uint16_t *>(p.o);
    a.lse = p.lse;
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
    a.causal = p.causal;
    a.n_qtiles = (p.N + W * 32 - 1) / (W * 32);
    a.negate_q = p.scale < 0.f ? 1 : 0;
    // |scale| below 1e-30 is raised to 1e-30: every probability still rounds to
    // exactly 1 (the scale-0 result), and the reference max stays finite.
    a.scale = fmaxf(fabsf(p.scale), 1e-30f);
    a.scale_log2 = a.scale * kLog2e;
    const long long items = (long long)a.n_qtiles * p.B * p.Hq;
    if (items == 0) return hipSuccess;
    if (items > 0x7fffffffLL) return hipErrorInvalidValue;
    // per-head byte offsets, including the padded last query tile, must fit 32 bits
    if ((long long)(a.n_qtiles * W * 32) * p.head_dim * 2 > 0xffffffffLL) return hipErrorInvalidValue;
    a.n_items = (int)items;
    return p.head_dim == 128 ? launch<128, W>(a, stream) : launch<64, W>(a, stream);
}

}  // namespace attn
