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
//   * 8 waves per workgroup; each wave walks 32-token steps of the chunk with its
//     own online-softmax state, and the eight states are merged through LDS at
//     the end (the same combine rule, inside the workgroup).
//   * Scores use v_mfma_f32_16x16x32_bf16 on S^T = K Q^T: the A operand is read
//     straight from the cache (lane = token, 16 bytes of its row), the B operand
//     holds the group's query rows (padded to 16 with zeros) for the whole
//     kernel.  A lane of the accumulator then owns one query head and four
//     tokens, so the softmax is in-register plus two half-wave exchanges.
//   * The output is accumulated as O^T += V^T P^T on the same instruction; the
//     score accumulator (rounded to bf16) is the B operand as it stands, and V
//     is transposed through a wave-private LDS slab in the matching token order.
//   * The next step's key/value loads are issued before the current step is
//     computed (two register buffers), so a workgroup keeps its whole chunk in
//     flight for the chunk sizes used at batch 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStep = 32;          // tokens per wave step (two 16-token score blocks)
constexpr int kVS = kStep + 8;     // transposed-V row stride in LDS (bf16 elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct SplitArgs {
    const uint16_t *q, *k, *v;
    const int32_t *bt, *seq_lens;
    float *o_parts, *lse_parts;
    int Hq, Hkv, group, page, max_blocks, chunk, max_chunks;
    long long seq_tokens;  // contiguous layout: tokens per sequence
    float scale_log2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Element offset of token t's row for KV head 0 (add hk * D).  `t` is a
// multiple-of-4 group or block start plus an in-page offset; pages hold a
// multiple of 16 tokens, so any 16-aligned block stays inside one page.
__device__ __forceinline__ size_t row_of(const SplitArgs &a, int b, int t)
{
    if (a.bt) {
        const int page = a.bt[(size_t)b * a.max_blocks + t / a.page];
        return ((size_t)page * a.page + (size_t)(t % a.page)) * a.Hkv;
    }
    return ((size_t)b * a.seq_tokens + (size_t)t) * a.Hkv;
}

template <int D>
struct StepRegs {
    uint4 k[2][D / 32];                    // score A operands: [block][k-step]
    uint4 v[(kStep / 4) * (D / 8) / 64][4]; // V units: [unit][token within group]
};

// Slot of 4-token group tg inside a transposed-V row: lane group G reads
// positions 8G..8G+7 = tokens {4G..4G+3} of block 0 then {16+4G..} of block 1.
__device__ __forceinline__ int vt_pos(int tg) { return (tg < 4) ? 8 * tg : 8 * (tg - 4) + 4; }

template <int D>
__device__ __forceinline__ void load_step(const SplitArgs &a, StepRegs<D> &r, int b, int hk, int tb,
                                          int t_end, int lane)
{
    const int l16 = lane & 15, G = lane >> 4;
    // one block-table lookup per 16-token block (a block never crosses a page);
    // blocks starting at or past t_end are never dereferenced
    size_t rb[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) rb[blk] = (tb + 16 * blk < t_end) ? row_of(a, b, tb + 16 * blk) + hk : 0;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int t = tb + 16 * blk + l16;
        if (t < t_end) {
            const uint16_t *row = a.k + (rb[blk] + (size_t)l16 * a.Hkv) * D;
#pragma unroll
            for (int s = 0; s < D / 32; ++s) r.k[blk][s] = *reinterpret_cast<const uint4 *>(row + 32 * s + 8 * G);
        } else {
#pragma unroll
            for (int s = 0; s < D / 32; ++s) r.k[blk][s] = make_uint4(0, 0, 0, 0);
        }
    }
    constexpr int UPL = (kStep / 4) * (D / 8) / 64;  // V units per lane
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int un = lane + 64 * u;
        const int tg = un & 7, dc = un >> 3;
        const int blk = tg >> 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int o = 4 * (tg & 3) + j;  // offset inside the 16-token block
            if (tb + 16 * blk + o < t_end)
                r.v[u][j] = *reinterpret_cast<const uint4 *>(a.v + (rb[blk] + (size_t)o * a.Hkv) * D + 8 * dc);
            else
                r.v[u][j] = make_uint4(0, 0, 0, 0);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(SplitArgs a)
{
    constexpr int VT_BYTES = kWaves * D * kVS * 2;
    constexpr int CMB_BYTES = kWaves * 16 * (D + 2) * 4;
    constexpr int LDS_BYTES = VT_BYTES > CMB_BYTES ? VT_BYTES : CMB_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];

    const int chunk = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    // lengths outside [0, capacity] are clamped so no read leaves the sequence's cache
    const int L = max(0, (int)min((long long)a.seq_lens[b], a.seq_tokens));
    const int t_begin = chunk * a.chunk;
    if (t_begin >= L) return;  // whole workgroup exits together: this chunk is empty
    const int t_end = min(t_begin + a.chunk, L);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, G = lane >> 4;
    const int g = a.group;

    // Query fragments (B operand of S^T = K Q^T); rows >= g are zero padding.
    bf16x8_t qf[D / 32];
    {
        const uint16_t *qrow = a.q + ((size_t)b * a.Hq + (size_t)hk * g + l16) * D;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (l16 < g) u = *reinterpret_cast<const uint4 *>(qrow + 32 * s + 8 * G);
            qf[s] = as_bf16x8(u);
        }
    }

    f32x4_t acc[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] = 0.f;
    float m = -INFINITY, l = 0.f;

    uint16_t *vt = reinterpret_cast<uint16_t *>(lds) + wave * D * kVS;  // this wave's slab

    auto compute_step = [&](const StepRegs<D> &r, int tb) {
        // scores for two 16-token blocks
        f32x4_t st[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) st[blk][i] = 0.f;
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
                st[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.k[blk][s]), qf[s], st[blk], 0, 0, 0);
        }
        // transpose V into the slab while the scores are in flight
        constexpr int UPL = (kStep / 4) * (D / 8) / 64;
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int un = lane + 64 * u;
            const int tg = un & 7, dc = un >> 3;
            const int pos = vt_pos(tg);
            const uint32_t w[4][4] = {{r.v[u][0].x, r.v[u][0].y, r.v[u][0].z, r.v[u][0].w},
                                      {r.v[u][1].x, r.v[u][1].y, r.v[u][1].z, r.v[u][1].w},
                                      {r.v[u][2].x, r.v[u][2].y, r.v[u][2].z, r.v[u][2].w},
                                      {r.v[u][3].x, r.v[u][3].y, r.v[u][3].z, r.v[u][3].w}};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint2 lo, hi;
                lo.x = (w[0][p] & 0xffffu) | (w[1][p] << 16);
                lo.y = (w[2][p] & 0xffffu) | (w[3][p] << 16);
                hi.x = (w[0][p] >> 16) | (w[1][p] & 0xffff0000u);
                hi.y = (w[2][p] >> 16) | (w[3][p] & 0xffff0000u);
                *reinterpret_cast<uint2 *>(&vt[(8 * dc + 2 * p) * kVS + pos]) = lo;
                *reinterpret_cast<uint2 *>(&vt[(8 * dc + 2 * p + 1) * kVS + pos]) = hi;
            }
        }
        // online softmax over this step (lane: query l16, tokens 4G+i of each block)
        const bool tail = tb + kStep > t_end;
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float xv = st[blk][i] * a.scale_log2;
                if (tail && tb + 16 * blk + 4 * G + i >= t_end) xv = -INFINITY;
                x[4 * blk + i] = xv;
                mx = fmaxf(mx, xv);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float c = __builtin_amdgcn_exp2f(m - m_use);
        float rs = 0.f;
        bf16x8_t pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(x[j] - m_use);
            rs += p;
            pf[j] = (__bf16)p;
        }
        l = l * c + rs;
        m = m_new;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[nb][i] *= c;
        // the slab writes of all lanes must land before any lane reads them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
            const bf16x8_t vf = *reinterpret_cast<const bf16x8_t *>(&vt[(16 * nb + l16) * kVS + 8 * G]);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[nb], 0, 0, 0);
        }
        // the next step may overwrite the slab only after every lane has read it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // two register buffers: the next step's loads are in flight during this step's math
    const int stride = kWaves * kStep;
    int tb = t_begin + wave * kStep;
    StepRegs<D> r0, r1;
    if (tb < t_end) load_step<D>(a, r0, b, hk, tb, t_end, lane);
    while (tb < t_end) {
        int tn = tb + stride;
        if (tn < t_end) load_step<D>(a, r1, b, hk, tn, t_end, lane);
        compute_step(r0, tb);
        tb = tn;
        if (tb >= t_end) break;
        tn = tb + stride;
        if (tn < t_end) load_step<D>(a, r0, b, hk, tn, t_end, lane);
        compute_step(r1, tb);
        tb = tn;
    }

    // ---- merge the eight wave states (combine rule) ------------------------------
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    __syncthreads();  // every wave is done with its slab
    float *wm = reinterpret_cast<float *>(lds);  // [kWaves][16]
    float *wl = wm + kWaves * 16;                // [kWaves][16]
    float *wo = wl + kWaves * 16;                // [kWaves][16][D]
    if (G == 0) {
        wm[wave * 16 + l16] = m;
        wl[wave * 16 + l16] = lt;
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
        *reinterpret_cast<f32x4_t *>(&wo[(wave * 16 + l16) * D + 16 * nb + 4 * G]) = acc[nb];
    __syncthreads();
    for (int idx = tid; idx < g * D; idx += kThreads) {
        const int n = idx / D, d = idx % D;
        float ms = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, wm[w * 16 + n]);
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float e = __builtin_amdgcn_exp2f(wm[w * 16 + n] - ms);  // 0 for a wave that saw no token
            lsum += e * wl[w * 16 + n];
            osum += e * wo[(w * 16 + n) * D + d];
        }
        const size_t row = (size_t)b * a.Hq + (size_t)hk * g + n;
        a.o_parts[(row * a.max_chunks + chunk) * D + d] = osum / lsum;
        if (d == 0) a.lse_parts[row * a.max_chunks + chunk] = (ms + log2f(lsum)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Combine: one workgroup per row (sequence x query head).
// ---------------------------------------------------------------------------
struct CombineArgs {
    const float *o_parts, *lse_parts;
    const int32_t *n_splits;  // explicit per-row split counts, or NULL
    const int32_t *seq_lens;  // decode: splits = ceil(seq_lens[row / Hq] / chunk), or NULL
    int Hq, chunk, max_splits, capacity;
    void *o;
    int o_bf16;
    float *lse;
};

constexpr int kCombineThreads = 256;

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <int D>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(CombineArgs a)
{
    constexpr int NWV = kCombineThreads / 64;
    constexpr int DPL = D / 64;  // output dims per lane
    __shared__ float red[NWV];
    __shared__ float red2[NWV];
    __shared__ float obuf[NWV][D];

    const size_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int ns;
    if (a.seq_lens) {
        const int L = max(0, min(a.seq_lens[row / a.Hq], a.capacity));
        ns = (L + a.chunk - 1) / a.chunk;
    } else if (a.n_splits) {
        ns = a.n_splits[row];
    } else {
        ns = a.max_splits;
    }
    ns = max(0, min(ns, a.max_splits));
    const float *lam = a.lse_parts + row * a.max_splits;
    const float *op = a.o_parts + row * a.max_splits * D;

    float mx = -INFINITY;
    for (int kx = tid; kx < ns; kx += kCombineThreads) mx = fmaxf(mx, lam[kx]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) mx = fmaxf(mx, red[w]);

    float z = 0.f;
    if (mx != -INFINITY)
        for (int kx = tid; kx < ns; kx += kCombineThreads) z += expf(lam[kx] - mx);
    z = wave_sum(z);
    if (lane == 0) red2[wave] = z;
    __syncthreads();
    z = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) z += red2[w];
    const bool empty = (mx == -INFINITY);
    const float Lam = empty ? -INFINITY : mx + logf(z);

    float accv[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) accv[e] = 0.f;
    if (!empty) {
        for (int kx = wave; kx < ns; kx += NWV) {
            const float wk = expf(lam[kx] - Lam);
            const float *src = op + (size_t)kx * D + lane * DPL;
#pragma unroll
            for (int e = 0; e < DPL; ++e) accv[e] = fmaf(wk, src[e], accv[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) obuf[wave][lane * DPL + e] = accv[e];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) s += obuf[w][tid];
        if (a.o_bf16) {
            const __bf16 r = (__bf16)s;
            static_cast<uint16_t *>(a.o)[row * D + tid] = __builtin_bit_cast(uint16_t, r);
        } else {
            static_cast<float *>(a.o)[row * D + tid] = s;
        }
    }
    if (tid == 0 && a.lse) a.lse[row] = Lam;
}

template <int D>
hipError_t launch_combine(const CombineArgs &c, int rows, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(lse_combine_kernel<D>, dim3((unsigned)rows), dim3(kCombineThreads), 0, stream, c);
    return hipGetLastError();
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
    a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
    a.page = p.page_size; a.max_blocks = p.max_blocks;
    a.chunk = p.chunk; a.max_chunks = p.max_chunks;
    a.seq_tokens = (long long)p.max_blocks * p.page_size;
    a.scale_log2 = p.scale * kLog2e;
    const dim3 grid((unsigned)p.max_chunks, (unsigned)p.Hkv, (unsigned)p.B);
    if (p.head_dim == 128)
        hipLaunchKernelGGL(decode_split_kernel<128>, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_split_kernel<64>, grid, dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    CombineArgs c;
    c.o_parts = p.o_parts; c.lse_parts = p.lse_parts;
    c.n_splits = nullptr; c.seq_lens = p.seq_lens;
    c.Hq = p.Hq; c.chunk = p.chunk; c.max_splits = p.max_chunks;
    c.capacity = p.max_blocks * p.page_size;
    c.o = p.o; c.o_bf16 = 1; c.lse = p.lse;
    const int rows = p.B * p.Hq;
    return p.head_dim == 128 ? launch_combine<128>(c, rows, stream) : launch_combine<64>(c, rows, stream);
}

hipError_t launch_lse_combine(const CombineParams &p, hipStream_t stream)
{
    CombineArgs c;
    c.o_parts = p.o_parts; c.lse_parts = p.lse_parts;
    c.n_splits = p.n_splits; c.seq_lens = nullptr;
    c.Hq = 1; c.chunk = 1; c.max_splits = p.max_splits; c.capacity = 0;
    c.o = p.o; c.o_bf16 = p.o_bf16 ? 1 : 0; c.lse = p.lse;
    return p.head_dim == 128 ? launch_combine<128>(c, p.rows, stream) : launch_combine<64>(c, p.rows, stream);
}

}  // namespace attn
