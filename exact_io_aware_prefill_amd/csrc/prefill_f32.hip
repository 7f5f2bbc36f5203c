// Tiled exact prefill attention in float32 arithmetic (gfx950 vector ALUs).
//
// Same method as the bf16 kernel (pofe.ai, "FlashAttention for inference: tiled
// prefill and split-KV decoding", sections "Prefill: tiles, loop order and the
// tensor cores" and "The online softmax, with every symbol defined"), for
// float32 inputs whose results must stay within float32 rounding: no bf16
// rounding anywhere, natural-base exponentials from the accurate device math
// library.  One wave per (sequence, head, query tile); 32-key tiles of K and V are
// staged in LDS and read as broadcasts.  Head dims up to 128 take one query row per
// lane (64-row tiles); d = 256 splits each row over two lanes (lane r and r + 32
// hold dims 0..127 and 128..255 of row r; 32-row tiles), which add their partial
// dot products with one cross-lane exchange, so q and the accumulator fit in
// registers.
// Sliding windows and logit soft-capping (two of the variants the page's section
// "Interaction with post-trained models" lists) are run-time options here:
// window >= 0 starts the key loop at the tile of row q0 - window and masks keys
// before row - window; softcap > 0 maps each score s to softcap * tanh(s / softcap)
// before masking, with the device library's tanhf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

namespace attn {
namespace {

constexpr int kLanes = 64;  // one wave per workgroup
constexpr int kKeys = 32;   // keys per tile
template <int D> constexpr int lanes_per_row() { return D > 128 ? 2 : 1; }
template <int D> constexpr int rows_per_tile() { return kLanes / lanes_per_row<D>(); }

// Padded batch: q, o [B, Hq, N, d], k, v [B, Hkv, N, d], lse [B, Hq, N]
// (cu_seqlens NULL).  Packed variable-length batch: sequence b is tokens
// cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, o [T, Hq, d], k, v [T, Hkv, d], lse [Hq, T].
struct Args {
    const float *q, *k, *v;
    float *o, *lse;
    const int32_t *cu_seqlens;
    int B, N, Hq, Hkv, group, causal, n_qtiles, T;
    float scale;
    int window;     // -1: none
    float softcap;  // 0: none
};

template <int D>
__global__ __launch_bounds__(kLanes) void prefill_f32_kernel(Args a)
{
    constexpr int LPR = lanes_per_row<D>();
    constexpr int ROWS = rows_per_tile<D>();
    constexpr int DH = D / LPR;  // dims held by one lane
    __shared__ __attribute__((aligned(16))) float Ks[kKeys * D];
    __shared__ __attribute__((aligned(16))) float Vs[kKeys * D];

    const int tid = threadIdx.x;
    const int half = tid / ROWS;  // which dims of its row this lane holds (0 unless d = 256)
    const int nbh = a.B * a.Hq;
    const int qtile = a.n_qtiles - 1 - (int)(blockIdx.x / nbh);
    const int bh = (int)(blockIdx.x % nbh);
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const int q0 = qtile * ROWS;
    const int qrow = q0 + tid % ROWS;
    // this sequence's rows: first element of row 0 and the stride between rows
    int N;
    size_t qbase, kvbase, qstride, kvstride, lsebase;
    if (a.cu_seqlens) {  // offsets outside [0, T] and lengths above N are clamped
        const int s0 = min(max(a.cu_seqlens[b], 0), a.T);
        const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.T);
        N = min(s1 - s0, a.N);
        qbase = ((size_t)s0 * a.Hq + h) * D;
        kvbase = ((size_t)s0 * a.Hkv + hk) * D;
        qstride = (size_t)a.Hq * D;
        kvstride = (size_t)a.Hkv * D;
        lsebase = (size_t)h * a.T + s0;
    } else {
        N = a.N;
        qbase = (size_t)bh * a.N * D;
        kvbase = (size_t)(b * a.Hkv + hk) * a.N * D;
        qstride = D;
        kvstride = D;
        lsebase = (size_t)bh * a.N;
    }
    if (q0 >= N) return;  // whole workgroup: no query row of this tile exists
    const float *kp = a.k + kvbase;
    const float *vp = a.v + kvbase;

    float q[DH], acc[DH];
#pragma unroll
    for (int d = 0; d < DH; ++d) {
        q[d] = (qrow < N) ? a.q[qbase + (size_t)qrow * qstride + half * DH + d] : 0.f;
        acc[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    const int kend = a.causal ? min(N, q0 + ROWS) : N;
    const int kbeg = a.window >= 0 ? max(0, q0 - a.window) / kKeys * kKeys : 0;
    for (int k0 = kbeg; k0 < kend; k0 += kKeys) {
        __syncthreads();
        for (int idx = tid; idx < kKeys * D / 4; idx += kLanes) {
            const int r = idx / (D / 4), c = idx % (D / 4);
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (k0 + r < N) {
                kv = *reinterpret_cast<const float4 *>(kp + (size_t)(k0 + r) * kvstride + 4 * c);
                vv = *reinterpret_cast<const float4 *>(vp + (size_t)(k0 + r) * kvstride + 4 * c);
            }
            *reinterpret_cast<float4 *>(&Ks[r * D + 4 * c]) = kv;
            *reinterpret_cast<float4 *>(&Vs[r * D + 4 * c]) = vv;
        }
        __syncthreads();

        float s[kKeys];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < kKeys; ++t) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < DH; ++d) dot = fmaf(q[d], Ks[t * D + half * DH + d], dot);
            // both lanes of a row form the same sum (float addition commutes)
            if (LPR == 2) dot += __shfl_xor(dot, ROWS);
            float x = dot * a.scale;
            if (a.softcap > 0.f) x = a.softcap * tanhf(x / a.softcap);
            const int key = k0 + t;
            if (key >= N || (a.causal && key > qrow) || (a.window >= 0 && key < qrow - a.window)) x = -INFINITY;
            s[t] = x;
            mx = fmaxf(mx, x);
        }
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // nothing visible yet
        const float c = expf(m - m_use);
        l *= c;
#pragma unroll
        for (int d = 0; d < DH; ++d) acc[d] *= c;
#pragma unroll
        for (int t = 0; t < kKeys; ++t) {
            const float p = expf(s[t] - m_use);
            l += p;
#pragma unroll
            for (int d = 0; d < DH; ++d) acc[d] = fmaf(p, Vs[t * D + half * DH + d], acc[d]);
        }
        m = m_new;
    }

    if (qrow < N) {
        float *orow = a.o + qbase + (size_t)qrow * qstride + half * DH;
        if (l > 0.f) {
            const float inv = 1.f / l;
#pragma unroll
            for (int d = 0; d < DH; ++d) orow[d] = acc[d] * inv;
            if (half == 0) a.lse[lsebase + qrow] = m + logf(l);
        } else {  // no visible key (not reachable for square causal or full attention)
#pragma unroll
            for (int d = 0; d < DH; ++d) orow[d] = 0.f;
            if (half == 0) a.lse[lsebase + qrow] = -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams &p, hipStream_t stream)
{
    Args a;
    a.q = static_cast<const float *>(p.q);
    a.k = static_cast<const float *>(p.k);
    a.v = static_cast<const float *>(p.v);
    a.o = static_cast<float *>(p.o);
    a.lse = p.lse;
    a.cu_seqlens = p.cu_seqlens;
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
    a.T = p.cu_seqlens ? p.total : p.B * p.N;
    a.causal = p.causal;
    const int rows = p.head_dim == 256 ? rows_per_tile<256>() : rows_per_tile<128>();
    a.n_qtiles = (p.N + rows - 1) / rows;
    a.scale = p.scale;
    a.window = (p.window >= 0 && p.window < p.N) ? p.window : -1;  // a longer window limits nothing
    a.softcap = p.softcap > 0.f ? p.softcap : 0.f;
    const long long nblk = (long long)a.n_qtiles * p.B * p.Hq;
    if (nblk == 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (p.head_dim == 128)
        hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)nblk), dim3(kLanes), 0, stream, a);
    else if (p.head_dim == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)nblk), dim3(kLanes), 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<256>, dim3((unsigned)nblk), dim3(kLanes), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
