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
//   * workgroup = 4 waves x 32 query rows = 128 rows; key/value tile = 64 keys.
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
//   * Exponentials run in base 2 with scale*log2(e) folded into the scores.
//   * Query tiles are issued longest-first (causal rows near the end see the
//     most keys).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockM = kWaves * 32;  // query rows per workgroup
constexpr int kBlockN = 64;           // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Args {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int B, N, Hq, Hkv, group, causal, n_qtiles;
    float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Position of key group `sub` (keys 4*sub..4*sub+3 of a 16-key step) inside
// the transposed V row: lanes of the lower half-wave read keys {0-3, 8-11},
// the upper half {4-7, 12-15}, matching the 32x32 accumulator rows.
__device__ __forceinline__ int vt_slot(int sub) { return ((sub & 1) << 3) | ((sub & 2) << 1); }

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(Args a)
{
    constexpr int KS = D + 8;         // K row stride in LDS (bf16): 16-byte aligned, bank-rotating
    constexpr int VS = kBlockN + 8;   // transposed-V row stride in LDS (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kBlockN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int nbh = a.B * a.Hq;
    const int qtile = a.n_qtiles - 1 - (int)(blockIdx.x / nbh);  // longest tiles first
    const int bh = (int)(blockIdx.x % nbh);
    const int b = bh / a.Hq, h = bh % a.Hq, hk = h / a.group;
    const int q0 = qtile * kBlockM;
    const uint16_t *qp = a.q + (size_t)bh * a.N * D;
    const uint16_t *kp = a.k + (size_t)(b * a.Hkv + hk) * a.N * D;
    const uint16_t *vp = a.v + (size_t)(b * a.Hkv + hk) * a.N * D;

    const int wrow0 = q0 + wave * 32;  // first query row of this wave
    const int qrow = wrow0 + l32;      // the query row this lane owns

    // Q fragments (B operand of S^T = K Q^T), resident for the whole kernel.
    bf16x8_t qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qrow < a.N) u = *reinterpret_cast<const uint4 *>(qp + (size_t)qrow * D + 16 * s + 8 * hh);
        qf[s] = as_bf16x8(u);
    }

    f32x16_t acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    float m = -INFINITY;  // running max of scaled scores, base-2 units
    float l = 0.f;        // this lane's share of the running sum (its 16-of-32 keys)

    const int kend = a.causal ? min(a.N, q0 + kBlockM) : a.N;  // keys this tile may see
    const int ntiles = (kend + kBlockN - 1) / kBlockN;

    for (int jt = 0; jt < ntiles; ++jt) {
        const int k0 = jt * kBlockN;
        __syncthreads();  // the previous tile's LDS reads are done
        // ---- stage K (row-major) -------------------------------------------
        {
            constexpr int CPR = D / 8;            // 16-byte chunks per row
            constexpr int RPP = kThreads / CPR;   // rows per pass
            const int c = tid % CPR;
#pragma unroll
            for (int r = tid / CPR; r < kBlockN; r += RPP) {
                uint4 u = make_uint4(0, 0, 0, 0);
                if (k0 + r < a.N) u = *reinterpret_cast<const uint4 *>(kp + (size_t)(k0 + r) * D + 8 * c);
                *reinterpret_cast<uint4 *>(&Ks[r * KS + 8 * c]) = u;
            }
        }
        // ---- stage V transposed: Vt[d][key slot] ----------------------------
        {
            constexpr int UNITS = (kBlockN / 4) * (D / 8);  // 4 keys x 8 dims each
#pragma unroll
            for (int u0 = 0; u0 < UNITS; u0 += kThreads) {
                const int un = u0 + tid;
                if (UNITS % kThreads == 0 || un < UNITS) {
                    const int kg = un % (kBlockN / 4);  // key group (4 keys)
                    const int dc = un / (kBlockN / 4);  // 8-dim chunk
                    uint32_t w[4][4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint4 x = make_uint4(0, 0, 0, 0);
                        const int key = k0 + 4 * kg + j;
                        if (key < a.N) x = *reinterpret_cast<const uint4 *>(vp + (size_t)key * D + 8 * dc);
                        w[j][0] = x.x; w[j][1] = x.y; w[j][2] = x.z; w[j][3] = x.w;
                    }
                    const int pos = 16 * (kg >> 2) + vt_slot(kg & 3);
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        // dims 8*dc+2p (low halves) and 8*dc+2p+1 (high halves)
                        uint2 lo, hi;
                        lo.x = (w[0][p] & 0xffffu) | (w[1][p] << 16);
                        lo.y = (w[2][p] & 0xffffu) | (w[3][p] << 16);
                        hi.x = (w[0][p] >> 16) | (w[1][p] & 0xffff0000u);
                        hi.y = (w[2][p] >> 16) | (w[3][p] & 0xffff0000u);
                        *reinterpret_cast<uint2 *>(&Vt[(8 * dc + 2 * p) * VS + pos]) = lo;
                        *reinterpret_cast<uint2 *>(&Vt[(8 * dc + 2 * p + 1) * VS + pos]) = hi;
                    }
                }
            }
        }
        __syncthreads();

        // A wave whose rows all precede this tile's first key (or lie past N) has nothing to add.
        if ((a.causal && k0 > wrow0 + 31) || wrow0 >= a.N) continue;

        // ---- S^T = K Q^T for two 32-key blocks -----------------------------
        f32x16_t st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) st[kb][i] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(&Ks[(kb * 32 + l32) * KS + 16 * s + 8 * hh]);
                st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[kb], 0, 0, 0);
            }
        }

        // ---- scale, mask, online softmax -----------------------------------
        const bool need_mask = (a.causal && k0 + kBlockN - 1 > wrow0) || (k0 + kBlockN > a.N);
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = st[kb][i] * a.scale_log2;
                if (need_mask) {
                    const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
                    if (key >= a.N || (a.causal && key > qrow)) x = -INFINITY;
                }
                st[kb][i] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no visible key yet: state unchanged
        const float c = __builtin_amdgcn_exp2f(m - m_use);
        float rs = 0.f;
        bf16x8_t pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(st[kb][i] - m_use);
                rs += p;
                pf[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
            }
        }
        l = l * c + rs;
        m = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= c;

        // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x8_t vf = *reinterpret_cast<const bf16x8_t *>(&Vt[(db * 32 + l32) * VS + 16 * ks + 8 * hh]);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], acc[db], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2 ----------------------
    const float lt = l + __shfl_xor(l, 32);
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
        if (hh == 0) a.lse[(size_t)bh * a.N + qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
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
    a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.group = p.Hq / p.Hkv;
    a.causal = p.causal;
    a.n_qtiles = (p.N + kBlockM - 1) / kBlockM;
    a.scale_log2 = p.scale * kLog2e;
    const long long nblk = (long long)a.n_qtiles * p.B * p.Hq;
    if (nblk == 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk), block(kThreads);
    if (p.head_dim == 128)
        hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn
