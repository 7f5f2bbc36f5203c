"""GPU parity of the FP8 (E4M3) prefill against the fp64 oracle on the same codes.

The oracle computes attention on the dequantised inputs with no rounding of the
probabilities.  The kernel rounds each probability to E4M3 before the P*V product
(nearest even; 3 mantissa bits, so at most 2^-4 relative error, or 2^-10 absolute
below the normal range) and writes O in bf16.  With p_j relative to the row's true
max, l = sum_j p_j and n visible keys, that bounds the error of a row by

    |dO| <= descale_v * max|v8| * (2^-4 + n 2^-10 / l) + 2^-8 |O| + 1e-5,

which the tests check element by element; the LSE keeps the bf16 path's 1e-3 bar
(the row sums use the unrounded float32 probabilities).  A second, typical-error
check asserts the RMS error is far below that worst case."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, check, dev, say

pytestmark = pytest.mark.gpu
LSE_TOL = 1e-3


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def row_bounds(x, rows=None):
    """Per-row error bound of the formula above, from the dequantised inputs."""
    q = oracle.e4m3_decode(x.q8); k = oracle.e4m3_decode(x.k8); v = oracle.e4m3_decode(x.v8)
    B, Hq, N, d = q.shape
    g = Hq // k.shape[1]
    dq = x.descale_q.double().numpy(); dk = x.descale_k.double().numpy(); dv = x.descale_v.double().numpy()
    rows = np.arange(N) if rows is None else rows
    bound = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            s = (q[b, h, rows] @ k[b, hk].T) * (x.scale * dq[b, hk] * dk[b, hk])
            if x.causal:
                s = np.where(np.arange(N)[None, :] <= rows[:, None], s, -np.inf)
            n = np.isfinite(s).sum(axis=1)
            mx = s.max(axis=1)
            lsum = np.exp(s - mx[:, None]).sum(axis=1)
            vmax = np.abs(v[b, hk]).max() * dv[b, hk]
            bound[b, h] = vmax * (2.0 ** -4 + n * 2.0 ** -10 / lsum)
    return bound


def check_fp8(name, o, lse, ro, rl, bound):
    og = o.float().cpu().numpy(); lg = lse.cpu().numpy()
    err = np.abs(og - ro)
    lim = bound[..., None] + 2.0 ** -8 * np.abs(ro) + 1e-5
    worst = float((err / lim).max())
    rms = float(np.sqrt(np.mean(err ** 2)))
    rms_ref = float(np.sqrt(np.mean(ro ** 2)))
    el = float(np.abs(lg - rl).max())
    say("%s: O max_abs=%.3e rms=%.3e (ref rms %.3e) worst err/bound=%.3f | LSE max_abs=%.3e"
        % (name, float(err.max()), rms, rms_ref, worst, el))
    assert worst <= 1.0, name
    assert rms <= 2.0 ** -4 * max(rms_ref, 1e-3), name  # typical error well inside the worst case
    assert el <= LSE_TOL, name


def run(attn, x):
    o, lse = attn.prefill_fp8(dev(x.q8), dev(x.k8), dev(x.v8), dev(x.descale_q), dev(x.descale_k),
                              dev(x.descale_v), x.causal, x.scale)
    torch.cuda.synchronize()
    return o, lse


def test_fp8_worked_example(attn):
    """The page's worked example, every value exact in E4M3: row 3 is 1.1381 up to the
    E4M3 rounding of the four probabilities."""
    say("case: fp8 worked example")
    N, d = 4, 64
    q8 = torch.zeros(1, 1, N, d, dtype=torch.uint8); k8 = torch.zeros_like(q8); v8 = torch.zeros_like(q8)
    q8[0, 0, :, 0] = 0x38
    k8[0, 0, :, 0] = torch.tensor([0x40, 0x38, 0x48, 0x44], dtype=torch.uint8)
    v8[0, 0, :, 0] = torch.tensor([0x38, 0x00, 0x40, 0xb8], dtype=torch.uint8)
    o, lse = attn.prefill_fp8(dev(q8), dev(k8), dev(v8), None, None, None, True, 1.0)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_fp8(q8, k8, v8, None, None, None, True, 1.0)
    assert abs(ro[0, 0, 3, 0] - 1.1381) < 5e-5
    assert abs(float(o[0, 0, 3, 0]) - ro[0, 0, 3, 0]) <= 2 * 2.0 ** -4 + 2.0 ** -8 * 1.2
    assert np.max(np.abs(lse.cpu().numpy() - rl)) <= 1e-5
    assert (o[0, 0, :, 1:] == 0).all()


@pytest.mark.parametrize("N", [1, 63, 64, 65, 300, 1000])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_ragged(attn, N, d, causal):
    say("case: fp8 prefill N=%d d=%d causal=%s" % (N, d, causal))
    x = W.prefill_fp8_inputs(3000 + N + d, 2, 8, 2, N, d, causal=causal)
    o, lse = run(attn, x)
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, causal, x.scale)
    check_fp8("fp8 N=%d d=%d causal=%d" % (N, d, causal), o, lse, ro, rl, row_bounds(x))


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.0])
def test_fp8_prefill_scales(attn, scale):
    """A negative scale (Q's sign bits are flipped instead), zero (uniform weights) and
    a large one (peaky rows)."""
    say("case: fp8 prefill scale=%g" % scale)
    x = W.prefill_fp8_inputs(3100, 1, 4, 2, 333, 128, scale=scale)
    o, lse = run(attn, x)
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, True, scale)
    check_fp8("fp8 scale=%g" % scale, o, lse, ro, rl, row_bounds(x))


def test_fp8_prefill_without_descales(attn):
    """NULL descales mean 1: the codes are the values."""
    say("case: fp8 prefill, no descales")
    x = W.prefill_fp8_inputs(3200, 1, 4, 4, 200, 64)
    x.descale_q = torch.ones_like(x.descale_q); x.descale_k = torch.ones_like(x.descale_k)
    x.descale_v = torch.ones_like(x.descale_v)
    # the raw codes reach 448: scale the scores back to the O(1) range the LSE bar assumes
    x.scale = 1.0 / (float(x.q8.float().std()) * float(x.k8.float().std()) * math.sqrt(64))
    o, lse = attn.prefill_fp8(dev(x.q8), dev(x.k8), dev(x.v8), None, None, None, True, x.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, None, None, None, True, x.scale)
    check_fp8("fp8 no descales", o, lse, ro, rl, row_bounds(x))


def test_fp8_prefill_d256_8k_sampled_rows(attn):
    """d = 256 (one wave per SIMD, 256-byte rows) at 8k tokens, 16 query / 8 KV heads,
    every 31st row."""
    N, step = 8192, 31
    say("case: fp8 prefill d=256 N=%d sampled every %d" % (N, step))
    x = W.prefill_fp8_inputs(3150, 1, 16, 8, N, 256)
    o, lse = run(attn, x)
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, True, x.scale,
                                row_step=step)
    rows = np.arange(0, N, step)
    check_fp8("fp8 d=256 8k (sampled)", o[:, :, rows], lse[:, :, rows], ro[:, :, rows], rl[:, :, rows],
              row_bounds(x, rows))


def test_fp8_prefill_16k_sampled_rows(attn):
    """The 16k-token prompt (28 query / 4 KV heads, d = 128) in FP8, every 61st row."""
    N, step = 16384, 61
    say("case: fp8 prefill N=%d sampled every %d" % (N, step))
    x = W.prefill_fp8_inputs(3, 1, 28, 4, N, 128)
    o, lse = run(attn, x)
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, True, x.scale,
                                row_step=step)
    rows = np.arange(0, N, step)
    check_fp8("fp8 16k (sampled)", o[:, :, rows], lse[:, :, rows], ro[:, :, rows], rl[:, :, rows],
              row_bounds(x, rows))


# ------------------------------------------------------------------ decode over an E4M3 cache
DEC_LENS = [1, 15, 16, 17, 100, 511, 513, 1000]


@pytest.mark.parametrize("g", [1, 4, 16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("chunk", [16, 256, 0])
def test_fp8_cache_decode(attn, g, d, paged, chunk):
    """The E4M3 codes convert to bf16 exactly and the descales fold into the score
    scale and the output, so the bf16 decode's bars apply (2e-2 on O, 1e-3 on LSE)."""
    say("case: fp8-cache decode g=%d d=%d paged=%s chunk=%d" % (g, d, paged, chunk))
    x = W.decode_fp8_inputs(3300 + g + d + chunk, len(DEC_LENS), g * 2, 2, d, DEC_LENS, 1024, paged)
    o, lse = attn.decode_fp8(dev(x.q), dev(x.k_cache8), dev(x.v_cache8), dev(x.block_table), dev(x.seq_lens),
                             x.page_size, x.max_blocks, dev(x.descale_k), dev(x.descale_v), x.scale, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_fp8(x.q, x.k_cache8, x.v_cache8, x.descale_k, x.descale_v, x.block_table, x.seq_lens,
                               x.scale, x.page_size, x.max_blocks)
    check("fp8-cache decode g=%d d=%d paged=%d chunk=%d" % (g, d, paged, chunk), o, lse, ro, rl, BF16_TOL)


def test_fp8_cache_decode_32k(attn):
    """The 32k-token decode (28 query / 4 KV heads, 64 chunks of 512) over an E4M3 cache."""
    say("case: fp8-cache decode 32k")
    x = W.decode_fp8_inputs(4, 1, 28, 4, 128, [32768], 32768, False)
    o, lse = attn.decode_fp8(dev(x.q), dev(x.k_cache8), dev(x.v_cache8), None, dev(x.seq_lens), x.page_size,
                             x.max_blocks, dev(x.descale_k), dev(x.descale_v), x.scale, 512)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_fp8(x.q, x.k_cache8, x.v_cache8, x.descale_k, x.descale_v, None, x.seq_lens, x.scale,
                               x.page_size, x.max_blocks)
    check("fp8-cache decode 32k", o, lse, ro, rl, BF16_TOL)


def test_fp8_cache_decode_matches_bf16_decode_of_the_same_values(attn):
    """With NULL descales the E4M3 codes are the values themselves, each exactly a bf16
    value, so the bf16 decode over the same cache widened to bf16 sums the same terms
    (in another order): LSE agrees to 1e-3 and O to bf16 rounding of values up to 448.
    Both are also held to the oracle, which reads NULL descales as 1."""
    say("case: fp8-cache decode vs bf16 decode, no descales")
    x = W.decode_fp8_inputs(3400, len(DEC_LENS), 8, 2, 128, DEC_LENS, 1024, True)
    scale = 1.0 / (float(x.k_cache8.float().std()) * math.sqrt(128))  # scores stay O(1)
    q, k8, v8 = dev(x.q), dev(x.k_cache8), dev(x.v_cache8)
    bt, sl = dev(x.block_table), dev(x.seq_lens)
    o8, l8 = attn.decode_fp8(q, k8, v8, bt, sl, x.page_size, x.max_blocks, None, None, scale, 64)
    o, lse = attn.decode(q, k8.to(torch.bfloat16), v8.to(torch.bfloat16), bt, sl, x.page_size, x.max_blocks,
                         scale, 64)
    torch.cuda.synchronize()
    o_tol = 448.0 * 2.0 ** -7
    assert float((l8 - lse).abs().max()) <= 1e-3
    assert float((o8.float() - o.float()).abs().max()) <= o_tol
    ro, rl = oracle.decode_fp8(x.q, x.k_cache8, x.v_cache8, None, None, x.block_table, x.seq_lens, scale,
                               x.page_size, x.max_blocks)
    assert np.max(np.abs(l8.cpu().numpy() - rl)) <= 1e-3
    assert np.max(np.abs(o8.float().cpu().numpy() - ro)) <= o_tol


# ------------------------------------------------------------------ packed (variable-length) FP8 prefill
def packed_row_bounds(x):
    """row_bounds for each sequence of a packed batch, assembled as [T, Hq]."""
    cu = x.cu_seqlens.tolist()
    Hq = x.q8.shape[1]
    out = np.zeros((x.q8.shape[0], Hq))
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        seq = W.Fp8PrefillInputs(x.q8[s0:s1].permute(1, 0, 2)[None], x.k8[s0:s1].permute(1, 0, 2)[None],
                                 x.v8[s0:s1].permute(1, 0, 2)[None], x.descale_q[b:b + 1], x.descale_k[b:b + 1],
                                 x.descale_v[b:b + 1], x.causal, x.scale)
        out[s0:s1] = row_bounds(seq)[0].T
    return out


def run_packed(attn, x):
    o, lse = attn.prefill_fp8_varlen(dev(x.q8), dev(x.k8), dev(x.v8), dev(x.cu_seqlens), x.max_seqlen,
                                     dev(x.descale_q), dev(x.descale_k), dev(x.descale_v), x.causal, x.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_varlen_ragged(attn, d, causal):
    lens = [1, 7, 0, 128, 129, 300, 64]
    say("case: fp8 varlen d=%d causal=%s lens=%s" % (d, causal, lens))
    x = W.prefill_fp8_packed_inputs(3500 + d, lens, 8, 2, d, causal=causal)
    o, lse = run_packed(attn, x)
    ro, rl = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, x.cu_seqlens,
                                       causal, x.scale)
    check_fp8("fp8 varlen d=%d causal=%d" % (d, causal), o, lse, ro, rl, packed_row_bounds(x))


def test_fp8_prefill_varlen_long_mix(attn):
    """Four prompts of 3000, 1, 2048 and 777 tokens, 8 query / 2 KV heads, d = 128."""
    lens = [3000, 1, 2048, 777]
    say("case: fp8 varlen long mix %s" % lens)
    x = W.prefill_fp8_packed_inputs(3600, lens, 8, 2, 128)
    o, lse = run_packed(attn, x)
    ro, rl = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, x.cu_seqlens,
                                       True, x.scale)
    check_fp8("fp8 varlen long mix", o, lse, ro, rl, packed_row_bounds(x))


def test_fp8_prefill_varlen_one_sequence_equals_padded(attn):
    """One packed sequence runs the padded kernel's arithmetic: bit for bit equal."""
    say("case: fp8 varlen one sequence = padded")
    N = 333
    x = W.prefill_fp8_packed_inputs(3700, [N], 8, 2, 128)
    o, lse = run_packed(attn, x)
    op, lp = attn.prefill_fp8(dev(x.q8.permute(1, 0, 2)[None]), dev(x.k8.permute(1, 0, 2)[None]),
                              dev(x.v8.permute(1, 0, 2)[None]), dev(x.descale_q), dev(x.descale_k),
                              dev(x.descale_v), True, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, op[0].permute(1, 0, 2)) and torch.equal(lse, lp[0])


def _random_case(seed):
    """Batch 1..3, KV heads 1/2/4/8, group 1/2/4/7, d 64/128/256, length 1..2000, causal
    or full, padded or packed (packed lengths 0..N, one of them N); the work kept below
    1e10 (batch x query heads x N^2 x d) for the oracle and the per-row bounds."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7]))
    d = int(rng.choice([64, 128, 256]))
    causal = bool(rng.integers(0, 2))
    packed = bool(rng.integers(0, 2))
    N = int(rng.integers(1, 2001))
    N = max(1, min(N, int((1e10 / (B * g * Hkv * d)) ** 0.5)))
    lens = rng.integers(0, N + 1, size=B)
    lens[int(rng.integers(0, B))] = N
    return B, Hkv, g, d, N, causal, packed, lens.tolist()


@pytest.mark.parametrize("seed", list(range(12)))
def test_fp8_prefill_random_shapes(attn, seed):
    """Seeded random shapes across the FP8 kernel's layouts, head sizes and masks."""
    B, Hkv, g, d, N, causal, packed, lens = _random_case(seed)
    Hq = g * Hkv
    say("case: fp8 prefill random seed=%d B=%d Hq=%d Hkv=%d d=%d N=%d causal=%s packed=%s lens=%s"
        % (seed, B, Hq, Hkv, d, N, causal, packed, lens if packed else "-"))
    if packed:
        x = W.prefill_fp8_packed_inputs(7000 + seed, lens, Hq, Hkv, d, causal=causal)
        o, lse = run_packed(attn, x)
        ro, rl = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, x.cu_seqlens,
                                           causal, x.scale)
        check_fp8("fp8 random seed=%d" % seed, o, lse, ro, rl, packed_row_bounds(x))
    else:
        x = W.prefill_fp8_inputs(7000 + seed, B, Hq, Hkv, N, d, causal=causal)
        o, lse = run(attn, x)
        ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, causal, x.scale)
        check_fp8("fp8 random seed=%d" % seed, o, lse, ro, rl, row_bounds(x))
