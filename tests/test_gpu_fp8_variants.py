"""GPU parity of the FP8 (E4M3) prefill with a sliding window and logit soft-capping
(attn_prefill_fp8_ext) against the fp64 oracle on the dequantised codes.  The error
bar is the FP8 prefill's per-row bound (tests/test_gpu_fp8.py), taken over each
row's visible keys (causal limit and window) and the capped scores: the kernel rounds
each probability to E4M3 before the P*V product; the LSE keeps the 1e-3 bar."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import dev, say
from test_gpu_fp8 import check_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def visible_scores(qv, kv, eff, causal, window, softcap, rows, N):
    """Scaled (and capped) scores of the given rows with the invisible keys at -inf."""
    s = (qv[rows] @ kv.T) * eff
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    j = np.arange(N)[None, :]
    i = rows[:, None]
    vis = np.ones_like(s, dtype=bool)
    if causal:
        vis &= j <= i
    if window >= 0:
        vis &= j >= i - window
    return np.where(vis, s, -np.inf)


def bound_rows(q, k, v, dq, dk, dv, scale, causal, window, softcap, rows, N, g):
    """Per-row bound descale_v * max|v8| * (2^-4 + n 2^-10 / l) of each head (shape [Hq, rows])."""
    Hq = q.shape[0]
    out = np.zeros((Hq, len(rows)))
    for h in range(Hq):
        hk = h // g
        s = visible_scores(q[h], k[hk], scale * dq[hk] * dk[hk], causal, window, softcap, rows, N)
        n = np.isfinite(s).sum(axis=1)
        mx = s.max(axis=1)
        lsum = np.exp(s - mx[:, None]).sum(axis=1)
        out[h] = np.abs(v[hk]).max() * dv[hk] * (2.0 ** -4 + n * 2.0 ** -10 / lsum)
    return out


def padded_bounds(x, window, softcap, rows=None):
    q, k, v = (oracle.e4m3_decode(t) for t in (x.q8, x.k8, x.v8))
    B, Hq, N, d = q.shape
    g = Hq // k.shape[1]
    rows = np.arange(N) if rows is None else rows
    dq, dk, dv = (t.double().numpy() for t in (x.descale_q, x.descale_k, x.descale_v))
    return np.stack([bound_rows(q[b], k[b], v[b], dq[b], dk[b], dv[b], x.scale, x.causal, window, softcap, rows, N, g)
                     for b in range(B)])


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window,softcap", [(0, 0.0), (37, 0.0), (200, 0.0), (-1, 20.0), (64, 5.0)])
def test_fp8_window_softcap_padded(attn, d, causal, window, softcap):
    N = 333
    say("case: fp8 ext N=%d d=%d causal=%s window=%d softcap=%g" % (N, d, causal, window, softcap))
    x = W.prefill_fp8_inputs(4000 + d + window, 2, 8, 2, N, d, causal=causal)
    o, lse = attn.prefill_fp8(dev(x.q8), dev(x.k8), dev(x.v8), dev(x.descale_q), dev(x.descale_k), dev(x.descale_v),
                              causal, x.scale, window_left=window, softcap=softcap)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, causal, x.scale,
                                window=window, softcap=softcap)
    check_fp8("fp8 ext d=%d causal=%d w=%d cap=%g" % (d, causal, window, softcap), o, lse, ro, rl,
              padded_bounds(x, window, softcap))


def test_fp8_ext_without_options_is_the_plain_kernel(attn):
    """window -1 and softcap 0 through the variant entry point run the plain kernel: bit for bit."""
    x = W.prefill_fp8_inputs(4100, 1, 8, 2, 500, 128)
    args = (dev(x.q8), dev(x.k8), dev(x.v8))
    ds = (dev(x.descale_q), dev(x.descale_k), dev(x.descale_v))
    o0, l0 = attn.prefill_fp8(*args, *ds, True, x.scale)
    o1 = torch.empty_like(o0)
    l1 = torch.empty_like(l0)
    attn.attn_prefill_fp8_ext(*args, o1, l1, *ds, None, 500, True, x.scale, -1, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_fp8_window_softcap_packed(attn):
    """A packed batch of ragged prompts with a window of 100 and a cap of 30."""
    lens = [1, 7, 0, 128, 129, 300, 64, 1000]
    window, softcap = 100, 30.0
    say("case: fp8 ext packed lens=%s window=%d softcap=%g" % (lens, window, softcap))
    x = W.prefill_fp8_packed_inputs(4200, lens, 8, 2, 128)
    cu = dev(x.cu_seqlens)
    o, lse = attn.prefill_fp8_varlen(dev(x.q8), dev(x.k8), dev(x.v8), cu, max(lens), dev(x.descale_q),
                                     dev(x.descale_k), dev(x.descale_v), True, x.scale, window_left=window,
                                     softcap=softcap)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, x.cu_seqlens,
                                       True, x.scale, window=window, softcap=softcap)
    q, k, v = (oracle.e4m3_decode(t) for t in (x.q8, x.k8, x.v8))
    dq, dk, dv = (t.double().numpy() for t in (x.descale_q, x.descale_k, x.descale_v))
    cuh = x.cu_seqlens.numpy()
    Hq, Hkv = q.shape[1], k.shape[1]
    bound = np.zeros((Hq, q.shape[0]))
    for b in range(len(lens)):
        s0, s1 = int(cuh[b]), int(cuh[b + 1])
        if s1 <= s0:
            continue
        bound[:, s0:s1] = bound_rows(q[s0:s1].transpose(1, 0, 2), k[s0:s1].transpose(1, 0, 2),
                                     v[s0:s1].transpose(1, 0, 2), dq[b], dk[b], dv[b], x.scale, True, window, softcap,
                                     np.arange(s1 - s0), s1 - s0, Hq // Hkv)
    # packed layout: o [T, Hq, d], lse [Hq, T]; check_fp8 takes the bound per (head, token)
    check_fp8("fp8 ext packed", o.permute(1, 0, 2), lse, ro.transpose(1, 0, 2), rl, bound)


def test_fp8_window_softcap_long_sampled_rows(attn):
    """N = 8192, 28 query / 4 KV heads, d = 128, window 4096, cap 30: every 97th row."""
    N, step, window, softcap = 8192, 97, 4096, 30.0
    say("case: fp8 ext N=%d window=%d cap=%g sampled every %d" % (N, window, softcap, step))
    x = W.prefill_fp8_inputs(3, 1, 28, 4, N, 128)
    o, lse = attn.prefill_fp8(dev(x.q8), dev(x.k8), dev(x.v8), dev(x.descale_q), dev(x.descale_k), dev(x.descale_v),
                              True, x.scale, window_left=window, softcap=softcap)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, True, x.scale, row_step=step,
                                window=window, softcap=softcap)
    rows = np.arange(0, N, step)
    check_fp8("fp8 ext 8k (sampled)", o[:, :, rows], lse[:, :, rows], ro[:, :, rows], rl[:, :, rows],
              padded_bounds(x, window, softcap, rows))


# ------------------------------------------------------------------ decode over an E4M3 cache
DEC_LENS = [1, 15, 16, 17, 100, 511, 513, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("window,softcap", [(0, 0.0), (40, 0.0), (300, 0.0), (-1, 15.0), (100, 5.0)])
def test_fp8_cache_decode_window_softcap(attn, d, paged, window, softcap):
    """The E4M3 codes convert to bf16 exactly and the descales fold into the scale (the
    cap acts on the descaled score), so the bf16 decode's bars hold: 2e-2 on O, 1e-3 on LSE."""
    from gpu_common import BF16_TOL, check
    say("case: fp8-cache decode d=%d paged=%s window=%d softcap=%g" % (d, paged, window, softcap))
    x = W.decode_fp8_inputs(4300 + d + window, len(DEC_LENS), 8, 2, d, DEC_LENS, 1024, paged)
    o, lse = attn.decode_fp8(dev(x.q), dev(x.k_cache8), dev(x.v_cache8), dev(x.block_table), dev(x.seq_lens),
                             x.page_size, x.max_blocks, dev(x.descale_k), dev(x.descale_v), x.scale, 64,
                             window_left=window, softcap=softcap)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_fp8(x.q, x.k_cache8, x.v_cache8, x.descale_k, x.descale_v, x.block_table, x.seq_lens,
                               x.scale, x.page_size, x.max_blocks, window=window, softcap=softcap)
    check("fp8-cache decode d=%d paged=%d w=%d cap=%g" % (d, paged, window, softcap), o, lse, ro, rl, BF16_TOL)


def test_fp8_cache_decode_ext_without_options_is_the_plain_kernel(attn):
    x = W.decode_fp8_inputs(4400, len(DEC_LENS), 8, 2, 128, DEC_LENS, 1024, True)
    args = (dev(x.q), dev(x.k_cache8), dev(x.v_cache8), dev(x.descale_k), dev(x.descale_v), dev(x.block_table),
            dev(x.seq_lens))
    o0, l0 = attn.decode_fp8(args[0], args[1], args[2], args[5], args[6], x.page_size, x.max_blocks, args[3],
                             args[4], x.scale, 64)
    ws = torch.empty(attn.attn_decode_workspace_bytes(len(DEC_LENS), 8, 2, 128, x.page_size, x.max_blocks, 64),
                     dtype=torch.uint8, device="cuda")
    o1, l1 = torch.empty_like(o0), torch.empty_like(l0)
    attn.attn_decode_fp8_ext(*args, o1, l1, x.page_size, x.max_blocks, x.scale, -1, 0.0, 64, ws)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("seed", list(range(10)))
def test_fp8_window_softcap_random_shapes(attn, seed):
    """Window and soft-cap on the FP8 prefill over seeded random padded shapes: batch
    1..2, KV heads 1/2/4, group 1/3/4, d 64/128/256, length 1..1500, causal or full;
    the window -1 or 0..N+49, the cap 0 or 1/5/20/50."""
    rng = np.random.default_rng(9500 + seed)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 3, 4]))
    d = int(rng.choice([64, 128, 256]))
    causal = bool(rng.integers(0, 2))
    N = int(rng.integers(1, 1501))
    window = -1 if rng.random() < 0.3 else int(rng.integers(0, N + 50))
    softcap = 0.0 if rng.random() < 0.4 else float(rng.choice([1.0, 5.0, 20.0, 50.0]))
    say("case: fp8 ext random seed=%d B=%d Hq=%d Hkv=%d d=%d N=%d causal=%s window=%d softcap=%g"
        % (seed, B, g * Hkv, Hkv, d, N, causal, window, softcap))
    x = W.prefill_fp8_inputs(9600 + seed, B, g * Hkv, Hkv, N, d, causal=causal)
    o, lse = attn.prefill_fp8(dev(x.q8), dev(x.k8), dev(x.v8), dev(x.descale_q), dev(x.descale_k), dev(x.descale_v),
                              causal, x.scale, window_left=window, softcap=softcap)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_fp8(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, x.descale_v, causal, x.scale,
                                window=window, softcap=softcap)
    check_fp8("fp8 ext random seed=%d" % seed, o, lse, ro, rl, padded_bounds(x, window, softcap))


@pytest.mark.parametrize("seed", list(range(10)))
def test_fp8_cache_decode_window_softcap_random_shapes(attn, seed):
    """Window and soft-cap on the E4M3-cache decode over seeded random batches: 1..12
    sequences of 0..capacity tokens, KV heads 1..8, group 1..7, d 64/128, contiguous or
    paged, chunks automatic or explicit; the bf16 decode's bars."""
    from gpu_common import BF16_TOL, check
    rng = np.random.default_rng(9700 + seed)
    B = int(rng.integers(1, 13))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7]))
    d = int(rng.choice([64, 128]))
    cap = int(rng.integers(64, 3001))
    paged = bool(rng.integers(0, 2))
    chunk = int(rng.choice([0, 16, 64, 256]))
    lens = rng.integers(0, cap + 1, size=B)
    lens[rng.random(B) < 0.15] = 0
    window = -1 if rng.random() < 0.3 else int(rng.integers(0, cap + 50))
    softcap = 0.0 if rng.random() < 0.4 else float(rng.choice([1.0, 5.0, 20.0, 50.0]))
    say("case: fp8-cache decode random seed=%d B=%d Hkv=%d g=%d d=%d cap=%d paged=%s chunk=%d window=%d softcap=%g"
        % (seed, B, Hkv, g, d, cap, paged, chunk, window, softcap))
    x = W.decode_fp8_inputs(9800 + seed, B, g * Hkv, Hkv, d, lens.tolist(), -(-cap // 16) * 16, paged)
    o, lse = attn.decode_fp8(dev(x.q), dev(x.k_cache8), dev(x.v_cache8), dev(x.block_table), dev(x.seq_lens),
                             x.page_size, x.max_blocks, dev(x.descale_k), dev(x.descale_v), x.scale, chunk,
                             window_left=window, softcap=softcap)
    torch.cuda.synchronize()
    ro, rl = oracle.decode_fp8(x.q, x.k_cache8, x.v_cache8, x.descale_k, x.descale_v, x.block_table, x.seq_lens,
                               x.scale, x.page_size, x.max_blocks, window=window, softcap=softcap)
    check("fp8-cache decode random seed=%d" % seed, o, lse, ro, rl, BF16_TOL)
