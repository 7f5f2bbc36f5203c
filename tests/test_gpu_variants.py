"""GPU parity of the sliding-window and logit soft-cap variants (attn_prefill_ext,
attn_decode_ext) against the fp64 oracle, element by element on seeded inputs, with
the bars of the plain paths: float32 inputs max |err| <= 1e-5, bf16 inputs
<= 2e-2 on O and <= 1e-3 on LSE.  Windows cover the degenerate ones (0: a row sees
only itself; 1; tile-sized and tile-crossing; longer than the sequence) and soft-caps
from strongly to barely active."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, F32_TOL, check, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def run_prefill(attn, x, window, cap):
    o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), x.causal, x.scale, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------------ prefill, padded layout
WINDOWS = [0, 1, 32, 100, 257, 5000]


@pytest.mark.parametrize("N", [1, 130, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", WINDOWS)
def test_bf16_prefill_window(attn, N, d, causal, window):
    say("case: bf16 prefill window=%d N=%d d=%d causal=%s" % (window, N, d, causal))
    x = W.prefill_inputs(1100 + N + d + window, 1, 8, 2, N, d, W.BF16, causal=causal)
    o, lse = run_prefill(attn, x, window, 0.0)
    ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale, window=window)
    check("bf16 window=%d N=%d d=%d causal=%d" % (window, N, d, causal), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("scale,cap", [(None, 1.0), (None, 30.0), (1.0, 30.0), (0.5, 5.0), (-0.4, 3.0)])
def test_bf16_prefill_softcap(attn, d, causal, scale, cap):
    """Scale 1/sqrt(d) keeps N(0,1) scores mostly below the cap; scale 1 or 0.5 pushes
    them to many times the cap, where tanh saturates; a negative scale flips them."""
    say("case: bf16 prefill softcap=%g scale=%s d=%d causal=%s" % (cap, scale, d, causal))
    x = W.prefill_inputs(1200 + d + int(cap), 1, 4, 2, 333, d, W.BF16, causal=causal, scale=scale)
    o, lse = run_prefill(attn, x, -1, cap)
    ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale, softcap=cap)
    check("bf16 softcap=%g scale=%g" % (cap, x.scale), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window,cap", [(0, 20.0), (64, 20.0), (200, 2.0)])
def test_bf16_prefill_window_and_softcap(attn, d, window, cap):
    say("case: bf16 prefill window=%d softcap=%g d=%d" % (window, cap, d))
    x = W.prefill_inputs(1300 + d + window, 2, 8, 2, 700, d, W.BF16, scale=0.3)
    o, lse = run_prefill(attn, x, window, cap)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, window=window, softcap=cap)
    check("bf16 window=%d softcap=%g" % (window, cap), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("N", [1, 65, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window,cap", [(0, 0.0), (17, 0.0), (64, 0.0), (-1, 2.0), (40, 10.0)])
def test_f32_prefill_variants(attn, N, d, window, cap):
    say("case: f32 prefill window=%d softcap=%g N=%d d=%d" % (window, cap, N, d))
    x = W.prefill_inputs(1400 + N + d, 1, 4, 2, N, d, W.F32, scale=0.25)
    o, lse = run_prefill(attn, x, window, cap)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, window=window, softcap=cap)
    check("f32 window=%d softcap=%g N=%d d=%d" % (window, cap, N, d), o, lse, ro, rl, F32_TOL)


def test_long_prefill_window_sampled_rows(attn):
    """A 16k-token prompt with a 4096-token window and a soft-cap, checked on every
    61st row (every position inside a tile is hit)."""
    cfg = W.prefill_long(16384)
    say("case: %s window=4096 softcap=30 sampled" % cfg["name"])
    x = W.make_prefill(cfg)
    o, lse = run_prefill(attn, x, 4096, 30.0)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, row_step=61, window=4096, softcap=30.0)
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    rows = np.arange(cfg["N"]) % 61 == 0
    check("16k window=4096 softcap=30 (sampled)", o[:, :, rows].float().cpu().numpy(),
          lse[:, :, rows].cpu().numpy(), ro[:, :, rows], rl[:, :, rows], BF16_TOL)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prefill_ext_without_options_is_the_plain_call(attn, dtype):
    """window -1 / softcap 0, or a window at least as long as the sequence, runs the
    plain kernel: bit-identical outputs."""
    say("case: prefill ext == plain (%s)" % dtype)
    x = W.prefill_inputs(1500, 1, 8, 2, 300, 128, dtype)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    o0, l0 = attn.prefill(q, k, v, True, x.scale)
    for window in (-1, 300, 1 << 30):
        o = torch.empty_like(o0)
        lse = torch.empty_like(l0)
        attn.attn_prefill_ext(q, k, v, o, lse, None, 300, True, x.scale, window, 0.0)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(lse, l0), window


# ------------------------------------------------------------------ prefill, packed layout
VARLEN_LENS = [1, 7, 0, 128, 129, 300, 1000]


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("window,cap", [(0, 0.0), (50, 0.0), (-1, 4.0), (96, 15.0)])
def test_prefill_varlen_variants(attn, dtype, window, cap):
    say("case: varlen %s window=%d softcap=%g" % (dtype, window, cap))
    x = W.prefill_packed_inputs(1600 + window, VARLEN_LENS, 8, 2, 128, dtype, scale=0.3)
    o, lse = attn.prefill_varlen(dev(x.q), dev(x.k), dev(x.v), dev(x.cu_seqlens), x.max_seqlen, x.causal,
                                 x.scale, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, True, x.scale, window=window, softcap=cap)
    tol = BF16_TOL if dtype == W.BF16 else F32_TOL
    check("varlen %s window=%d softcap=%g" % (dtype, window, cap), o, lse, ro, rl, tol)


# ------------------------------------------------------------------ decode
LENS = [1, 15, 16, 17, 100, 511, 513, 1000]


@pytest.mark.parametrize("g", [1, 4])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("chunk", [16, 0])
@pytest.mark.parametrize("window", [0, 1, 16, 100, 511, 5000])
def test_decode_window(attn, g, d, paged, chunk, window):
    say("case: decode window=%d g=%d d=%d paged=%s chunk=%d" % (window, g, d, paged, chunk))
    Hkv = 2
    seed = 1700 + g + d + window
    if paged:
        x = W.decode_paged_inputs(seed, len(LENS), g * Hkv, Hkv, d, 16, 1, 1024, lengths=LENS)
    else:
        x = W.decode_contiguous_inputs(seed, len(LENS), g * Hkv, Hkv, 1024, d, seq_lens=LENS)
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                         x.page_size, x.max_blocks, x.scale, chunk, window_left=window)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size,
                           x.max_blocks, window=window)
    check("decode window=%d g=%d d=%d paged=%d chunk=%d" % (window, g, d, paged, chunk), o, lse, ro, rl,
          BF16_TOL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale,cap,window", [(None, 1.0, -1), (1.0, 30.0, -1), (-0.5, 4.0, -1),
                                              (0.5, 10.0, 300), (None, 50.0, 0)])
def test_decode_softcap(attn, d, scale, cap, window):
    say("case: decode softcap=%g scale=%s window=%d d=%d" % (cap, scale, window, d))
    x = W.decode_paged_inputs(1800 + d, len(LENS), 16, 4, d, 16, 1, 1024, lengths=LENS)
    if scale is not None:
        x.scale = scale
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                         x.page_size, x.max_blocks, x.scale, 64, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size,
                           x.max_blocks, window=window, softcap=cap)
    check("decode softcap=%g scale=%g window=%d" % (cap, x.scale, window), o, lse, ro, rl, BF16_TOL)


def test_decode_32k_window(attn):
    """The 32k-token single-sequence decode with a 4096-token window and a soft-cap:
    only the last 9 of 64 chunks are read."""
    cfg = W.DECODE_32K
    say("case: %s window=4096 softcap=30" % cfg["name"])
    x = W.make_decode_32k(cfg)
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), None, dev(x.seq_lens), x.page_size,
                         x.max_blocks, x.scale, cfg["chunk"], window_left=4096, softcap=30.0)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, None, x.seq_lens, x.scale, x.page_size, x.max_blocks,
                           window=4096, softcap=30.0)
    check("decode 32k window=4096 softcap=30", o, lse, ro, rl, BF16_TOL)


APPEND_LENS = [0, 1, 15, 16, 17, 255, 511, 512, 1023]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("window,cap", [(0, 0.0), (20, 0.0), (300, 8.0), (-1, 2.0)])
def test_decode_append_variants(attn, paged, window, cap):
    say("case: decode append window=%d softcap=%g paged=%s" % (window, cap, paged))
    Hkv, cap_tokens, B, d, g = 2, 1024, len(APPEND_LENS), 128, 4
    seed = 1900 + window
    if paged:
        x = W.decode_paged_inputs(seed, B, g * Hkv, Hkv, d, 16, 1, cap_tokens, lengths=[L + 1 for L in APPEND_LENS])
    else:
        x = W.decode_contiguous_inputs(seed, B, g * Hkv, Hkv, cap_tokens, d, seq_lens=APPEND_LENS)
    cached = torch.tensor(APPEND_LENS, dtype=torch.int32)
    kn, vn = W.decode_new_rows(seed + 1, B, Hkv, d)
    kc, vc = dev(x.k_cache), dev(x.v_cache)
    o, lse = attn.decode_append(dev(x.q), dev(kn), dev(vn), kc, vc, dev(x.block_table), dev(cached), x.page_size,
                                x.max_blocks, x.scale, 32, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl, rk, rv = oracle.decode_append(x.q, kn, vn, x.k_cache, x.v_cache, x.block_table, cached, x.scale,
                                          x.page_size, x.max_blocks, window=window, softcap=cap)
    check("append window=%d softcap=%g paged=%d" % (window, cap, paged), o, lse, ro, rl, BF16_TOL)
    assert np.array_equal(kc.cpu().double().numpy(), rk) and np.array_equal(vc.cpu().double().numpy(), rv)


def test_decode_ext_without_options_is_the_plain_call(attn):
    say("case: decode ext == plain")
    x = W.decode_paged_inputs(2000, len(LENS), 8, 2, 128, 16, 1, 1024, lengths=LENS)
    args = (dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens), x.page_size,
            x.max_blocks, x.scale, 64)
    o0, l0 = attn.decode(*args)
    for window in (-1, 1024, 1 << 30):
        o = torch.empty_like(o0)
        lse = torch.empty_like(l0)
        ws = torch.empty(attn.attn_decode_workspace_bytes(len(LENS), 8, 2, 128, 16, x.max_blocks, 64),
                         dtype=torch.uint8, device="cuda")
        attn.attn_decode_ext(args[0], None, None, args[1], args[2], args[3], args[4], o, lse, x.page_size,
                             x.max_blocks, x.scale, window, 0.0, 64, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(lse, l0), window


# ------------------------------------------------------------------ seeded random shapes
def _draw_options(rng, n, d):
    """A window (-1: none, else 0..n+49) and a soft-cap (0: none, else 1..50); the scale
    is the workloads' 1/sqrt(d) without a cap, and with one anything with |scale| sqrt(d)
    <= 4 (scores of N(0,1) inputs spread up to 4 times the workloads', enough to
    saturate caps 1 and 5).  Wider spreads make rows that one or two keys dominate,
    where rounding the probabilities and O to bf16 alone can pass the 2e-2 bar (about
    2^-9 (max|v - O| + |O|) with |v| near 4)."""
    window = -1 if rng.random() < 0.3 else int(rng.integers(0, n + 50))
    cap = 0.0 if rng.random() < 0.4 else float(rng.choice([1.0, 5.0, 20.0, 50.0]))
    scale = None if cap == 0.0 else float(rng.uniform(-4.0, 4.0)) / d ** 0.5
    return window, cap, scale


@pytest.mark.parametrize("seed", list(range(16)))
def test_prefill_variants_random_shapes(attn, seed):
    """Window and soft-cap over seeded random prefill shapes: batch 1..2, KV heads
    1/2/4, group 1/3/4, d 64/128/256, length 1..2500, causal or full, padded or
    packed (lengths 0..N, one of them N)."""
    rng = np.random.default_rng(8000 + seed)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 3, 4]))
    d = int(rng.choice([64, 128, 256]))
    causal = bool(rng.integers(0, 2))
    packed = bool(rng.integers(0, 2))
    N = int(rng.integers(1, 2501))
    N = max(1, min(N, int((1e10 / (B * g * Hkv * d)) ** 0.5)))
    window, cap, scale = _draw_options(rng, N, d)
    Hq = g * Hkv
    say("case: prefill variants random seed=%d B=%d Hq=%d Hkv=%d d=%d N=%d causal=%s packed=%s window=%d cap=%g "
        "scale=%s" % (seed, B, Hq, Hkv, d, N, causal, packed, window, cap, scale))
    if packed:
        lens = rng.integers(0, N + 1, size=B)
        lens[int(rng.integers(0, B))] = N
        x = W.prefill_packed_inputs(8100 + seed, lens.tolist(), Hq, Hkv, d, W.BF16, causal=causal, scale=scale)
        o, lse = attn.prefill_varlen(dev(x.q), dev(x.k), dev(x.v), dev(x.cu_seqlens), x.max_seqlen, causal, x.scale,
                                     window_left=window, softcap=cap)
        torch.cuda.synchronize()
        ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, causal, x.scale, window=window, softcap=cap)
    else:
        x = W.prefill_inputs(8100 + seed, B, Hq, Hkv, N, d, W.BF16, causal=causal, scale=scale)
        o, lse = run_prefill(attn, x, window, cap)
        ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale, window=window, softcap=cap)
    check("prefill variants random seed=%d" % seed, o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("seed", list(range(16)))
def test_decode_variants_random_shapes(attn, seed):
    """Window and soft-cap over seeded random decode batches: 1..12 sequences of
    0..capacity tokens (capacity 64..3000), KV heads 1/2/4/8, group 1/2/4/7, d
    64/128/256, contiguous or paged, automatic or explicit chunks."""
    rng = np.random.default_rng(8200 + seed)
    B = int(rng.integers(1, 13))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7]))
    d = int(rng.choice([64, 128, 256]))
    cap_tokens = int(rng.integers(64, 3001))
    paged = bool(rng.integers(0, 2))
    chunk = int(rng.choice([0, 16, 64, 256]))
    lens = rng.integers(0, cap_tokens + 1, size=B)
    lens[rng.random(B) < 0.15] = 0
    window, cap, scale = _draw_options(rng, cap_tokens, d)
    say("case: decode variants random seed=%d B=%d Hkv=%d g=%d d=%d capacity=%d paged=%s chunk=%d window=%d cap=%g "
        "scale=%s" % (seed, B, Hkv, g, d, cap_tokens, paged, chunk, window, cap, scale))
    if paged:
        x = W.decode_paged_inputs(8300 + seed, B, g * Hkv, Hkv, d, 16, 1, cap_tokens, lengths=lens.tolist())
    else:
        capc = -(-cap_tokens // 16) * 16
        x = W.decode_contiguous_inputs(8300 + seed, B, g * Hkv, Hkv, capc, d, seq_lens=lens.tolist())
    if scale is not None:
        x.scale = scale
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                         x.page_size, x.max_blocks, x.scale, chunk, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size,
                           x.max_blocks, window=window, softcap=cap)
    check("decode variants random seed=%d" % seed, o, lse, ro, rl, BF16_TOL)
