"""GPU parity for head_dim 256 (prefill bf16 and float32, packed prefill, decode with
and without the append, windows and soft-caps) against the fp64
oracle, element by element on seeded inputs, with the bars of the other head sizes:
float32 inputs max |err| <= 1e-5; bf16 inputs <= 2e-2 on O and <= 1e-3 on LSE."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, F32_TOL, check, dev, say

pytestmark = pytest.mark.gpu
D = 256


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


@pytest.mark.parametrize("N", [1, 31, 129, 300, 1000])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_prefill_d256(attn, N, causal):
    say("case: bf16 prefill d=256 N=%d causal=%s" % (N, causal))
    x = W.prefill_inputs(2100 + N, 1, 8, 4, N, D, W.BF16, causal=causal)
    o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), causal, x.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale)
    check("bf16 d=256 N=%d causal=%d" % (N, causal), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("window,cap", [(0, 0.0), (100, 0.0), (-1, 50.0), (64, 30.0)])
def test_bf16_prefill_d256_variants(attn, window, cap):
    say("case: bf16 prefill d=256 window=%d softcap=%g" % (window, cap))
    x = W.prefill_inputs(2200 + window, 2, 8, 4, 700, D, W.BF16, scale=0.2)
    o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), True, x.scale, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, window=window, softcap=cap)
    check("bf16 d=256 window=%d softcap=%g" % (window, cap), o, lse, ro, rl, BF16_TOL)


def test_bf16_prefill_d256_long_sampled_rows(attn):
    """8192 tokens, 16 query / 8 KV heads, every 37th row against the oracle."""
    N, step = 8192, 37
    say("case: bf16 prefill d=256 N=%d sampled every %d" % (N, step))
    x = W.prefill_inputs(2300, 1, 16, 8, N, D, W.BF16)
    o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), True, x.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, row_step=step)
    rows = np.arange(N) % step == 0
    check("bf16 d=256 N=8192 (sampled)", o[:, :, rows].float().cpu().numpy(), lse[:, :, rows].cpu().numpy(),
          ro[:, :, rows], rl[:, :, rows], BF16_TOL)


@pytest.mark.parametrize("N", [1, 33, 64, 200])
@pytest.mark.parametrize("window,cap", [(-1, 0.0), (20, 0.0), (-1, 5.0)])
def test_f32_prefill_d256(attn, N, window, cap):
    say("case: f32 prefill d=256 N=%d window=%d softcap=%g" % (N, window, cap))
    x = W.prefill_inputs(2400 + N, 1, 4, 2, N, D, W.F32, scale=0.1)
    o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), True, x.scale, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, window=window, softcap=cap)
    check("f32 d=256 N=%d window=%d softcap=%g" % (N, window, cap), o, lse, ro, rl, F32_TOL)


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prefill_varlen_d256(attn, dtype):
    say("case: varlen d=256 %s" % dtype)
    x = W.prefill_packed_inputs(2500, [1, 7, 0, 128, 129, 300], 8, 4, D, dtype, scale=0.1)
    o, lse = attn.prefill_varlen(dev(x.q), dev(x.k), dev(x.v), dev(x.cu_seqlens), x.max_seqlen, x.causal, x.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, True, x.scale)
    check("varlen d=256 %s" % dtype, o, lse, ro, rl, BF16_TOL if dtype == W.BF16 else F32_TOL)


LENS = [1, 15, 16, 17, 100, 511, 513, 1000]


@pytest.mark.parametrize("g", [1, 2, 8, 16])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("chunk", [16, 128, 0])
def test_decode_d256(attn, g, paged, chunk):
    say("case: decode d=256 g=%d paged=%s chunk=%d" % (g, paged, chunk))
    Hkv = 2
    if paged:
        x = W.decode_paged_inputs(2600 + g, len(LENS), g * Hkv, Hkv, D, 16, 1, 1024, lengths=LENS)
    else:
        x = W.decode_contiguous_inputs(2600 + g, len(LENS), g * Hkv, Hkv, 1024, D, seq_lens=LENS)
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                         x.page_size, x.max_blocks, x.scale, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size,
                           x.max_blocks)
    check("decode d=256 g=%d paged=%d chunk=%d" % (g, paged, chunk), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("window,cap", [(-1, 0.0), (0, 0.0), (300, 30.0), (-1, 5.0)])
def test_decode_append_d256(attn, window, cap):
    say("case: decode append d=256 window=%d softcap=%g" % (window, cap))
    lens = [0, 1, 15, 16, 255, 511, 1023]
    B, Hkv, g = len(lens), 2, 4
    x = W.decode_paged_inputs(2700 + window, B, g * Hkv, Hkv, D, 16, 1, 1024, lengths=[L + 1 for L in lens])
    cached = torch.tensor(lens, dtype=torch.int32)
    kn, vn = W.decode_new_rows(2701, B, Hkv, D)
    kc, vc = dev(x.k_cache), dev(x.v_cache)
    o, lse = attn.decode_append(dev(x.q), dev(kn), dev(vn), kc, vc, dev(x.block_table), dev(cached), x.page_size,
                                x.max_blocks, x.scale, 64, window_left=window, softcap=cap)
    torch.cuda.synchronize()
    ro, rl, rk, rv = oracle.decode_append(x.q, kn, vn, x.k_cache, x.v_cache, x.block_table, cached, x.scale,
                                          x.page_size, x.max_blocks, window=window, softcap=cap)
    check("append d=256 window=%d softcap=%g" % (window, cap), o, lse, ro, rl, BF16_TOL)
    assert np.array_equal(kc.cpu().double().numpy(), rk) and np.array_equal(vc.cpu().double().numpy(), rv)
