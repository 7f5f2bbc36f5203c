"""GPU parity of attn_decode_fp8_append: decode over an E4M3 KV cache with the new
token's codes written into the cache in place first (the page's "Minimal
implementation" decode step on the 8-bit cache).  The codes convert to bf16 exactly,
so the bf16 decode bars apply; the cache after the call must equal the oracle's byte
for byte (only the new token's slot changes) and cache_seqlens is left to the caller."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, check, dev, say

pytestmark = pytest.mark.gpu

APPEND_LENS = [0, 1, 15, 16, 17, 255, 511, 512, 1023]  # tokens cached before the new one


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def _u8(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


@pytest.mark.parametrize("g", [1, 7])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("chunk", [16, 512, 0])
def test_fp8_cache_decode_append(attn, g, d, paged, chunk):
    say("case: fp8-cache decode append g=%d d=%d paged=%s chunk=%d" % (g, d, paged, chunk))
    Hkv, cap, B = 2, 1024, len(APPEND_LENS)
    seed = 3700 + g + d + chunk
    # pages (or rows) for the cached tokens and the new one
    x = W.decode_fp8_inputs(seed, B, g * Hkv, Hkv, d, [L + 1 for L in APPEND_LENS], cap, paged)
    cached = torch.tensor(APPEND_LENS, dtype=torch.int32)
    kn8, vn8 = W.decode_fp8_new_rows(seed + 1, d, x.descale_k, x.descale_v)
    kc, vc, sl = dev(x.k_cache8), dev(x.v_cache8), dev(cached)
    o, lse = attn.decode_fp8_append(dev(x.q), dev(kn8), dev(vn8), kc, vc, dev(x.block_table), sl, x.page_size,
                                    x.max_blocks, dev(x.descale_k), dev(x.descale_v), x.scale, chunk)
    torch.cuda.synchronize()
    ro, rl, rk, rv = oracle.decode_fp8_append(x.q, kn8, vn8, x.k_cache8, x.v_cache8, x.descale_k, x.descale_v,
                                              x.block_table, cached, x.scale, x.page_size, x.max_blocks)
    check("fp8 append g=%d d=%d paged=%d chunk=%d" % (g, d, paged, chunk), o, lse, ro, rl, BF16_TOL)
    assert np.array_equal(_u8(kc).cpu().numpy(), rk), "K cache after the append differs"
    assert np.array_equal(_u8(vc).cpu().numpy(), rv), "V cache after the append differs"
    assert torch.equal(sl.cpu(), cached), "cache_seqlens must be left to the caller"


def test_fp8_append_of_a_cached_row_is_decode_of_one_more_token(attn):
    """Appending the codes already cached at token L writes no new byte, so the output
    is attn_decode_fp8 over L + 1 tokens, bit for bit (the same split and combine)."""
    say("case: fp8-cache append of a cached row vs decode_fp8")
    lens = [300, 16, 999]
    x = W.decode_fp8_inputs(3790, 3, 8, 2, 128, [L + 1 for L in lens], 1024, True)
    bt = x.block_table
    kn8 = torch.stack([x.k_cache8[bt[b, L // 16], L % 16] for b, L in enumerate(lens)])
    vn8 = torch.stack([x.v_cache8[bt[b, L // 16], L % 16] for b, L in enumerate(lens)])
    args = dict(page_size=x.page_size, max_blocks_per_seq=x.max_blocks, descale_k=dev(x.descale_k),
                descale_v=dev(x.descale_v), scale=x.scale, chunk_tokens=64)
    o1, l1 = attn.decode_fp8_append(dev(x.q), dev(kn8), dev(vn8), dev(x.k_cache8), dev(x.v_cache8), dev(bt),
                                    dev(torch.tensor(lens, dtype=torch.int32)), **args)
    o2, l2 = attn.decode_fp8(dev(x.q), dev(x.k_cache8), dev(x.v_cache8), dev(bt),
                             dev(torch.tensor([L + 1 for L in lens], dtype=torch.int32)), **args)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
