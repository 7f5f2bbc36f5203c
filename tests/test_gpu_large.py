"""GPU parity on large launch grids: many sequences per call (the decode grid's batch
dimension at its limit of 65535, thousands of paged sequences, thousands of packed
prompts, a wide padded batch), each checked element by element against the fp64
oracle with the bf16 bars: max |err| <= 2e-2 on O and <= 1e-3 on LSE."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, check, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def test_decode_batch_at_grid_limit(attn):
    """65535 sequences (the largest batch the decode accepts), one query and one KV
    head of 64 dims, contiguous 16-token caches holding 0..16 tokens each (empty
    sequences give O = 0, LSE = -inf)."""
    B, S = 65535, 16
    say("case: decode B=%d contiguous S=%d" % (B, S))
    lens = np.random.default_rng(61).integers(0, S + 1, size=B).tolist()
    x = W.decode_contiguous_inputs(60, B, 1, 1, S, 64, seq_lens=lens)
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), None, dev(x.seq_lens), x.page_size,
                         x.max_blocks, x.scale, 0)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, None, x.seq_lens, x.scale, x.page_size, x.max_blocks)
    check("decode B=65535", o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("chunk", [0, 32])
def test_decode_many_paged_sequences(attn, chunk):
    """4096 paged sequences of 1..100 tokens, 8 query / 2 KV heads, d = 128."""
    say("case: decode 4096 paged sequences chunk=%d" % chunk)
    x = W.decode_paged_inputs(62, 4096, 8, 2, 128, 16, 1, 100)
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                         x.page_size, x.max_blocks, x.scale, chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size,
                           x.max_blocks)
    check("decode 4096 paged chunk=%d" % chunk, o, lse, ro, rl, BF16_TOL)


def test_prefill_varlen_many_prompts(attn):
    """2000 packed prompts of 0..150 tokens (about 150k tokens), 4 query / 2 KV heads."""
    lens = np.random.default_rng(63).integers(0, 151, size=2000).tolist()
    say("case: varlen prefill, %d prompts, %d tokens" % (len(lens), sum(lens)))
    x = W.prefill_packed_inputs(64, lens, 4, 2, 64, W.BF16)
    o, lse = attn.prefill_varlen(dev(x.q), dev(x.k), dev(x.v), dev(x.cu_seqlens), x.max_seqlen, x.causal, x.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, True, x.scale)
    check("varlen 2000 prompts", o, lse, ro, rl, BF16_TOL)


def test_prefill_wide_padded_batch(attn):
    """512 sequences of 100 tokens, 4 query heads sharing one KV head, d = 128."""
    say("case: padded prefill B=512 N=100")
    x = W.prefill_inputs(65, 512, 4, 1, 100, 128, W.BF16)
    o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), True, x.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale)
    check("padded B=512 N=100", o, lse, ro, rl, BF16_TOL)
