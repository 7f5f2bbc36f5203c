"""attn_decode_noalloc (the decode with its partials in the library's static
per-GPU scratch, for callers that cannot allocate) against attn_decode with a
caller workspace: two calls in a row, the second on a smaller input, each bit for
bit equal to attn_decode's result and within the bf16 bars of the oracle."""
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


def _pair(attn, x, chunk):
    q, kc, vc, bt, sl = dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens)
    B, Hq, d = q.shape
    Hkv = kc.shape[-2]
    need = attn.attn_decode_workspace_bytes(B, Hq, Hkv, d, x.page_size, x.max_blocks, chunk)
    assert 0 < need <= attn.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ref = torch.empty_like(q)
    l_ref = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    attn.attn_decode(q, kc, vc, bt, sl, o_ref, l_ref, x.page_size, x.max_blocks, x.scale, chunk, ws)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    attn.attn_decode_noalloc(q, kc, vc, bt, sl, o, lse, x.page_size, x.max_blocks, x.scale, chunk)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_decode_matches_workspace_decode_twice(attn):
    big = W.make_decode_paged()                                                    # 32 sequences, auto chunk
    small = W.decode_contiguous_inputs(31, 3, 8, 2, 1024, 128, seq_lens=[1000, 1, 300])
    for name, x, chunk in (("paged batch-32", big, 0), ("contiguous batch-3", small, 64)):
        say("case: attn_decode_noalloc", name)
        o, lse, o_ref, l_ref = _pair(attn, x, chunk)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), name
        ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size,
                               x.max_blocks)
        check("noalloc " + name, o, lse, ro, rl, BF16_TOL)


def test_noalloc_rejects_partials_beyond_the_scratch(attn):
    say("case: attn_decode_noalloc beyond its scratch")
    q = torch.zeros(4096, 32, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(4096, 16, 8, 128, dtype=torch.bfloat16, device="cuda")
    sl = torch.full((4096,), 16, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    need = attn.attn_decode_workspace_bytes(4096, 32, 8, 128, 16, 1, 16)
    assert need > attn.NOALLOC_SCRATCH_BYTES
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode_noalloc(q, kc, kc, None, sl, o, None, 16, 1, 0.1, 16)
    assert e.value.status == attn.ATTN_ERR_SCRATCH
