"""GPU invariances the method guarantees: the result does not depend on the split
count (within tolerance), on where pages sit in the pool (bitwise, same schedule),
on GQA sharing versus explicitly expanded K/V (bitwise), or on the run (bitwise
determinism: no atomics); and decoding query i against keys 0..i agrees with row i
of the causal prefill (within tolerance: different kernels, different rounding)."""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, check, dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def decode(attn, q, kc, vc, bt, sl, P, maxb, scale, chunk):
    o, lse = attn.decode(dev(q), dev(kc), dev(vc), dev(bt), dev(sl), P, maxb, scale, chunk)
    torch.cuda.synchronize()
    return o, lse


@pytest.fixture(scope="module")
def long_seq():
    # 2 sequences, 28/4 heads, 8192-token contiguous cache
    return W.decode_contiguous_inputs(41, 2, 28, 4, 8192, 128, seq_lens=[8192, 5000])


def test_decode_split_count_invariance(attn, long_seq):
    x = long_seq
    ro, rl = oracle.decode(x.q, x.k_cache, x.v_cache, None, x.seq_lens, x.scale, 16, x.max_blocks)
    outs = []
    for chunk in (256, 512, 1024, 2048, 8192):
        say("case: decode chunk=%d" % chunk)
        o, lse = decode(attn, x.q, x.k_cache, x.v_cache, None, x.seq_lens, 16, x.max_blocks, x.scale, chunk)
        check("chunk=%d" % chunk, o, lse, ro, rl, BF16_TOL)
        outs.append((o.float().cpu(), lse.cpu()))
    for o, l in outs[1:]:
        assert (o - outs[0][0]).abs().max().item() <= 2 * BF16_TOL["o"]
        assert (l - outs[0][1]).abs().max().item() <= 2 * BF16_TOL["lse"]


def _scatter_pages(kc, lens, P, perm_seed):
    """contiguous [B,S,Hkv,d] -> pool [pages,P,Hkv,d] + block table (identity if perm_seed is None)."""
    B, S, Hkv, d = kc.shape
    maxb = S // P
    pages = [-(-int(L) // P) for L in lens]
    pool = sum(pages)
    order = np.arange(pool) if perm_seed is None else np.random.default_rng(perm_seed).permutation(pool)
    bt = torch.full((B, maxb), -1, dtype=torch.int32)
    kp = torch.zeros((pool, P, Hkv, d), dtype=kc.dtype)
    off = 0
    for b in range(B):
        for p in range(pages[b]):
            phys = int(order[off + p])
            bt[b, p] = phys
            kp[phys] = kc[b, p * P:(p + 1) * P]
        off += pages[b]
    return kp, bt


def test_paging_is_bitwise_invisible(attn, long_seq):
    x = long_seq
    lens = x.seq_lens.tolist()
    ref = decode(attn, x.q, x.k_cache, x.v_cache, None, x.seq_lens, 16, x.max_blocks, x.scale, 512)
    for seed in (None, 3):
        say("case: paged copy, permutation seed=%s" % seed)
        kp, bt = _scatter_pages(x.k_cache, lens, 16, seed)
        vp, bt2 = _scatter_pages(x.v_cache, lens, 16, seed)
        assert torch.equal(bt, bt2)
        o, lse = decode(attn, x.q, kp, vp, bt, x.seq_lens, 16, x.max_blocks, x.scale, 512)
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])


def test_decode_is_deterministic(attn, long_seq):
    x = long_seq
    say("case: decode run-to-run")
    a = decode(attn, x.q, x.k_cache, x.v_cache, None, x.seq_lens, 16, x.max_blocks, x.scale, 0)
    for _ in range(3):
        b = decode(attn, x.q, x.k_cache, x.v_cache, None, x.seq_lens, 16, x.max_blocks, x.scale, 0)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_prefill_is_deterministic(attn):
    say("case: prefill run-to-run")
    x = W.prefill_inputs(42, 1, 8, 2, 1500, 128, W.BF16)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    a = attn.prefill(q, k, v, True, x.scale)
    for _ in range(3):
        b = attn.prefill(q, k, v, True, x.scale)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_gqa_equals_expanded_heads_bitwise(attn):
    say("case: GQA vs expanded K/V")
    x = W.prefill_inputs(43, 1, 8, 2, 700, 128, W.BF16)
    q = dev(x.q)
    a = attn.prefill(q, dev(x.k), dev(x.v), True, x.scale)
    b = attn.prefill(q, dev(x.k.repeat_interleave(4, dim=1)), dev(x.v.repeat_interleave(4, dim=1)),
                     True, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_row_matches_prefill_row(attn):
    say("case: decode of query i vs prefill row i")
    N = 1000
    x = W.prefill_inputs(44, 1, 8, 2, N, 128, W.BF16)
    po, pl = attn.prefill(dev(x.q), dev(x.k), dev(x.v), True, x.scale)
    kc = x.k.permute(0, 2, 1, 3).contiguous()  # [1, N, Hkv, d]
    vc = x.v.permute(0, 2, 1, 3).contiguous()
    kc = torch.cat([kc, torch.zeros(1, 1008 - N, 2, 128, dtype=kc.dtype)], dim=1)
    vc = torch.cat([vc, torch.zeros(1, 1008 - N, 2, 128, dtype=vc.dtype)], dim=1)
    for i in (0, 17, 500, 999):
        o, lse = decode(attn, x.q[:, :, i].contiguous(), kc, vc, None,
                        torch.tensor([i + 1], dtype=torch.int32), 16, 1008 // 16, x.scale, 256)
        assert (o.float() - po[:, :, i].float()).abs().max().item() <= BF16_TOL["o"]
        assert (lse - pl[:, :, i]).abs().max().item() <= BF16_TOL["lse"]


def test_launches_follow_the_callers_stream(attn):
    """Prefill and decode launched on a side stream (default priority) that first
    waits for the inputs: the same results as on the current stream, bit for bit,
    once that stream is synchronised."""
    say("case: calls on a side stream")
    x = W.prefill_inputs(71, 1, 8, 2, 700, 128, W.BF16)
    y = W.decode_paged_inputs(72, 3, 8, 2, 128, 16, 1, 900, lengths=[900, 17, 512])
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    args = (dev(y.q), dev(y.k_cache), dev(y.v_cache), dev(y.block_table), dev(y.seq_lens), y.page_size,
            y.max_blocks, y.scale, 64)
    o0, l0 = attn.prefill(q, k, v, True, x.scale)
    d0, m0 = attn.decode(*args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o1, l1 = attn.prefill(q, k, v, True, x.scale, stream=side)
        d1, m1 = attn.decode(*args, stream=side)
    side.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(d0, d1) and torch.equal(m0, m1)


def test_stream_argument_without_stream_context(attn):
    """stream= names a side stream while the current stream stays the default one: the
    outputs and the decode workspace are allocated on the side stream, so memory that
    the current stream allocates and fills right after the calls (before any
    synchronisation) cannot be the memory the kernels still use."""
    say("case: stream= without a stream context")
    x = W.prefill_inputs(73, 1, 8, 2, 700, 128, W.BF16)
    y = W.decode_paged_inputs(74, 3, 8, 2, 128, 16, 1, 900, lengths=[900, 17, 512])
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    args = (dev(y.q), dev(y.k_cache), dev(y.v_cache), dev(y.block_table), dev(y.seq_lens), y.page_size,
            y.max_blocks, y.scale, 64)
    o0, l0 = attn.prefill(q, k, v, True, x.scale)
    d0, m0 = attn.decode(*args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        o1, l1 = attn.prefill(q, k, v, True, x.scale, stream=side)
        d1, m1 = attn.decode(*args, stream=side)
        # the current stream allocates and overwrites memory while the side stream runs
        junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(8)]
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(d0, d1) and torch.equal(m0, m1)
