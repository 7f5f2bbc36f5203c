"""The decode's balanced split (automatic chunking, two or more sequences): each KV
head's tokens of all sequences are cut into equal contiguous shares, one per
workgroup, across sequence boundaries, and the combine merges every sequence's
pieces (pofe.ai page, section "Decode: a different bottleneck": split-KV over the
keys, merged by the combine rule).  Cases that stress the share boundaries:
empty sequences inside the batch, more than 64 sequences (the device-side unit
scan runs over several blocks of 64), many short sequences per workgroup, all
head sizes, and the E4M3 cache, against the fp64 oracle."""
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


def run(attn, x, chunk=0):
    o, lse = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                         x.page_size, x.max_blocks, x.scale, chunk)
    torch.cuda.synchronize()
    return o, lse


def reference(x):
    return oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, x.page_size, x.max_blocks)


RAGGED = [0, 1, 255, 256, 257, 4000, 0, 9000, 31, 17000]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 4, 7])
@pytest.mark.parametrize("paged", [False, True])
def test_balanced_decode_ragged_batch(attn, d, g, paged):
    say("case: balanced decode d=%d g=%d paged=%s lengths=%s" % (d, g, paged, RAGGED))
    Hkv, cap = 2, 17024
    if paged:
        x = W.decode_paged_inputs(900 + d + g, len(RAGGED), g * Hkv, Hkv, d, 16, 1, cap, lengths=RAGGED)
    else:
        x = W.decode_contiguous_inputs(900 + d + g, len(RAGGED), g * Hkv, Hkv, cap, d, seq_lens=RAGGED)
    o, lse = run(attn, x)
    for b, L in enumerate(RAGGED):
        if L == 0:  # an empty sequence: output 0, log-sum-exp -inf
            assert (o[b] == 0).all() and torch.isneginf(lse[b]).all()
    ro, rl = reference(x)
    check("balanced d=%d g=%d paged=%d" % (d, g, paged), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("B,Hkv,g,d,lmax", [(200, 32, 1, 64, 600), (100, 2, 4, 128, 3000), (65, 8, 4, 128, 2048)])
def test_balanced_decode_many_sequences(attn, B, Hkv, g, d, lmax):
    """More than 64 sequences (several scan blocks), many of them per workgroup share
    (32 KV heads leave 8 workgroups per head), zero lengths among them."""
    rng = np.random.default_rng(B + Hkv)
    lens = rng.integers(0, lmax + 1, size=B)
    lens[::17] = 0
    say("case: balanced decode B=%d Hkv=%d g=%d d=%d, lengths up to %d" % (B, Hkv, g, d, lmax))
    x = W.decode_paged_inputs(1000 + B, B, g * Hkv, Hkv, d, 16, 1, lmax, lengths=lens.tolist())
    o, lse = run(attn, x)
    ro, rl = reference(x)
    check("balanced many B=%d Hkv=%d" % (B, Hkv), o, lse, ro, rl, BF16_TOL)


def run_fp8(attn, x, chunk=0):
    o, lse = attn.decode_fp8(dev(x.q), dev(x.k_cache8), dev(x.v_cache8), dev(x.block_table), dev(x.seq_lens),
                             x.page_size, x.max_blocks, dev(x.descale_k), dev(x.descale_v), x.scale, chunk)
    torch.cuda.synchronize()
    return o, lse


def reference_fp8(x):
    return oracle.decode_fp8(x.q, x.k_cache8, x.v_cache8, x.descale_k, x.descale_v, x.block_table, x.seq_lens,
                             x.scale, x.page_size, x.max_blocks)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 7])
@pytest.mark.parametrize("paged", [False, True])
def test_balanced_fp8_cache_decode_ragged_batch(attn, d, g, paged):
    """The balanced split over an E4M3 cache (d = 128 moves K rows through the wave's
    LDS slab as the bf16 cache does): the ragged batch with empty sequences, against
    the oracle's plain decode of the dequantised cache."""
    say("case: balanced fp8-cache decode d=%d g=%d paged=%s lengths=%s" % (d, g, paged, RAGGED))
    x = W.decode_fp8_inputs(1900 + d + g, len(RAGGED), g * 2, 2, d, RAGGED, 17024, paged)
    o, lse = run_fp8(attn, x)
    for b, L in enumerate(RAGGED):
        if L == 0:
            assert (o[b] == 0).all() and torch.isneginf(lse[b]).all()
    ro, rl = reference_fp8(x)
    check("balanced fp8 d=%d g=%d paged=%d" % (d, g, paged), o, lse, ro, rl, BF16_TOL)


def test_balanced_fp8_cache_decode_many_sequences(attn):
    """More than 64 sequences over an E4M3 cache: several unit-scan blocks, many short
    sequences per workgroup share, zero lengths among them."""
    B, Hkv, g, d, lmax = 90, 4, 4, 128, 2500
    rng = np.random.default_rng(77)
    lens = rng.integers(0, lmax + 1, size=B)
    lens[::13] = 0
    say("case: balanced fp8-cache decode B=%d Hkv=%d g=%d d=%d, lengths up to %d" % (B, Hkv, g, d, lmax))
    x = W.decode_fp8_inputs(1950, B, g * Hkv, Hkv, d, lens.tolist(), lmax, True)
    o, lse = run_fp8(attn, x)
    ro, rl = reference_fp8(x)
    check("balanced fp8 many B=%d" % B, o, lse, ro, rl, BF16_TOL)


def test_balanced_fp8_cache_decode_matches_per_chunk_split(attn):
    """Same E4M3 cache, balanced split against explicit 256-token chunks: the same exact
    decode, within the float32 rounding of the two merges."""
    x = W.decode_fp8_inputs(1960, len(RAGGED), 8, 2, 128, RAGGED, 17024, True)
    o0, l0 = run_fp8(attn, x, 0)
    o1, l1 = run_fp8(attn, x, 256)
    assert (o0.float() - o1.float()).abs().max().item() <= 1e-2
    live = torch.isfinite(l1)
    assert torch.equal(torch.isfinite(l0), live)
    assert (l0[live] - l1[live]).abs().max().item() <= 1e-4


def test_balanced_and_per_chunk_splits_agree(attn):
    """The two splits group the keys differently; both are the same exact decode, so
    they agree with each other within the float32 rounding of their merges."""
    x = W.decode_paged_inputs(1234, len(RAGGED), 8, 2, 128, 16, 1, 17024, lengths=RAGGED)
    ob, lb = run(attn, x, 0)
    oc, lc = run(attn, x, 512)
    fin = torch.isfinite(lc)
    assert torch.equal(torch.isneginf(lb), torch.isneginf(lc))
    assert (ob.float() - oc.float()).abs().max().item() <= 1e-2
    assert (lb[fin] - lc[fin]).abs().max().item() <= 1e-5


def test_balanced_decode_is_deterministic(attn):
    """Fixed shares and a fixed merge order: two calls give the same bits."""
    x = W.decode_paged_inputs(77, len(RAGGED), 28, 4, 128, 16, 1, 17024, lengths=RAGGED)
    o1, l1 = run(attn, x)
    o2, l2 = run(attn, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _random_case(seed):
    """A seeded random batch shape for the balanced split: batch 2..160 (fewer for large
    heads and capacities), KV heads 1..32,
    group 1..16 (at most 16 query heads per KV head), d 64/128/256, lengths 0..capacity
    with zeros among them, paged or contiguous."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(2, 161))
    Hkv = int(rng.choice([1, 2, 4, 8, 32]))
    g = int(rng.choice([1, 2, 4, 7, 16]))
    d = int(rng.choice([64, 128, 256]))
    cap = int(rng.choice([256, 1024, 3000]))
    # at most about 200 MB of K/V at full capacity, so the fp64 oracle finishes in seconds
    B = max(2, min(B, int(200e6 // (cap * Hkv * d * 4))))
    lens = rng.integers(0, cap + 1, size=B)
    lens[rng.random(B) < 0.15] = 0
    paged = bool(rng.integers(0, 2))
    return B, Hkv, g, d, cap, lens.tolist(), paged


@pytest.mark.parametrize("seed", list(range(24)))
def test_balanced_decode_random_shapes(attn, seed):
    B, Hkv, g, d, cap, lens, paged = _random_case(seed)
    say("case: balanced decode random seed=%d B=%d Hkv=%d g=%d d=%d cap=%d paged=%s" % (seed, B, Hkv, g, d, cap, paged))
    if paged:
        x = W.decode_paged_inputs(5000 + seed, B, g * Hkv, Hkv, d, 16, 1, cap, lengths=lens)
    else:
        capc = -(-cap // 16) * 16
        x = W.decode_contiguous_inputs(5000 + seed, B, g * Hkv, Hkv, capc, d, seq_lens=lens)
    o, lse = run(attn, x)
    ro, rl = reference(x)
    check("balanced random seed=%d" % seed, o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("paged", [False, True])
def test_balanced_decode_append(attn, d, paged):
    """The in-place append under the balanced split: the new rows land in their slots
    (bit for bit) and the query attends them, for a batch whose sequences cross
    workgroup shares; compared with the oracle's append."""
    lens = [0, 1, 255, 256, 4000, 9000, 31, 2000, 700]
    B, Hkv, g, cap = len(lens), 4, 4, 9216
    say("case: balanced decode append d=%d paged=%s" % (d, paged))
    seed = 7000 + d + paged
    if paged:
        x = W.decode_paged_inputs(seed, B, g * Hkv, Hkv, d, 16, 1, cap, lengths=[L + 1 for L in lens])
    else:
        x = W.decode_contiguous_inputs(seed, B, g * Hkv, Hkv, cap, d, seq_lens=lens)
    cached = torch.tensor(lens, dtype=torch.int32)
    kn, vn = W.decode_new_rows(seed + 1, B, Hkv, d)
    kc, vc = dev(x.k_cache), dev(x.v_cache)
    o, lse = attn.decode_append(dev(x.q), dev(kn), dev(vn), kc, vc, dev(x.block_table), dev(cached), x.page_size,
                                x.max_blocks, x.scale, 0)
    torch.cuda.synchronize()
    ro, rl, rk, rv = oracle.decode_append(x.q, kn, vn, x.k_cache, x.v_cache, x.block_table, cached, x.scale,
                                          x.page_size, x.max_blocks)
    check("balanced append d=%d paged=%d" % (d, paged), o, lse, ro, rl, BF16_TOL)
    assert np.array_equal(kc.cpu().double().numpy(), rk), "K cache after the append differs"
    assert np.array_equal(vc.cpu().double().numpy(), rv), "V cache after the append differs"


@pytest.mark.parametrize("seed", list(range(12)))
def test_fp8_cache_decode_random_shapes(attn, seed):
    """Seeded random batches over an E4M3 cache: 1..100 sequences (1 runs the per-chunk
    split, more the balanced one), KV heads 1..8, group 1..7, d 64/128, lengths
    0..capacity with zeros among them, contiguous or paged, automatic or explicit
    chunks; against the oracle's plain decode of the dequantised cache."""
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.choice([1, 2, 7, 33, 100]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7]))
    d = int(rng.choice([64, 128]))
    cap = int(rng.choice([256, 1024, 3000]))
    B = max(1, min(B, int(200e6 // (cap * Hkv * d * 4))))
    lens = rng.integers(0, cap + 1, size=B)
    lens[rng.random(B) < 0.15] = 0
    paged = bool(rng.integers(0, 2))
    chunk = int(rng.choice([0, 0, 64, 256]))
    say("case: fp8-cache decode random seed=%d B=%d Hkv=%d g=%d d=%d cap=%d paged=%s chunk=%d"
        % (seed, B, Hkv, g, d, cap, paged, chunk))
    x = W.decode_fp8_inputs(9100 + seed, B, g * Hkv, Hkv, d, lens.tolist(), -(-cap // 16) * 16, paged)
    o, lse = run_fp8(attn, x, chunk)
    ro, rl = reference_fp8(x)
    check("fp8-cache decode random seed=%d" % seed, o, lse, ro, rl, BF16_TOL)
