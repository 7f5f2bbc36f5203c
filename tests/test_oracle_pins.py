"""Pins for the fp64 oracle, against things other than itself.

* values the pofe.ai page prints for its worked example (tests/golden/worked_example.json);
* closed forms of that example (each causal row is a small softmax written out by hand);
* a library routine: PyTorch's float64 scaled_dot_product_attention and logsumexp on CPU;
* a second, hand-written numpy softmax;
* invariances the method guarantees in exact arithmetic: tile size, split count,
  page placement, GQA = MHA on expanded K/V, score shifts, and special cases.

Each test is chosen so that a plausible slip in the oracle (dropped term, wrong sign
or index, transposed operand, wrong head group, wrong log base, off-by-one causal
limit, wrong page index) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from exact_io_aware_prefill_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
E = math.e


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example
def test_worked_example_trace_matches_page(golden):
    tr = oracle.online_trace(golden["scores"], golden["values"], golden["block"])
    tol = 0.5 * 10 ** (-golden["printed_decimals"]) + 1e-12
    b1, b2 = golden["block1"], golden["block2"]
    assert len(tr["m"]) == 2
    assert tr["m"][0] == b1["m"] and tr["m"][1] == b2["m"]
    assert abs(tr["l"][0] - b1["l"]) <= tol
    assert abs(tr["o_tilde"][0] - b1["o_tilde"]) <= tol
    assert abs(tr["o_tilde"][0] / tr["l"][0] - b1["interim_output"]) <= tol
    assert abs(tr["c"][1] - b2["c"]) <= tol
    assert abs(tr["l"][1] - b2["l"]) <= tol
    assert abs(tr["o_tilde"][1] - b2["o_tilde"]) <= tol
    assert abs(tr["o"] - golden["result"]) <= tol
    # the page's direct computation: e^s and their sum
    es = np.exp(np.asarray(golden["scores"], dtype=np.float64))
    assert np.allclose(es, golden["direct_exp_scores"], atol=5e-4)
    assert abs(math.exp(tr["lse"]) - golden["direct_exp_sum"]) <= 5e-4


def test_worked_example_closed_form():
    tr = oracle.online_trace([2, 1, 4, 3], [1, 0, 2, -1], 2)
    num = E**2 * 1 + E**1 * 0 + E**4 * 2 + E**3 * (-1)
    den = E**2 + E**1 + E**4 + E**3
    assert abs(tr["o"] - num / den) < 1e-14
    assert abs(tr["o"] - 1.1380900204) < 1e-10
    assert abs(tr["lse"] - math.log(den)) < 1e-14
    assert abs(tr["lse"] - 4.4401896986) < 1e-10
    # first block correction is exp(-inf) = 0, second is e^(2-4)
    assert tr["c"][0] == 0.0
    assert abs(tr["c"][1] - math.exp(-2.0)) < 1e-16


@pytest.mark.parametrize("block", [1, 2, 3, 4, 7])
def test_worked_example_block_size_invariant(block):
    tr = oracle.online_trace([2, 1, 4, 3], [1, 0, 2, -1], block)
    assert abs(tr["o"] - 1.1380900204) < 1e-10
    assert abs(tr["lse"] - 4.4401896986) < 1e-10


def _embedded_example(d=8):
    s = [2.0, 1.0, 4.0, 3.0]
    vals = [1.0, 0.0, 2.0, -1.0]
    q = np.zeros((1, 1, 4, d)); k = np.zeros((1, 1, 4, d)); v = np.zeros((1, 1, 4, d))
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = s
    v[0, 0, :, 0] = vals
    return q, k, v


# closed forms of the causal prefixes of the example: row i sees keys 0..i
ROWS_O = [1.0,
          E**2 / (E**2 + E),
          (E**2 + 2 * E**4) / (E**2 + E + E**4),
          (E**2 + 2 * E**4 - E**3) / (E**2 + E + E**4 + E**3)]
ROWS_LSE = [2.0, math.log(E**2 + E), math.log(E**2 + E + E**4), math.log(E**2 + E + E**4 + E**3)]


@pytest.mark.parametrize("tiles", [None, (4, 2), (2, 2), (1, 2), (4, 1), (3, 3), (2, 4)])
def test_worked_example_as_causal_prefill(golden, tiles):
    q, k, v = _embedded_example()
    if tiles is None:
        o, lse = oracle.prefill(q, k, v, causal=True, scale=1.0)
    else:
        o, lse = oracle.prefill_tiled(q, k, v, True, 1.0, *tiles)
    assert np.allclose(o[0, 0, :, 0], ROWS_O, atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 0], ROWS_LSE, atol=1e-14, rtol=0)
    assert np.all(o[0, 0, :, 1:] == 0.0)
    # row 1 is the page's interim output after block 1; row 3 is its result
    assert abs(o[0, 0, 1, 0] - golden["block1"]["interim_output"]) < 5e-5
    assert abs(o[0, 0, 3, 0] - golden["result"]) < 5e-5
    assert abs(ROWS_O[3] - 1.1380900204) < 1e-10
    assert abs(ROWS_LSE[1] - 2.3132616875) < 1e-10
    assert abs(ROWS_O[2] - 1.8017846683) < 1e-10


def test_combine_of_the_two_example_blocks(golden):
    o1, l1 = E**2 / (E**2 + E), math.log(E**2 + E)          # block (2, 1)
    o2, l2 = (2 * E**4 - E**3) / (E**4 + E**3), math.log(E**4 + E**3)  # block (4, 3)
    o, lse = oracle.lse_combine(np.array([[[o1], [o2]]]), np.array([[l1, l2]]))
    assert abs(o[0, 0] - 1.1380900204) < 1e-10
    assert abs(o[0, 0] - golden["result"]) < 5e-5
    assert abs(lse[0] - 4.4401896986) < 1e-10
    # the merge weights are softmax(lambda): 0.1192..., 0.8807...
    w1 = 1.0 / (1.0 + math.exp(l2 - l1))
    assert abs(w1 - 0.1192029220) < 1e-9


# --------------------------------------------------- library cross-check (SDPA)
def _torch_ref(q, k, v, causal, scale):
    """PyTorch float64 CPU reference; K/V expanded to Hq heads in contiguous groups."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = s.shape[-1]
        mask = torch.ones(n, n, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


CASES = [
    # B, Hq, Hkv, N, d, causal
    (1, 1, 1, 1, 4, True),
    (1, 1, 1, 5, 4, False),
    (2, 4, 2, 17, 8, True),
    (1, 6, 3, 33, 16, True),
    (2, 6, 3, 33, 16, False),
    (1, 6, 2, 64, 12, True),
    (1, 3, 1, 9, 24, True),
]


@pytest.mark.parametrize("case", CASES)
def test_plain_prefill_matches_torch_sdpa(case):
    B, Hq, Hkv, N, d, causal = case
    rng = np.random.default_rng(1000 + N + d)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    scale = 0.3 + rng.random()
    o, lse = oracle.prefill(q, k, v, causal, scale)
    ro, rl = _torch_ref(q, k, v, causal, scale)
    assert np.max(np.abs(o - ro)) < 1e-12
    assert np.max(np.abs(lse - rl)) < 1e-12


def test_plain_prefill_matches_handwritten_numpy_softmax():
    rng = np.random.default_rng(7)
    N, d = 23, 5
    q = rng.standard_normal((1, 1, N, d)); k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    o, lse = oracle.prefill(q, k, v, True, 0.7)
    for i in range(N):
        s = 0.7 * (k[0, 0, : i + 1] @ q[0, 0, i])
        p = np.exp(s - s.max()); p /= p.sum()
        assert np.max(np.abs(o[0, 0, i] - p @ v[0, 0, : i + 1])) < 1e-13
        assert abs(lse[0, 0, i] - (s.max() + np.log(np.exp(s - s.max()).sum()))) < 1e-13


def test_gqa_equals_mha_on_expanded_kv_bitwise():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, d = 2, 8, 2, 19, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    o1, l1 = oracle.prefill(q, k, v, True, 0.5)
    o2, l2 = oracle.prefill(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1),
                            True, 0.5)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_row_sampling_computes_only_sampled_rows():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 40, 8)); k = rng.standard_normal((1, 1, 40, 8))
    v = rng.standard_normal((1, 1, 40, 8))
    o_all, l_all = oracle.prefill(q, k, v, True, 0.35)
    o_s, l_s = oracle.prefill(q, k, v, True, 0.35, row_step=7)
    rows = np.arange(40) % 7 == 0
    assert np.array_equal(o_s[:, :, rows], o_all[:, :, rows])
    assert np.array_equal(l_s[:, :, rows], l_all[:, :, rows])
    assert np.all(np.isnan(l_s[:, :, ~rows]))


# ----------------------------------------------------- the pages' tiled algorithm
@pytest.mark.parametrize("causal", [True, False])
def test_tiled_prefill_is_independent_of_tile_size(causal):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, N, d = 1, 4, 2, 300, 16
    q = rng.standard_normal((B, Hq, N, d)); k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    o0, l0 = oracle.prefill(q, k, v, causal, 0.25)
    for br, bc in [(1, 1), (2, 2), (3, 7), (7, 3), (64, 64), (64, 16), (16, 64), (N, N), (300, 1)]:
        o, l = oracle.prefill_tiled(q, k, v, causal, 0.25, br, bc)
        assert np.max(np.abs(o - o0)) < 1e-12, (br, bc)
        assert np.max(np.abs(l - l0)) < 1e-12, (br, bc)


def test_tiled_prefill_toy_run_magnitude():
    """The page's toy run: 2,048-token causal prefill, d=128, 64x64 tiles, fp64:
    tiled and standard differ only by rounding (it reports 1.1e-15)."""
    rng = np.random.default_rng(0)
    N, d = 2048, 128
    q = rng.standard_normal((1, 1, N, d)); k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    s = 1.0 / math.sqrt(d)
    o0, l0 = oracle.prefill(q, k, v, True, s)
    o1, l1 = oracle.prefill_tiled(q, k, v, True, s, 64, 64)
    assert np.max(np.abs(o1 - o0)) < 1e-13
    assert np.max(np.abs(l1 - l0)) < 1e-13


# --------------------------------------------------------------------- decode
def _to_cache(k):
    """[B, Hkv, S, d] -> contiguous decode cache [B, S, Hkv, d]."""
    return np.ascontiguousarray(np.transpose(k, (0, 2, 1, 3)))


def _page(kc, lens, P, rng):
    """Scatter a contiguous [B, S, Hkv, d] cache into a randomly permuted page pool.
    Built directly here (not through the oracle) so the oracle's page gather is checked."""
    B, S, Hkv, d = kc.shape
    pages = [-(-int(L) // P) for L in lens]
    pool = sum(pages)
    perm = rng.permutation(pool)
    maxb = -(-S // P)
    bt = np.full((B, maxb), -1, dtype=np.int32)
    kp = np.zeros((pool, P, Hkv, d))
    off = 0
    for b in range(B):
        for p in range(pages[b]):
            phys = perm[off + p]
            bt[b, p] = phys
            n = min(P, int(lens[b]) - p * P)
            kp[phys, :n] = kc[b, p * P: p * P + n]
        off += pages[b]
    return kp, bt


def test_decode_matches_torch_sdpa():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, S, d, P = 3, 6, 2, 96, 16, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, S, d)); v = rng.standard_normal((B, Hkv, S, d))
    lens = np.array([96, 1, 37], dtype=np.int32)
    o, lse = oracle.decode(q, _to_cache(k), _to_cache(v), None, lens, 0.4, P, S // P)
    for b in range(B):
        L = int(lens[b])
        ro, rl = _torch_ref(q[b][None, :, None, :], k[b][None, :, :L], v[b][None, :, :L], False, 0.4)
        assert np.max(np.abs(o[b] - ro[0, :, 0])) < 1e-12
        assert np.max(np.abs(lse[b] - rl[0, :, 0])) < 1e-12


def test_decode_paging_invariance_bitwise():
    rng = np.random.default_rng(22)
    B, Hq, Hkv, S, d, P = 4, 8, 4, 160, 8, 16
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, S, Hkv, d)); vc = rng.standard_normal((B, S, Hkv, d))
    lens = np.array([160, 17, 1, 100], dtype=np.int32)
    o0, l0 = oracle.decode(q, kc, vc, None, lens, 0.3, P, S // P)
    kp, bt = _page(kc, lens, P, np.random.default_rng(5))
    vp, bt2 = _page(vc, lens, P, np.random.default_rng(5))
    assert np.array_equal(bt, bt2)
    o1, l1 = oracle.decode(q, kp, vp, bt, lens, 0.3, P, S // P)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("chunk", [1, 2, 16, 512, 1024])
def test_split_decode_is_independent_of_chunk(chunk):
    rng = np.random.default_rng(23)
    B, Hq, Hkv, S, d, P = 2, 4, 2, 1024, 16, 16
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, S, Hkv, d)); vc = rng.standard_normal((B, S, Hkv, d))
    lens = np.array([1024, 333], dtype=np.int32)
    o0, l0 = oracle.decode(q, kc, vc, None, lens, 0.25, P, S // P)
    for block in (1, 7, 64):
        o, l = oracle.split_decode(q, kc, vc, None, lens, 0.25, P, S // P, chunk, block)
        assert np.max(np.abs(o - o0)) < 1e-12
        assert np.max(np.abs(l - l0)) < 1e-12


def test_split_decode_toy_run_magnitude():
    """The page's toy run: four query heads against a 32,768-token cache with
    1,024-token chunks; split and standard differ only by rounding (it reports 3.0e-16)."""
    rng = np.random.default_rng(0)
    S, d, P = 32768, 128, 16
    q = rng.standard_normal((1, 4, d))
    kc = rng.standard_normal((1, S, 4, d)); vc = rng.standard_normal((1, S, 4, d))
    lens = np.array([S], dtype=np.int32)
    s = 1.0 / math.sqrt(d)
    o0, l0 = oracle.decode(q, kc, vc, None, lens, s, P, S // P)
    o1, l1 = oracle.split_decode(q, kc, vc, None, lens, s, P, S // P, 1024, 1024)
    assert np.max(np.abs(o1 - o0)) < 1e-14
    assert np.max(np.abs(l1 - l0)) < 1e-13


def test_split_parts_recombine():
    rng = np.random.default_rng(24)
    q = rng.standard_normal((1, 2, 8))
    kc = rng.standard_normal((1, 64, 1, 8)); vc = rng.standard_normal((1, 64, 1, 8))
    lens = np.array([50], dtype=np.int32)
    o, l, op, lp = oracle.split_decode(q, kc, vc, None, lens, 0.5, 16, 4, 16, 4, return_parts=True)
    assert lp.shape == (2, 4) and np.isfinite(lp[:, :4]).all()
    o2, l2 = oracle.lse_combine(op, lp)
    assert np.array_equal(o2, o.reshape(2, 8)) and np.array_equal(l2, l.reshape(2))
    # each partial is the plain softmax over its own chunk
    for c in range(4):
        t1 = min(50, 16 * c + 16)
        ro, rl = oracle.decode(q, kc[:, 16 * c:16 * c + 16], vc[:, 16 * c:16 * c + 16], None,
                               np.array([t1 - 16 * c], dtype=np.int32), 0.5, 16, 1)
        assert np.max(np.abs(op[:, c] - ro[0])) < 1e-13
        assert np.max(np.abs(lp[:, c] - rl[0])) < 1e-13


def test_prefill_row_equals_decode_of_that_row_bitwise():
    rng = np.random.default_rng(25)
    B, Hq, Hkv, N, d = 1, 4, 2, 48, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    o, lse = oracle.prefill(q, k, v, True, 0.3)
    for i in (0, 1, 15, 16, 47):
        od, ld = oracle.decode(q[:, :, i], _to_cache(k), _to_cache(v), None,
                               np.array([i + 1], dtype=np.int32), 0.3, 16, N // 16)
        assert np.array_equal(od, o[:, :, i]) and np.array_equal(ld, lse[:, :, i])


# -------------------------------------------------------------- special cases
def test_single_key_gives_its_value():
    rng = np.random.default_rng(26)
    q = rng.standard_normal((1, 1, 1, 8)); k = rng.standard_normal((1, 1, 1, 8))
    v = rng.standard_normal((1, 1, 1, 8))
    o, lse = oracle.prefill(q, k, v, True, 0.6)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    assert abs(lse[0, 0, 0] - 0.6 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-15


def test_equal_scores_give_prefix_means():
    rng = np.random.default_rng(27)
    N, d = 30, 6
    q = np.zeros((1, 1, N, d)); k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    o, lse = oracle.prefill(q, k, v, True, 1.0)
    means = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert np.max(np.abs(o[0, 0] - means)) < 1e-14
    assert np.max(np.abs(lse[0, 0] - np.log(np.arange(1, N + 1)))) < 1e-14
    o, lse = oracle.prefill(q, k, v, False, 1.0)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(axis=0))) < 1e-14
    assert np.max(np.abs(lse[0, 0] - math.log(N))) < 1e-14


def test_shifting_a_rows_scores_shifts_only_its_lse():
    rng = np.random.default_rng(28)
    N, d = 20, 6
    q = rng.standard_normal((1, 1, N, d)); k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    shift = rng.standard_normal(N) * 5.0
    # extra coordinate: q'_i = [q_i, shift_i], k'_j = [k_j, 1]  ->  s'_ij = s_ij + shift_i
    q2 = np.concatenate([q, shift[None, None, :, None]], axis=-1)
    k2 = np.concatenate([k, np.ones((1, 1, N, 1))], axis=-1)
    v2 = np.concatenate([v, np.zeros((1, 1, N, 1))], axis=-1)
    o1, l1 = oracle.prefill(q, k, v, True, 1.0)
    o2, l2 = oracle.prefill(q2, k2, v2, True, 1.0)
    assert np.max(np.abs(o2[..., :d] - o1)) < 1e-12
    assert np.max(np.abs(l2 - (l1 + shift))) < 1e-12


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(29)
    N, d = 16, 4
    q = np.zeros((1, 1, N, d)); q[..., 0] = 1.0
    k = np.zeros((1, 1, N, d)); k[0, 0, 5, 0] = 80.0
    v = rng.standard_normal((1, 1, N, d))
    o, lse = oracle.prefill(q, k, v, False, 1.0)
    assert np.max(np.abs(o[0, 0] - v[0, 0, 5])) < 1e-30 + 1e-12
    assert np.max(np.abs(lse[0, 0] - (80.0 + math.log1p((N - 1) * math.exp(-80.0))))) < 1e-12


def test_empty_sequence_and_empty_combine():
    q = np.ones((2, 2, 4))
    kc = np.ones((2, 16, 1, 4)); vc = np.ones((2, 16, 1, 4))
    o, lse = oracle.decode(q, kc, vc, None, np.array([0, 3], dtype=np.int32), 1.0, 16, 1)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    assert np.allclose(o[1], 1.0) and np.allclose(lse[1], 4.0 + math.log(3.0))
    o, lse = oracle.split_decode(q, kc, vc, None, np.array([0, 3], dtype=np.int32), 1.0, 16, 1, 2, 1)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    oc, lc = oracle.lse_combine(np.ones((1, 3, 4)), np.zeros((1, 3)), np.array([0], dtype=np.int32))
    assert np.all(oc == 0.0) and np.isneginf(lc[0])


def test_one_split_combine_is_identity():
    rng = np.random.default_rng(30)
    op = rng.standard_normal((5, 1, 7)); lp = rng.standard_normal((5, 1)) * 10
    o, l = oracle.lse_combine(op, lp)
    assert np.array_equal(o, op[:, 0]) and np.array_equal(l, lp[:, 0])


def test_combine_ignores_splits_past_n_splits():
    rng = np.random.default_rng(31)
    op = rng.standard_normal((3, 4, 5)); lp = rng.standard_normal((3, 4))
    ns = np.array([4, 2, 1], dtype=np.int32)
    o, l = oracle.lse_combine(op, lp, ns)
    for r in range(3):
        o2, l2 = oracle.lse_combine(op[r:r + 1, :ns[r]], lp[r:r + 1, :ns[r]])
        assert np.array_equal(o[r], o2[0]) and l[r] == l2[0]


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.prefill(np.zeros((1, 3, 4, 8)), np.zeros((1, 2, 4, 8)), np.zeros((1, 2, 4, 8)),
                       True, 1.0)
    with pytest.raises(ValueError):
        oracle.decode(np.zeros((1, 2, 4)), np.zeros((1, 16, 1, 4)), np.zeros((1, 16, 1, 4)), None,
                      np.array([17], dtype=np.int32), 1.0, 16, 1)


# ---------------------------------------------------------------------------
# Decode with in-place append (pofe.ai page, section "Minimal implementation")
# ---------------------------------------------------------------------------
def test_append_into_empty_cache_is_the_new_token_alone():
    """With nothing cached, the query sees only the new key: the softmax has one
    term, so O = v_new and LSE = scale * <q, k_new> (closed form)."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, d, P, nb = 2, 4, 2, 8, 16, 3
    q = rng.standard_normal((B, Hq, d))
    kn = rng.standard_normal((B, Hkv, d)); vn = rng.standard_normal((B, Hkv, d))
    kc = rng.standard_normal((B, nb * P, Hkv, d)); vc = rng.standard_normal((B, nb * P, Hkv, d))
    o, lse, kc2, vc2 = oracle.decode_append(q, kn, vn, kc, vc, None, np.zeros(B, np.int32), 0.3, P, nb)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(o[b, h], vn[b, h // g])
            assert abs(lse[b, h] - 0.3 * float(q[b, h] @ kn[b, h // g])) < 1e-12
    assert np.array_equal(kc2[:, 0], kn) and np.array_equal(vc2[:, 0], vn)


def test_append_of_a_cached_row_equals_decode_of_one_more_token():
    """Appending the row the cache already holds at position L changes no data, so
    the result is plain decode over L + 1 tokens, bit for bit, and the cache is
    unchanged; paged and contiguous layouts, including page boundaries."""
    rng = np.random.default_rng(32)
    B, Hq, Hkv, d, P = 4, 6, 3, 16, 16
    S = 80
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, S, d)); v = rng.standard_normal((B, Hkv, S, d))
    kc, vc = _to_cache(k), _to_cache(v)
    lens = np.array([0, 15, 16, 63], dtype=np.int32)
    kn = np.stack([kc[b, lens[b]] for b in range(B)]); vn = np.stack([vc[b, lens[b]] for b in range(B)])
    o, lse, kc2, vc2 = oracle.decode_append(q, kn, vn, kc, vc, None, lens, 0.25, P, S // P)
    ro, rl = oracle.decode(q, kc, vc, None, lens + 1, 0.25, P, S // P)
    assert np.array_equal(o, ro) and np.array_equal(lse, rl)
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)
    # the same through a permuted page pool
    kp, bt = _page(kc, lens + 1, P, np.random.default_rng(5))
    vp, _ = _page(vc, lens + 1, P, np.random.default_rng(5))
    o3, lse3, kp2, vp2 = oracle.decode_append(q, kn, vn, kp, vp, bt, lens, 0.25, P, bt.shape[1])
    assert np.array_equal(o3, ro) and np.array_equal(lse3, rl)
    assert np.array_equal(kp2, kp) and np.array_equal(vp2, vp)


def test_append_writes_only_the_new_slot():
    """The new rows land at token L (page bt[b][L // P], slot L % P) and nowhere else;
    a length at or past the capacity puts them in the last slot."""
    rng = np.random.default_rng(33)
    B, Hq, Hkv, d, P, nb = 3, 2, 2, 4, 16, 2
    pool = 7
    kp = rng.standard_normal((pool, P, Hkv, d)); vp = rng.standard_normal((pool, P, Hkv, d))
    bt = np.array([[3, 5], [0, 6], [2, 1]], dtype=np.int32)
    lens = np.array([17, 5, 99], dtype=np.int32)  # the last is past the capacity 32
    kn = rng.standard_normal((B, Hkv, d)); vn = rng.standard_normal((B, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    _, _, kp2, vp2 = oracle.decode_append(q, kn, vn, kp, vp, bt, lens, 1.0, P, nb)
    expect_k, expect_v = kp.copy(), vp.copy()
    for b, (page, slot) in enumerate([(5, 1), (0, 5), (1, 15)]):
        expect_k[page, slot] = kn[b]; expect_v[page, slot] = vn[b]
    assert np.array_equal(kp2, expect_k) and np.array_equal(vp2, expect_v)


# ---------------------------------------------------------------------------
# Packed variable-length prefill (pofe.ai page, section "Interaction with
# post-trained models": engines batch prompts of different lengths without padding)
# ---------------------------------------------------------------------------
def _packed(rng, lens, Hq, Hkv, d):
    T = sum(lens)
    return (rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hkv, d)),
            np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))


def test_varlen_sequences_do_not_see_each_other():
    """Changing every token of one sequence leaves the others' outputs bit for bit."""
    rng = np.random.default_rng(41)
    lens = [5, 0, 17, 9]
    q, k, v, cu = _packed(rng, lens, 4, 2, 8)
    o, lse = oracle.prefill_varlen(q, k, v, cu, True, 0.35)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    s0, s1 = cu[2], cu[3]
    q2[s0:s1] += 1.5; k2[s0:s1] -= 0.7; v2[s0:s1] *= 3.0
    o2, lse2 = oracle.prefill_varlen(q2, k2, v2, cu, True, 0.35)
    keep = np.r_[0:s0, s1:cu[-1]]
    assert np.array_equal(o[keep], o2[keep]) and np.array_equal(lse[:, keep], lse2[:, keep])
    assert not np.array_equal(o[s0:s1], o2[s0:s1])


def test_varlen_packing_order_does_not_matter():
    """Packing the same sequences in another order permutes the outputs, bit for bit."""
    rng = np.random.default_rng(42)
    lens = [3, 11, 1, 7]
    q, k, v, cu = _packed(rng, lens, 2, 1, 8)
    o, lse = oracle.prefill_varlen(q, k, v, cu, True, 0.5)
    order = [2, 0, 3, 1]
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    cu2 = np.concatenate([[0], np.cumsum([lens[b] for b in order])]).astype(np.int32)
    o2, lse2 = oracle.prefill_varlen(q[idx], k[idx], v[idx], cu2, True, 0.5)
    assert np.array_equal(o2, o[idx]) and np.array_equal(lse2, lse[:, idx])


def test_varlen_single_token_sequence_is_its_value():
    """A one-token sequence attends only to itself: O = v, LSE = scale * <q, k>."""
    rng = np.random.default_rng(43)
    q, k, v, cu = _packed(rng, [4, 1, 6], 2, 2, 8)
    o, lse = oracle.prefill_varlen(q, k, v, cu, True, 0.8)
    t = cu[1]
    for h in range(2):
        assert np.array_equal(o[t, h], v[t, h])
        assert abs(lse[h, t] - 0.8 * float(q[t, h] @ k[t, h])) < 1e-12


# ---------------------------------------------------------------------------
# Variants the pofe.ai page lists (section "Interaction with post-trained
# models"): sliding windows and logit soft-capping
# ---------------------------------------------------------------------------
def test_window_matches_torch_sdpa_with_a_band_mask():
    """Row i sees keys max(0, i - W) .. i: PyTorch float64 SDPA with the same
    boolean band mask (a library routine) agrees to 1e-12."""
    rng = np.random.default_rng(51)
    B, Hq, Hkv, N, d, W = 2, 4, 2, 70, 16, 9
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    o, lse = oracle.prefill(q, k, v, True, 0.3, window=W)
    i = torch.arange(N)[:, None]; j = torch.arange(N)[None, :]
    allowed = (j <= i) & (j >= i - W)
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    kt = kt.repeat_interleave(2, dim=1); vt = vt.repeat_interleave(2, dim=1)
    ro = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=0.3)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * 0.3
    rl = torch.logsumexp(s.masked_fill(~allowed, float("-inf")), dim=-1)
    assert np.max(np.abs(o - ro.numpy())) < 1e-12 and np.max(np.abs(lse - rl.numpy())) < 1e-12


def test_window_special_cases():
    rng = np.random.default_rng(52)
    B, Hq, Hkv, N, d = 1, 2, 1, 40, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    full = oracle.prefill(q, k, v, True, 0.4)
    # a window as long as the sequence changes nothing, bit for bit
    wide = oracle.prefill(q, k, v, True, 0.4, window=N - 1)
    assert np.array_equal(wide[0], full[0]) and np.array_equal(wide[1], full[1])
    # window 0: each row sees only itself, O = v_i and LSE = scale * <q_i, k_i>
    o0, l0 = oracle.prefill(q, k, v, True, 0.4, window=0)
    for h in range(Hq):
        assert np.array_equal(o0[0, h], v[0, 0])
        assert np.max(np.abs(l0[0, h] - 0.4 * np.einsum("nd,nd->n", q[0, h], k[0, 0]))) < 1e-12
    # decode of token i with a window = prefill row i with the same window, bit for bit
    ow, lw = oracle.prefill(q, k, v, True, 0.4, window=5)
    for i in (0, 3, 17, 39):
        od, ld = oracle.decode(q[:, :, i], _to_cache(k), _to_cache(v), None, np.array([i + 1], np.int32), 0.4, 8,
                               N // 8, window=5)
        assert np.array_equal(od, ow[:, :, i]) and np.array_equal(ld, lw[:, :, i])


def test_softcap_limits():
    """softcap * tanh(s / softcap) differs from s by at most |s|^3 / (3 softcap^2): with a
    large cap the result is the uncapped one within that bound; with a tiny cap every
    score is within +-cap, so the weights are uniform up to exp(+-2 cap) and O is the
    mean of the visible values within 4 cap max|v|."""
    rng = np.random.default_rng(53)
    B, Hq, Hkv, N, d = 1, 2, 2, 30, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    scale = 0.35
    o, lse = oracle.prefill(q, k, v, True, scale)
    smax = float(np.max(np.abs(np.einsum("bhnd,bhmd->bhnm", q, k)))) * scale
    C = 1000.0
    oc, lc = oracle.prefill(q, k, v, True, scale, softcap=C)
    bound = smax ** 3 / (3 * C * C)
    assert np.max(np.abs(lc - lse)) <= bound * 1.01 + 1e-12
    assert np.max(np.abs(oc - o)) <= 4 * bound * float(np.max(np.abs(v))) + 1e-12
    c = 1e-3
    ot, lt = oracle.prefill(q, k, v, True, scale, softcap=c)
    for i in range(N):
        mean = v[0, :, : i + 1].mean(axis=1)
        assert np.max(np.abs(ot[0, :, i] - mean)) <= 4 * c * float(np.max(np.abs(v))) + 1e-12
        assert np.max(np.abs(lt[0, :, i] - np.log(i + 1))) <= c + 1e-12


def test_softcap_applies_to_the_scaled_score():
    """The cap bounds the scaled score s = scale * <q, k>, not the raw dot product: with a
    large scale and a tiny cap every capped score is still within +-cap, so the weights
    stay uniform (capping <q, k> first and scaling after would leave scores up to
    scale * cap apart and fail the bound below)."""
    rng = np.random.default_rng(54)
    B, Hq, Hkv, N, d = 1, 2, 1, 24, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d)); v = rng.standard_normal((B, Hkv, N, d))
    scale, c = 40.0, 1e-3
    ot, lt = oracle.prefill(q, k, v, True, scale, softcap=c)
    for i in range(N):
        mean = v[0, 0, : i + 1].mean(axis=0)
        assert np.max(np.abs(ot[0, :, i] - mean)) <= 4 * c * float(np.max(np.abs(v))) + 1e-12
        assert np.max(np.abs(lt[0, :, i] - np.log(i + 1))) <= c + 1e-12
    # the same holds for decode of the last token
    kc = k[0].transpose(1, 0, 2)[None].copy()  # [1, N, Hkv, d]
    vc = v[0].transpose(1, 0, 2)[None].copy()
    od, ld = oracle.decode(q[:, :, N - 1], kc, vc, None, np.array([N], dtype=np.int32), scale, N, 1, softcap=c)
    assert np.max(np.abs(od[0] - v[0, 0].mean(axis=0))) <= 4 * c * float(np.max(np.abs(v))) + 1e-12


# ---------------------------------------------------------------- FP8 (E4M3) inputs
def test_e4m3_decode_matches_the_format_and_torch():
    """Every byte code decodes as PyTorch's float8_e4m3fn does (a library routine), and
    the format's landmarks hold: largest 448, smallest normal 2^-6, smallest subnormal
    2^-9, 1.0 = 0x38, the sign bit, and NaN only at 0x7f / 0xff."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.flatnonzero(np.isnan(got)).tolist() == [0x7f, 0xff]
    assert got[0x7e] == 448.0 and np.nanmax(got) == 448.0
    assert got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xb8] == -1.0 and got[0x00] == 0.0 and np.signbit(got[0x80])
    # within a binade the 8 mantissa steps are 1/8 apart
    assert np.allclose(np.diff(got[0x38:0x40]), 0.125, rtol=0, atol=0)


def test_fp8_prefill_reproduces_the_worked_example():
    """The page's worked example with every value exact in E4M3 (codes written by hand
    from the format: 1 = 0x38, 2 = 0x40, 3 = 0x44, 4 = 0x48, -1 = 0xb8, 0 = 0x00):
    row 3 is the printed 1.1381 and the closed form."""
    N, d = 4, 16
    q8 = np.zeros((1, 1, N, d), np.uint8); k8 = np.zeros_like(q8); v8 = np.zeros_like(q8)
    q8[0, 0, :, 0] = 0x38
    k8[0, 0, :, 0] = [0x40, 0x38, 0x48, 0x44]
    v8[0, 0, :, 0] = [0x38, 0x00, 0x40, 0xb8]
    o, lse = oracle.prefill_fp8(q8, k8, v8, None, None, None, True, 1.0)
    e = math.e
    assert abs(o[0, 0, 3, 0] - (e**2 + 2 * e**4 - e**3) / (e**2 + e + e**4 + e**3)) < 1e-12
    assert round(o[0, 0, 3, 0], 4) == 1.1381
    assert abs(lse[0, 0, 3] - math.log(e**2 + e + e**4 + e**3)) < 1e-12


def test_fp8_prefill_descale_invariants():
    """Descales are per (sequence, KV head) multipliers of the decoded values: doubling
    descale_q and halving scale changes nothing; tripling descale_v triples O and keeps
    the LSE; changing one KV head's descale_k changes only that group's query heads."""
    rng = np.random.default_rng(61)
    B, Hq, Hkv, N, d = 2, 4, 2, 40, 16
    codes = lambda shape: rng.integers(0, 256, size=shape).astype(np.uint8) & 0x7e | (
        rng.integers(0, 2, size=shape).astype(np.uint8) << 7)  # no NaN codes, and both signs
    q8, k8, v8 = codes((B, Hq, N, d)), codes((B, Hkv, N, d)), codes((B, Hkv, N, d))
    # keep scores moderate: small exponents only
    q8 &= 0xbf; k8 &= 0xbf
    dq = rng.uniform(0.001, 0.01, (B, Hkv)); dk = rng.uniform(0.001, 0.01, (B, Hkv)); dv = rng.uniform(0.5, 2, (B, Hkv))
    o, lse = oracle.prefill_fp8(q8, k8, v8, dq, dk, dv, True, 0.25)
    o2, lse2 = oracle.prefill_fp8(q8, k8, v8, 2 * dq, dk, dv, True, 0.125)
    assert np.max(np.abs(o2 - o)) < 1e-12 and np.max(np.abs(lse2 - lse)) < 1e-12
    o3, lse3 = oracle.prefill_fp8(q8, k8, v8, dq, dk, 3 * dv, True, 0.25)
    assert np.max(np.abs(o3 - 3 * o)) < 1e-12 and np.max(np.abs(lse3 - lse)) < 1e-12
    dk2 = dk.copy(); dk2[1, 0] *= 2
    o4, lse4 = oracle.prefill_fp8(q8, k8, v8, dq, dk2, dv, True, 0.25)
    g = Hq // Hkv
    changed = np.zeros((B, Hq), bool); changed[1, 0:g] = True
    assert np.array_equal(o4[~changed], o[~changed]) and np.array_equal(lse4[~changed], lse[~changed])
    assert np.max(np.abs(o4[changed] - o[changed])) > 1e-6
    # the changed group equals the same call with the scale doubled for that sequence
    o5, lse5 = oracle.prefill_fp8(q8[1:], k8[1:], v8[1:], dq[1:], dk[1:], dv[1:], True, 0.5)
    assert np.max(np.abs(o5[0, 0:g] - o4[1, 0:g])) < 1e-12


def test_fp8_varlen_oracle_is_the_padded_fp8_oracle_per_sequence():
    """The packed FP8 oracle against the (pinned) padded one on each sequence alone
    with that sequence's descale row; an empty sequence owns no rows; another
    sequence's codes do not reach a sequence; descale_v[b] scales sequence b's
    output only, and descale_q * descale_k is all the scores see."""
    lens = [5, 0, 70, 33]
    x = W.prefill_fp8_packed_inputs(41, lens, 6, 2, 64, scale=0.3)
    args = (x.descale_q, x.descale_k, x.descale_v, x.cu_seqlens, True, x.scale)
    o, lse = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, *args)
    cu = x.cu_seqlens.tolist()
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        sl = lambda t: t[s0:s1].permute(1, 0, 2)[None]  # noqa: E731
        ro, rl = oracle.prefill_fp8(sl(x.q8), sl(x.k8), sl(x.v8), x.descale_q[b:b + 1], x.descale_k[b:b + 1],
                                    x.descale_v[b:b + 1], True, x.scale)
        assert np.abs(ro[0].transpose(1, 0, 2) - o[s0:s1]).max() <= 1e-12
        assert np.abs(rl[0] - lse[:, s0:s1]).max() <= 1e-12
    assert not np.isnan(o).any() and not np.isnan(lse).any()  # the empty sequence leaves no row unwritten
    # isolation: new codes for sequence 0 leave sequences 2 and 3 unchanged
    q2 = x.q8.clone()
    q2[:5] = torch.flip(q2[:5], dims=[0])
    k2 = x.k8.clone()
    k2[:5] = torch.flip(k2[:5], dims=[0])
    o2, l2 = oracle.prefill_fp8_varlen(q2, k2, x.v8, *args)
    assert np.array_equal(o2[5:], o[5:]) and np.array_equal(l2[:, 5:], lse[:, 5:])
    # descale_v[2] x 2: sequence 2's output doubles, the rest is unchanged
    dv = x.descale_v.clone()
    dv[2] *= 2
    o3, l3 = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, x.descale_q, x.descale_k, dv, x.cu_seqlens, True, x.scale)
    assert np.abs(o3[5:75] - 2 * o[5:75]).max() <= 1e-12
    assert np.array_equal(o3[75:], o[75:]) and np.array_equal(o3[:5], o[:5]) and np.array_equal(l3, lse)
    # descale_q x 4 with descale_k / 4: the same scores
    o4, l4 = oracle.prefill_fp8_varlen(x.q8, x.k8, x.v8, x.descale_q * 4, x.descale_k / 4, x.descale_v,
                                       x.cu_seqlens, True, x.scale)
    assert np.abs(o4 - o).max() <= 1e-12 and np.abs(l4 - lse).max() <= 1e-12


def test_fp8_decode_worked_example_and_invariants():
    """Decode over an E4M3 cache: the worked example (codes by hand, as for the FP8
    prefill) gives the printed 1.1381 for the last token; doubling descale_k while
    halving scale changes nothing; descale_v scales O; one sequence's descales touch
    only that sequence; decode of token L-1 equals FP8 prefill row L-1, bitwise."""
    d = 16
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 1.0
    k8 = np.zeros((1, 4, 1, d), np.uint8); v8 = np.zeros_like(k8)
    k8[0, :, 0, 0] = [0x40, 0x38, 0x48, 0x44]
    v8[0, :, 0, 0] = [0x38, 0x00, 0x40, 0xb8]
    o, lse = oracle.decode_fp8(q, k8, v8, None, None, None, np.array([4], np.int32), 1.0, 4, 1)
    assert round(o[0, 0, 0], 4) == 1.1381
    e = math.e
    assert abs(lse[0, 0] - math.log(e**2 + e + e**4 + e**3)) < 1e-12

    rng = np.random.default_rng(71)
    B, Hq, Hkv, S, d = 3, 4, 2, 48, 16
    codes = lambda shape: (rng.integers(0, 256, size=shape).astype(np.uint8) & 0x3e) | (
        rng.integers(0, 2, size=shape).astype(np.uint8) << 7)
    qq = rng.standard_normal((B, Hq, d))
    kc, vc = codes((B, S, Hkv, d)), codes((B, S, Hkv, d))
    sl = np.array([1, 30, 48], np.int32)
    dk = rng.uniform(0.5, 2, (B, Hkv)); dv = rng.uniform(0.5, 2, (B, Hkv))
    o, lse = oracle.decode_fp8(qq, kc, vc, dk, dv, None, sl, 0.3, 16, 3)
    o2, lse2 = oracle.decode_fp8(qq, kc, vc, 2 * dk, dv, None, sl, 0.15, 16, 3)
    assert np.max(np.abs(o2 - o)) < 1e-12 and np.max(np.abs(lse2 - lse)) < 1e-12
    o3, lse3 = oracle.decode_fp8(qq, kc, vc, dk, 3 * dv, None, sl, 0.3, 16, 3)
    assert np.max(np.abs(o3 - 3 * o)) < 1e-12 and np.max(np.abs(lse3 - lse)) < 1e-12
    dv4 = dv.copy(); dv4[2] *= 5
    o4, _ = oracle.decode_fp8(qq, kc, vc, dk, dv4, None, sl, 0.3, 16, 3)
    assert np.array_equal(o4[:2], o[:2]) and not np.allclose(o4[2], o[2])
    # token L-1 of sequence 2 against the FP8 prefill of the same rows (query at row L-1)
    L = 48
    q8 = np.zeros((1, Hq, L, d), np.uint8)
    qp = np.zeros((1, Hq, L, d)); qp[0, :, L - 1] = qq[2]
    # the prefill takes E4M3 queries: compare on a query that is exact in E4M3
    qx = oracle.e4m3_decode(codes((Hq, d)))
    q8[0, :, L - 1] = 0  # placeholder rows; only row L-1 is compared
    qcodes = torch.from_numpy(qx).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q8[0, :, L - 1] = qcodes
    kp = kc[2].transpose(1, 0, 2)[None].copy(); vp = vc[2].transpose(1, 0, 2)[None].copy()
    op, lp = oracle.prefill_fp8(q8, kp, vp, None, dk[2:3], dv[2:3], True, 0.3)
    od, ld = oracle.decode_fp8(qx[None], kc[2:3], vc[2:3], dk[2:3], dv[2:3], None, np.array([L], np.int32),
                               0.3, 16, 3)
    assert np.array_equal(op[0, :, L - 1], od[0]) and np.array_equal(lp[0, :, L - 1], ld[0])


def _e4m3_codes(rng, shape):
    """Random finite E4M3 codes (exponent fields below 15 and the sign bit random)."""
    return (rng.integers(0, 256, size=shape).astype(np.uint8) & 0x77) | (
        rng.integers(0, 2, size=shape).astype(np.uint8) << 7)


def test_fp8_append_into_empty_cache_is_the_new_token_alone():
    """E4M3 cache, nothing cached: the softmax has the new key alone, so O is the new
    value row dequantised, descale_v * e4m3(v_new), and LSE = scale * descale_k *
    <q, e4m3(k_new)> (closed form, with the E4M3 values from the format definition)."""
    rng = np.random.default_rng(34)
    B, Hq, Hkv, d, P, nb = 2, 4, 2, 8, 16, 2
    q = rng.standard_normal((B, Hq, d))
    kn, vn = _e4m3_codes(rng, (B, Hkv, d)), _e4m3_codes(rng, (B, Hkv, d))
    kc, vc = _e4m3_codes(rng, (B, nb * P, Hkv, d)), _e4m3_codes(rng, (B, nb * P, Hkv, d))
    dk = rng.uniform(0.5, 2, (B, Hkv)); dv = rng.uniform(0.5, 2, (B, Hkv))
    o, lse, kc2, vc2 = oracle.decode_fp8_append(q, kn, vn, kc, vc, dk, dv, None, np.zeros(B, np.int32), 0.3, P, nb)
    g = Hq // Hkv
    val = np.vectorize(lambda c: math.ldexp(1 + (int(c) & 7) / 8, ((int(c) >> 3) & 15) - 7) if (int(c) >> 3) & 15
                       else math.ldexp((int(c) & 7) / 8, -6))
    sign = lambda c: np.where(c >> 7, -1.0, 1.0)
    ke, ve = val(kn) * sign(kn), val(vn) * sign(vn)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            assert np.max(np.abs(o[b, h] - dv[b, hk] * ve[b, hk])) < 1e-12
            assert abs(lse[b, h] - 0.3 * dk[b, hk] * float(q[b, h] @ ke[b, hk])) < 1e-12
    assert np.array_equal(kc2[:, 0], kn) and np.array_equal(vc2[:, 0], vn)
    assert np.array_equal(kc2[:, 1:], kc[:, 1:]) and np.array_equal(vc2[:, 1:], vc[:, 1:])


def test_fp8_append_of_a_cached_row_equals_decode_of_one_more_token():
    """Appending the codes the E4M3 cache already holds at token L changes no byte, so
    the result is decode_fp8 over L + 1 tokens, bit for bit; paged and contiguous; and a
    paged append writes only slot L % P of page bt[b][L // P]."""
    rng = np.random.default_rng(35)
    B, Hq, Hkv, d, P, nb = 3, 4, 2, 16, 16, 4
    q = rng.standard_normal((B, Hq, d))
    kc, vc = _e4m3_codes(rng, (B, nb * P, Hkv, d)), _e4m3_codes(rng, (B, nb * P, Hkv, d))
    dk = rng.uniform(0.5, 2, (B, Hkv)); dv = rng.uniform(0.5, 2, (B, Hkv))
    lens = np.array([15, 16, 63], np.int32)
    kn = np.stack([kc[b, lens[b]] for b in range(B)]); vn = np.stack([vc[b, lens[b]] for b in range(B)])
    o, lse, kc2, vc2 = oracle.decode_fp8_append(q, kn, vn, kc, vc, dk, dv, None, lens, 0.25, P, nb)
    ro, rl = oracle.decode_fp8(q, kc, vc, dk, dv, None, lens + 1, 0.25, P, nb)
    assert np.array_equal(o, ro) and np.array_equal(lse, rl)
    assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)
    # paged: pool of 9 pages, sequence b's logical page j at bt[b, j]
    bt = np.array([[4, 0, 7, 2], [8, 1, 3, 6], [5, 2, 0, 1]], np.int32)
    kp, vp = _e4m3_codes(rng, (9, P, Hkv, d)), _e4m3_codes(rng, (9, P, Hkv, d))
    kn2, vn2 = _e4m3_codes(rng, (B, Hkv, d)), _e4m3_codes(rng, (B, Hkv, d))
    lens2 = np.array([17, 5, 40], np.int32)
    _, _, kp2, vp2 = oracle.decode_fp8_append(q, kn2, vn2, kp, vp, dk, dv, bt, lens2, 0.25, P, nb)
    ek, ev = kp.copy(), vp.copy()
    for b, (page, slot) in enumerate([(0, 1), (8, 5), (0, 8)]):
        ek[page, slot] = kn2[b]; ev[page, slot] = vn2[b]
    assert np.array_equal(kp2, ek) and np.array_equal(vp2, ev)


def test_oracle_result_does_not_depend_on_its_thread_count():
    """The oracle's threads split rows and heads, never one row's sums, so its results
    are bitwise the same on one thread as on all of them (the single-core timing
    therefore measures the same computation)."""
    x = W.prefill_inputs(21, 1, 4, 2, 97, 64, W.BF16)
    y = W.decode_paged_inputs(22, 3, 4, 2, 64, 16, 1, 300, lengths=[300, 17, 129])
    n0 = oracle.num_threads()
    try:
        outs = []
        for n in (1, max(2, n0)):
            assert oracle.set_num_threads(n) == n
            assert oracle.threads_used() == n  # the request holds in the parallel regions
            o, l = oracle.prefill(x.q, x.k, x.v, True, x.scale)
            od, ld = oracle.decode(y.q, y.k_cache, y.v_cache, y.block_table, y.seq_lens, y.scale,
                                   y.page_size, y.max_blocks)
            outs.append((o, l, od, ld))
    finally:
        oracle.set_num_threads(n0)
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
