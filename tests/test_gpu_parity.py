"""GPU parity: the HIP path through the C-ABI against the fp64 oracle, element by
element on the same seeded inputs.  Bars: float32 inputs max |err| <= 1e-5 on O and
LSE; bf16 inputs (float32 accumulation) max |err| <= 2e-2 on O and <= 1e-3 on LSE.
The long-prefill workloads are compared on every row at N = 8192 and N = 16384, and
on every 7th row at N = 30720 (a prime stride, so every position inside a tile is
hit).  Each case prints its measured max-abs, max-relative and RMS errors."""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_prefill_amd import workloads as W
from gpu_common import BF16_TOL, F32_TOL, check, dev, say, stats

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    from exact_io_aware_prefill_amd import attn as a  # raises if libattn.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return a


def run_prefill(attn, x):
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    o, lse = attn.prefill(q, k, v, x.causal, x.scale)
    torch.cuda.synchronize()
    return o, lse


# ------------------------------------------------------------------ prefill fp32
def test_worked_example_through_f32_prefill(attn):
    say("case: worked example, f32 prefill N=4 d=64")
    x = W.worked_example_inputs(64)
    o, lse = run_prefill(attn, x)
    e = math.e
    rows_o = [1.0, e**2 / (e**2 + e), (e**2 + 2 * e**4) / (e**2 + e + e**4),
              (e**2 + 2 * e**4 - e**3) / (e**2 + e + e**4 + e**3)]
    rows_l = [2.0, math.log(e**2 + e), math.log(e**2 + e + e**4), math.log(e**2 + e + e**4 + e**3)]
    oc = o.cpu().numpy()[0, 0]
    assert np.max(np.abs(oc[:, 0] - rows_o)) <= 1e-5
    assert np.max(np.abs(lse.cpu().numpy()[0, 0] - rows_l)) <= 1e-5
    assert abs(oc[3, 0] - 1.1381) < 5e-5  # the page's printed result
    assert np.all(oc[:, 1:] == 0.0)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, 1.0)
    check("worked-example", o, lse, ro, rl, F32_TOL)


def test_small_f32_prefill_workload(attn):
    cfg = W.PREFILL_SMALL_F32
    say("case:", cfg["name"])
    x = W.make_prefill(cfg)
    assert x.scale == 1.0 / 8.0
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale)
    check(cfg["name"], o, lse, ro, rl, F32_TOL)


@pytest.mark.parametrize("N", [1, 7, 64, 65, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_f32_prefill_ragged(attn, N, d, causal):
    say("case: f32 prefill B=2 Hq=4 Hkv=2 N=%d d=%d causal=%s" % (N, d, causal))
    x = W.prefill_inputs(100 + N + d, 2, 4, 2, N, d, W.F32, causal=causal)
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale)
    check("f32 N=%d d=%d" % (N, d), o, lse, ro, rl, F32_TOL)


# ------------------------------------------------------------------ prefill bf16
def test_prefill_2k_workload(attn):
    cfg = W.PREFILL_2K
    say("case:", cfg["name"])
    x = W.make_prefill(cfg)
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale)
    check(cfg["name"], o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("N", [1, 5, 64, 127, 129, 300, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_prefill_ragged(attn, N, d, causal):
    say("case: bf16 prefill B=2 Hq=6 Hkv=2 N=%d d=%d causal=%s" % (N, d, causal))
    x = W.prefill_inputs(200 + N + d, 2, 6, 2, N, d, W.BF16, causal=causal)
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale)
    check("bf16 N=%d d=%d causal=%d" % (N, d, causal), o, lse, ro, rl, BF16_TOL)


def test_bf16_prefill_peaky_softmax(attn):
    """Queries scaled by 10: near one-hot rows, frequent rescaling (c << 1)."""
    say("case: bf16 prefill peaky (q x10) N=777 d=128")
    x = W.prefill_inputs(7, 1, 4, 1, 777, 128, W.BF16)
    x.q = (x.q.float() * 10.0).to(torch.bfloat16)
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale)
    check("peaky", o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("N,row_step", [(8192, 1), (16384, 1), (30720, 7)])
def test_long_prefill_workloads(attn, N, row_step):
    """The long-prompt workloads against the oracle: every row of every head at
    N = 8192 and at the headline N = 16384; every 7th row at N = 30720 (the oracle's
    full run there takes over a minute of host time)."""
    cfg = W.prefill_long(N)
    say("case:", cfg["name"], "all rows" if row_step == 1 else "rows sampled every %d" % row_step)
    x = W.make_prefill(cfg)
    o, lse = run_prefill(attn, x)
    assert torch.isfinite(lse).all() and torch.isfinite(o.float()).all()
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, x.scale, row_step=row_step)
    if row_step == 1:
        check(cfg["name"], o, lse, ro, rl, BF16_TOL)
    else:
        rows = np.arange(N) % row_step == 0
        check(cfg["name"], o[:, :, rows].float().cpu().numpy(), lse[:, :, rows].cpu().numpy(),
              ro[:, :, rows], rl[:, :, rows], BF16_TOL)
    del ro, rl
    # a property at every row: LSE >= the row's own (diagonal) scaled score
    diag = (x.q.float() * x.k.float().repeat_interleave(7, dim=1)).sum(-1) * x.scale
    assert (lse.cpu() >= diag - 1e-3).all()


# ------------------------------------------------------------------ combine
def test_worked_example_through_lse_combine(attn):
    say("case: worked example through attn_lse_combine")
    e = math.e
    o1, l1 = e**2 / (e**2 + e), math.log(e**2 + e)
    o2, l2 = (2 * e**4 - e**3) / (e**4 + e**3), math.log(e**4 + e**3)
    op = torch.zeros(1, 2, 64, dtype=torch.float32)
    op[0, 0, 0], op[0, 1, 0] = o1, o2
    lp = torch.tensor([[l1, l2]], dtype=torch.float32)
    o = torch.empty(1, 64, dtype=torch.float32, device="cuda")
    lse = torch.empty(1, dtype=torch.float32, device="cuda")
    attn.attn_lse_combine(dev(op), dev(lp), None, o, lse)
    torch.cuda.synchronize()
    assert abs(o[0, 0].item() - 1.1380900204) <= 1e-5
    assert abs(lse[0].item() - 4.4401896986) <= 1e-5
    assert (o[0, 1:] == 0).all()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16])
def test_lse_combine_random_partials(attn, d, odt):
    say("case: lse_combine random partials d=%d out=%s" % (d, odt))
    g = torch.Generator().manual_seed(d)
    rows, S = 37, 300
    op = torch.randn(rows, S, d, generator=g)
    lp = torch.randn(rows, S, generator=g) * 4
    lp[3, 7] = float("-inf")   # an empty partial
    lp[5, :] = float("-inf")   # a row with only empty partials
    ns = torch.randint(0, S + 1, (rows,), generator=g, dtype=torch.int32)
    ns[0], ns[1], ns[5] = 0, 1, S
    o = torch.empty(rows, d, dtype=odt, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    attn.attn_lse_combine(dev(op), dev(lp), dev(ns), o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_combine(op, lp, ns)
    tol = F32_TOL if odt == torch.float32 else dict(o=1e-2, lse=1e-5)
    check("combine d=%d" % d, o, lse, ro, rl, tol)


# ------------------------------------------------------------------ decode
def run_decode(attn, x, chunk):
    out = attn.decode(dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens),
                      x.page_size, x.max_blocks, x.scale, chunk)
    torch.cuda.synchronize()
    return out


def oracle_decode(x):
    return oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale,
                         x.page_size, x.max_blocks)


def test_decode_32k_workload(attn):
    cfg = W.DECODE_32K
    say("case:", cfg["name"])
    x = W.make_decode_32k(cfg)
    assert attn.attn_decode_chunk_tokens(1, 4, x.page_size, x.max_blocks, 512) == 512
    assert -(-cfg["S"] // 512) == 64
    o, lse = run_decode(attn, x, cfg["chunk"])
    ro, rl = oracle_decode(x)
    check(cfg["name"], o, lse, ro, rl, BF16_TOL)


def test_decode_paged_workload(attn):
    cfg = W.DECODE_PAGED
    say("case:", cfg["name"])
    x = W.make_decode_paged(cfg)
    o, lse = run_decode(attn, x, 0)
    ro, rl = oracle_decode(x)
    check(cfg["name"], o, lse, ro, rl, BF16_TOL)


LENS = [1, 15, 16, 17, 100, 511, 513, 1000]


@pytest.mark.parametrize("g", [1, 4, 7, 16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("chunk", [16, 256, 512])
def test_decode_ragged(attn, g, d, paged, chunk):
    say("case: decode g=%d d=%d paged=%s chunk=%d" % (g, d, paged, chunk))
    Hkv = 2
    if paged:
        x = W.decode_paged_inputs(300 + g + d, len(LENS), g * Hkv, Hkv, d, 16, 1, 1024, lengths=LENS)
    else:
        x = W.decode_contiguous_inputs(300 + g + d, len(LENS), g * Hkv, Hkv, 1024, d, seq_lens=LENS)
    o, lse = run_decode(attn, x, chunk)
    ro, rl = oracle_decode(x)
    check("decode g=%d d=%d paged=%d chunk=%d" % (g, d, paged, chunk), o, lse, ro, rl, BF16_TOL)


def test_decode_empty_sequence(attn):
    say("case: decode with seq_len 0")
    x = W.decode_contiguous_inputs(9, 3, 8, 2, 64, 128, seq_lens=[0, 5, 0])
    o, lse = run_decode(attn, x, 32)
    assert (o[0] == 0).all() and torch.isneginf(lse[0]).all()
    assert (o[2] == 0).all() and torch.isneginf(lse[2]).all()
    ro, rl = oracle_decode(x)
    check("decode empty", o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_prefill_unusual_scales(attn, scale, dtype):
    """Negative scale (the kernel negates Q instead), zero scale (uniform weights) and a
    large scale (peaky rows)."""
    say("case: prefill scale=%g dtype=%s" % (scale, dtype))
    x = W.prefill_inputs(8, 1, 4, 2, 333, 128, dtype, scale=scale)
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, True, scale)
    # The fixed bars hold at the workloads' scale 1/sqrt(d).  Terms that come from
    # float32 rounding of a score s = scale * <q, k> grow with |s|, i.e. |scale| *
    # sqrt(d) times larger here for N(0,1) inputs: an absolute error u|s| in each
    # score moves the LSE by up to that much and each weight by that factor.  So
    # only the bars that such terms dominate are widened by that factor: float32 O
    # and LSE, and the bf16 path's LSE (its row sums and reference stay float32).
    # The bf16 O error comes from rounding P and O to bf16 (2^-9 relative each),
    # which does not depend on the scale, so its bar stays at 2e-2.
    grow = max(1.0, abs(scale) * math.sqrt(128))
    if dtype == W.BF16:
        tol = dict(o=BF16_TOL["o"], lse=BF16_TOL["lse"] * grow)
    else:
        tol = {k_: v_ * grow for k_, v_ in F32_TOL.items()}
    check("scale=%g" % scale, o, lse, ro, rl, tol)


# ------------------------------------------------------------------ decode with append
APPEND_LENS = [0, 1, 15, 16, 17, 255, 511, 512, 1023]  # tokens cached before the new one


@pytest.mark.parametrize("g", [1, 7])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("chunk", [16, 512, 0])
def test_decode_append(attn, g, d, paged, chunk):
    """The new token's rows go into the cache in place (only its slot changes, bit for
    bit) and the query attends the cached tokens plus the new one."""
    say("case: decode append g=%d d=%d paged=%s chunk=%d" % (g, d, paged, chunk))
    Hkv, cap, B = 2, 1024, len(APPEND_LENS)
    seed = 700 + g + d + chunk
    if paged:  # pages for the cached tokens and the new one
        x = W.decode_paged_inputs(seed, B, g * Hkv, Hkv, d, 16, 1, cap, lengths=[L + 1 for L in APPEND_LENS])
    else:
        x = W.decode_contiguous_inputs(seed, B, g * Hkv, Hkv, cap, d, seq_lens=APPEND_LENS)
    cached = torch.tensor(APPEND_LENS, dtype=torch.int32)
    kn, vn = W.decode_new_rows(seed + 1, B, Hkv, d)
    kc, vc, sl = dev(x.k_cache), dev(x.v_cache), dev(cached)
    o, lse = attn.decode_append(dev(x.q), dev(kn), dev(vn), kc, vc, dev(x.block_table), sl, x.page_size,
                                x.max_blocks, x.scale, chunk)
    torch.cuda.synchronize()
    ro, rl, rk, rv = oracle.decode_append(x.q, kn, vn, x.k_cache, x.v_cache, x.block_table, cached, x.scale,
                                          x.page_size, x.max_blocks)
    check("append g=%d d=%d paged=%d chunk=%d" % (g, d, paged, chunk), o, lse, ro, rl, BF16_TOL)
    assert np.array_equal(kc.cpu().double().numpy(), rk), "K cache after the append differs"
    assert np.array_equal(vc.cpu().double().numpy(), rv), "V cache after the append differs"
    assert torch.equal(sl.cpu(), cached), "cache_seqlens must be left to the caller"


def test_decode_append_full_cache_uses_last_slot(attn):
    """A length at or past the capacity is clamped: the new rows replace the last slot."""
    say("case: decode append into a full cache")
    lens = [64, 500, 63]
    x = W.decode_contiguous_inputs(41, 3, 8, 2, 64, 128, seq_lens=[64, 64, 63])
    cached = torch.tensor(lens, dtype=torch.int32)
    kn, vn = W.decode_new_rows(42, 3, 2, 128)
    kc, vc = dev(x.k_cache), dev(x.v_cache)
    o, lse = attn.decode_append(dev(x.q), dev(kn), dev(vn), kc, vc, None, dev(cached), x.page_size, x.max_blocks,
                                x.scale, 16)
    torch.cuda.synchronize()
    ro, rl, rk, rv = oracle.decode_append(x.q, kn, vn, x.k_cache, x.v_cache, None, cached, x.scale, x.page_size,
                                          x.max_blocks)
    check("append full cache", o, lse, ro, rl, BF16_TOL)
    assert np.array_equal(kc.cpu().double().numpy(), rk) and np.array_equal(vc.cpu().double().numpy(), rv)


# ------------------------------------------------------------------ packed variable-length prefill
VARLEN_LENS = [1, 7, 0, 128, 129, 300, 1000, 2047]


def run_varlen(attn, x):
    o, lse = attn.prefill_varlen(dev(x.q), dev(x.k), dev(x.v), dev(x.cu_seqlens), x.max_seqlen, x.causal, x.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_varlen_bf16(attn, d, causal):
    say("case: varlen bf16 d=%d causal=%s" % (d, causal))
    x = W.prefill_packed_inputs(900 + d + causal, VARLEN_LENS, 8, 2, d, W.BF16, causal=causal)
    o, lse = run_varlen(attn, x)
    ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, causal, x.scale)
    check("varlen bf16 d=%d causal=%d" % (d, causal), o, lse, ro, rl, BF16_TOL)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_varlen_f32(attn, d):
    say("case: varlen f32 d=%d" % d)
    x = W.prefill_packed_inputs(950 + d, [1, 33, 0, 64, 65, 200], 4, 4, d, W.F32)
    o, lse = run_varlen(attn, x)
    ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, True, x.scale)
    check("varlen f32 d=%d" % d, o, lse, ro, rl, F32_TOL)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_varlen_key_split(attn, d):
    """A packed batch small enough for the key-split instantiation (at most 512 query
    tiles of 128 rows: 16 tiles x 8 sequences x 4 heads): most of its 64-row work items
    lie past their sequence's end and exit, the others split their key walks in two."""
    lens = [0, 1, 63, 64, 65, 700, 2047, 1300]
    say("case: varlen key split d=%d lengths=%s" % (d, lens))
    x = W.prefill_packed_inputs(970 + d, lens, 4, 2, d, W.BF16)
    o, lse = run_varlen(attn, x)
    ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, True, x.scale)
    check("varlen key split d=%d" % d, o, lse, ro, rl, BF16_TOL)


def test_prefill_varlen_one_sequence_equals_padded(attn):
    """A packed batch of one sequence runs the same arithmetic as the padded layout,
    so the outputs agree bit for bit."""
    say("case: varlen single sequence vs padded")
    x = W.prefill_inputs(960, 1, 8, 2, 777, 128, W.BF16)
    o_p, lse_p = run_prefill(attn, x)
    q = x.q[0].transpose(0, 1).contiguous()  # [N, Hq, d]
    k = x.k[0].transpose(0, 1).contiguous()
    v = x.v[0].transpose(0, 1).contiguous()
    cu = torch.tensor([0, 777], dtype=torch.int32)
    o, lse = attn.prefill_varlen(dev(q), dev(k), dev(v), dev(cu), 777, True, x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.transpose(0, 1).cpu(), o_p[0].cpu())
    assert torch.equal(lse.cpu(), lse_p[0].cpu())


# ------------------------------------------------------------------ decode without the LSE output
@pytest.mark.parametrize("paged", [False, True])
def test_decode_without_lse_output(attn, paged):
    """lse_or_null = NULL: the combine writes O only.  O matches the oracle and is bit for
    bit the O of the same call with an LSE buffer (the same kernels and partials)."""
    say("case: decode with lse NULL paged=%s" % paged)
    lens = [1, 700, 513, 0, 2048]
    if paged:
        x = W.decode_paged_inputs(811, len(lens), 28, 4, 128, 16, 1, 2048, lengths=lens)
    else:
        x = W.decode_contiguous_inputs(812, len(lens), 28, 4, 2048, 128, seq_lens=lens)
    q, kc, vc, bt, sl = dev(x.q), dev(x.k_cache), dev(x.v_cache), dev(x.block_table), dev(x.seq_lens)
    ws = torch.empty(attn.attn_decode_workspace_bytes(len(lens), 28, 4, 128, x.page_size, x.max_blocks, 0),
                     dtype=torch.uint8, device="cuda")
    o1 = torch.full_like(q, float("nan"))
    attn.attn_decode(q, kc, vc, bt, sl, o1, None, x.page_size, x.max_blocks, x.scale, 0, ws)
    o2 = torch.empty_like(q)
    l2 = torch.empty(len(lens), 28, dtype=torch.float32, device="cuda")
    attn.attn_decode(q, kc, vc, bt, sl, o2, l2, x.page_size, x.max_blocks, x.scale, 0, ws)
    torch.cuda.synchronize()
    ro, rl = oracle_decode(x)
    so = stats(o1.float().cpu().numpy(), ro)
    say("decode lse NULL paged=%d: O max_abs=%.3e rms=%.3e" % (paged, so["max_abs"], so["rms"]))
    assert so["max_abs"] <= BF16_TOL["o"], so
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("N,causal", [(2000, True), (1111, False)])
def test_prefill_key_split_odd_tile_counts(attn, N, causal):
    """Short prompts run the key-split instantiation (two wave groups per query tile,
    each over half of its key tiles, merged by the combine rule).  With N = 2000 the
    last query tile has 63 key tiles (causal), with N = 1111 every tile has 35
    (full): the second group's last tile lies wholly past the diagonal or past N."""
    say("case: key-split prefill N=%d causal=%s" % (N, causal))
    x = W.prefill_inputs(1300 + N, 1, 28, 4, N, 128, W.BF16, causal=causal)
    o, lse = run_prefill(attn, x)
    ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale)
    check("key split N=%d causal=%d" % (N, causal), o, lse, ro, rl, BF16_TOL)
