"""Seeded random prefill shapes against the fp64 oracle (pofe.ai page, section
"Prefill: tiles, loop order and the tensor cores": the tiled walk must give the exact
attention for any shape).  The draws cross the launcher's choices: the plain kernel,
the key split for grids of at most 512 query tiles, the one-wave d = 256 kernel on
small grids, the XCD placement when the (sequence, KV head) pairs divide 8, ragged
last tiles, causal or full masks, and the padded or packed layout with empty
sequences."""
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


def _random_case(seed):
    """Batch 1..3, KV heads 1/2/4/8, group 1/2/4/7, d 64/128/256, length 1..3000,
    causal or full, padded or packed (packed lengths 0..N, one of them N).  The work
    (batch x query heads x N^2 x d) stays below 2e10 so the oracle finishes in about
    a second."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7]))
    d = int(rng.choice([64, 128, 256]))
    causal = bool(rng.integers(0, 2))
    packed = bool(rng.integers(0, 2))
    N = int(rng.integers(1, 3001))
    N = max(1, min(N, int((2e10 / (B * g * Hkv * d)) ** 0.5)))
    lens = rng.integers(0, N + 1, size=B)
    lens[int(rng.integers(0, B))] = N
    return B, Hkv, g, d, N, causal, packed, lens.tolist()


@pytest.mark.parametrize("seed", list(range(24)))
def test_prefill_random_shapes(attn, seed):
    B, Hkv, g, d, N, causal, packed, lens = _random_case(seed)
    Hq = g * Hkv
    say("case: prefill random seed=%d B=%d Hq=%d Hkv=%d d=%d N=%d causal=%s packed=%s lens=%s"
        % (seed, B, Hq, Hkv, d, N, causal, packed, lens if packed else "-"))
    if packed:
        x = W.prefill_packed_inputs(6000 + seed, lens, Hq, Hkv, d, W.BF16, causal=causal)
        o, lse = attn.prefill_varlen(dev(x.q), dev(x.k), dev(x.v), dev(x.cu_seqlens), x.max_seqlen, causal, x.scale)
        torch.cuda.synchronize()
        ro, rl = oracle.prefill_varlen(x.q, x.k, x.v, x.cu_seqlens, causal, x.scale)
    else:
        x = W.prefill_inputs(6000 + seed, B, Hq, Hkv, N, d, W.BF16, causal=causal)
        o, lse = attn.prefill(dev(x.q), dev(x.k), dev(x.v), causal, x.scale)
        torch.cuda.synchronize()
        ro, rl = oracle.prefill(x.q, x.k, x.v, causal, x.scale)
    check("prefill random seed=%d" % seed, o, lse, ro, rl, BF16_TOL)
