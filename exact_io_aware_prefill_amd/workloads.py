"""Seeded synthetic inputs for the attention path (no attention arithmetic here).

Both the GPU library's tests/benchmark and the fp64 oracle consume exactly the
arrays produced here, so an error measures the kernel, not the input cast.

Recipe (stands in for the activations of the model the pages serve; no weights,
prompts or datasets are involved):
  * values are drawn with numpy ``default_rng(seed)`` (PCG64) ``standard_normal``
    in float64, cast to float32, and for bf16 workloads rounded to bfloat16
    (round to nearest even, done by PyTorch's CPU cast);
  * draw order: Q, then K, then V (prefill and contiguous decode); for the paged
    decode workload: Q, sequence lengths, page permutation, K pool, V pool;
  * big tensors are drawn one head-slab at a time from the same generator, which
    yields the same stream as one large draw while bounding host memory.

Layouts (all contiguous, row-major):
  prefill      q, o: [B, Hq, N, d]      k, v: [B, Hkv, N, d]
  decode       q, o: [B, Hq, d]
               contiguous cache  k, v: [B, S, Hkv, d]
               paged cache       k, v: [num_pages, page_size, Hkv, d]
               block_table int32 [B, max_blocks] (unused slots = -1), seq_lens int32 [B]
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

_SLAB = 1 << 22  # values per draw (32 MiB of float64)


def _draw(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    """N(0,1) draw of `shape`, float64 -> float32 (-> bfloat16 RNE), as a CPU tensor."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=torch.float32 if dtype == F32 else torch.bfloat16)
    pos = 0
    while pos < n:
        m = min(_SLAB, n - pos)
        x = rng.standard_normal(m).astype(np.float32)
        out[pos:pos + m] = torch.from_numpy(x).to(out.dtype)
        pos += m
    return out.view(*shape)


@dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    causal: bool
    scale: float
    dtype: str


def prefill_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str,
                   causal: bool = True, scale: Optional[float] = None) -> PrefillInputs:
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, N, d), dtype)
    k = _draw(rng, (B, Hkv, N, d), dtype)
    v = _draw(rng, (B, Hkv, N, d), dtype)
    return PrefillInputs(q, k, v, causal, 1.0 / math.sqrt(d) if scale is None else scale, dtype)


@dataclass
class PackedPrefillInputs:
    q: torch.Tensor           # [T, Hq, d]
    k: torch.Tensor           # [T, Hkv, d]
    v: torch.Tensor
    cu_seqlens: torch.Tensor  # [B + 1] int32
    max_seqlen: int
    causal: bool
    scale: float
    dtype: str


def prefill_packed_inputs(seed: int, lens, Hq: int, Hkv: int, d: int, dtype: str, causal: bool = True,
                          scale: Optional[float] = None) -> PackedPrefillInputs:
    """A packed batch of sequences with the given lengths (draw order: Q, K, V)."""
    lens = [int(x) for x in lens]
    T = sum(lens)
    rng = np.random.default_rng(seed)
    q = _draw(rng, (T, Hq, d), dtype)
    k = _draw(rng, (T, Hkv, d), dtype)
    v = _draw(rng, (T, Hkv, d), dtype)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    return PackedPrefillInputs(q, k, v, cu, max(lens) if lens else 0, causal,
                               1.0 / math.sqrt(d) if scale is None else scale, dtype)


@dataclass
class Fp8PrefillInputs:
    q8: torch.Tensor  # [B, Hq, N, d] float8_e4m3fn codes
    k8: torch.Tensor  # [B, Hkv, N, d]
    v8: torch.Tensor
    descale_q: torch.Tensor  # [B, Hkv] float32
    descale_k: torch.Tensor
    descale_v: torch.Tensor
    causal: bool
    scale: float


def _to_e4m3(x: torch.Tensor, descale: torch.Tensor, group: int) -> torch.Tensor:
    """x [B, H, N, d] float32 -> E4M3 codes of x / descale[b, h // group] (PyTorch's
    round-to-nearest conversion; |x| / descale <= 448 by construction)."""
    ds = descale.repeat_interleave(group, dim=1)[:, :, None, None]
    return (x / ds).to(torch.float8_e4m3fn)


def prefill_fp8_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, causal: bool = True,
                       scale: Optional[float] = None) -> Fp8PrefillInputs:
    """Q, K, V drawn as in prefill_inputs (float32), then quantised to E4M3 with one
    descale per (sequence, KV head): the group's largest magnitude maps to 448."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, N, d), F32)
    k = _draw(rng, (B, Hkv, N, d), F32)
    v = _draw(rng, (B, Hkv, N, d), F32)
    g = Hq // Hkv

    def descale(x):  # heads of one KV group are adjacent, so [B, Hkv, rest]
        return torch.clamp(x.abs().reshape(B, Hkv, -1).amax(dim=-1), min=1e-12) / 448.0
    dq, dk, dv = descale(q), descale(k), descale(v)
    return Fp8PrefillInputs(_to_e4m3(q, dq, g), _to_e4m3(k, dk, 1), _to_e4m3(v, dv, 1), dq.float(), dk.float(),
                            dv.float(), causal, 1.0 / math.sqrt(d) if scale is None else scale)


@dataclass
class Fp8PackedPrefillInputs:
    q8: torch.Tensor  # [T, Hq, d] E4M3 codes
    k8: torch.Tensor  # [T, Hkv, d]
    v8: torch.Tensor
    descale_q: torch.Tensor  # [B, Hkv] float32
    descale_k: torch.Tensor
    descale_v: torch.Tensor
    cu_seqlens: torch.Tensor  # [B + 1] int32
    max_seqlen: int
    causal: bool
    scale: float


def prefill_fp8_packed_inputs(seed: int, lens, Hq: int, Hkv: int, d: int, causal: bool = True,
                              scale: Optional[float] = None) -> Fp8PackedPrefillInputs:
    """The float32 draws of prefill_packed_inputs, quantised to E4M3 with one descale
    per (sequence, KV head): the largest magnitude of the sequence's rows of that KV
    head (and, for Q, of its query heads) maps to 448."""
    x = prefill_packed_inputs(seed, lens, Hq, Hkv, d, F32, causal, scale)
    lens = [int(n) for n in lens]
    B, g = len(lens), Hq // Hkv
    cu = x.cu_seqlens.tolist()
    dq, dk, dv = torch.ones(B, Hkv), torch.ones(B, Hkv), torch.ones(B, Hkv)
    q8 = torch.zeros(x.q.shape, dtype=torch.float8_e4m3fn)
    k8 = torch.zeros(x.k.shape, dtype=torch.float8_e4m3fn)
    v8 = torch.zeros(x.v.shape, dtype=torch.float8_e4m3fn)
    for b in range(B):
        s0, s1 = cu[b], cu[b + 1]
        if s1 <= s0:
            continue
        qs = x.q[s0:s1].reshape(s1 - s0, Hkv, g, d)  # the query heads of one KV head are adjacent
        dq[b] = torch.clamp(qs.abs().amax(dim=(0, 2, 3)), min=1e-12) / 448.0
        dk[b] = torch.clamp(x.k[s0:s1].abs().amax(dim=(0, 2)), min=1e-12) / 448.0
        dv[b] = torch.clamp(x.v[s0:s1].abs().amax(dim=(0, 2)), min=1e-12) / 448.0
        q8[s0:s1] = (qs / dq[b][None, :, None, None]).reshape(s1 - s0, Hq, d).to(torch.float8_e4m3fn)
        k8[s0:s1] = (x.k[s0:s1] / dk[b][None, :, None]).to(torch.float8_e4m3fn)
        v8[s0:s1] = (x.v[s0:s1] / dv[b][None, :, None]).to(torch.float8_e4m3fn)
    return Fp8PackedPrefillInputs(q8, k8, v8, dq.float(), dk.float(), dv.float(), x.cu_seqlens, x.max_seqlen,
                                  causal, x.scale)


def worked_example_inputs(d: int = 64) -> PrefillInputs:
    """The pofe.ai worked example (section "A worked example by hand": scores
    (2, 1, 4, 3), scalar values (1, 0, 2, -1)) embedded in a 4-token causal
    prefill: q_i = e0, k_j = s_j e0, v_j = value_j e0, scale 1, float32.
    Row 3 of the causal output is the page's example; rows 0..2 are its prefixes."""
    s = [2.0, 1.0, 4.0, 3.0]
    vals = [1.0, 0.0, 2.0, -1.0]
    q = torch.zeros(1, 1, 4, d, dtype=torch.float32)
    k = torch.zeros(1, 1, 4, d, dtype=torch.float32)
    v = torch.zeros(1, 1, 4, d, dtype=torch.float32)
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor(s)
    v[0, 0, :, 0] = torch.tensor(vals)
    return PrefillInputs(q, k, v, True, 1.0, F32)


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, d]
    k_cache: torch.Tensor      # [B, S, Hkv, d] or [num_pages, P, Hkv, d]
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor]  # int32 [B, max_blocks] or None (contiguous)
    seq_lens: torch.Tensor     # int32 [B]
    page_size: int
    max_blocks: int
    scale: float
    dtype: str


def decode_contiguous_inputs(seed: int, B: int, Hq: int, Hkv: int, S: int, d: int,
                             dtype: str = BF16, page_size: int = 16,
                             seq_lens: Optional[list] = None) -> DecodeInputs:
    """One query token per sequence over a contiguous [B, S, Hkv, d] cache."""
    assert S % page_size == 0
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, d), dtype)
    k = _draw(rng, (B, S, Hkv, d), dtype)
    v = _draw(rng, (B, S, Hkv, d), dtype)
    sl = torch.tensor(seq_lens if seq_lens is not None else [S] * B, dtype=torch.int32)
    return DecodeInputs(q, k, v, None, sl, page_size, S // page_size, 1.0 / math.sqrt(d), dtype)


def decode_paged_inputs(seed: int, B: int, Hq: int, Hkv: int, d: int, page_size: int,
                        len_min: int, len_max: int, dtype: str = BF16,
                        lengths: Optional[list] = None) -> DecodeInputs:
    """Paged cache: sequence b has L_b ~ U{len_min..len_max} tokens (or `lengths`),
    stored in ceil(L_b / page_size) pages of a shared pool; a seeded random
    permutation of the pool assigns logical page p of sequence b to physical
    page perm[off_b + p].  Unused block-table slots hold -1 (never read)."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, d), dtype)
    if lengths is None:
        lens = rng.integers(len_min, len_max + 1, size=B).astype(np.int64)
    else:
        lens = np.asarray(lengths, dtype=np.int64)
    pages = (lens + page_size - 1) // page_size
    pool = int(pages.sum())
    perm = rng.permutation(pool) if pool > 0 else np.zeros(0, dtype=np.int64)
    max_blocks = max(1, -(-len_max // page_size))
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    kc = _draw(rng, (max(pool, 1), page_size, Hkv, d), dtype)
    vc = _draw(rng, (max(pool, 1), page_size, Hkv, d), dtype)
    return DecodeInputs(q, kc, vc, torch.from_numpy(bt), torch.from_numpy(lens.astype(np.int32)),
                        page_size, max_blocks, 1.0 / math.sqrt(d), dtype)


def decode_paged_layout(seed: int, B: int, Hq: int, d: int, page_size: int, len_min: int, len_max: int):
    """The query, lengths and block table of decode_paged_inputs(seed, ...) without
    the cache contents: the same draws in the same order up to the page permutation,
    so the layout equals that workload's.  Returns (q [B, Hq, d] bf16, block_table
    [B, max_blocks] int32, seq_lens [B] int32, pool pages, max_blocks)."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, d), BF16)
    lens = rng.integers(len_min, len_max + 1, size=B).astype(np.int64)
    pages = (lens + page_size - 1) // page_size
    pool = int(pages.sum())
    perm = rng.permutation(pool) if pool > 0 else np.zeros(0, dtype=np.int64)
    max_blocks = max(1, -(-len_max // page_size))
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += int(pages[b])
    return q, torch.from_numpy(bt), torch.from_numpy(lens.astype(np.int32)), max(pool, 1), max_blocks


@dataclass
class Fp8DecodeInputs:
    q: torch.Tensor                      # [B, Hq, d] bf16
    k_cache8: torch.Tensor               # E4M3 codes, layout as DecodeInputs
    v_cache8: torch.Tensor
    descale_k: torch.Tensor              # [B, Hkv] float32
    descale_v: torch.Tensor
    block_table: Optional[torch.Tensor]
    seq_lens: torch.Tensor
    page_size: int
    max_blocks: int
    scale: float


def decode_fp8_inputs(seed: int, B: int, Hq: int, Hkv: int, d: int, lengths, capacity: int, paged: bool,
                      page_size: int = 16) -> Fp8DecodeInputs:
    """The float32 draws of decode_paged_inputs / decode_contiguous_inputs (q kept in
    bf16), with each sequence's cache rows quantised to E4M3 per KV head: the
    sequence's largest magnitude of that head maps to 448 (PyTorch's conversion)."""
    if paged:
        x = decode_paged_inputs(seed, B, Hq, Hkv, d, page_size, 1, capacity, dtype=F32, lengths=lengths)
    else:
        x = decode_contiguous_inputs(seed, B, Hq, Hkv, capacity, d, dtype=F32, page_size=page_size,
                                     seq_lens=lengths)
    kc, vc = x.k_cache.clone(), x.v_cache.clone()
    dk = torch.ones(B, Hkv); dv = torch.ones(B, Hkv)
    k8 = torch.zeros(kc.shape, dtype=torch.float8_e4m3fn)
    v8 = torch.zeros(vc.shape, dtype=torch.float8_e4m3fn)
    for b in range(B):
        L = int(x.seq_lens[b])
        if paged:
            pages = x.block_table[b, :-(-L // page_size)].long() if L > 0 else torch.zeros(0, dtype=torch.long)
            rows_k, rows_v = kc[pages], vc[pages]            # [np, P, Hkv, d]
        else:
            rows_k, rows_v = kc[b:b + 1, :max(L, 1)], vc[b:b + 1, :max(L, 1)]
        for h in range(Hkv):
            for src, ds in ((rows_k, dk), (rows_v, dv)):
                amax = float(src[..., h, :].abs().max()) if src.numel() else 0.0
                ds[b, h] = max(amax, 1e-12) / 448.0
        for h in range(Hkv):
            if paged:
                k8[pages, :, h] = (kc[pages, :, h] / dk[b, h]).to(torch.float8_e4m3fn)
                v8[pages, :, h] = (vc[pages, :, h] / dv[b, h]).to(torch.float8_e4m3fn)
            else:
                k8[b, :, h] = (kc[b, :, h] / dk[b, h]).clamp(-448, 448).to(torch.float8_e4m3fn)
                v8[b, :, h] = (vc[b, :, h] / dv[b, h]).clamp(-448, 448).to(torch.float8_e4m3fn)
    return Fp8DecodeInputs(x.q.to(torch.bfloat16), k8, v8, dk.float(), dv.float(), x.block_table, x.seq_lens,
                           x.page_size, x.max_blocks, x.scale)


def decode_new_rows(seed: int, B: int, Hkv: int, d: int, dtype: str = BF16):
    """The appended token's key and value rows [B, Hkv, d] (draw order: K, then V)."""
    rng = np.random.default_rng(seed)
    return _draw(rng, (B, Hkv, d), dtype), _draw(rng, (B, Hkv, d), dtype)


def decode_fp8_new_rows(seed: int, d: int, descale_k, descale_v):
    """The appended token's rows for an E4M3 cache: float32 draws [B, Hkv, d] (as
    decode_new_rows) quantised to E4M3 codes with the cache's per-(sequence, KV head)
    descales [B, Hkv] (code = value / descale, clamped to +-448, PyTorch's conversion)."""
    B, Hkv = descale_k.shape
    kn, vn = decode_new_rows(seed, B, Hkv, d, F32)
    k8 = (kn / descale_k[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    v8 = (vn / descale_v[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    return k8, v8


# --------------------------------------------------------------------------
# Named workloads: the pages' shapes (Qwen2.5-7B attention layout for prefill
# and single-sequence decode, Llama-3-8B layout for batched paged decode).
# --------------------------------------------------------------------------
PREFILL_SMALL_F32 = dict(name="prefill-causal-f32-b1-h1-n256-d64", seed=0, B=1, Hq=1, Hkv=1,
                         N=256, d=64, dtype=F32)
PREFILL_2K = dict(name="prefill-causal-bf16-b1-h28x4-n2048-d128", seed=2, B=1, Hq=28, Hkv=4,
                  N=2048, d=128, dtype=BF16)


def prefill_long(N: int) -> dict:
    assert N in (8192, 16384, 30720)
    return dict(name="prefill-causal-bf16-b1-h28x4-n%d-d128" % N, seed=3, B=1, Hq=28, Hkv=4,
                N=N, d=128, dtype=BF16)


DECODE_32K = dict(name="decode-splitkv-bf16-b1-h28x4-s32768-d128-chunk512", seed=4, B=1, Hq=28,
                  Hkv=4, S=32768, d=128, chunk=512)
DECODE_PAGED = dict(name="decode-paged-bf16-b32-h32x8-len1024to32768-d128-page16", seed=5, B=32,
                    Hq=32, Hkv=8, d=128, page_size=16, len_min=1024, len_max=32768, chunk=0)


def make_prefill(cfg: dict) -> PrefillInputs:
    return prefill_inputs(cfg["seed"], cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["d"],
                          cfg["dtype"])


def make_decode_32k(cfg: dict = DECODE_32K) -> DecodeInputs:
    return decode_contiguous_inputs(cfg["seed"], cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["d"])


def make_decode_paged(cfg: dict = DECODE_PAGED) -> DecodeInputs:
    return decode_paged_inputs(cfg["seed"], cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"],
                               cfg["page_size"], cfg["len_min"], cfg["len_max"])
