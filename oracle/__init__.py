"""Exact-attention oracle (fp64, CPU) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The GPU library and its Python
binding never import, load or call it, and it shares no code with them.

The arithmetic lives in ``oracle.c`` (plain C, double precision), which follows
the pofe.ai page "FlashAttention for inference: tiled prefill and split-KV
decoding": the plain definition of attention (section "The bottleneck it
attacks"), the online-softmax update and the combine rule (section "The online
softmax, with every symbol defined"), the tiled prefill loop (section "Prefill:
tiles, loop order and the tensor cores") and split-KV decoding over a paged cache
(section "Decode: a different bottleneck").  This module only builds the C file,
converts arrays to contiguous float64 and calls it.

Parity status: every function here is pinned by CPU tests against values the
page prints (its worked example), closed forms, a library routine (PyTorch's
float64 ``scaled_dot_product_attention`` and ``logsumexp``) and invariances; see
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        dbl = ctypes.c_double
        lib.oracle_prefill.argtypes = [P, P, P, P, P, i, i, i, i, i, i, dbl, i]
        lib.oracle_prefill_ext.argtypes = [P, P, P, P, P, i, i, i, i, i, i, dbl, i, dbl, i]
        lib.oracle_decode_ext.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i, dbl, i, dbl]
        lib.oracle_prefill_tiled.argtypes = [P, P, P, P, P, i, i, i, i, i, i, dbl, i, i]
        lib.oracle_decode.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i, dbl]
        lib.oracle_split_decode.argtypes = [P, P, P, P, P, P, P, i, i, i, i, i, i, dbl, i, i, P, P]
        lib.oracle_lse_combine.argtypes = [P, P, P, i, i, i, P, P]
        lib.oracle_online_trace.argtypes = [P, P, i, i, P, P, P, P, P, P]
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.argtypes = [i]
        lib.oracle_threads_used.argtypes = []
        lib.oracle_e4m3_decode.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_e4m3_decode.restype = ctypes.c_int
        for f in (lib.oracle_prefill, lib.oracle_prefill_ext, lib.oracle_decode_ext,
                  lib.oracle_prefill_tiled, lib.oracle_decode,
                  lib.oracle_split_decode, lib.oracle_lse_combine, lib.oracle_online_trace,
                  lib.oracle_num_threads, lib.oracle_set_num_threads, lib.oracle_threads_used):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Contiguous float64 copy/view of an array-like (torch tensors included)."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def threads_used() -> int:
    """Threads one of the oracle's parallel regions actually runs with."""
    return int(_load().oracle_threads_used())


def set_num_threads(n: int) -> int:
    """Use n OpenMP threads from now on (n > 0); returns the count in effect."""
    return int(_load().oracle_set_num_threads(int(n)))


def prefill(q, k, v, causal: bool, scale: float, row_step: int = 1, window: int = -1, softcap: float = 0.0):
    """Plain-definition prefill.  q: [B,Hq,N,d]; k, v: [B,Hkv,N,d].

    Returns (o [B,Hq,N,d], lse [B,Hq,N]) in float64.  With row_step > 1 only rows
    i with i % row_step == 0 are computed; the rest are NaN.  window >= 0: row i
    also needs j >= i - window (sliding window); softcap > 0: every score s
    becomes softcap * tanh(s / softcap) before the softmax.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == k.shape
    o = np.full_like(q, np.nan)
    lse = np.full((B, Hq, N), np.nan)
    rc = _load().oracle_prefill_ext(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Hq, Hkv, N, d,
                                    int(bool(causal)), float(scale), int(window), float(softcap),
                                    int(row_step))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return o, lse


def prefill_varlen(q, k, v, cu_seqlens, causal: bool, scale: float, window: int = -1, softcap: float = 0.0):
    """Prefill of a packed batch without padding (the variable-length interface of the
    pofe.ai page, section "Interaction with post-trained models"): sequence b is tokens
    cu_seqlens[b] .. cu_seqlens[b+1]-1 of q [T, Hq, d], k, v [T, Hkv, d] and attends
    only to itself; each sequence is the plain prefill above.  Returns (o [T, Hq, d],
    lse [Hq, T]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = _i32(cu_seqlens)
    T, Hq, d = q.shape
    o = np.full_like(q, np.nan)
    lse = np.full((Hq, T), np.nan)
    for b in range(cu.shape[0] - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 <= s0:
            continue
        ob, lb = prefill(q[s0:s1].transpose(1, 0, 2)[None], k[s0:s1].transpose(1, 0, 2)[None],
                         v[s0:s1].transpose(1, 0, 2)[None], causal, scale, window=window, softcap=softcap)
        o[s0:s1] = ob[0].transpose(1, 0, 2)
        lse[:, s0:s1] = lb[0]
    return o, lse


def prefill_tiled(q, k, v, causal: bool, scale: float, br: int, bc: int):
    """The pages' tiled online-softmax prefill with Br x Bc tiles (same layouts)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    o = np.full_like(q, np.nan)
    lse = np.full((B, Hq, N), np.nan)
    rc = _load().oracle_prefill_tiled(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Hq, Hkv, N, d,
                                      int(bool(causal)), float(scale), int(br), int(bc))
    if rc != 0:
        raise ValueError("oracle_prefill_tiled rejected its arguments")
    return o, lse


def decode(q, k_cache, v_cache, block_table, seq_lens, scale: float, page_size: int,
           max_blocks: int, window: int = -1, softcap: float = 0.0):
    """Plain-definition decode.  q: [B,Hq,d].  Cache [nblk,P,Hkv,d] with a block table
    [B,max_blocks], or contiguous [B,S,Hkv,d] when block_table is None (S = max_blocks*P).
    The query is token seq_lens[b] - 1; window >= 0 limits it to keys
    seq_lens[b] - 1 - window ..; softcap as in prefill.
    Returns (o [B,Hq,d], lse [B,Hq]) in float64."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, d = q.shape
    Hkv = kc.shape[-2]
    bt = None if block_table is None else _i32(block_table)
    sl = _i32(seq_lens)
    o = np.full_like(q, np.nan)
    lse = np.full((B, Hq), np.nan)
    rc = _load().oracle_decode_ext(_p(q), _p(kc), _p(vc), _p(bt), _p(sl), _p(o), _p(lse), B, Hq,
                                   Hkv, d, int(page_size), int(max_blocks), float(scale), int(window),
                                   float(softcap))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return o, lse


def decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, scale: float,
                  page_size: int, max_blocks: int, window: int = -1, softcap: float = 0.0):
    """Decode step with the new token appended in place first (pofe.ai page, section
    "Minimal implementation": the cache and block table take the new keys and values,
    cache_seqlens counts the tokens already cached).  The new rows k_new, v_new
    [B, Hkv, d] go to token t = cache_seqlens[b] of sequence b -- slot t % P of page
    block_table[b][t // P], or row t of a contiguous cache -- and the query attends
    t + 1 tokens.  t is clamped into [0, capacity - 1], the library's reading for a
    value outside the cache.  Returns (o, lse, k_cache_after, v_cache_after) in
    float64; the arguments are not modified."""
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    kn, vn = _f64(k_new), _f64(v_new)
    sl = _i32(cache_seqlens)
    bt = None if block_table is None else _i32(block_table)
    cap = int(max_blocks) * int(page_size)
    t_new = np.clip(sl.astype(np.int64), 0, cap - 1)
    for b in range(sl.shape[0]):
        t = int(t_new[b])
        if bt is None:
            kc[b, t] = kn[b]
            vc[b, t] = vn[b]
        else:
            page = int(bt[b, t // page_size])
            kc[page, t % page_size] = kn[b]
            vc[page, t % page_size] = vn[b]
    o, lse = decode(q, kc, vc, bt, (t_new + 1).astype(np.int32), scale, page_size, max_blocks, window=window,
                    softcap=softcap)
    return o, lse, kc, vc


def split_decode(q, k_cache, v_cache, block_table, seq_lens, scale: float, page_size: int,
                 max_blocks: int, chunk: int, block: int = 64, return_parts: bool = False):
    """The pages' split-KV decode: per-chunk online softmax, then the combine rule."""
    q, kc, vc = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, d = q.shape
    Hkv = kc.shape[-2]
    bt = None if block_table is None else _i32(block_table)
    sl = _i32(seq_lens)
    o = np.full_like(q, np.nan)
    lse = np.full((B, Hq), np.nan)
    max_chunks = -(-(max_blocks * page_size) // chunk)
    op = lp = None
    if return_parts:
        op = np.full((B * Hq, max_chunks, d), np.nan)
        lp = np.full((B * Hq, max_chunks), np.nan)
    rc = _load().oracle_split_decode(_p(q), _p(kc), _p(vc), _p(bt), _p(sl), _p(o), _p(lse),
                                     B, Hq, Hkv, d, int(page_size), int(max_blocks),
                                     float(scale), int(chunk), int(block), _p(op), _p(lp))
    if rc != 0:
        raise ValueError("oracle_split_decode rejected its arguments")
    if return_parts:
        return o, lse, op, lp
    return o, lse


def lse_combine(o_parts, lse_parts, n_splits=None):
    """Combine rule.  o_parts [rows, S, d], lse_parts [rows, S] -> (o [rows,d], lse [rows])."""
    op, lp = _f64(o_parts), _f64(lse_parts)
    rows, S, d = op.shape
    ns = None if n_splits is None else _i32(n_splits)
    o = np.full((rows, d), np.nan)
    lse = np.full((rows,), np.nan)
    rc = _load().oracle_lse_combine(_p(op), _p(lp), _p(ns), rows, S, d, _p(o), _p(lse))
    if rc != 0:
        raise ValueError("oracle_lse_combine rejected its arguments")
    return o, lse


def online_trace(scores, values, block: int):
    """Online update on one row with given scores and scalar values.

    Returns dict with per-block m, l, o_tilde, c and the final o, lse."""
    s, v = _f64(scores), _f64(values)
    n = s.shape[0]
    nb = max(1, -(-n // block))
    m, l, ot, c = (np.zeros(nb) for _ in range(4))
    o = np.zeros(1)
    lse = np.zeros(1)
    cnt = _load().oracle_online_trace(_p(s), _p(v), n, int(block), _p(m), _p(l), _p(ot), _p(c),
                                      _p(o), _p(lse))
    if cnt < 0:
        raise ValueError("oracle_online_trace rejected its arguments")
    return {"m": m[:cnt], "l": l[:cnt], "o_tilde": ot[:cnt], "c": c[:cnt],
            "o": float(o[0]), "lse": float(lse[0])}


def _u8(a) -> np.ndarray:
    """Contiguous uint8 view of byte codes (torch float8 / uint8 tensors or arrays)."""
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if a.dtype != __import__("torch").uint8:
            a = a.view(__import__("torch").uint8)
        a = a.numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def e4m3_decode(codes) -> np.ndarray:
    """FP8 E4M3 (OCP, finite-only variant) byte codes -> float64 values, from the
    format definition in oracle.c (NaN for the two NaN codes)."""
    c = _u8(codes)
    out = np.empty(c.shape, dtype=np.float64)
    if _load().oracle_e4m3_decode(_p(c), _p(out), c.size) != 0:
        raise ValueError("oracle_e4m3_decode rejected its arguments")
    return out


def prefill_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal: bool, scale: float, row_step: int = 1,
                window: int = -1, softcap: float = 0.0):
    """Attention on FP8 inputs: the plain prefill of the dequantised tensors.

    q8 [B, Hq, N, d], k8, v8 [B, Hkv, N, d] are E4M3 byte codes; descale_* are
    [B, Hkv] float factors (None = 1), shared by the query heads of one KV head:
    Q = descale_q[b, h / g] * decode(q8), K and V likewise.  The result is
    prefill(Q, K, V, causal, scale) in float64 -- what the method computes on the
    dequantised inputs, with no rounding of the probabilities.  window / softcap are
    those of prefill (the cap acts on the scaled score scale * <Q, K>)."""
    q, k, v = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv

    def ds(x):
        return np.ones((B, Hkv)) if x is None else _f64(x).reshape(B, Hkv)
    dq, dk, dv = ds(descale_q), ds(descale_k), ds(descale_v)
    q = q * np.repeat(dq, g, axis=1)[:, :, None, None]
    k = k * dk[:, :, None, None]
    v = v * dv[:, :, None, None]
    return prefill(q, k, v, causal, scale, row_step=row_step, window=window, softcap=softcap)


def prefill_fp8_varlen(q8, k8, v8, descale_q, descale_k, descale_v, cu_seqlens, causal: bool, scale: float,
                       window: int = -1, softcap: float = 0.0):
    """FP8 inputs in the packed layout: q8 [T, Hq, d], k8, v8 [T, Hkv, d] E4M3 codes;
    sequence b (tokens cu_seqlens[b] .. cu_seqlens[b+1]-1) reads its own descales
    descale_*[b, hk] (None = 1) for KV head hk and the query heads that share it.
    The dequantised packed tensors then go through prefill_varlen above.  Returns
    (o [T, Hq, d], lse [Hq, T]) in float64."""
    q, k, v = e4m3_decode(q8), e4m3_decode(k8), e4m3_decode(v8)
    cu = _i32(cu_seqlens)
    B = cu.shape[0] - 1
    Hq, Hkv = q.shape[1], k.shape[1]
    g = Hq // Hkv

    def ds(x):
        return np.ones((B, Hkv)) if x is None else _f64(x).reshape(B, Hkv)
    dq, dk, dv = ds(descale_q), ds(descale_k), ds(descale_v)
    for b in range(B):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        q[s0:s1] *= np.repeat(dq[b], g)[None, :, None]
        k[s0:s1] *= dk[b][None, :, None]
        v[s0:s1] *= dv[b][None, :, None]
    return prefill_varlen(q, k, v, cu, causal, scale, window=window, softcap=softcap)


def decode_fp8(q, k_cache8, v_cache8, descale_k, descale_v, block_table, seq_lens, scale: float,
               page_size: int, max_blocks: int, window: int = -1, softcap: float = 0.0):
    """Decode over an E4M3 cache: sequence b reads descale_k[b, hk] * decode(k8) and
    descale_v[b, hk] * decode(v8) for KV head hk (None = 1), then the plain decode
    (with decode's window and soft-cap, the cap acting on scale * <q, K>)."""
    k, v = e4m3_decode(k_cache8), e4m3_decode(v_cache8)
    qq = _f64(q)
    B, Hkv = qq.shape[0], k.shape[-2]

    def ds(x):
        return np.ones((B, Hkv)) if x is None else _f64(x).reshape(B, Hkv)
    dk, dv = ds(descale_k), ds(descale_v)
    sl = _i32(seq_lens)
    bt = None if block_table is None else _i32(block_table)
    o = np.empty(qq.shape)
    lse = np.empty(qq.shape[:2])
    for b in range(B):
        if bt is None:  # contiguous [B, S, Hkv, d]: this sequence's rows only
            kb = k[b:b + 1] * dk[b][None, None, :, None]
            vb = v[b:b + 1] * dv[b][None, None, :, None]
            ob, lb = decode(qq[b:b + 1], kb, vb, None, sl[b:b + 1], scale, page_size, max_blocks, window, softcap)
        else:  # paged pool [pages, P, Hkv, d] through this sequence's table row
            kb = k * dk[b][None, None, :, None]
            vb = v * dv[b][None, None, :, None]
            ob, lb = decode(qq[b:b + 1], kb, vb, bt[b:b + 1], sl[b:b + 1], scale, page_size, max_blocks, window,
                            softcap)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse


def decode_fp8_append(q, k_new8, v_new8, k_cache8, v_cache8, descale_k, descale_v, block_table, cache_seqlens,
                      scale: float, page_size: int, max_blocks: int):
    """Decode over an E4M3 cache with the new token appended in place first (pofe.ai
    page, section "Minimal implementation", on the 8-bit cache of decode_fp8): the new
    rows' codes k_new8, v_new8 [B, Hkv, d] go to token t = cache_seqlens[b] of sequence
    b (slot t % P of page block_table[b][t // P], or row t of a contiguous cache), t
    clamped into [0, capacity - 1], and the query attends t + 1 tokens of the cache
    with its per-(sequence, KV head) descales.  Returns (o, lse, k_cache8_after,
    v_cache8_after); the arguments are not modified."""
    kc, vc = _u8(k_cache8).copy(), _u8(v_cache8).copy()
    kn, vn = _u8(k_new8), _u8(v_new8)
    sl = _i32(cache_seqlens)
    bt = None if block_table is None else _i32(block_table)
    cap = int(max_blocks) * int(page_size)
    t_new = np.clip(sl.astype(np.int64), 0, cap - 1)
    for b in range(sl.shape[0]):
        t = int(t_new[b])
        if bt is None:
            kc[b, t] = kn[b]
            vc[b, t] = vn[b]
        else:
            page = int(bt[b, t // page_size])
            kc[page, t % page_size] = kn[b]
            vc[page, t % page_size] = vn[b]
    o, lse = decode_fp8(q, kc, vc, descale_k, descale_v, bt, (t_new + 1).astype(np.int32), scale, page_size,
                        max_blocks)
    return o, lse, kc, vc
