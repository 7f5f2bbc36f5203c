"""ctypes binding to libattn.so (declared in include/attn.h), same entry-point names.

Argument marshalling only: tensors are passed as device pointers with their sizes
read from the tensor shapes, and the current PyTorch HIP stream is passed as the
stream.  Every step of the computation runs in the library's HIP kernels; there is
no other implementation behind these functions.  Importing this module raises if
the library has not been built (python -m exact_io_aware_prefill_amd.build).
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError("libattn.so is not built: run `python -m exact_io_aware_prefill_amd.build` "
                      "(hipcc for gfx950); there is no fallback implementation")
lib = ctypes.CDLL(_LIB_PATH)

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_GQA = -3
ATTN_ERR_UNSUPPORTED = -4
ATTN_ERR_WORKSPACE = -5
ATTN_ERR_ALIGN = -6
ATTN_ERR_HIP = -7
ATTN_ERR_SCRATCH = -8
ATTN_F32 = 0
ATTN_BF16 = 1

EXPORTS = ("attn_prefill", "attn_prefill_varlen", "attn_prefill_ext", "attn_prefill_fp8", "attn_prefill_fp8_varlen",
           "attn_prefill_fp8_ext",
           "attn_decode", "attn_decode_noalloc", "attn_decode_append", "attn_decode_ext", "attn_decode_fp8",
           "attn_decode_fp8_append", "attn_decode_fp8_ext",
           "attn_decode_chunk_tokens",
           "attn_decode_workspace_bytes", "attn_lse_combine", "attn_decode_check_tables", "attn_status_string")

_P = ctypes.c_void_p
_I = ctypes.c_int
lib.attn_prefill.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
lib.attn_prefill.restype = _I
lib.attn_prefill_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
lib.attn_prefill_varlen.restype = _I
lib.attn_prefill_ext.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                 ctypes.c_float, _P]
lib.attn_prefill_ext.restype = _I
lib.attn_prefill_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P]
lib.attn_prefill_fp8.restype = _I
lib.attn_prefill_fp8_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                        ctypes.c_float, _P]
lib.attn_prefill_fp8_varlen.restype = _I
lib.attn_prefill_fp8_ext.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                     ctypes.c_float, _P]
lib.attn_prefill_fp8_ext.restype = _I
lib.attn_decode_ext.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                ctypes.c_float, _I, _P, ctypes.c_size_t, _P]
lib.attn_decode_ext.restype = _I
lib.attn_decode_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P,
                                ctypes.c_size_t, _P]
lib.attn_decode_fp8.restype = _I
lib.attn_decode_fp8_append.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                       ctypes.c_float, _I, _P, ctypes.c_size_t, _P]
lib.attn_decode_fp8_append.restype = _I
lib.attn_decode_fp8_ext.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                    ctypes.c_float, _I, _P, ctypes.c_size_t, _P]
lib.attn_decode_fp8_ext.restype = _I
lib.attn_decode.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                            _I, _P, ctypes.c_size_t, _P]
lib.attn_decode.restype = _I
lib.attn_decode_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _P]
lib.attn_decode_noalloc.restype = _I
lib.attn_decode_append.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float,
                                   _I, _P, ctypes.c_size_t, _P]
lib.attn_decode_append.restype = _I
lib.attn_decode_check_tables.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P]
lib.attn_decode_check_tables.restype = _I
lib.attn_decode_chunk_tokens.argtypes = [_I, _I, _I, _I, _I]
lib.attn_decode_chunk_tokens.restype = _I
lib.attn_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I]
lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
lib.attn_lse_combine.argtypes = [_P, _P, _P, _I, _I, _I, _P, _I, _P, _P]
lib.attn_lse_combine.restype = _I
lib.attn_status_string.argtypes = [_I]
lib.attn_status_string.restype = ctypes.c_char_p
# measurement helpers of include/attn_bench.h (not part of the attention path)
BENCH_EXPORTS = ("attn_bench_stream_read", "attn_bench_empty")
lib.attn_bench_stream_read.argtypes = [_P, _P, ctypes.c_size_t, _I, _P, _P]
lib.attn_bench_stream_read.restype = _I
lib.attn_bench_empty.argtypes = [_P]
lib.attn_bench_empty.restype = _I


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (status %d)" % (where, attn_status_string(status), status))
        self.status = status


def attn_status_string(status: int) -> str:
    return lib.attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    return -1


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc: int, where: str):
    if rc != ATTN_OK:
        raise AttnError(rc, where)


def attn_prefill(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """q, o: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (bf16 or f32, contiguous, on the GPU);
    lse: [B, Hq, N] float32.  Writes o and lse."""
    B, Hq, N, d = q.shape
    rc = lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, N, Hq, k.shape[1], d,
                          _dtype_code(q), int(bool(causal)), float(scale), _stream(stream))
    _check(rc, "attn_prefill")


def attn_prefill_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, causal: bool, scale: float,
                        stream=None) -> None:
    """Packed batch: q, o [T, Hq, d]; k, v [T, Hkv, d]; lse [Hq, T] float32; cu_seqlens
    [B+1] int32 on the GPU; max_seqlen >= every sequence length.  Writes o and lse."""
    T, Hq, d = q.shape
    B = cu_seqlens.numel() - 1
    rc = lib.attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), B,
                                 int(max_seqlen), T, Hq, k.shape[1], d, _dtype_code(q), int(bool(causal)),
                                 float(scale), _stream(stream))
    _check(rc, "attn_prefill_varlen")


def attn_prefill_ext(q, k, v, o, lse, cu_seqlens, max_seqlen: int, causal: bool, scale: float,
                     window_left: int = -1, softcap: float = 0.0, stream=None) -> None:
    """attn_prefill (cu_seqlens None: q [B, Hq, N, d]) or attn_prefill_varlen (q [T, Hq, d],
    max_seqlen the longest sequence) with a sliding window (window_left >= 0: keys j >= i -
    window_left) and logit soft-capping (softcap > 0)."""
    if cu_seqlens is None:
        B, Hq, N, d = q.shape
        T, Hkv = 0, k.shape[1]
    else:
        T, Hq, d = q.shape
        B, N, Hkv = cu_seqlens.numel() - 1, int(max_seqlen), k.shape[1]
    rc = lib.attn_prefill_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), B, N, T, Hq, Hkv, d,
                              _dtype_code(q), int(bool(causal)), float(scale), int(window_left), float(softcap),
                              _stream(stream))
    _check(rc, "attn_prefill_ext")


def attn_prefill_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal: bool, scale: float,
                     stream=None) -> None:
    """q8 [B, Hq, N, d], k8, v8 [B, Hkv, N, d]: E4M3 codes (torch.float8_e4m3fn or uint8);
    o [B, Hq, N, d] bf16, lse [B, Hq, N] float32; descale_* [B, Hkv] float32 or None."""
    B, Hq, N, d = q8.shape
    rc = lib.attn_prefill_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), _ptr(descale_q), _ptr(descale_k),
                              _ptr(descale_v), B, N, Hq, k8.shape[1], d, int(bool(causal)), float(scale),
                              _stream(stream))
    _check(rc, "attn_prefill_fp8")


def attn_prefill_fp8_varlen(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, cu_seqlens, max_seqlen: int,
                            causal: bool, scale: float, stream=None) -> None:
    """Packed batch: q8 [T, Hq, d], k8, v8 [T, Hkv, d] E4M3 codes; o [T, Hq, d] bf16; lse [Hq, T]
    float32; descale_* [B, Hkv] float32 or None; cu_seqlens [B+1] int32 on the GPU."""
    T, Hq, d = q8.shape
    B = cu_seqlens.numel() - 1
    rc = lib.attn_prefill_fp8_varlen(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), _ptr(descale_q),
                                     _ptr(descale_k), _ptr(descale_v), _ptr(cu_seqlens), B, int(max_seqlen), T, Hq,
                                     k8.shape[1], d, int(bool(causal)), float(scale), _stream(stream))
    _check(rc, "attn_prefill_fp8_varlen")


def attn_prefill_fp8_ext(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, cu_seqlens, max_seqlen: int,
                         causal: bool, scale: float, window_left: int, softcap: float, stream=None) -> None:
    """attn_prefill_fp8 (cu_seqlens None: padded [B, H, N, d]) or attn_prefill_fp8_varlen (packed
    [T, H, d] with cu_seqlens) with a sliding window (-1: none) and a logit soft-cap (0: none)."""
    if cu_seqlens is None:
        B, Hq, N, d = q8.shape
        Hkv, T, seq = k8.shape[1], 0, N
    else:
        T, Hq, d = q8.shape
        B, Hkv, seq = cu_seqlens.numel() - 1, k8.shape[1], int(max_seqlen)
    rc = lib.attn_prefill_fp8_ext(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), _ptr(descale_q), _ptr(descale_k),
                                  _ptr(descale_v), _ptr(cu_seqlens), B, seq, T, Hq, Hkv, d, int(bool(causal)),
                                  float(scale), int(window_left), float(softcap), _stream(stream))
    _check(rc, "attn_prefill_fp8_ext")


def attn_decode_chunk_tokens(batch: int, n_kv_heads: int, page_size: int, max_blocks_per_seq: int,
                             chunk_tokens: int = 0) -> int:
    r = lib.attn_decode_chunk_tokens(batch, n_kv_heads, page_size, max_blocks_per_seq, chunk_tokens)
    _check(min(r, 0), "attn_decode_chunk_tokens")
    return r


def attn_decode_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                                page_size: int, max_blocks_per_seq: int, chunk_tokens: int = 0) -> int:
    return int(lib.attn_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, page_size,
                                               max_blocks_per_seq, chunk_tokens))


def attn_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, page_size: int,
                max_blocks_per_seq: int, scale: float, chunk_tokens: int, workspace,
                stream=None) -> None:
    """q, o: [B, Hq, d]; caches [num_pages, P, Hkv, d] with block_table [B, max_blocks] int32,
    or [B, S, Hkv, d] with block_table None; seq_lens [B] int32; lse [B, Hq] float32 or None;
    workspace: a uint8 device tensor of at least attn_decode_workspace_bytes(...) bytes."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[-2]
    rc = lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                         _ptr(o), _ptr(lse), B, Hq, Hkv, d, int(page_size), int(max_blocks_per_seq),
                         _dtype_code(q), float(scale), int(chunk_tokens), _ptr(workspace),
                         0 if workspace is None else workspace.numel() * workspace.element_size(),
                         _stream(stream))
    _check(rc, "attn_decode")


def attn_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, page_size: int,
                        max_blocks_per_seq: int, scale: float, chunk_tokens: int, stream=None) -> None:
    """attn_decode with the partials in the library's static per-GPU scratch
    (ATTN_DECODE_NOALLOC_SCRATCH_BYTES) instead of a caller workspace: no device
    memory is allocated.  Calls that overlap on one GPU race on that scratch."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[-2]
    rc = lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
                                 _ptr(o), _ptr(lse), B, Hq, Hkv, d, int(page_size), int(max_blocks_per_seq),
                                 _dtype_code(q), float(scale), int(chunk_tokens), _stream(stream))
    _check(rc, "attn_decode_noalloc")


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_DECODE_NOALLOC_SCRATCH_BYTES of include/attn.h


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, o, lse,
                       page_size: int, max_blocks_per_seq: int, scale: float, chunk_tokens: int, workspace,
                       stream=None) -> None:
    """attn_decode after writing k_new, v_new [B, Hkv, d] into the caches at token
    cache_seqlens[b] (the tokens already cached); the query attends cache_seqlens[b] + 1
    tokens.  cache_seqlens is not modified."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[-2]
    rc = lib.attn_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_table), _ptr(cache_seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv, d,
                                int(page_size), int(max_blocks_per_seq), _dtype_code(q), float(scale),
                                int(chunk_tokens), _ptr(workspace),
                                0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(rc, "attn_decode_append")


def attn_decode_ext(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, o, lse, page_size: int,
                    max_blocks_per_seq: int, scale: float, window_left: int, softcap: float, chunk_tokens: int,
                    workspace, stream=None) -> None:
    """attn_decode (k_new, v_new None) or attn_decode_append (both given) with a sliding
    window (the query, token L-1, sees tokens >= L-1-window_left) and logit soft-capping."""
    B, Hq, d = q.shape
    Hkv = k_cache.shape[-2]
    rc = lib.attn_decode_ext(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                             _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv, d, int(page_size),
                             int(max_blocks_per_seq), _dtype_code(q), float(scale), int(window_left),
                             float(softcap), int(chunk_tokens), _ptr(workspace),
                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check(rc, "attn_decode_ext")


def attn_decode_fp8(q, k_cache8, v_cache8, descale_k, descale_v, block_table, seq_lens, o, lse, page_size: int,
                    max_blocks_per_seq: int, scale: float, chunk_tokens: int, workspace, stream=None) -> None:
    """attn_decode over an E4M3 cache (torch.float8_e4m3fn or uint8 codes, layouts as
    attn_decode); descale_k, descale_v [B, Hkv] float32 or None; q, o bf16."""
    B, Hq, d = q.shape
    Hkv = k_cache8.shape[-2]
    rc = lib.attn_decode_fp8(_ptr(q), _ptr(k_cache8), _ptr(v_cache8), _ptr(descale_k), _ptr(descale_v),
                             _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv, d, int(page_size),
                             int(max_blocks_per_seq), float(scale), int(chunk_tokens), _ptr(workspace),
                             0 if workspace is None else workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check(rc, "attn_decode_fp8")


def attn_decode_fp8_append(q, k_new8, v_new8, k_cache8, v_cache8, descale_k, descale_v, block_table, cache_seqlens,
                           o, lse, page_size: int, max_blocks_per_seq: int, scale: float, chunk_tokens: int, workspace,
                           stream=None) -> None:
    """attn_decode_fp8 after writing the new token's E4M3 codes k_new8, v_new8 [B, Hkv, d]
    into the caches at token cache_seqlens[b]; the query attends cache_seqlens[b] + 1
    tokens.  cache_seqlens is not modified."""
    B, Hq, d = q.shape
    Hkv = k_cache8.shape[-2]
    rc = lib.attn_decode_fp8_append(_ptr(q), _ptr(k_new8), _ptr(v_new8), _ptr(k_cache8), _ptr(v_cache8),
                                    _ptr(descale_k), _ptr(descale_v), _ptr(block_table), _ptr(cache_seqlens), _ptr(o),
                                    _ptr(lse), B, Hq, Hkv, d, int(page_size), int(max_blocks_per_seq), float(scale),
                                    int(chunk_tokens), _ptr(workspace),
                                    0 if workspace is None else workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _check(rc, "attn_decode_fp8_append")


def attn_decode_fp8_ext(q, k_cache8, v_cache8, descale_k, descale_v, block_table, seq_lens, o, lse, page_size: int,
                        max_blocks_per_seq: int, scale: float, window_left: int, softcap: float, chunk_tokens: int,
                        workspace, stream=None) -> None:
    """attn_decode_fp8 with a sliding window (-1: none) and a logit soft-cap (0: none)."""
    B, Hq, d = q.shape
    Hkv = k_cache8.shape[-2]
    rc = lib.attn_decode_fp8_ext(_ptr(q), _ptr(k_cache8), _ptr(v_cache8), _ptr(descale_k), _ptr(descale_v),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv, d, int(page_size),
                                 int(max_blocks_per_seq), float(scale), int(window_left), float(softcap),
                                 int(chunk_tokens), _ptr(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _check(rc, "attn_decode_fp8_ext")


def decode_fp8(q, k_cache8, v_cache8, block_table, seq_lens, page_size: int, max_blocks_per_seq: int,
               descale_k=None, descale_v=None, scale: float | None = None, chunk_tokens: int = 0, stream=None,
               workspace=None, window_left: int = -1, softcap: float = 0.0):
    with _on(stream):
        B, Hq, d = q.shape
        Hkv = k_cache8.shape[-2]
        need = attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, max_blocks_per_seq, chunk_tokens)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_decode_fp8(q, k_cache8, v_cache8, descale_k, descale_v, block_table, seq_lens, o, lse, page_size,
                            max_blocks_per_seq, scale, chunk_tokens, workspace, stream)
        else:
            attn_decode_fp8_ext(q, k_cache8, v_cache8, descale_k, descale_v, block_table, seq_lens, o, lse, page_size,
                                max_blocks_per_seq, scale, window_left, softcap, chunk_tokens, workspace, stream)
        return o, lse


def decode_fp8_append(q, k_new8, v_new8, k_cache8, v_cache8, block_table, cache_seqlens, page_size: int,
                      max_blocks_per_seq: int, descale_k=None, descale_v=None, scale: float | None = None,
                      chunk_tokens: int = 0, stream=None, workspace=None):
    with _on(stream):
        B, Hq, d = q.shape
        Hkv = k_cache8.shape[-2]
        need = attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, max_blocks_per_seq, chunk_tokens)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        scale = d ** -0.5 if scale is None else scale
        attn_decode_fp8_append(q, k_new8, v_new8, k_cache8, v_cache8, descale_k, descale_v, block_table, cache_seqlens,
                               o, lse, page_size, max_blocks_per_seq, scale, chunk_tokens, workspace, stream)
        return o, lse


def attn_lse_combine(o_parts, lse_parts, n_splits, o, lse, stream=None) -> None:
    """o_parts [rows, S, d] f32; lse_parts [rows, S] f32; n_splits [rows] int32 or None;
    o [rows, d] (bf16 or f32); lse [rows] f32 or None."""
    rows, S, d = o_parts.shape
    rc = lib.attn_lse_combine(_ptr(o_parts), _ptr(lse_parts), _ptr(n_splits), rows, S, d, _ptr(o),
                              _dtype_code(o), _ptr(lse), _stream(stream))
    _check(rc, "attn_lse_combine")



def attn_decode_check_tables(block_table, seq_lens, page_size: int, max_blocks_per_seq: int, num_blocks: int,
                             appended: bool, bad_out, stream=None) -> None:
    """block_table [B, max_blocks] int32 or None; seq_lens [B] int32; bad_out: a one-element
    int32 device tensor, overwritten with the number of out-of-range lengths and used table
    entries (read it after synchronising)."""
    rc = lib.attn_decode_check_tables(_ptr(block_table), _ptr(seq_lens), int(seq_lens.shape[0]), int(page_size),
                                      int(max_blocks_per_seq), int(num_blocks), 1 if appended else 0, _ptr(bad_out),
                                      _stream(stream))
    _check(rc, "attn_decode_check_tables")

def attn_bench_stream_read(a, b, workgroups: int, sink, stream=None) -> None:
    """Read device tensors a and b (same byte size) once in one kernel on `workgroups`
    workgroups (the floor of a decode that reads them); sink: int32 tensor of at least
    4 * workgroups elements."""
    nbytes = a.numel() * a.element_size()
    assert b.numel() * b.element_size() == nbytes and sink.numel() >= 4 * workgroups
    rc = lib.attn_bench_stream_read(_ptr(a), _ptr(b), nbytes, int(workgroups), _ptr(sink), _stream(stream))
    if rc != 0:
        raise RuntimeError("attn_bench_stream_read failed (%d)" % rc)


def attn_bench_empty(stream=None) -> None:
    """One empty kernel: the cost of a further dependent launch."""
    rc = lib.attn_bench_empty(_stream(stream))
    if rc != 0:
        raise RuntimeError("attn_bench_empty failed (%d)" % rc)


# ---- conveniences that allocate outputs with PyTorch (allocation only) ----------
# Outputs and the decode workspace are allocated on the stream the kernels run on,
# so PyTorch's caching allocator orders any reuse of that memory (in particular of
# the temporary workspace, released when the function returns) after the launch.
def _plain(window_left, softcap) -> bool:
    return window_left == -1 and softcap == 0.0


def _on(stream):
    """Allocation context for a launch on `stream` (None: the current stream)."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def prefill(q, k, v, causal: bool = True, scale: float | None = None, stream=None, window_left: int = -1,
            softcap: float = 0.0):
    with _on(stream):
        B, Hq, N, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_prefill(q, k, v, o, lse, causal, scale, stream)
        else:
            attn_prefill_ext(q, k, v, o, lse, None, N, causal, scale, window_left, softcap, stream)
        return o, lse


def prefill_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = True, scale: float | None = None,
                   stream=None, window_left: int = -1, softcap: float = 0.0):
    with _on(stream):
        T, Hq, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_prefill_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen, causal, scale, stream)
        else:
            attn_prefill_ext(q, k, v, o, lse, cu_seqlens, max_seqlen, causal, scale, window_left, softcap, stream)
        return o, lse


def prefill_fp8(q8, k8, v8, descale_q=None, descale_k=None, descale_v=None, causal: bool = True,
                scale: float | None = None, stream=None, window_left: int = -1, softcap: float = 0.0):
    with _on(stream):
        B, Hq, N, d = q8.shape
        o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q8.device)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_prefill_fp8(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, causal, scale, stream)
        else:
            attn_prefill_fp8_ext(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, None, N, causal, scale, window_left,
                                 softcap, stream)
        return o, lse


def prefill_fp8_varlen(q8, k8, v8, cu_seqlens, max_seqlen: int, descale_q=None, descale_k=None, descale_v=None,
                       causal: bool = True, scale: float | None = None, stream=None, window_left: int = -1,
                       softcap: float = 0.0):
    with _on(stream):
        T, Hq, d = q8.shape
        o = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=q8.device)
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q8.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_prefill_fp8_varlen(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, cu_seqlens, max_seqlen, causal,
                                    scale, stream)
        else:
            attn_prefill_fp8_ext(q8, k8, v8, o, lse, descale_q, descale_k, descale_v, cu_seqlens, max_seqlen, causal,
                                 scale, window_left, softcap, stream)
        return o, lse


def decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, page_size: int,
                  max_blocks_per_seq: int, scale: float | None = None, chunk_tokens: int = 0, stream=None,
                  workspace=None, window_left: int = -1, softcap: float = 0.0):
    """Decode step with the new token's k_new, v_new [B, Hkv, d] written into the caches
    in place at token cache_seqlens[b]; returns (o, lse) over cache_seqlens[b] + 1 tokens."""
    with _on(stream):
        B, Hq, d = q.shape
        Hkv = k_cache.shape[-2]
        need = attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, max_blocks_per_seq, chunk_tokens)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, o, lse, page_size,
                               max_blocks_per_seq, scale, chunk_tokens, workspace, stream)
        else:
            attn_decode_ext(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, o, lse, page_size,
                            max_blocks_per_seq, scale, window_left, softcap, chunk_tokens, workspace, stream)
        return o, lse


def decode(q, k_cache, v_cache, block_table, seq_lens, page_size: int, max_blocks_per_seq: int,
           scale: float | None = None, chunk_tokens: int = 0, stream=None, workspace=None, window_left: int = -1,
           softcap: float = 0.0):
    with _on(stream):
        B, Hq, d = q.shape
        Hkv = k_cache.shape[-2]
        need = attn_decode_workspace_bytes(B, Hq, Hkv, d, page_size, max_blocks_per_seq, chunk_tokens)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        scale = d ** -0.5 if scale is None else scale
        if _plain(window_left, softcap):
            attn_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, page_size, max_blocks_per_seq, scale,
                        chunk_tokens, workspace, stream)
        else:
            attn_decode_ext(q, None, None, k_cache, v_cache, block_table, seq_lens, o, lse, page_size,
                            max_blocks_per_seq, scale, window_left, softcap, chunk_tokens, workspace, stream)
        return o, lse
