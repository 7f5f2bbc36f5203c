"""C-ABI boundary tests that need no GPU: the library loads, exports every entry
point include/attn.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented status codes."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

attn = pytest.importorskip("exact_io_aware_prefill_amd.attn",
                           reason="libattn.so not built (python -m exact_io_aware_prefill_amd.build)")

FAKE = 0x10000  # a 16-byte aligned, never dereferenced address
MIS = FAKE + 4  # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(attn_[a-z_0-9]+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(attn.EXPORTS)


BENCH_HEADER = os.path.join(ROOT, "include", "attn_bench.h")


def test_bench_header_declares_the_measurement_helpers():
    text = open(BENCH_HEADER).read()
    names = sorted(set(re.findall(r"^\s*int\s+(attn_bench_[a-z_0-9]+)\s*\(", text, flags=re.M)))
    assert names == sorted(attn.BENCH_EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", attn._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(attn_\w+)$", out, flags=re.M))
    assert set(names) <= exported
    # host-side argument checks, before any HIP call
    f = attn.lib.attn_bench_stream_read
    assert f(None, P(FAKE), 16, 1, P(FAKE), None) == -1
    assert f(P(FAKE), P(FAKE), 15, 1, P(FAKE), None) == -2
    assert f(P(FAKE), P(MIS), 16, 1, P(FAKE), None) == -2
    assert f(P(FAKE), P(FAKE), 16, 0, P(FAKE), None) == -2
    assert f(P(FAKE), P(FAKE), 0, 4, P(FAKE), None) == 0


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(attn.lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", attn._LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(attn_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name in ("ATTN_OK", "ATTN_ERR_NULL", "ATTN_ERR_SHAPE", "ATTN_ERR_GQA", "ATTN_ERR_UNSUPPORTED",
                 "ATTN_ERR_WORKSPACE", "ATTN_ERR_ALIGN", "ATTN_ERR_HIP", "ATTN_F32", "ATTN_BF16"):
        m = re.search(r"#define\s+%s\s+(-?\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(attn, name), name
    for code in range(-8, 1):
        s = attn.attn_status_string(code)
        assert s and s != "unknown status"
    assert attn.attn_status_string(-99) == "unknown status"


def P(x):
    return ctypes.c_void_p(x)


def prefill(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, N=16, Hq=4, Hkv=2, d=128, dtype=1, causal=1):
    return attn.lib.attn_prefill(P(q), P(k), P(v), P(o), P(lse), B, N, Hq, Hkv, d, dtype, causal,
                                 0.1, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(lse=0), attn.ATTN_ERR_NULL),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(N=-5), attn.ATTN_ERR_SHAPE),
    (dict(Hq=0), attn.ATTN_ERR_SHAPE),
    (dict(d=0), attn.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=512), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), attn.ATTN_ERR_UNSUPPORTED),
    (dict(k=MIS), attn.ATTN_ERR_ALIGN),
    (dict(o=MIS), attn.ATTN_ERR_ALIGN),
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0), attn.ATTN_OK),   # empty call: nothing to do
    (dict(N=0, q=0, k=0, v=0, o=0, lse=0), attn.ATTN_OK),
])
def test_prefill_argument_errors(kw, code):
    assert prefill(**kw) == code


def varlen(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, B=3, maxs=100, T=250, Hq=8, Hkv=2, d=128,
           dtype=1):
    return attn.lib.attn_prefill_varlen(P(q), P(k), P(v), P(o), P(lse), P(cu), B, maxs, T, Hq, Hkv, d, dtype,
                                        1, 0.1, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=0), attn.ATTN_ERR_NULL),
    (dict(lse=0), attn.ATTN_ERR_NULL),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(maxs=-1), attn.ATTN_ERR_SHAPE),
    (dict(T=-5), attn.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=3), attn.ATTN_ERR_UNSUPPORTED),
    (dict(cu=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(o=MIS), attn.ATTN_ERR_ALIGN),
    (dict(maxs=1 << 20, Hq=64, Hkv=8), attn.ATTN_ERR_UNSUPPORTED),   # a head's rows past 32-bit offsets
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0, cu=0), attn.ATTN_OK),
    (dict(T=0, q=0, k=0, v=0, o=0, lse=0, cu=0), attn.ATTN_OK),
])
def test_prefill_varlen_argument_errors(kw, code):
    assert varlen(**kw) == code


def prefill_ext(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=0, B=2, N=100, T=0, Hq=8, Hkv=2, d=128, dtype=1,
                causal=1, window=-1, cap=0.0):
    return attn.lib.attn_prefill_ext(P(q), P(k), P(v), P(o), P(lse), P(cu), B, N, T, Hq, Hkv, d, dtype, causal,
                                     0.1, window, cap, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-2), attn.ATTN_ERR_SHAPE),
    (dict(cap=-1.0), attn.ATTN_ERR_SHAPE),
    (dict(cap=float("inf")), attn.ATTN_ERR_SHAPE),
    (dict(cap=float("nan")), attn.ATTN_ERR_SHAPE),
    (dict(window=-2, q=0), attn.ATTN_ERR_SHAPE),          # option errors come before pointer checks
    (dict(q=0, window=3), attn.ATTN_ERR_NULL),
    (dict(lse=0, cap=30.0), attn.ATTN_ERR_NULL),
    (dict(Hq=6, Hkv=4, window=3), attn.ATTN_ERR_GQA),
    (dict(d=96, cap=5.0), attn.ATTN_ERR_UNSUPPORTED),
    (dict(o=MIS, window=0), attn.ATTN_ERR_ALIGN),
    (dict(cu=FAKE + 2, T=250), attn.ATTN_ERR_ALIGN),      # packed: cu_seqlens must be 4-byte aligned
    (dict(cu=FAKE, T=-1), attn.ATTN_ERR_SHAPE),           # packed: total_tokens >= 0
    (dict(cu=0, T=-1, q=0, window=5), attn.ATTN_ERR_NULL),  # padded: total_tokens is ignored
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0, window=7, cap=1.0), attn.ATTN_OK),
    (dict(cu=FAKE, T=0, q=0, k=0, v=0, o=0, lse=0), attn.ATTN_OK),
])
def test_prefill_ext_argument_errors(kw, code):
    assert prefill_ext(**kw) == code


def prefill_fp8(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dq=0, dk=0, dv=0, B=1, N=16, Hq=4, Hkv=2, d=128,
                causal=1):
    return attn.lib.attn_prefill_fp8(P(q), P(k), P(v), P(o), P(lse), P(dq), P(dk), P(dv), B, N, Hq, Hkv, d, causal,
                                     0.1, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(lse=0), attn.ATTN_ERR_NULL),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(N=-1), attn.ATTN_ERR_SHAPE),
    (dict(Hkv=0), attn.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=512), attn.ATTN_ERR_UNSUPPORTED),     # fp8 prefill: head sizes 64, 128 and 256
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(k=MIS), attn.ATTN_ERR_ALIGN),
    (dict(dv=FAKE + 2), attn.ATTN_ERR_ALIGN),     # descales are float arrays: 4-byte aligned
    (dict(dq=FAKE + 4, q=0), attn.ATTN_ERR_NULL),  # 4-byte aligned descale is fine; NULL q is not
    (dict(N=1 << 30), attn.ATTN_ERR_UNSUPPORTED),  # a head's rows past 32-bit offsets
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0), attn.ATTN_OK),
])
def test_prefill_fp8_argument_errors(kw, code):
    assert prefill_fp8(**kw) == code


def prefill_fp8_varlen(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dq=0, dk=0, dv=0, cu=FAKE, B=2, N=16, T=20, Hq=4,
                       Hkv=2, d=128, causal=1):
    return attn.lib.attn_prefill_fp8_varlen(P(q), P(k), P(v), P(o), P(lse), P(dq), P(dk), P(dv), P(cu), B, N, T, Hq,
                                            Hkv, d, causal, 0.1, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=0), attn.ATTN_ERR_NULL),
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(cu=FAKE + 2), attn.ATTN_ERR_ALIGN),      # cu_seqlens is int32: 4-byte aligned
    (dict(cu=FAKE + 4, q=0), attn.ATTN_ERR_NULL),  # 4-byte aligned offsets are fine; NULL q is not
    (dict(v=MIS), attn.ATTN_ERR_ALIGN),
    (dict(T=-1), attn.ATTN_ERR_SHAPE),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=512), attn.ATTN_ERR_UNSUPPORTED),
    (dict(N=1 << 24, Hq=32), attn.ATTN_ERR_UNSUPPORTED),  # a packed row holds all heads: 32-bit offsets
    (dict(T=0, q=0, k=0, v=0, o=0, lse=0, cu=0), attn.ATTN_OK),
    (dict(N=0, q=0, k=0, v=0, o=0, lse=0, cu=0), attn.ATTN_OK),
])
def test_prefill_fp8_varlen_argument_errors(kw, code):
    assert prefill_fp8_varlen(**kw) == code


def decode(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, d=128, P_=16,
           maxb=8, dtype=1, chunk=0, ws=FAKE, wsb=1 << 30):
    return attn.lib.attn_decode(P(q), P(kc), P(vc), P(bt), P(sl), P(o), P(lse), B, Hq, Hkv, d, P_,
                                maxb, dtype, 0.1, chunk, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(sl=0), attn.ATTN_ERR_NULL),
    (dict(o=0), attn.ATTN_ERR_NULL),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(P_=0), attn.ATTN_ERR_SHAPE),
    (dict(maxb=0), attn.ATTN_ERR_SHAPE),
    (dict(chunk=-16), attn.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=0), attn.ATTN_ERR_UNSUPPORTED),          # decode is bf16 only
    (dict(Hq=34, Hkv=2), attn.ATTN_ERR_UNSUPPORTED),     # group of 17 > 16
    (dict(chunk=24), attn.ATTN_ERR_UNSUPPORTED),         # not a multiple of 16
    (dict(P_=8), attn.ATTN_ERR_UNSUPPORTED),             # paged blocks would straddle pages
    (dict(ws=0), attn.ATTN_ERR_WORKSPACE),
    (dict(wsb=16), attn.ATTN_ERR_WORKSPACE),
    (dict(vc=MIS), attn.ATTN_ERR_ALIGN),
    (dict(ws=MIS), attn.ATTN_ERR_ALIGN),
    (dict(lse=MIS), attn.ATTN_ERR_ALIGN),
    (dict(B=0, q=0, kc=0, vc=0, bt=0, sl=0, o=0, ws=0), attn.ATTN_OK),
])
def test_decode_argument_errors(kw, code):
    assert decode(**kw) == code


def decode_append(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2,
                  d=128, P_=16, maxb=8, dtype=1, chunk=0, ws=FAKE, wsb=1 << 30):
    return attn.lib.attn_decode_append(P(q), P(kn), P(vn), P(kc), P(vc), P(bt), P(sl), P(o), P(lse), B, Hq, Hkv,
                                       d, P_, maxb, dtype, 0.1, chunk, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=0), attn.ATTN_ERR_NULL),
    (dict(vn=0), attn.ATTN_ERR_NULL),
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(kn=MIS), attn.ATTN_ERR_ALIGN),
    (dict(vn=MIS), attn.ATTN_ERR_ALIGN),
    (dict(B=-1, kn=0), attn.ATTN_ERR_SHAPE),        # shape errors come before pointer checks
    (dict(d=80, kn=0), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=0), attn.ATTN_ERR_WORKSPACE),
    (dict(B=0, q=0, kn=0, vn=0, kc=0, vc=0, bt=0, sl=0, o=0, ws=0), attn.ATTN_OK),
])
def test_decode_append_argument_errors(kw, code):
    assert decode_append(**kw) == code


def decode_ext(q=FAKE, kn=0, vn=0, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, d=128,
               P_=16, maxb=8, dtype=1, window=-1, cap=0.0, chunk=0, ws=FAKE, wsb=1 << 30):
    return attn.lib.attn_decode_ext(P(q), P(kn), P(vn), P(kc), P(vc), P(bt), P(sl), P(o), P(lse), B, Hq, Hkv, d,
                                    P_, maxb, dtype, 0.1, window, cap, chunk, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-5), attn.ATTN_ERR_SHAPE),
    (dict(cap=-0.5), attn.ATTN_ERR_SHAPE),
    (dict(cap=float("inf")), attn.ATTN_ERR_SHAPE),
    (dict(kn=FAKE), attn.ATTN_ERR_NULL),                  # append needs both new rows
    (dict(vn=FAKE), attn.ATTN_ERR_NULL),
    (dict(kn=MIS, vn=FAKE), attn.ATTN_ERR_ALIGN),
    (dict(q=0, window=4), attn.ATTN_ERR_NULL),
    (dict(d=80, cap=3.0), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=0, window=4), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=0, window=4), attn.ATTN_ERR_WORKSPACE),
    (dict(B=0, q=0, kc=0, vc=0, bt=0, sl=0, o=0, ws=0, window=4, cap=2.0), attn.ATTN_OK),
])
def test_decode_ext_argument_errors(kw, code):
    assert decode_ext(**kw) == code


def decode_fp8(q=FAKE, kc=FAKE, vc=FAKE, dk=0, dv=0, bt=FAKE, sl=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, d=128,
               P_=16, maxb=8, chunk=0, ws=FAKE, wsb=1 << 30):
    return attn.lib.attn_decode_fp8(P(q), P(kc), P(vc), P(dk), P(dv), P(bt), P(sl), P(o), P(lse), B, Hq, Hkv, d, P_,
                                    maxb, 0.1, chunk, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(kc=0), attn.ATTN_ERR_NULL),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=256), attn.ATTN_ERR_UNSUPPORTED),      # E4M3 cache: head sizes 64 and 128
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
    (dict(P_=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=0), attn.ATTN_ERR_WORKSPACE),
    (dict(dk=FAKE + 2), attn.ATTN_ERR_ALIGN),      # descales are float arrays: 4-byte aligned
    (dict(vc=MIS), attn.ATTN_ERR_ALIGN),
    (dict(B=0, q=0, kc=0, vc=0, bt=0, sl=0, o=0, ws=0), attn.ATTN_OK),
])
def test_decode_fp8_argument_errors(kw, code):
    assert decode_fp8(**kw) == code


def test_decode_contiguous_accepts_any_page_size_for_capacity():
    # page_size only fixes capacity when block_table is NULL; with a NULL workspace the
    # host check stops at ERR_WORKSPACE, i.e. after the page-size checks passed
    assert decode(bt=0, P_=8, ws=0) == attn.ATTN_ERR_WORKSPACE


def test_workspace_formula_and_chunk_choice():
    # explicit chunk: B * Hq * ceil(cap / chunk) * (d + 1) * 4
    assert attn.attn_decode_workspace_bytes(1, 28, 4, 128, 16, 2048, 512) == 1 * 28 * 64 * 129 * 4
    assert attn.attn_decode_workspace_bytes(3, 8, 2, 64, 16, 10, 48) == 3 * 8 * 4 * 65 * 4
    assert attn.attn_decode_chunk_tokens(1, 4, 16, 2048, 512) == 512
    # automatic choice: a multiple of 256 tokens between 256 and 2048; with several
    # sequences the workspace also holds the balanced split's partials, at most
    # min(256 / Hkv, ceil(capacity / unit)) per sequence, unit 256 tokens (128 at d = 256)
    for B, Hkv, maxb in [(1, 4, 2048), (32, 8, 2048), (1, 1, 1), (128, 8, 64), (4, 2, 100000), (3, 32, 8)]:
        c = attn.attn_decode_chunk_tokens(B, Hkv, 16, maxb, 0)
        assert 256 <= c <= 2048 and c % 256 == 0
        for d, unit in ((128, 256), (256, 128)):
            splits = -(-(maxb * 16) // c)
            if B >= 2:
                splits = max(splits, min(max(1, 256 // Hkv), -(-(maxb * 16) // unit)))
            assert attn.attn_decode_workspace_bytes(B, 4 * Hkv, Hkv, d, 16, maxb, 0) == \
                B * 4 * Hkv * splits * (d + 1) * 4, (B, Hkv, maxb, d)
    # the c5 batch: 32 splits of the balanced split (256 / 8 KV heads) against 16 chunks of 2048
    assert attn.attn_decode_workspace_bytes(32, 32, 8, 128, 16, 2048, 0) == 32 * 32 * 32 * 129 * 4
    assert attn.attn_decode_workspace_bytes(1, 28, 4, 128, 16, 2048, 24) == 0
    with pytest.raises(attn.AttnError):
        attn.attn_decode_chunk_tokens(1, 4, 16, 2048, 20)


def combine(op=FAKE, lp=FAKE, ns=0, rows=4, S=3, d=128, o=FAKE, odt=1, lse=0):
    return attn.lib.attn_lse_combine(P(op), P(lp), P(ns), rows, S, d, P(o), odt, P(lse), None)


@pytest.mark.parametrize("kw,code", [
    (dict(op=0), attn.ATTN_ERR_NULL),
    (dict(o=0), attn.ATTN_ERR_NULL),
    (dict(rows=-1), attn.ATTN_ERR_SHAPE),
    (dict(S=0), attn.ATTN_ERR_SHAPE),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(odt=5), attn.ATTN_ERR_UNSUPPORTED),
    (dict(lp=MIS), attn.ATTN_ERR_ALIGN),
    (dict(rows=0, op=0, lp=0, o=0), attn.ATTN_OK),
])
def test_combine_argument_errors(kw, code):
    assert combine(**kw) == code


def check_tables(bt=FAKE, sl=FAKE, B=4, page=16, mb=8, nb=32, app=0, out=FAKE):
    return attn.lib.attn_decode_check_tables(P(bt), P(sl), B, page, mb, nb, app, P(out), None)


@pytest.mark.parametrize("kw,code", [
    (dict(sl=0), attn.ATTN_ERR_NULL),
    (dict(out=0), attn.ATTN_ERR_NULL),
    (dict(B=0, out=0), attn.ATTN_ERR_NULL),
    (dict(B=-1), attn.ATTN_ERR_SHAPE),
    (dict(page=0), attn.ATTN_ERR_SHAPE),
    (dict(mb=0), attn.ATTN_ERR_SHAPE),
    (dict(nb=-1), attn.ATTN_ERR_SHAPE),
    (dict(app=2), attn.ATTN_ERR_SHAPE),
    (dict(out=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(sl=FAKE + 1), attn.ATTN_ERR_ALIGN),
    (dict(bt=FAKE + 2), attn.ATTN_ERR_ALIGN),
])
def test_check_tables_argument_errors(kw, code):
    assert check_tables(**kw) == code


def prefill_fp8_ext(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dq=0, dk=0, dv=0, cu=0, B=2, N=16, T=0, Hq=4, Hkv=2,
                    d=128, causal=1, window=8, cap=10.0):
    return attn.lib.attn_prefill_fp8_ext(P(q), P(k), P(v), P(o), P(lse), P(dq), P(dk), P(dv), P(cu), B, N, T, Hq, Hkv,
                                         d, causal, 0.1, window, cap, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-2), attn.ATTN_ERR_SHAPE),
    (dict(cap=-1.0), attn.ATTN_ERR_SHAPE),
    (dict(cap=float("nan")), attn.ATTN_ERR_SHAPE),
    (dict(cap=float("inf")), attn.ATTN_ERR_SHAPE),
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(cu=FAKE, T=20, q=0), attn.ATTN_ERR_NULL),   # packed form: same checks as the varlen call
    (dict(cu=FAKE + 2, T=20), attn.ATTN_ERR_ALIGN),
    (dict(o=MIS), attn.ATTN_ERR_ALIGN),
    (dict(dk=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
    (dict(d=512), attn.ATTN_ERR_UNSUPPORTED),
    (dict(B=0, q=0, k=0, v=0, o=0, lse=0), attn.ATTN_OK),
])
def test_prefill_fp8_ext_argument_errors(kw, code):
    assert prefill_fp8_ext(**kw) == code


def decode_fp8_ext(q=FAKE, kc=FAKE, vc=FAKE, dk=0, dv=0, bt=FAKE, sl=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, d=128,
                   page=16, mb=8, window=16, cap=10.0, chunk=0, ws=FAKE, wsb=1 << 30):
    return attn.lib.attn_decode_fp8_ext(P(q), P(kc), P(vc), P(dk), P(dv), P(bt), P(sl), P(o), P(lse), B, Hq, Hkv, d,
                                        page, mb, 0.1, window, cap, chunk, P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-2), attn.ATTN_ERR_SHAPE),
    (dict(cap=-0.5), attn.ATTN_ERR_SHAPE),
    (dict(cap=float("inf")), attn.ATTN_ERR_SHAPE),
    (dict(q=0), attn.ATTN_ERR_NULL),
    (dict(ws=0), attn.ATTN_ERR_WORKSPACE),
    (dict(wsb=16), attn.ATTN_ERR_WORKSPACE),
    (dict(d=256), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dk=FAKE + 2), attn.ATTN_ERR_ALIGN),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_GQA),
])
def test_decode_fp8_ext_argument_errors(kw, code):
    assert decode_fp8_ext(**kw) == code


def test_decode_noalloc_host_checks():
    """attn_decode_noalloc checks its arguments on the host before any HIP call: the
    argument errors of attn_decode, and ATTN_ERR_SCRATCH when the partials would not
    fit its static scratch (no workspace argument to grow)."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+ATTN_DECODE_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == attn.NOALLOC_SCRATCH_BYTES
    assert re.search(r"#define\s+ATTN_ERR_SCRATCH\s+-8", text) and attn.ATTN_ERR_SCRATCH == -8
    assert attn.attn_status_string(attn.ATTN_ERR_SCRATCH) != "unknown status"

    def call(B=4, Hq=8, Hkv=2, d=128, page=16, maxb=64, chunk=0, q=FAKE, sl=FAKE):
        return attn.lib.attn_decode_noalloc(P(q), P(FAKE), P(FAKE), None, P(sl), P(FAKE), None, B, Hq, Hkv, d,
                                            page, maxb, 1, 0.1, chunk, None)
    assert call(q=0) == attn.ATTN_ERR_NULL
    assert call(Hq=6, Hkv=4) == attn.ATTN_ERR_GQA
    assert call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert call(B=0) == attn.ATTN_OK
    # 4096 x 32 rows x one 16-token chunk x 129 floats = 67.6 MB > 16 MiB
    assert attn.attn_decode_workspace_bytes(4096, 32, 8, 128, 16, 1, 16) > attn.NOALLOC_SCRATCH_BYTES
    assert call(B=4096, Hq=32, Hkv=8, maxb=1, chunk=16) == attn.ATTN_ERR_SCRATCH
    # exactly at the limit is accepted by the size check (checked via the workspace formula)
    rows = attn.NOALLOC_SCRATCH_BYTES // (129 * 4)
    assert attn.attn_decode_workspace_bytes(rows, 1, 1, 128, 16, 1, 16) <= attn.NOALLOC_SCRATCH_BYTES


def test_decode_fp8_append_host_checks():
    """attn_decode_fp8_append: the append's rows are required and aligned, head sizes
    64 and 128 only, and the workspace is checked, all on the host."""
    def call(kn=FAKE, vn=FAKE, d=128, ws=FAKE, wsb=1 << 30, B=2, q=FAKE):
        return attn.lib.attn_decode_fp8_append(P(q), P(kn) if kn else None, P(vn) if vn else None, P(FAKE),
                                               P(FAKE), None, None, None, P(FAKE), P(FAKE), None, B, 8, 2, d, 16,
                                               64, 0.1, 0, P(ws) if ws else None, wsb, None)
    assert call(kn=0) == attn.ATTN_ERR_NULL
    assert call(vn=0) == attn.ATTN_ERR_NULL
    assert call(q=0) == attn.ATTN_ERR_NULL
    assert call(kn=MIS) == attn.ATTN_ERR_ALIGN
    assert call(d=256) == attn.ATTN_ERR_UNSUPPORTED
    assert call(d=96) == attn.ATTN_ERR_UNSUPPORTED
    assert call(ws=0) == attn.ATTN_ERR_WORKSPACE
    assert call(wsb=16) == attn.ATTN_ERR_WORKSPACE
    assert call(B=0) == attn.ATTN_OK


def test_paged_layout_helper_matches_the_paged_workload():
    """bench.py's paged decode leg takes its lengths and page placement from
    decode_paged_layout; they must be the paged workload's own (same seeded draws)."""
    from exact_io_aware_prefill_amd import workloads as W
    import torch
    for seed, B, lo, hi in ((5, 4, 100, 300), (9, 7, 1, 64)):
        q, bt, sl, pool, mb = W.decode_paged_layout(seed, B, 8, 64, 16, lo, hi)
        x = W.decode_paged_inputs(seed, B, 8, 2, 64, 16, lo, hi)
        assert torch.equal(q, x.q) and torch.equal(bt, x.block_table) and torch.equal(sl, x.seq_lens)
        assert pool == x.k_cache.shape[0] and mb == x.max_blocks
