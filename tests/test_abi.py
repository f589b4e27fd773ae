"""CPU checks of the C ABI: the library loads, exports every function include/attn.h declares,
and rejects invalid arguments with the documented status codes before touching a device.

No call here reaches a kernel launch: every argument set below fails host-side validation.
"""
import ctypes
import os
import re

import pytest

import attention_attn_prefill_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("attn_prefill", "attn_decode_paged", "kv_cache_append", "attn_decode_workspace_size",
              "attn_prefill_paged", "attn_decode_paged_multi", "attn_decode_multi_workspace_size",
              "attn_status_str", "attn_last_error"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = A.lib()
    for n in _declared():
        assert hasattr(L, n), f"libattn.so does not export {n}"
    assert set(_declared()) == set(A._SIGS), "binding signatures out of sync with the header"


def test_status_strings():
    L = A.lib()
    assert L.attn_status_str(0) == b"ok"
    assert L.attn_status_str(A.ATTN_ERR_WORKSPACE).startswith(b"workspace")
    assert L.attn_status_str(99) == b"unknown status"


def _prefill(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, dtype=A.ATTN_BF16, B=1, S=8, Hq=4, Hkv=2,
                D=64, scale=0.125, causal=1, window=0)
    args.update(kw)
    return A.lib().attn_prefill(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dtype"],
                                args["B"], args["S"], args["Hq"], args["Hkv"], args["D"], args["scale"],
                                args["causal"], args["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(o=None), A.ATTN_ERR_NULL),
    (dict(dtype=A.ATTN_I8), A.ATTN_ERR_DTYPE), (dict(dtype=7), A.ATTN_ERR_DTYPE),
    (dict(B=0), A.ATTN_ERR_SHAPE), (dict(S=0), A.ATTN_ERR_SHAPE), (dict(Hq=3), A.ATTN_ERR_SHAPE),
    (dict(window=-1), A.ATTN_ERR_SHAPE), (dict(scale=0.0), A.ATTN_ERR_SHAPE),
    (dict(scale=float("nan")), A.ATTN_ERR_SHAPE), (dict(D=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(D=256), A.ATTN_ERR_UNSUPPORTED),
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code
    assert A.lib().attn_last_error() != b""


def _decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None, table=FAKE, ctx=FAKE, o=FAKE,
             kv=A.ATTN_BF16, B=2, Hq=8, Hkv=2, D=64, bs=16, mb=4, nb=8, maxctx=64, scale=0.125,
             window=0, split=0, ws=None, wsb=0)
    a.update(kw)
    return A.lib().attn_decode_paged(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["table"], a["ctx"],
                                     a["o"], a["kv"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"],
                                     a["nb"], a["maxctx"], a["scale"], a["window"], a["split"], a["ws"],
                                     a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(table=None), A.ATTN_ERR_NULL), (dict(ctx=None), A.ATTN_ERR_NULL),
    (dict(kv=A.ATTN_F32), A.ATTN_ERR_DTYPE), (dict(kv=A.ATTN_I8), A.ATTN_ERR_NULL),
    (dict(ks=FAKE, vs=FAKE), A.ATTN_ERR_SHAPE), (dict(Hq=6, Hkv=4), A.ATTN_ERR_SHAPE),
    (dict(maxctx=0), A.ATTN_ERR_SHAPE), (dict(window=-2), A.ATTN_ERR_SHAPE), (dict(split=-16), A.ATTN_ERR_SHAPE),
    (dict(split=24), A.ATTN_ERR_SHAPE), (dict(D=80), A.ATTN_ERR_UNSUPPORTED), (dict(bs=8), A.ATTN_ERR_UNSUPPORTED),
    # more than 16 query heads per KV head, byte cache: virtual KV heads, which stage partials
    (dict(Hq=34, Hkv=2, kv=A.ATTN_I8, ks=FAKE, vs=FAKE), A.ATTN_ERR_WORKSPACE),
    (dict(split=8208), A.ATTN_ERR_UNSUPPORTED),
    (dict(maxctx=5000, split=64), A.ATTN_ERR_WORKSPACE),
    (dict(maxctx=5000, split=64, ws=FAKE, wsb=16), A.ATTN_ERR_WORKSPACE),
    # every tensor the kernels read or write in 16-byte pieces must be 16-byte aligned
    (dict(q=ctypes.c_void_p(0x1008)), A.ATTN_ERR_SHAPE), (dict(o=ctypes.c_void_p(0x1004)), A.ATTN_ERR_SHAPE),
    (dict(kc=ctypes.c_void_p(0x1002)), A.ATTN_ERR_SHAPE),
    (dict(kv=A.ATTN_I8, ks=FAKE, vs=ctypes.c_void_p(0x1002)), A.ATTN_ERR_SHAPE),
])
def test_decode_validation(kw, code):
    assert _decode(**kw) == code


def _multi(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None, table=FAKE, ctx=FAKE, o=FAKE,
             kv=A.ATTN_BF16, B=2, ql=4, Hq=8, Hkv=2, D=64, bs=16, mb=4, nb=8, maxctx=64, scale=0.125,
             window=0, split=0, ws=None, wsb=0)
    a.update(kw)
    return A.lib().attn_decode_paged_multi(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["table"],
                                           a["ctx"], a["o"], a["kv"], a["B"], a["ql"], a["Hq"], a["Hkv"],
                                           a["D"], a["bs"], a["mb"], a["nb"], a["maxctx"], a["scale"],
                                           a["window"], a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(ql=0), A.ATTN_ERR_SHAPE), (dict(ql=-1), A.ATTN_ERR_SHAPE),
    # 4 heads per KV head x 5 rows > 16 columns, byte cache: virtual KV heads (one query head
    # each), which stage partials; more than 16 rows: refused (a bf16 cache goes through the
    # prefill kernel)
    (dict(ql=5, kv=A.ATTN_I8, ks=FAKE, vs=FAKE), A.ATTN_ERR_WORKSPACE),
    (dict(Hq=16, Hkv=1, ql=2, kv=A.ATTN_FP8, ks=FAKE, vs=FAKE), A.ATTN_ERR_WORKSPACE),
    (dict(ql=17, kv=A.ATTN_I8, ks=FAKE, vs=FAKE), A.ATTN_ERR_UNSUPPORTED),
    (dict(Hq=2, Hkv=2, ql=17, kv=A.ATTN_FP8, ks=FAKE, vs=FAKE), A.ATTN_ERR_UNSUPPORTED),
    (dict(ql=5, split=24), A.ATTN_ERR_SHAPE), (dict(ql=5, window=-1), A.ATTN_ERR_SHAPE),
    (dict(B=40000), A.ATTN_ERR_SHAPE), (dict(ql=5, B=70000), A.ATTN_ERR_SHAPE),
    (dict(), A.ATTN_ERR_WORKSPACE),                     # the balanced shape stages partials
    (dict(kv=A.ATTN_FP8, ks=ctypes.c_void_p(0x1008), vs=FAKE), A.ATTN_ERR_SHAPE),
])
def test_decode_multi_validation(kw, code):
    assert _multi(**kw) == code


def test_wide_decode_workspace_is_that_of_the_virtual_kv_heads():
    """More than 16 query columns per KV head: the size is that of the byte-cache path, R
    virtual KV heads per cache head (R the smallest divisor of Hq/Hkv that brings a virtual
    head's columns to 16); a bf16 cache runs on the prefill kernel and needs none of it."""
    wm, ws = A.attn_decode_multi_workspace_size, A.attn_decode_workspace_size
    assert wm(3, 8, 32, 8, 64, 4096, 0, 0) == wm(3, 8, 32, 16, 64, 4096, 0, 0) > 0  # 4 x 8: R = 2
    assert wm(3, 5, 20, 4, 128, 7000, 0, 0) == wm(3, 5, 20, 20, 128, 7000, 0, 0) > 0  # 5 x 5: R = 5
    assert ws(3, 64, 2, 64, 4096, 0, 0) == ws(3, 64, 4, 64, 4096, 0, 0) > 0  # 32 heads: R = 2
    assert wm(3, 17, 8, 8, 64, 4096, 0, 0) == 0  # 17 rows: no byte-cache path


def test_multi_workspace_matches_single_row():
    ws, wm = A.attn_decode_workspace_size, A.attn_decode_multi_workspace_size
    for args in ((2, 8, 2, 64, 5000, 0, 64), (3, 32, 8, 128, 4096, 0, 0), (2, 8, 2, 64, 700, 100, 0)):
        B, rest = args[0], args[1:]
        assert wm(B, 1, *rest) == ws(B, *rest)
    assert wm(3, 4, 32, 8, 128, 4096, 0, 0) > ws(3, 32, 8, 128, 4096, 0, 0)


def test_workspace_size_rules():
    ws = A.attn_decode_workspace_size
    assert ws(2, 8, 2, 64, 64, 0, 64) == 0  # one split: no workspace
    n = ws(2, 8, 2, 64, 5000, 0, 64)        # 79 splits
    assert n >= 2 * 8 * 79 * (64 + 1) * 4
    assert ws(2, 8, 2, 64, 5000, 100, 64) < n  # the window bounds the splits
    assert ws(0, 8, 2, 64, 64, 0, 0) == 0
    # library's choice, no window: the balanced shape always stages partials (prefix + slots)
    assert ws(2, 8, 2, 64, 64, 0, 0) >= (2 * 2 + 4) * 4 * (64 + 1) * 4
    # library's choice with a window covering the whole span: one split, no workspace
    assert ws(2, 8, 2, 64, 64, 100, 0) == 0


def _append(**kw):
    a = dict(kn=FAKE, vn=FAKE, seq=FAKE, pos=FAKE, table=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None,
             dt=A.ATTN_BF16, T=4, Hkv=2, D=64, bs=16, ns=2, mb=4, nb=8)
    a.update(kw)
    return A.lib().kv_cache_append(a["kn"], a["vn"], a["seq"], a["pos"], a["table"], a["kc"], a["vc"],
                                   a["ks"], a["vs"], a["dt"], a["T"], a["Hkv"], a["D"], a["bs"],
                                   a["ns"], a["mb"], a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), A.ATTN_ERR_NULL), (dict(kc=None), A.ATTN_ERR_NULL),
    (dict(dt=A.ATTN_I8), A.ATTN_ERR_NULL), (dict(dt=A.ATTN_F32), A.ATTN_ERR_DTYPE),
    (dict(T=-1), A.ATTN_ERR_SHAPE), (dict(Hkv=0), A.ATTN_ERR_SHAPE), (dict(D=32), A.ATTN_ERR_UNSUPPORTED),
    (dict(bs=32), A.ATTN_ERR_UNSUPPORTED), (dict(T=0, kn=None), A.ATTN_OK),
])
def test_append_validation(kw, code):
    assert _append(**kw) == code


def _paged(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, table=FAKE, cu=FAKE, ctx=FAKE, o=FAKE, lse=None,
             B=2, Hq=8, Hkv=2, D=64, bs=16, mb=4, nb=8, mq=16, tq=20, scale=0.125, causal=1, window=0)
    a.update(kw)
    return A.lib().attn_prefill_paged(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["table"], a["cu"],
                                      a["ctx"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                      a["mb"], a["nb"], a["mq"], a["tq"], a["scale"], a["causal"],
                                      a["window"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(cu=None), A.ATTN_ERR_NULL), (dict(kn=None), A.ATTN_ERR_NULL),
    (dict(tq=-1), A.ATTN_ERR_SHAPE), (dict(Hq=6, Hkv=4), A.ATTN_ERR_SHAPE), (dict(window=-1), A.ATTN_ERR_SHAPE),
    (dict(scale=-1.0), A.ATTN_ERR_SHAPE), (dict(D=96), A.ATTN_ERR_UNSUPPORTED), (dict(bs=32), A.ATTN_ERR_UNSUPPORTED),
    (dict(tq=0, q=None), A.ATTN_OK),
    # 1024 sequences x 16 heads x 2^20 rows: 2^27 workgroups of 256 threads, past a 2^32-thread grid
    (dict(B=1024, Hq=16, Hkv=16, mq=1 << 20, tq=1 << 30), A.ATTN_ERR_SHAPE),
])
def test_prefill_paged_validation(kw, code):
    assert _paged(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(base=0.0), A.ATTN_ERR_SHAPE), (dict(base=float("nan")), A.ATTN_ERR_SHAPE),
    (dict(base=-5.0), A.ATTN_ERR_SHAPE), (dict(D=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(kn=None), A.ATTN_ERR_NULL), (dict(T=0, kn=None), A.ATTN_OK),
])
def test_append_rope_validation(kw, code):
    a = dict(kn=FAKE, T=4, D=64, base=10000.0)
    a.update(kw)
    r = A.lib().kv_cache_append_rope(a["kn"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                     A.ATTN_BF16, a["T"], 2, a["D"], 16, 2, 4, 8, a["base"], None)
    assert r == code


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), A.ATTN_ERR_SHAPE), (dict(T=-1), A.ATTN_ERR_SHAPE), (dict(D=32), A.ATTN_ERR_UNSUPPORTED),
    (dict(base=0.0), A.ATTN_ERR_SHAPE), (dict(x=None), A.ATTN_ERR_NULL), (dict(T=0, x=None), A.ATTN_OK),
])
def test_rope_inplace_validation(kw, code):
    a = dict(x=FAKE, T=3, H=2, D=64, base=10000.0)
    a.update(kw)
    assert A.lib().attn_rope_inplace(a["x"], FAKE, a["T"], a["H"], a["D"], a["base"], None) == code


def test_fp8_cache_validation():
    assert _decode(kv=A.ATTN_FP8) == A.ATTN_ERR_NULL            # fp8 cache without scales
    assert _decode(kv=A.ATTN_FP8, ks=FAKE) == A.ATTN_ERR_NULL
    assert _decode(kv=4) == A.ATTN_ERR_DTYPE
    assert _append(dt=A.ATTN_FP8) == A.ATTN_ERR_NULL
    assert _append(dt=A.ATTN_FP8, T=0, kn=None) == A.ATTN_OK


def _noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=None, vs=None, table=FAKE, ctx=FAKE, o=FAKE,
             kv=A.ATTN_BF16, B=2, Hq=8, Hkv=2, D=64, bs=16, mb=4, nb=8, maxctx=64, scale=0.125,
             window=0, split=0)
    a.update(kw)
    return A.lib().attn_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["table"],
                                             a["ctx"], a["o"], a["kv"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                             a["bs"], a["mb"], a["nb"], a["maxctx"], a["scale"],
                                             a["window"], a["split"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), A.ATTN_ERR_NULL), (dict(kv=A.ATTN_F32), A.ATTN_ERR_DTYPE),
    (dict(Hq=6, Hkv=4), A.ATTN_ERR_SHAPE), (dict(D=80), A.ATTN_ERR_UNSUPPORTED),
    (dict(o=ctypes.c_void_p(0x1004)), A.ATTN_ERR_SHAPE),
    # partials of 2048 sequences x 16 query heads per KV head x D = 128 exceed the 32 MiB array
    (dict(B=2048, Hq=128, Hkv=8, D=128, maxctx=1000), A.ATTN_ERR_WORKSPACE),
    (dict(B=512, Hq=64, Hkv=8, D=128, maxctx=100000, split=64), A.ATTN_ERR_WORKSPACE),
])
def test_noalloc_validation(kw, code):
    """Rejected before the device is touched (no GPU here), oversized requests with a message
    that names the static scratch's size."""
    assert _noalloc(**kw) == code
    if code == A.ATTN_ERR_WORKSPACE:
        assert b"static scratch holds 33554432" in A.lib().attn_last_error()
