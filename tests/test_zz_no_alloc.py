"""GPU check of attn_decode_paged_noalloc (through the C ABI): its output equals
attn_decode_paged's bit for bit on the same inputs, on two calls in a row, the second with a
smaller input (the static scratch keeps the first call's contents), and on further calls with an
INT8 cache (one of them with more than 16 query heads per KV head)."""
import numpy as np
import pytest

from synth import DecodeWorkload, context_lens, decode_query, int8_pool, paged_table, pool
from tests.gpu_util import dev, dev_bf16, host_bits, torch

pytestmark = pytest.mark.gpu


def _case(name, seed, kv, B, Hq, Hkv, D, lo, hi, window=0):
    wl = DecodeWorkload(name, seed, kv, B, Hq, Hkv, D, lo, hi, 16, window)
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, 16, wl.seed, 2, True)
    qbits, _ = decode_query(wl)
    if kv == "bf16":
        kc, vc = dev_bf16(pool(wl, "k", nb)), dev_bf16(pool(wl, "v", nb))
        ks = vs = None
    else:
        k8, k_s = int8_pool(wl, "k", nb)
        v8, v_s = int8_pool(wl, "v", nb)
        kc, vc, ks, vs = dev(k8), dev(v8), dev(k_s), dev(v_s)
    return wl, dict(q=dev_bf16(qbits), kc=kc, vc=vc, ks=ks, vs=vs, table=dev(table), ctx=dev(ctx),
                    mx=int(ctx.max()))


def _both(wl, c):
    import attention_attn_prefill_amd as A
    kw = dict(k_scale=c["ks"], v_scale=c["vs"], scale=wl.scale, window=wl.window)
    ref = A.attn_decode_paged(c["q"], c["kc"], c["vc"], c["table"], c["ctx"], c["mx"], **kw)
    got = A.attn_decode_paged_noalloc(c["q"], c["kc"], c["vc"], c["table"], c["ctx"], c["mx"], **kw)
    torch().cuda.synchronize()
    return host_bits(ref), host_bits(got)


def test_noalloc_matches_workspace_entry_point():
    # first call: Llama-shaped heads, ragged contexts, the balanced shape (partials in scratch)
    wl1, c1 = _case("na1", 3101, "bf16", 48, 32, 8, 64, 1, 3000)
    ref1, got1 = _both(wl1, c1)
    assert np.array_equal(ref1, got1)
    # second call, smaller: 5 sequences, D = 128, a window (fixed splits merged from scratch)
    wl2, c2 = _case("na2", 3102, "bf16", 5, 16, 2, 128, 200, 900, window=100)
    ref2, got2 = _both(wl2, c2)
    assert np.array_equal(ref2, got2)
    # third: an INT8 cache, balanced shape, 3 sequences
    wl3, c3 = _case("na3", 3103, "i8", 3, 8, 1, 128, 100, 5000)
    ref3, got3 = _both(wl3, c3)
    assert np.array_equal(ref3, got3)
    # fourth: an INT8 cache with 32 query heads per KV head (two virtual KV heads per cache head)
    wl4, c4 = _case("na4", 3104, "i8", 6, 64, 2, 64, 50, 2000)
    ref4, got4 = _both(wl4, c4)
    assert np.array_equal(ref4, got4)
    # the first input again after the others: same bits as before
    _, again = _both(wl1, c1)
    assert np.array_equal(again, got1)
