"""Seeded random sweep of the GPU path against the fp64 oracle: each case draws its own
combination of head dim, head counts, batch, ragged and empty contexts, window, cache dtype,
split policy and draft rows (decode), or batch, length, heads, mask and window (prefill), so
combinations no hand-written case names are exercised too. Sizes stay small enough for the
oracle; every draw is printed in the test id. ATTN_RANDOM_SCALE=k multiplies the number of cases
(k = 1 by default), for a longer sweep run by hand."""
import os

import numpy as np
import pytest

import oracle
from synth import (DecodeWorkload, PrefillWorkload, bf16_bits, bf16_value, fp8_pool, int8_pool,
                   new_tokens, paged_table, pool, prefill_inputs)
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu


def _decode_case(i):
    r = np.random.default_rng(9000 + i)
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    QL = int(r.choice([1, 1, 1, 2, 3, 4]))
    G = int(r.choice([g for g in (1, 2, 3, 4, 5, 6, 8, 16) if g * QL <= 16]))
    B = int(r.integers(1, 13))
    ctx = []
    for _ in range(B):
        u = r.random()
        if u < 0.1 and QL == 1:
            ctx.append(0)
        elif u < 0.35:
            ctx.append(int(r.integers(QL, 41)))
        else:
            ctx.append(int(r.integers(max(QL, 41), 1501)))
    window = 0 if r.random() < 0.6 else int(r.integers(1, 601))
    kv = str(r.choice(["bf16", "bf16", "i8", "fp8"]))
    split = 0 if r.random() < 0.5 else 16 * int(r.integers(1, 33))
    spare = int(r.integers(0, 6))
    return dict(D=D, Hkv=Hkv, G=G, QL=QL, ctx=tuple(ctx), window=window, kv=kv, split=split, spare=spare,
                seed=9000 + i)


def _wide_decode_case(i):
    """Draft rows x query heads per KV head above 16 (bf16 cache): the paged prefill kernel's
    path of attn_decode_paged / attn_decode_paged_multi."""
    r = np.random.default_rng(9300 + i)
    QL = int(r.choice([1, 2, 3, 5, 6, 8]))
    G = int(r.choice([g for g in (3, 4, 5, 6, 8, 12, 16, 20, 32) if 16 < g * QL <= 64]))
    B = int(r.integers(1, 9))
    ctx = [int(r.integers(QL, 41)) if r.random() < 0.3 else int(r.integers(max(QL, 41), 1201))
           for _ in range(B)]
    window = 0 if r.random() < 0.6 else int(r.integers(1, 401))
    return dict(D=int(r.choice([64, 128])), Hkv=int(r.choice([1, 2, 4])), G=G, QL=QL, ctx=tuple(ctx),
                window=window, kv="bf16", split=0 if r.random() < 0.5 else 16 * int(r.integers(1, 9)),
                spare=int(r.integers(0, 4)), seed=9300 + i)


def _wide_byte_decode_case(i):
    """The same widths with an INT8 or FP8 cache: virtual KV heads (each cache head split into
    groups of query heads of at most 16 columns)."""
    c = _wide_decode_case(10000 + i)
    c["kv"] = "i8" if i % 2 == 0 else "fp8"
    return c


SCALE = max(1, int(os.environ.get("ATTN_RANDOM_SCALE", "1")))
DECODE_CASES = [_decode_case(i) for i in range(60 * SCALE)] + \
    [_wide_decode_case(i) for i in range(15 * SCALE)] + \
    [_wide_byte_decode_case(i) for i in range(10 * SCALE)]


def _dec_id(c):
    return (f"D{c['D']}-Hkv{c['Hkv']}-G{c['G']}-QL{c['QL']}-B{len(c['ctx'])}-w{c['window']}-{c['kv']}"
            f"-split{c['split']}")


@pytest.mark.parametrize("c", DECODE_CASES, ids=_dec_id)
def test_random_decode(c):
    import attention_attn_prefill_amd as A
    D, Hkv, G, QL, window, seed = c["D"], c["Hkv"], c["G"], c["QL"], c["window"], c["seed"]
    Hq = G * Hkv
    ctx = np.array(c["ctx"], np.int32)
    B = len(ctx)
    wl = DecodeWorkload("random", seed, "bf16" if c["kv"] == "bf16" else "i8", B, Hq, Hkv, D, 1,
                        max(1, int(ctx.max())), 16, window)
    table, nb = paged_table(np.maximum(ctx, 1), 16, seed, c["spare"], True)
    qb, qf = new_tokens(seed + 3, B * QL, Hq, D, "k")
    if c["kv"] == "bf16":
        kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
        kc, vc, ks, vs = dev_bf16(kb), dev_bf16(vb), None, None
        kf, vf = bf16_value(kb), bf16_value(vb)
    elif c["kv"] == "i8":
        (k8, k_s), (v8, v_s) = int8_pool(wl, "k", nb), int8_pool(wl, "v", nb)
        kc, vc, ks, vs = dev(k8), dev(v8), dev(k_s), dev(v_s)
        kf, vf = oracle.dequantize_int8(k8, k_s), oracle.dequantize_int8(v8, v_s)
    else:
        (k8, k_s), (v8, v_s) = fp8_pool(wl, "k", nb), fp8_pool(wl, "v", nb)
        kc, vc, ks, vs = dev(k8), dev(v8), dev(k_s), dev(v_s)
        kf, vf = oracle.dequantize_fp8(k8, k_s), oracle.dequantize_fp8(v8, v_s)
    if QL == 1:
        o = A.attn_decode_paged(dev_bf16(qb.reshape(B, Hq, D)), kc, vc, dev(table), dev(ctx),
                                max(1, int(ctx.max())), k_scale=ks, v_scale=vs, scale=wl.scale,
                                window=window, split_tokens=c["split"])
    else:
        o = A.attn_decode_paged_multi(dev_bf16(qb.reshape(B, QL, Hq, D)), kc, vc, dev(table), dev(ctx),
                                      int(ctx.max()), k_scale=ks, v_scale=vs, scale=wl.scale,
                                      window=window, split_tokens=c["split"])
    torch().cuda.synchronize()
    got = host_f64(o).reshape(B, QL, Hq, D)
    live = ctx > 0
    assert (got[~live] == 0).all()
    seqs = np.nonzero(live)[0]
    q = qf.reshape(B, QL, Hq, D)[seqs].reshape(len(seqs) * QL, Hq, D)
    cu = np.arange(len(seqs) + 1) * QL
    ro, _ = oracle.prefill_paged(q, cu, kf, vf, table[seqs], ctx[seqs], wl.scale, 16, True, window)
    assert maxabs(got[seqs], ro.reshape(len(seqs), QL, Hq, D)) <= BF16_TOL


def _prefill_case(i):
    r = np.random.default_rng(9500 + i)
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 5, 8]))
    B = int(r.integers(1, 4))
    S = int(r.integers(1, 700))
    causal = bool(r.random() < 0.8)
    window = 0 if r.random() < 0.5 else int(r.integers(1, 400))
    return dict(D=D, Hkv=Hkv, G=G, B=B, S=S, causal=causal, window=window, seed=9500 + i)


PREFILL_CASES = [_prefill_case(i) for i in range(40 * SCALE)]


@pytest.mark.parametrize("c", PREFILL_CASES,
                         ids=lambda c: f"D{c['D']}-Hkv{c['Hkv']}-G{c['G']}-B{c['B']}-S{c['S']}"
                                       f"-{'causal' if c['causal'] else 'full'}-w{c['window']}")
def test_random_prefill(c):
    import attention_attn_prefill_amd as A
    wl = PrefillWorkload("random", c["seed"], "bf16", c["B"], c["S"], c["G"] * c["Hkv"], c["Hkv"], c["D"],
                         c["causal"], c["window"])
    x = prefill_inputs(wl)
    o = A.attn_prefill(*(dev_bf16(x[n + "_bits"]) for n in "qkv"), scale=wl.scale, causal=wl.causal,
                       window=wl.window)
    torch().cuda.synchronize()
    ro, _ = oracle.attention(x["q"], x["k"], x["v"], wl.scale, wl.causal, wl.window)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


def _chunk_case(i):
    r = np.random.default_rng(9800 + i)
    D = int(r.choice([64, 128]))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    B = int(r.integers(1, 5))
    ctx, ql = [], []
    for _ in range(B):
        n = int(r.integers(1, 1200))
        ctx.append(n)
        ql.append(int(r.integers(0, min(n, 300) + 1)))
    window = 0 if r.random() < 0.6 else int(r.integers(1, 500))
    return dict(D=D, Hkv=Hkv, G=G, ctx=tuple(ctx), ql=tuple(ql), window=window, seed=9800 + i)


CHUNK_CASES = [_chunk_case(i) for i in range(30 * SCALE)]


@pytest.mark.parametrize("c", CHUNK_CASES,
                         ids=lambda c: f"D{c['D']}-Hkv{c['Hkv']}-G{c['G']}-B{len(c['ctx'])}-w{c['window']}")
def test_random_prefill_paged(c):
    import attention_attn_prefill_amd as A
    t = torch()
    D, Hkv, Hq, seed, window = c["D"], c["Hkv"], c["G"] * c["Hkv"], c["seed"], c["window"]
    ctx = np.array(c["ctx"], np.int32)
    ql = np.array(c["ql"], np.int32)
    wl = DecodeWorkload("chunk", seed, "bf16", len(ctx), Hq, Hkv, D, 1, int(ctx.max()))
    table, nb = paged_table(ctx, 16, seed, 2, True)
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    T = int(ql.sum())
    kn, _ = new_tokens(seed + 1, T, Hkv, D, "k")
    vn, _ = new_tokens(seed + 2, T, Hkv, D, "v")
    qb, qf = new_tokens(seed + 3, T, Hq, D, "k")
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    seq = np.repeat(np.arange(len(ctx)), ql).astype(np.int32)
    pos = np.concatenate([np.arange(n - q, n) for n, q in zip(ctx, ql)]).astype(np.int32)
    kc, vc = dev_bf16(kb), dev_bf16(vb)
    o = A.attn_prefill_paged(dev_bf16(qb), kc, vc, dev(table), dev(cu), dev(ctx),
                             max(1, int(ql.max())), scale=D ** -0.5, causal=True, window=window,
                             k_new=dev_bf16(kn), v_new=dev_bf16(vn))
    t.cuda.synchronize()
    kexp = oracle.append_expected(bf16_value(kb), bf16_value(kn), seq, pos, table, 16)
    vexp = oracle.append_expected(bf16_value(vb), bf16_value(vn), seq, pos, table, 16)
    # the chunk's rows land in the cache bit for bit, every other slot is untouched
    assert np.array_equal(host_bits(kc), bf16_bits(kexp))
    assert np.array_equal(host_bits(vc), bf16_bits(vexp))
    if T == 0:
        return
    ro, _ = oracle.prefill_paged(qf, cu, kexp, vexp, table, ctx, D ** -0.5, 16, True, window)
    assert maxabs(host_f64(o), ro) <= BF16_TOL
