"""GPU parity of attn_decode_paged and kv_cache_append (through the C ABI) against the oracle."""
import numpy as np
import pytest

import oracle
from synth import (DecodeWorkload, WORKLOADS, bf16_value, context_lens, decode_query, int8_pool,
                   new_tokens, paged_table, pool, pool_blocks)
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu


def _decode(q, kc, vc, table, ctx, wl, max_ctx, ks=None, vs=None, split=0, window=None):
    import attention_attn_prefill_amd as A
    o = A.attn_decode_paged(q, kc, vc, table, ctx, max_ctx, k_scale=ks, v_scale=vs,
                            scale=wl.scale, window=wl.window if window is None else window,
                            split_tokens=split)
    torch().cuda.synchronize()
    return o


def _small(D, Hq, Hkv, window, kv="bf16", ctx=(1, 15, 16, 17, 100, 333), spare=3, seed=0):
    wl = DecodeWorkload("small", 500 + 7 * D + Hq + window + seed, kv, len(ctx), Hq, Hkv, D, 1,
                        max(ctx), 16, window)
    ctx = np.array(ctx, np.int32)
    table, nb = paged_table(ctx, 16, wl.seed, spare, True)
    qbits, qf = decode_query(wl)
    return wl, ctx, table, nb, qbits, qf


def _poison_unused(pool_arr, table, ctx, bs=16, value=None):
    """Fill every slot no live token occupies (test-side scan of the table)."""
    used = np.zeros(pool_arr.shape[0] * bs, bool)
    for b, c in enumerate(ctx):
        for t in range(int(c)):
            used[int(table[b][t // bs]) * bs + t % bs] = True
    out = pool_arr.copy()
    flat = out.reshape(pool_arr.shape[0], pool_arr.shape[1], bs, -1)
    for s in np.nonzero(~used)[0]:
        flat[s // bs, :, s % bs] = value
    return out


CASES = [(64, 8, 2, 0), (64, 32, 8, 5), (128, 8, 1, 0), (128, 4, 4, 40), (64, 16, 1, 0),
         (128, 64, 8, 0), (64, 6, 3, 17),
         # more than 16 query heads per KV head: two virtual KV heads per cache head (bf16 and
         # byte caches), three (byte caches; bf16 goes through the paged prefill kernel)
         (64, 64, 2, 0), (128, 40, 2, 17), (64, 48, 1, 0)]


@pytest.mark.parametrize("split", [0, 16, 48])
@pytest.mark.parametrize("D,Hq,Hkv,window", CASES)
def test_decode_bf16_small(D, Hq, Hkv, window, split):
    wl, ctx, table, nb, qbits, qf = _small(D, Hq, Hkv, window)
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    nan_bf16 = np.uint16(0x7FC0)
    kp, vp = _poison_unused(kb, table, ctx, value=nan_bf16), _poison_unused(vb, table, ctx, value=nan_bf16)
    o = _decode(dev_bf16(qbits), dev_bf16(kp), dev_bf16(vp), dev(table), dev(ctx), wl, int(ctx.max()),
                split=split)
    ro, _ = oracle.decode_paged(qf, bf16_value(kb), bf16_value(vb), table, ctx, wl.scale, 16, window)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("D,Hq,Hkv,window", CASES[:5])
def test_decode_int8_small(D, Hq, Hkv, window, split):
    wl, ctx, table, nb, qbits, qf = _small(D, Hq, Hkv, window, kv="i8")
    kc, ks = int8_pool(wl, "k", nb)
    vc, vs = int8_pool(wl, "v", nb)
    o = _decode(dev_bf16(qbits), dev(kc), dev(vc), dev(table), dev(ctx), wl, int(ctx.max()),
                ks=dev(ks), vs=dev(vs), split=split)
    ro, _ = oracle.decode_paged(qf, kc, vc, table, ctx, wl.scale, 16, window, k_scale=ks, v_scale=vs)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("D,Hq,Hkv,window", CASES[7:])
def test_decode_int8_more_than_16_heads_per_kv_head(D, Hq, Hkv, window, split):
    """32 and 20 query heads per KV head with an INT8 cache: virtual KV heads."""
    test_decode_int8_small(D, Hq, Hkv, window, split)


@pytest.mark.parametrize("kv", ["i8", "bf16"])
def test_virtual_kv_heads_equal_a_cache_with_repeated_heads(kv):
    """Splitting each cache head into R virtual heads computes, for every query head, exactly
    what a cache holding each head R times (and R times the KV heads) gives: bit for bit."""
    wl, ctx, table, nb, qbits, qf = _small(64, 64, 2, 0, kv=kv)  # 32 heads per KV head: R = 2
    rep = lambda x: np.repeat(x, 2, axis=1)  # [nb][Hkv][...] -> [nb][2 Hkv][...]
    if kv == "i8":
        (kc, ks), (vc, vs) = int8_pool(wl, "k", nb), int8_pool(wl, "v", nb)
        put = dev
    else:
        kc, vc, ks, vs = pool(wl, "k", nb), pool(wl, "v", nb), None, None
        put = dev_bf16
    opt = lambda x: None if x is None else dev(x)
    opt_rep = lambda x: None if x is None else dev(rep(x))
    for split in (0, 32):
        o = _decode(dev_bf16(qbits), put(kc), put(vc), dev(table), dev(ctx), wl, int(ctx.max()),
                    ks=opt(ks), vs=opt(vs), split=split)
        o2 = _decode(dev_bf16(qbits), put(rep(kc)), put(rep(vc)), dev(table), dev(ctx), wl,
                     int(ctx.max()), ks=opt_rep(ks), vs=opt_rep(vs), split=split)
        assert np.array_equal(host_bits(o), host_bits(o2)), split


def test_ctx_one_returns_v_exactly():
    wl, ctx, table, nb, qbits, qf = _small(128, 16, 2, 0, ctx=(1, 1, 1))
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    o = _decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, 1)
    got = host_bits(o)
    for b in range(3):
        want = np.repeat(vb[table[b][0], :, 0], 8, axis=0)
        assert np.array_equal(got[b], want)


def test_permutation_invariance_bit_exact():
    """Same logical K/V written through two different tables: identical outputs."""
    import attention_attn_prefill_amd as A
    t = torch()
    wl, ctx, _, _, qbits, qf = _small(64, 32, 8, 0, ctx=(700, 31, 1025, 16, 300))
    T = int(ctx.sum())
    kn, _ = new_tokens(11, T, wl.Hkv, wl.D, "k")
    vn, _ = new_tokens(11, T, wl.Hkv, wl.D, "v")
    seq = np.repeat(np.arange(len(ctx)), ctx).astype(np.int32)
    pos = np.concatenate([np.arange(c) for c in ctx]).astype(np.int32)
    outs = []
    for seed, permute, spare in ((1, False, 0), (2, True, 5), (3, True, 9)):
        table, nb = paged_table(ctx, 16, seed, spare, permute)
        kc = t.zeros((nb, wl.Hkv, 16, wl.D), dtype=t.bfloat16, device="cuda")
        vc = t.zeros_like(kc)
        dt = dev(table)
        A.kv_cache_append(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dt, kc, vc)
        outs.append(host_bits(_decode(dev_bf16(qbits), kc, vc, dt, dev(ctx), wl, int(ctx.max()), split=64)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_split_invariance_and_determinism():
    wl, ctx, table, nb, qbits, qf = _small(128, 32, 8, 0, ctx=(2000, 513, 64, 1500))
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    args = (dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, 2000)
    ro, _ = oracle.decode_paged(qf, bf16_value(kb), bf16_value(vb), table, ctx, wl.scale, 16)
    first = None
    for split in (16, 64, 128, 0):
        o = host_bits(_decode(*args, split=split))
        assert maxabs(bf16_value(o), ro) <= BF16_TOL
        again = host_bits(_decode(*args, split=split))
        assert np.array_equal(o, again)
        first = o if first is None else first


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_decode_balanced_tiny_and_empty_contexts(kv):
    """Default (balanced) shape with no window: many short and empty sequences, so one wave's
    range spans several (sequence, KV head) segments and segments split across waves."""
    ctx = (0, 1, 2, 15, 16, 17, 0, 33, 1, 100, 48, 0, 5, 64, 65, 3)
    wl, ctx, table, nb, qbits, qf = _small(64, 8, 2, 0, kv=kv, ctx=ctx, seed=11)
    live = ctx > 0
    if kv == "bf16":
        kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
        o = _decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, 100)
        ro, _ = oracle.decode_paged(qf[live], bf16_value(kb), bf16_value(vb), table[live], ctx[live],
                                    wl.scale, 16)
    else:
        (kc, ks), (vc, vs) = int8_pool(wl, "k", nb), int8_pool(wl, "v", nb)
        o = _decode(dev_bf16(qbits), dev(kc), dev(vc), dev(table), dev(ctx), wl, 100, ks=dev(ks), vs=dev(vs))
        ro, _ = oracle.decode_paged(qf[live], kc, vc, table[live], ctx[live], wl.scale, 16,
                                    k_scale=ks, v_scale=vs)
    got = host_f64(o)
    assert (got[~live] == 0).all()
    assert maxabs(got[live], ro) <= BF16_TOL


@pytest.mark.parametrize("Hq", [4, 8])
def test_decode_one_long_sequence_split_over_every_wave(Hq):
    """One sequence, one KV head, 20000 keys: the balanced shape gives each of ~1250 waves a
    single block, so the merge combines ~1250 partials of one segment (4 columns use the VALU
    PV form, 8 the MFMA form)."""
    wl, ctx, table, nb, qbits, qf = _small(64, Hq, 1, 0, ctx=(20000,), seed=13)
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    o = _decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, 20000)
    ro, _ = oracle.decode_paged(qf, bf16_value(kb), bf16_value(vb), table, ctx, wl.scale, 16)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


def test_decode_large_batch_uses_fixed_splits():
    """Beyond the balanced shape's batch limit the default falls back to fixed splits."""
    rng = np.random.default_rng(5)
    ctx = tuple(int(c) for c in rng.integers(1, 40, size=2100))
    wl, ctx, table, nb, qbits, qf = _small(64, 8, 2, 0, ctx=ctx, spare=0, seed=12)
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    o = _decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, 40)
    ro, _ = oracle.decode_paged(qf, bf16_value(kb), bf16_value(vb), table, ctx, wl.scale, 16)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


def test_zero_context_gives_zero():
    wl, ctx, table, nb, qbits, qf = _small(64, 8, 2, 0, ctx=(5, 3))
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    ctx0 = np.array([0, 3], np.int32)
    for split in (0, 16):
        o = host_f64(_decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx0), wl, 5,
                             split=split))
        assert (o[0] == 0).all()


# ---- kv_cache_append -------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("int8", [False, True])
def test_append_bit_exact(D, int8):
    import attention_attn_prefill_amd as A
    t = torch()
    Hkv, bs = 4, 16
    ctx = np.array([40, 7, 100], np.int32)
    table, nb = paged_table(ctx, bs, 31, 4, True)
    rng = np.random.default_rng(D + int8)
    T = 90
    seq = rng.integers(0, 3, T).astype(np.int32)
    pos = np.array([rng.integers(0, ctx[s]) for s in seq], np.int32)
    # make (seq, pos) unique so the expected pool is well defined
    _, first = np.unique(seq.astype(np.int64) * 100000 + pos, return_index=True)
    seq, pos = seq[np.sort(first)], pos[np.sort(first)]
    # rows that must be skipped: bad sequence, bad position, table entry -1
    seq = np.concatenate([seq, [3, -1, 0, 1]]).astype(np.int32)
    pos = np.concatenate([pos, [0, 0, 4 * bs * 10, 20]]).astype(np.int32)  # seq 1 pos 20 -> entry -1
    T = len(seq)
    kn, kf = new_tokens(40 + D, T, Hkv, D, "k")
    vn, vf = new_tokens(41 + D, T, Hkv, D, "v")
    valid = np.array([(0 <= s < 3) and (0 <= p < table.shape[1] * bs) and table[s][p // bs] >= 0
                      for s, p in zip(seq, pos)])
    dt = dev(table)
    if not int8:
        sentinel = np.full((nb, Hkv, bs, D), 0x1234, np.uint16)
        kc, vc = dev_bf16(sentinel), dev_bf16(sentinel)
        A.kv_cache_append(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dt, kc, vc)
        t.cuda.synchronize()
        for got, rows in ((kc, kn), (vc, vn)):
            want = oracle.append_expected(sentinel, rows[valid], seq[valid], pos[valid], table, bs)
            assert np.array_equal(host_bits(got), want)
    else:
        sent_c = np.full((nb, Hkv, bs, D), 77, np.int8)
        sent_s = np.full((nb, Hkv, bs), 3.0, np.float16)
        kc, vc, ks, vs = dev(sent_c), dev(sent_c), dev(sent_s), dev(sent_s)
        A.kv_cache_append(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dt, kc, vc, k_scale=ks, v_scale=vs)
        t.cuda.synchronize()
        for gc, gs, rows in ((kc, ks, kf), (vc, vs, vf)):
            codes, scales = oracle.quantize_int8(rows)
            want_c = oracle.append_expected(sent_c, codes[valid], seq[valid], pos[valid], table, bs)
            want_s = oracle.append_expected(sent_s, scales[valid], seq[valid], pos[valid], table, bs)
            assert np.array_equal(gc.cpu().numpy(), want_c)
            assert np.array_equal(gs.cpu().numpy().view(np.uint16), want_s.view(np.uint16))


# ---- full-size workloads -----------------------------------------------------------------------
def _full_bf16(wl):
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, wl.block_size, wl.seed)
    qbits, qf = decode_query(wl)
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    return ctx, table, nb, qbits, qf, kb, vb


def test_decode_llama1b_b64_all_outputs():
    wl = WORKLOADS["decode_llama1b_b64"]
    ctx, table, nb, qbits, qf, kb, vb = _full_bf16(wl)
    o = _decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, wl.ctx_hi)
    ro, _ = oracle.decode_paged(qf, bf16_value(kb), bf16_value(vb), table, ctx, wl.scale, 16)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


def _oracle_sampled(wl, qf, table, ctx, seqs, getter):
    """Oracle decode for a few sequences, from just their blocks (compact pool, identity table)."""
    worst = []
    for b in seqs:
        n = -(-int(ctx[b]) // wl.block_size)
        blocks = table[b, :n]
        parts = getter(blocks)
        tb = np.arange(n, dtype=np.int32)[None]
        ro, _ = oracle.decode_paged(qf[b:b + 1], *parts[:2], tb, ctx[b:b + 1], wl.scale, wl.block_size,
                                    wl.window, *parts[2:])
        worst.append((b, ro[0]))
    return worst


def test_decode_swa_b32_sampled():
    wl = WORKLOADS["decode_swa_b32"]
    ctx, table, nb, qbits, qf, kb, vb = _full_bf16(wl)
    o = host_f64(_decode(dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx), wl, wl.ctx_hi))
    for b, ro in _oracle_sampled(wl, qf, table, ctx, [0, 13, 31],
                                 lambda blk: (pool_blocks(wl, "k", blk), pool_blocks(wl, "v", blk))):
        assert maxabs(o[b], ro) <= BF16_TOL


def test_decode_int8_70b_b16_sampled():
    """Cache quantized on the GPU by kv_cache_append (checked bit-exact on sampled blocks) and
    read by the decode; the oracle quantizes the same bf16 rows with its own quantizer."""
    import attention_attn_prefill_amd as A
    t = torch()
    wl = WORKLOADS["decode_int8_70b_b16"]
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, 16, wl.seed)
    qbits, qf = decode_query(wl)
    caches = []
    ident = dev(np.arange(nb, dtype=np.int32)[None])
    T = nb * 16
    seq = dev(np.zeros(T, np.int32))
    pos = dev(np.arange(T, dtype=np.int32))
    for which in ("k", "v"):
        src = pool(wl, which, nb)  # [nb][Hkv][16][D] bf16 bits, physical order
        rows = dev_bf16(np.ascontiguousarray(src.transpose(0, 2, 1, 3)).reshape(T, wl.Hkv, wl.D))
        c = t.empty((nb, wl.Hkv, 16, wl.D), dtype=t.int8, device="cuda")
        s = t.empty((nb, wl.Hkv, 16), dtype=t.float16, device="cuda")
        A.kv_cache_append(rows, rows, seq, pos, ident, c, c, k_scale=s, v_scale=s)
        del rows, src
        caches += [c, s]
    t.cuda.synchronize()
    kc, ks, vc, vs = caches
    o = host_f64(_decode(dev_bf16(qbits), kc, vc, dev(table), dev(ctx), wl, wl.ctx_hi, ks=ks, vs=vs))

    def quantized(blk):
        kq, ksc = oracle.quantize_int8(pool_blocks(wl, "k", blk))
        vq, vsc = oracle.quantize_int8(pool_blocks(wl, "v", blk))
        return kq, vq, ksc, vsc

    probe = np.array([0, 1, 777, nb - 1])
    kq, vq, ksc, vsc = quantized(probe)
    assert np.array_equal(kc[probe].cpu().numpy(), kq) and np.array_equal(vc[probe].cpu().numpy(), vq)
    assert np.array_equal(ks[probe].cpu().numpy().view(np.uint16), ksc.view(np.uint16))
    assert np.array_equal(vs[probe].cpu().numpy().view(np.uint16), vsc.view(np.uint16))
    for b, ro in _oracle_sampled(wl, qf, table, ctx, [0, 9], quantized):
        assert maxabs(o[b], ro) <= BF16_TOL


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("D,window", [(64, 0), (128, 0), (128, 40)])
def test_byte_cache_query_range(kv, D, window):
    """Byte caches multiply on fp16: bf16 queries outside fp16's range (|q| >= 65520, or below its
    smallest subnormal) must still match the oracle. Heads take N(0,1) queries times 3e4
    (elements past 65504), 1e-30 and 1e-7 (below fp16's subnormals), 1, and one head mixes
    3e4 with 1e-30 inside the same vector."""
    import attention_attn_prefill_amd as A
    from synth import fp8_pool
    wl, ctx, table, nb, _, _ = _small(D, 8, 2, window, kv=kv, ctx=(2, 15, 16, 17, 100, 333))
    qf = decode_query(wl)[1].astype(np.float32)
    factors = np.array([3e4, 1e-30, 1e-7, 1.0, 3e4, 1.0, 1e-7, 1e-30], np.float32)
    qf = qf * factors[None, :, None]
    qf[:, 5, : D // 2] *= np.float32(3e4)
    qf[:, 5, D // 2:] *= np.float32(1e-30)
    from synth import bf16_bits
    qbits = bf16_bits(qf)
    qv = bf16_value(qbits).astype(np.float64)
    assert np.abs(qv).max() > 65520 and 0 < np.abs(qv[:, 1]).max() < 2.0 ** -24
    if kv == "i8":
        kc, ks = int8_pool(wl, "k", nb)
        vc, vs = int8_pool(wl, "v", nb)
        kf, vf = oracle.dequantize_int8(kc, ks), oracle.dequantize_int8(vc, vs)
    else:
        kc, ks = fp8_pool(wl, "k", nb)
        vc, vs = fp8_pool(wl, "v", nb)
        kf, vf = oracle.dequantize_fp8(kc, ks), oracle.dequantize_fp8(vc, vs)
    o = _decode(dev_bf16(qbits), dev(kc), dev(vc), dev(table), dev(ctx), wl, int(ctx.max()),
                ks=dev(ks), vs=dev(vs))
    ro, _ = oracle.decode_paged(qv, kf, vf, table, ctx, wl.scale, 16, window)
    assert maxabs(host_f64(o), ro) <= BF16_TOL
    # the same columns as draft rows of the multi-row decode (2 rows x 4 heads per KV head)
    q2 = qbits.reshape(len(ctx), 2, 4, D)
    om = A.attn_decode_paged_multi(dev_bf16(q2), dev(kc), dev(vc), dev(table), dev(ctx), int(ctx.max()),
                                   k_scale=dev(ks), v_scale=dev(vs), scale=wl.scale, window=window)
    torch().cuda.synchronize()
    cu = np.arange(len(ctx) + 1) * 2
    rm, _ = oracle.prefill_paged(qv.reshape(len(ctx) * 2, 4, D), cu, kf, vf, table, ctx, wl.scale, 16,
                                 True, window)
    assert maxabs(host_f64(om).reshape(len(ctx) * 2, 4, D), rm) <= BF16_TOL


def test_shared_workspace_bit_identical():
    """One workspace reused by calls of different shapes (balanced single-row, multi-row, fixed
    splits with and without a window, the balanced call again) gives the same bits as a fresh
    workspace per call: nothing a call leaves in the workspace reaches a later call."""
    import attention_attn_prefill_amd as A
    t = torch()
    wl, ctx, table, nb, qbits, qf = _small(64, 8, 2, 0, ctx=(1, 15, 16, 17, 100, 333, 2000, 40))
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    q, kc, vc, tb, cx = dev_bf16(qbits), dev_bf16(kb), dev_bf16(vb), dev(table), dev(ctx)
    mx = int(ctx.max())
    q2 = dev_bf16(np.concatenate([qbits, qbits[:, ::-1]], axis=1).reshape(len(ctx), 2, 8, 64))
    need = max(A.attn_decode_workspace_size(len(ctx), 8, 2, 64, mx, w, sp) for w, sp in ((0, 0), (0, 32), (300, 64)))
    need = max(need, A.attn_decode_multi_workspace_size(len(ctx), 2, 8, 2, 64, mx, 0, 0))
    ws = t.full((need,), 0x7F, dtype=t.uint8, device="cuda")  # starts as NaN-like garbage
    calls = [
        lambda w: A.attn_decode_paged(q, kc, vc, tb, cx, mx, scale=wl.scale, workspace=w),
        lambda w: A.attn_decode_paged_multi(q2, kc, vc, tb, cx, mx, scale=wl.scale, workspace=w),
        lambda w: A.attn_decode_paged(q, kc, vc, tb, cx, mx, scale=wl.scale, split_tokens=32, workspace=w),
        lambda w: A.attn_decode_paged(q, kc, vc, tb, cx, mx, scale=wl.scale, window=300, split_tokens=64,
                                      workspace=w),
        lambda w: A.attn_decode_paged(q, kc, vc, tb, cx, mx, scale=wl.scale, workspace=w),
    ]
    for call in calls + calls:
        shared = call(ws)
        fresh = call(None)
        t.cuda.synchronize()
        assert np.array_equal(host_bits(shared), host_bits(fresh))
    ro, _ = oracle.decode_paged(qf, bf16_value(kb), bf16_value(vb), table, ctx, wl.scale, 16)
    assert maxabs(host_f64(calls[0](ws)), ro) <= BF16_TOL
