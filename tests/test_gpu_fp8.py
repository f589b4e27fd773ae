"""GPU parity of the FP8 E4M3 KV cache: quantizing append (bit-exact codes and scales),
single-row and multi-row decode, and a 70B-shaped long-context decode."""
import numpy as np
import pytest

import oracle
from synth import (DecodeWorkload, WORKLOADS, bf16_bits, bf16_value, context_lens, decode_query,
                   fp8_pool, new_tokens, paged_table, pool, pool_blocks)
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_f64, maxabs, torch
from tests.test_gpu_decode import _oracle_sampled

pytestmark = pytest.mark.gpu


def _append_rows(rows_bits, D, Hkv=1):
    """Quantize rows [T][Hkv][D] (bf16 bits) into an FP8 cache with an identity table."""
    import attention_attn_prefill_amd as A
    t = torch()
    T = rows_bits.shape[0]
    nb = -(-T // 16)
    c = t.zeros((nb, Hkv, 16, D), dtype=t.uint8, device="cuda")
    s = t.zeros((nb, Hkv, 16), dtype=t.float16, device="cuda")
    r = dev_bf16(rows_bits)
    A.kv_cache_append(r, r, dev(np.zeros(T, np.int32)), dev(np.arange(T, dtype=np.int32)),
                      dev(np.arange(nb, dtype=np.int32)[None]), c, c, k_scale=s, v_scale=s)
    t.cuda.synchronize()
    codes = c.cpu().numpy().transpose(0, 2, 1, 3).reshape(nb * 16, Hkv, D)[:T]
    scales = s.cpu().numpy().transpose(0, 2, 1).reshape(nb * 16, Hkv)[:T]
    return codes, scales


def test_fp8_append_encodes_every_code_boundary():
    """Rows whose absmax is 448 get scale 1, so their codes are the E4M3 encoding of the inputs
    themselves: every code value, every midpoint between neighbours (ties to even), values one
    bf16 step either side of each midpoint, signed zeros and subnormals."""
    grid = oracle.fp8_e4m3_decode(np.arange(127, dtype=np.uint8))  # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2
    step = np.exp2(np.floor(np.log2(mids[1:])) - 7)  # one bf16 step at each midpoint
    vals = np.concatenate([grid, mids, mids[1:] + step, mids[1:] - step])
    vals = np.concatenate([vals, -vals, [-0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -11]])
    assert np.array_equal(bf16_value(bf16_bits(vals.astype(np.float32))), vals)  # all exact in bf16
    D = 128
    per_row = D - 1
    n = -(-len(vals) // per_row)
    x = np.zeros((n, 1, D), np.float32)
    x[:, 0, 0] = 448.0
    x.reshape(n, D)[:, 1:].flat[: len(vals)] = vals
    codes, scales = _append_rows(bf16_bits(x), D)
    want_c, want_s = oracle.quantize_fp8(x)
    assert np.array_equal(scales.view(np.uint16), want_s.view(np.uint16))
    assert (scales == 1.0).all()
    assert np.array_equal(codes, want_c)


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_append_random_rows_bit_exact(D):
    bits, f = new_tokens(5100 + D, 2000, 4, D, "k")
    f[7] *= 1e-3    # small and large rows
    f[8] *= 300.0
    f[9] = 0.0
    bits = bf16_bits(f)
    codes, scales = _append_rows(bits, D, Hkv=4)
    want_c, want_s = oracle.quantize_fp8(bf16_value(bits))
    assert np.array_equal(scales.view(np.uint16), want_s.view(np.uint16))
    assert np.array_equal(codes, want_c)


def _small(D, Hq, Hkv, window, ctx, seed):
    wl = DecodeWorkload("fp8", seed, "fp8", len(ctx), Hq, Hkv, D, 1, max(ctx), 16, window)
    ctx = np.array(ctx, np.int32)
    table, nb = paged_table(ctx, 16, wl.seed, 3, True)
    qbits, qf = decode_query(wl)
    (kc, ks), (vc, vs) = fp8_pool(wl, "k", nb), fp8_pool(wl, "v", nb)
    return wl, ctx, table, qbits, qf, kc, ks, vc, vs


CASES = [(64, 8, 2, 0), (64, 32, 8, 5), (128, 8, 1, 0), (128, 4, 4, 40), (128, 64, 8, 0), (64, 6, 3, 17)]


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("D,Hq,Hkv,window", CASES)
def test_fp8_decode_small(D, Hq, Hkv, window, split):
    import attention_attn_prefill_amd as A
    wl, ctx, table, qbits, qf, kc, ks, vc, vs = _small(D, Hq, Hkv, window, (1, 15, 16, 17, 100, 333), 5200 + D + Hq)
    o = A.attn_decode_paged(dev_bf16(qbits), dev(kc), dev(vc), dev(table), dev(ctx), int(ctx.max()),
                            k_scale=dev(ks), v_scale=dev(vs), scale=wl.scale, window=window, split_tokens=split)
    torch().cuda.synchronize()
    ro, _ = oracle.decode_paged(qf, oracle.dequantize_fp8(kc, ks), oracle.dequantize_fp8(vc, vs), table, ctx,
                                wl.scale, 16, window)
    assert maxabs(host_f64(o), ro) <= BF16_TOL


def test_fp8_decode_multi_rows():
    import attention_attn_prefill_amd as A
    wl, ctx, table, _, _, kc, ks, vc, vs = _small(128, 32, 8, 0, (9, 200, 1500), 5300)
    QL = 4
    qb, qf = new_tokens(5301, len(ctx) * QL, 32, 128, "k")
    o = A.attn_decode_paged_multi(dev_bf16(qb.reshape(len(ctx), QL, 32, 128)), dev(kc), dev(vc), dev(table),
                                  dev(ctx), int(ctx.max()), k_scale=dev(ks), v_scale=dev(vs), scale=wl.scale)
    torch().cuda.synchronize()
    ro, _ = oracle.prefill_paged(qf, np.arange(len(ctx) + 1) * QL, oracle.dequantize_fp8(kc, ks),
                                 oracle.dequantize_fp8(vc, vs), table, ctx, wl.scale, 16, True, 0)
    assert maxabs(host_f64(o).reshape(ro.shape), ro) <= BF16_TOL


@pytest.mark.parametrize("QL,Hq,Hkv", [(8, 32, 8), (3, 48, 2)])
def test_fp8_decode_multi_rows_more_than_16_columns(QL, Hq, Hkv):
    """8 drafts x 4 heads and 3 drafts x 24 heads per KV head: virtual KV heads."""
    import attention_attn_prefill_amd as A
    wl, ctx, table, _, _, kc, ks, vc, vs = _small(128, Hq, Hkv, 0, (9, 200, 1500), 5310 + QL)
    qb, qf = new_tokens(5311 + QL, len(ctx) * QL, Hq, 128, "k")
    o = A.attn_decode_paged_multi(dev_bf16(qb.reshape(len(ctx), QL, Hq, 128)), dev(kc), dev(vc), dev(table),
                                  dev(ctx), int(ctx.max()), k_scale=dev(ks), v_scale=dev(vs), scale=wl.scale)
    torch().cuda.synchronize()
    ro, _ = oracle.prefill_paged(qf, np.arange(len(ctx) + 1) * QL, oracle.dequantize_fp8(kc, ks),
                                 oracle.dequantize_fp8(vc, vs), table, ctx, wl.scale, 16, True, 0)
    assert maxabs(host_f64(o).reshape(ro.shape), ro) <= BF16_TOL


def test_fp8_decode_70b_b16_sampled():
    """The INT8 70B-shaped configuration with an FP8 cache: quantized on the GPU (bit-exact
    on sampled blocks), decoded, and checked on sampled sequences."""
    import attention_attn_prefill_amd as A
    t = torch()
    wl = WORKLOADS["decode_int8_70b_b16"]
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, 16, wl.seed)
    qbits, qf = decode_query(wl)
    ident = dev(np.arange(nb, dtype=np.int32)[None])
    T = nb * 16
    seq = dev(np.zeros(T, np.int32))
    pos = dev(np.arange(T, dtype=np.int32))
    caches = []
    for which in ("k", "v"):
        src = pool(wl, which, nb)
        rows = dev_bf16(np.ascontiguousarray(src.transpose(0, 2, 1, 3)).reshape(T, wl.Hkv, wl.D))
        c = t.empty((nb, wl.Hkv, 16, wl.D), dtype=t.uint8, device="cuda")
        s = t.empty((nb, wl.Hkv, 16), dtype=t.float16, device="cuda")
        A.kv_cache_append(rows, rows, seq, pos, ident, c, c, k_scale=s, v_scale=s)
        del rows, src
        caches += [c, s]
    t.cuda.synchronize()
    kc, ks, vc, vs = caches
    o = A.attn_decode_paged(dev_bf16(qbits), kc, vc, dev(table), dev(ctx), wl.ctx_hi, k_scale=ks, v_scale=vs,
                            scale=wl.scale)
    o = host_f64(o)

    def quantized(blk):
        kq, ksc = oracle.quantize_fp8(pool_blocks(wl, "k", blk))
        vq, vsc = oracle.quantize_fp8(pool_blocks(wl, "v", blk))
        return oracle.dequantize_fp8(kq, ksc), oracle.dequantize_fp8(vq, vsc), (kq, ksc, vq, vsc)

    probe = np.array([0, 1, 777, nb - 1])
    kf, vf, (kq, ksc, vq, vsc) = quantized(probe)
    assert np.array_equal(kc[probe].cpu().numpy(), kq) and np.array_equal(vc[probe].cpu().numpy(), vq)
    assert np.array_equal(ks[probe].cpu().numpy().view(np.uint16), ksc.view(np.uint16))
    for b, ro in _oracle_sampled(wl, qf, table, ctx, [0, 9], lambda blk: quantized(blk)[:2]):
        assert maxabs(o[b], ro) <= BF16_TOL


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_decode_ignores_nan_in_unwritten_slots(D, split):
    """Slots after a sequence's last token are never written, so they may hold any byte: fill
    them with E4M3 NaN codes (0x7F, 0xFF) and NaN scales. Their probabilities are 0, and the
    result must still match the oracle, which reads only visible tokens."""
    import attention_attn_prefill_amd as A
    wl, ctx, table, qbits, qf, kc, ks, vc, vs = _small(D, 16, 4, 0, (1, 15, 17, 100, 333), 5400 + D)
    kc, vc, ks, vs = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    for b, n in enumerate(ctx):
        if n % 16:
            pb = table[b, (n - 1) // 16]
            kc[pb, :, n % 16:, :] = 0x7F
            vc[pb, :, n % 16:, :] = 0xFF
            ks[pb, :, n % 16:] = np.float16(np.nan)
            vs[pb, :, n % 16:] = np.float16(np.nan)
    o = A.attn_decode_paged(dev_bf16(qbits), dev(kc), dev(vc), dev(table), dev(ctx), int(ctx.max()),
                            k_scale=dev(ks), v_scale=dev(vs), scale=wl.scale, split_tokens=split)
    torch().cuda.synchronize()
    o = host_f64(o)
    assert np.isfinite(o).all()
    visible = lambda c, s: oracle.dequantize_fp8(c, s)  # noqa: E731 -- NaN slots are never read
    ro, _ = oracle.decode_paged(qf, visible(kc, np.nan_to_num(ks)), visible(vc, np.nan_to_num(vs)), table, ctx,
                                wl.scale, 16, 0)
    assert np.isfinite(ro).all()  # the oracle reads visible tokens only
    assert maxabs(o, ro) <= BF16_TOL
