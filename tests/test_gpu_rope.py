"""GPU parity of the RoPE-fused cache append and the in-place query rotation."""
import numpy as np
import pytest

import oracle
from synth import DecodeWorkload, bf16_value, decode_query, new_tokens, paged_table, pool
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu


def _ulps_bf16(a_bits, b_bits):
    """Distance in bf16 ulps between two arrays of finite bf16 bit patterns."""
    def key(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return np.abs(key(a_bits) - key(b_bits))


@pytest.mark.parametrize("D,base", [(64, 10000.0), (128, 500000.0)])
def test_rope_inplace_matches_oracle(D, base):
    import attention_attn_prefill_amd as A
    T, H = 300, 6
    xb, xf = new_tokens(4100 + D, T, H, D, "k")
    pos = np.random.default_rng(D).integers(0, 40000, size=T).astype(np.int32)
    pos[:3] = (0, 1, 32767)
    x = dev_bf16(xb)
    A.attn_rope_inplace(x, dev(pos), rope_base=base)
    torch().cuda.synchronize()
    want = oracle.bf16_round(oracle.rope(xf, pos, base))
    got = host_bits(x)
    want_bits = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d = _ulps_bf16(got, want_bits)
    # the device reduces the angle in fp64 and takes sin/cos and the rotation in fp32, the
    # oracle works in fp64 throughout: the bf16 results differ by at most one unit, and only
    # where the fp32 result lies next to a bf16 rounding boundary
    assert d.max() <= 1 and (d == 0).mean() > 0.999
    assert np.array_equal(got[pos == 0], xb[pos == 0])  # position 0: identity


@pytest.mark.parametrize("int8", [False, True])
def test_append_rope_places_and_rotates(int8):
    import attention_attn_prefill_amd as A
    t = torch()
    Hkv, D, bs, base = 4, 128, 16, 10000.0
    ctx = np.array([40, 17, 70], np.int32)
    table, nb = paged_table(ctx, bs, 4200, 2, True)
    T = 25
    rng = np.random.default_rng(4201)
    seq = rng.integers(0, 3, size=T).astype(np.int32)
    pos = np.array([rng.integers(0, ctx[s]) for s in seq], np.int32)
    # distinct target slots
    _, first = np.unique(seq.astype(np.int64) * 1000 + pos, return_index=True)
    keep = np.sort(first)
    seq, pos, T = seq[keep], pos[keep], len(keep)
    kn, kf = new_tokens(4202, T, Hkv, D, "k")
    vn, vf = new_tokens(4203, T, Hkv, D, "v")
    if not int8:
        kc = t.full((nb, Hkv, bs, D), 0x7777, dtype=t.int16, device="cuda").view(t.bfloat16)
        vc = t.full((nb, Hkv, bs, D), 0x7777, dtype=t.int16, device="cuda").view(t.bfloat16)
        A.kv_cache_append_rope(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dev(table), kc, vc,
                               rope_base=base)
        t.cuda.synchronize()
        gk, gv = host_bits(kc), host_bits(vc)
        for i in range(T):
            blk, slot = table[seq[i]][pos[i] // bs], pos[i] % bs
            assert np.array_equal(gv[blk, :, slot], vn[i])  # V: the bits, at exactly this slot
            want = oracle.bf16_round(oracle.rope(kf[i:i + 1], pos[i:i + 1], base))[0]
            wb = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            assert _ulps_bf16(gk[blk, :, slot], wb).max() <= 1
            gk[blk, :, slot] = 0x7777
            gv[blk, :, slot] = 0x7777
        assert (gk == 0x7777).all() and (gv == 0x7777).all()  # nothing else written
    else:
        kc = t.zeros((nb, Hkv, bs, D), dtype=t.int8, device="cuda")
        vc = t.zeros_like(kc)
        ks = t.zeros((nb, Hkv, bs), dtype=t.float16, device="cuda")
        vs = t.zeros_like(ks)
        A.kv_cache_append_rope(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dev(table), kc, vc,
                               rope_base=base, k_scale=ks, v_scale=vs)
        t.cuda.synchronize()
        gk, gks = kc.cpu().numpy(), ks.cpu().numpy()
        gv, gvs = vc.cpu().numpy(), vs.cpu().numpy()
        for i in range(T):
            blk, slot = table[seq[i]][pos[i] // bs], pos[i] % bs
            wv, wvs = oracle.quantize_int8(vf[i])  # V: exact quantization of the bf16 values
            assert np.array_equal(gv[blk, :, slot], wv) and np.array_equal(gvs[blk, :, slot], wvs)
            rot = oracle.rope(kf[i:i + 1], pos[i:i + 1], base)[0].astype(np.float32)
            wk, wks = oracle.quantize_int8(rot)
            assert np.abs(gk[blk, :, slot].astype(int) - wk.astype(int)).max() <= 1
            assert np.allclose(gks[blk, :, slot].astype(np.float64), wks.astype(np.float64), rtol=2e-3)


def test_rope_end_to_end_decode():
    """Append K with RoPE, rotate Q in place, decode: equals attention over rotated Q and K."""
    import attention_attn_prefill_amd as A
    t = torch()
    B, Hq, Hkv, D, bs, base = 3, 8, 2, 64, 16, 500000.0
    ctx = np.array([33, 200, 1], np.int32)
    wl = DecodeWorkload("rope", 4300, "bf16", B, Hq, Hkv, D, 1, int(ctx.max()))
    table, nb = paged_table(ctx, bs, 4300, 1, True)
    T = int(ctx.sum())
    seq = np.repeat(np.arange(B), ctx).astype(np.int32)
    pos = np.concatenate([np.arange(c) for c in ctx]).astype(np.int32)
    kn, kf = new_tokens(4301, T, Hkv, D, "k")
    vn, vf = new_tokens(4302, T, Hkv, D, "v")
    kc = t.zeros((nb, Hkv, bs, D), dtype=t.bfloat16, device="cuda")
    vc = t.zeros_like(kc)
    A.kv_cache_append_rope(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dev(table), kc, vc, rope_base=base)
    qbits, qf = decode_query(wl)
    q = dev_bf16(qbits)
    A.attn_rope_inplace(q, dev(ctx - 1), rope_base=base)
    o = A.attn_decode_paged(q, kc, vc, dev(table), dev(ctx), int(ctx.max()), scale=wl.scale)
    t.cuda.synchronize()
    qr = oracle.rope(qf, ctx - 1, base)
    kr = oracle.rope(kf, pos, base)
    for b in range(B):
        rows = seq == b
        for h in range(Hq):
            ro, _ = oracle.attention_head(qr[b:b + 1, h], kr[rows, h // 4], vf[rows, h // 4], wl.scale,
                                          [ctx[b] - 1], True, 0)
            assert maxabs(host_f64(o)[b, h], ro[0]) <= BF16_TOL
