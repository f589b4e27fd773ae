"""GPU parity with every live cache block placed past the first 4 GiB of its pool.

The paged entry points address the pools with 64-bit byte offsets (a block id times 32 KiB for a
bf16 block of 8 KV heads at D = 128, 16 KiB for a byte cache). Here each pool is a little over
4 GiB and every block a sequence uses lies above the 2^32-byte mark, so an offset computed in
32 bits anywhere on the path (loads, the fused append's stores, the append kernel, scales) reads
or writes another block. The oracle works on a compact pool of just the used blocks with the
table renumbered; only the device table points into the high region.
"""
import numpy as np
import pytest

import oracle
from synth import DecodeWorkload, bf16_value, int8_pool, new_tokens, paged_table, pool
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu
LSE_TOL_BF16 = 4e-3  # l sums bf16-rounded probabilities: ln l within 2^-9 of the exact LSE
Hq, Hkv, D, BS = 32, 8, 128, 16


def _high_ids(nb_c, block_bytes, seed):
    """Physical ids for compact blocks 0 .. nb_c-1, all above the 4 GiB mark, and the pool size."""
    base = (1 << 32) // block_bytes
    rng = np.random.default_rng(seed)
    phys = (base + 1 + 3 * rng.permutation(nb_c)).astype(np.int64)
    return phys, int(base + 3 * nb_c + 4)


def _remap(table, phys):
    return np.where(table >= 0, phys[np.maximum(table, 0)], -1).astype(np.int32)


def _scatter(shape_tail, dtype, num_blocks, phys, compact):
    """A pool of num_blocks blocks (uninitialized) with the compact blocks written at phys."""
    t = torch()
    big = t.empty((num_blocks,) + shape_tail, dtype=dtype, device="cuda")
    big[t.from_numpy(phys).cuda()] = compact
    return big


def _gather(big, phys):
    t = torch()
    return big[t.from_numpy(phys).cuda()]


def _bf16_case(ctx, seed, spare=2):
    ctx = np.array(ctx, np.int32)
    wl = DecodeWorkload("high", seed, "bf16", len(ctx), Hq, Hkv, D, 1, int(ctx.max()))
    table, nb_c = paged_table(ctx, BS, seed, spare, True)
    phys, nb = _high_ids(nb_c, Hkv * BS * D * 2, seed + 1)
    kb, vb = pool(wl, "k", nb_c), pool(wl, "v", nb_c)
    t = torch()
    kc = _scatter((Hkv, BS, D), t.bfloat16, nb, phys, dev_bf16(kb))
    vc = _scatter((Hkv, BS, D), t.bfloat16, nb, phys, dev_bf16(vb))
    return dict(wl=wl, ctx=ctx, table=table, phys=phys, kb=kb, vb=vb, kc=kc, vc=vc,
                tdev=dev(_remap(table, phys)))


@pytest.fixture(scope="module")
def bf16_case():
    c = _bf16_case((5, 17, 700, 2049), seed=4242)  # every context holds the 5 draft rows
    yield c
    c.clear()
    torch().cuda.empty_cache()


def test_decode_bf16_blocks_above_4gib(bf16_case):
    import attention_attn_prefill_amd as A
    c = bf16_case
    assert c["kc"].numel() * 2 > (1 << 32) and int(c["phys"].min()) * Hkv * BS * D * 2 >= (1 << 32)
    qb, qf = new_tokens(4300, len(c["ctx"]), Hq, D, "k")
    ro, _ = oracle.decode_paged(qf, bf16_value(c["kb"]), bf16_value(c["vb"]), c["table"], c["ctx"],
                                c["wl"].scale, BS, 0)
    for split in (0, 64):
        o = A.attn_decode_paged(dev_bf16(qb), c["kc"], c["vc"], c["tdev"], dev(c["ctx"]),
                                int(c["ctx"].max()), scale=c["wl"].scale, split_tokens=split)
        torch().cuda.synchronize()
        assert maxabs(host_f64(o), ro) <= BF16_TOL, split


@pytest.mark.parametrize("QL", [3, 5])  # 12 columns per KV head: decode kernels; 20: paged prefill
def test_decode_multi_bf16_blocks_above_4gib(bf16_case, QL):
    import attention_attn_prefill_amd as A
    c = bf16_case
    B = len(c["ctx"])
    qb, qf = new_tokens(4400 + QL, B * QL, Hq, D, "k")
    o = A.attn_decode_paged_multi(dev_bf16(qb.reshape(B, QL, Hq, D)), c["kc"], c["vc"], c["tdev"],
                                  dev(c["ctx"]), int(c["ctx"].max()), scale=c["wl"].scale)
    torch().cuda.synchronize()
    ro, _ = oracle.prefill_paged(qf, np.arange(B + 1) * QL, bf16_value(c["kb"]), bf16_value(c["vb"]),
                                 c["table"], c["ctx"], c["wl"].scale, BS, True, 0)
    assert maxabs(host_f64(o).reshape(ro.shape), ro) <= BF16_TOL


def test_prefill_paged_fused_append_blocks_above_4gib():
    """Chunks appended into high blocks by the fused append and attended in the same call."""
    import attention_attn_prefill_amd as A
    t = torch()
    ctx = np.array([300, 1000, 129], np.int32)
    q_len = np.array([300, 77, 129], np.int32)
    c = _bf16_case(ctx, seed=4500)
    T = int(q_len.sum())
    kn, _ = new_tokens(4501, T, Hkv, D, "k")
    vn, _ = new_tokens(4502, T, Hkv, D, "v")
    qb, _ = new_tokens(4503, T, Hq, D, "k")
    cu = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
    seq = np.repeat(np.arange(len(ctx)), q_len).astype(np.int32)
    pos = np.concatenate([np.arange(n - m, n) for n, m in zip(ctx, q_len)]).astype(np.int32)
    L = t.empty((T, Hq), dtype=t.float32, device="cuda")
    o = A.attn_prefill_paged(dev_bf16(qb), c["kc"], c["vc"], c["tdev"], dev(cu), dev(ctx),
                             int(q_len.max()), scale=c["wl"].scale, lse=L,
                             k_new=dev_bf16(kn), v_new=dev_bf16(vn))
    t.cuda.synchronize()
    kexp = oracle.append_expected(bf16_value(c["kb"]), bf16_value(kn), seq, pos, c["table"], BS)
    vexp = oracle.append_expected(bf16_value(c["vb"]), bf16_value(vn), seq, pos, c["table"], BS)
    # the written high blocks hold exactly the expected rows (compact order)
    for big, want in ((c["kc"], kexp), (c["vc"], vexp)):
        got = host_bits(_gather(big, c["phys"]))
        assert np.array_equal(got, (np.asarray(want, np.float32).view(np.uint32) >> 16).astype(np.uint16))
    ro, rl = oracle.prefill_paged(bf16_value(qb), cu, kexp, vexp, c["table"], ctx, c["wl"].scale,
                                  BS, True, 0)
    assert maxabs(host_f64(o), ro) <= BF16_TOL
    assert maxabs(host_f64(L), rl) <= LSE_TOL_BF16
    c.clear()
    t.cuda.empty_cache()


def test_int8_append_and_decode_blocks_above_4gib():
    """kv_cache_append quantizing into high blocks (codes and scales bit-exact), then decode."""
    import attention_attn_prefill_amd as A
    t = torch()
    ctx = np.array([5, 1200, 333], np.int32)
    wl = DecodeWorkload("high_i8", 4600, "i8", len(ctx), Hq, Hkv, D, 1, int(ctx.max()))
    table, nb_c = paged_table(ctx, BS, 4600, 2, True)
    phys, nb = _high_ids(nb_c, Hkv * BS * D, 4601)
    (kc_c, ks_c), (vc_c, vs_c) = int8_pool(wl, "k", nb_c), int8_pool(wl, "v", nb_c)
    kc = _scatter((Hkv, BS, D), t.int8, nb, phys, dev(kc_c))
    vc = _scatter((Hkv, BS, D), t.int8, nb, phys, dev(vc_c))
    ks = _scatter((Hkv, BS), t.float16, nb, phys, dev(ks_c))
    vs = _scatter((Hkv, BS), t.float16, nb, phys, dev(vs_c))
    assert kc.numel() > (1 << 32) and int(phys.min()) * Hkv * BS * D >= (1 << 32)
    tdev = dev(_remap(table, phys))
    # overwrite the last 40 tokens of sequence 1 and all of sequence 2 through the append kernel
    seq = np.concatenate([np.full(40, 1), np.full(333, 2)]).astype(np.int32)
    pos = np.concatenate([np.arange(1160, 1200), np.arange(333)]).astype(np.int32)
    kn, kf = new_tokens(4602, len(seq), Hkv, D, "k")
    vn, vf = new_tokens(4603, len(seq), Hkv, D, "v")
    A.kv_cache_append(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), tdev, kc, vc, k_scale=ks, v_scale=vs)
    t.cuda.synchronize()
    want = {}
    for name, pc, ps, rows in (("k", kc_c, ks_c, kf), ("v", vc_c, vs_c, vf)):
        codes, scales = oracle.quantize_int8(rows)
        want[name] = (oracle.append_expected(pc, codes, seq, pos, table, BS),
                      oracle.append_expected(ps, scales, seq, pos, table, BS))
    for name, gc, gs in (("k", kc, ks), ("v", vc, vs)):
        assert np.array_equal(_gather(gc, phys).cpu().numpy(), want[name][0]), name
        assert np.array_equal(_gather(gs, phys).cpu().numpy().view(np.uint16),
                              want[name][1].view(np.uint16)), name
    qb, qf = new_tokens(4604, len(ctx), Hq, D, "k")
    o = A.attn_decode_paged(dev_bf16(qb), kc, vc, tdev, dev(ctx), int(ctx.max()), k_scale=ks,
                            v_scale=vs, scale=wl.scale)
    t.cuda.synchronize()
    ro, _ = oracle.decode_paged(qf, want["k"][0], want["v"][0], table, ctx, wl.scale, BS, 0,
                                k_scale=want["k"][1], v_scale=want["v"][1])
    assert maxabs(host_f64(o), ro) <= BF16_TOL
    del kc, vc, ks, vs
    t.cuda.empty_cache()


def test_prefill_contiguous_tensors_above_4gib():
    """Contiguous prefill with Q, K, V and O of 4.4 GB each (130 x 16384 rows, 8 heads, D = 128,
    causal window 32): rows of the batches whose offsets pass 2^31 and 2^32 bytes."""
    import attention_attn_prefill_amd as A
    t = torch()
    B, S, H, W = 130, 16384, 8, 32
    gen = t.Generator(device="cuda").manual_seed(4700)
    q, k, v = (t.randn((B, S, H, D), device="cuda", generator=gen, dtype=t.bfloat16) for _ in range(3))
    assert q.numel() * 2 > (1 << 32)
    L = t.empty((B, H, S), dtype=t.float32, device="cuda")
    o = A.attn_prefill(q, k, v, causal=True, window=W, lse=L)
    t.cuda.synchronize()
    rows = [0, 1, 31, 32, 33, 1000, 8191, 16383]
    for b in (64, 129):  # row offsets past 2^31 and past 2^32 bytes
        for h in (0, 7):
            qs = host_f64(q[b, rows, h])
            ks, vs = host_f64(k[b, :, h]), host_f64(v[b, :, h])
            ro, rl = oracle.attention_head(qs, ks, vs, D ** -0.5, rows, True, W)
            assert maxabs(host_f64(o[b, rows, h]), ro) <= BF16_TOL, (b, h)
            assert maxabs(host_f64(L[b, h, rows]), rl) <= LSE_TOL_BF16, (b, h)
    del q, k, v, o, L
    t.cuda.empty_cache()
