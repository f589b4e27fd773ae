"""GPU parity of attn_prefill_paged (chunked prefill over the paged cache, fused append)."""
import numpy as np
import pytest

import oracle
from synth import DecodeWorkload, bf16_value, decode_query, new_tokens, paged_table, pool
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu
LSE_TOL_BF16 = 4e-3  # l sums bf16-rounded probabilities: ln l within 2^-9 of the exact LSE


def _case(ctx, q_len, Hq, Hkv, D, seed, spare=3):
    """Pool holding every sequence's prefix (random), the chunk's new rows, packed queries."""
    ctx = np.array(ctx, np.int32)
    q_len = np.array(q_len, np.int32)
    wl = DecodeWorkload("chunk", seed, "bf16", len(ctx), Hq, Hkv, D, 1, int(ctx.max()))
    table, nb = paged_table(ctx, 16, seed, spare, True)
    kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
    T = int(q_len.sum())
    kn, _ = new_tokens(seed + 1, T, Hkv, D, "k")
    vn, _ = new_tokens(seed + 2, T, Hkv, D, "v")
    qb, _ = new_tokens(seed + 3, T, Hq, D, "k")  # packed query rows [T][Hq][D]
    cu = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
    seq = np.repeat(np.arange(len(ctx)), q_len).astype(np.int32)
    pos = np.concatenate([np.arange(c - n, c) for c, n in zip(ctx, q_len)]).astype(np.int32)
    return dict(ctx=ctx, q_len=q_len, table=table, nb=nb, kb=kb, vb=vb, kn=kn, vn=vn, qb=qb, cu=cu,
                seq=seq, pos=pos, scale=D ** -0.5)


def _bits(x):
    """bf16 bit patterns of bf16-representable values."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _run(c, window=0, causal=True, fused=True):
    import attention_attn_prefill_amd as A
    t = torch()
    kc, vc = dev_bf16(c["kb"]), dev_bf16(c["vb"])
    T, Hq = c["qb"].shape[0], c["qb"].shape[1]
    L = t.empty((T, Hq), dtype=t.float32, device="cuda")
    kw = dict(k_new=dev_bf16(c["kn"]), v_new=dev_bf16(c["vn"])) if fused else {}
    o = A.attn_prefill_paged(dev_bf16(c["qb"]), kc, vc, dev(c["table"]), dev(c["cu"]), dev(c["ctx"]),
                             int(c["q_len"].max()), scale=c["scale"], causal=causal, window=window,
                             lse=L, **kw)
    t.cuda.synchronize()
    return o, L, kc, vc


def _expected(c, window, causal=True):
    kexp = oracle.append_expected(bf16_value(c["kb"]), bf16_value(c["kn"]), c["seq"], c["pos"], c["table"], 16)
    vexp = oracle.append_expected(bf16_value(c["vb"]), bf16_value(c["vn"]), c["seq"], c["pos"], c["table"], 16)
    o, lse = oracle.prefill_paged(bf16_value(c["qb"]), c["cu"], kexp, vexp, c["table"], c["ctx"],
                                  c["scale"], 16, causal, window)
    return o, lse, kexp, vexp


CASES = [
    # ctx, q_len, Hq, Hkv, D, window
    ((300, 17, 1000, 64), (300, 1, 130, 64), 8, 2, 64, 0),     # whole, single row, ragged chunks
    ((200, 555, 33), (0, 200, 33), 4, 4, 128, 0),                # an empty chunk
    ((2000, 129), (700, 129), 32, 8, 128, 300),                  # window
    ((64, 65, 1), (64, 32, 1), 16, 2, 64, 1),                    # window 1
    ((900,), (257,), 12, 4, 64, 0),
    ((3000, 2500), (96, 96), 8, 1, 128, 0),
]


@pytest.mark.parametrize("ctx,q_len,Hq,Hkv,D,window", CASES)
def test_prefill_paged_matches_oracle(ctx, q_len, Hq, Hkv, D, window):
    c = _case(ctx, q_len, Hq, Hkv, D, seed=600 + D + window + len(ctx))
    o, L, kc, vc = _run(c, window)
    ro, rl, kexp, vexp = _expected(c, window)
    # fused append wrote exactly the chunk rows
    assert np.array_equal(host_bits(kc), _bits(kexp))
    assert np.array_equal(host_bits(vc), _bits(vexp))
    if o.shape[0]:
        assert maxabs(host_f64(o), ro) <= BF16_TOL
        assert maxabs(host_f64(L), rl) <= LSE_TOL_BF16


def test_prefill_paged_without_append_and_non_causal():
    c = _case((400, 90), (120, 90), 8, 2, 128, seed=777)
    # pre-fill the cache on the host side (test-side placement), then call without k_new/v_new
    kexp = oracle.append_expected(bf16_value(c["kb"]), bf16_value(c["kn"]), c["seq"], c["pos"], c["table"], 16)
    vexp = oracle.append_expected(bf16_value(c["vb"]), bf16_value(c["vn"]), c["seq"], c["pos"], c["table"], 16)
    c2 = dict(c)
    c2["kb"], c2["vb"] = _bits(kexp), _bits(vexp)
    for causal in (True, False):
        o, L, _, _ = _run(c2, 0, causal, fused=False)
        ro, rl = oracle.prefill_paged(bf16_value(c["qb"]), c["cu"], kexp, vexp, c["table"], c["ctx"],
                                      c["scale"], 16, causal, 0)
        assert maxabs(host_f64(o), ro) <= BF16_TOL


@pytest.mark.parametrize("D,window", [(64, 0), (128, 0), (64, 37), (128, 200)])
def test_prefill_paged_fused_append_reads_what_the_cache_holds(D, window):
    # The fused call takes the chunk's keys from k_new / v_new while it writes them to the
    # cache; a second call without k_new reads the same values from the cache. Same bf16 inputs
    # in the same order, so O and the LSE must agree bit for bit.
    c = _case((300, 61, 17), (100, 61, 17), 8, 2, D, seed=4242 + D + window)
    o1, L1, kc, vc = _run(c, window)
    import attention_attn_prefill_amd as A
    t = torch()
    L2 = t.empty_like(L1)
    o2 = A.attn_prefill_paged(dev_bf16(c["qb"]), kc, vc, dev(c["table"]), dev(c["cu"]), dev(c["ctx"]),
                              int(c["q_len"].max()), scale=c["scale"], causal=True, window=window, lse=L2)
    t.cuda.synchronize()
    assert np.array_equal(host_bits(o1), host_bits(o2))
    assert np.array_equal(L1.cpu().numpy().view(np.uint32), L2.cpu().numpy().view(np.uint32))


def test_prefill_paged_whole_sequence_equals_contiguous_prefill():
    """A chunk covering the whole sequence is ordinary prefill: compare with attn_prefill."""
    import attention_attn_prefill_amd as A
    t = torch()
    S, Hq, Hkv, D = 333, 8, 2, 64
    c = _case((S,), (S,), Hq, Hkv, D, seed=901, spare=0)
    o, _, _, _ = _run(c, 0)
    q = dev_bf16(c["qb"][None])
    k = dev_bf16(c["kn"][None])
    v = dev_bf16(c["vn"][None])
    oc = A.attn_prefill(q, k, v, scale=c["scale"], causal=True)
    t.cuda.synchronize()
    assert maxabs(host_f64(o), host_f64(oc)[0]) <= 1e-2


def test_prefill_paged_llama1b_chunk_sampled():
    """Llama-3.2-1B-shaped chunked prefill: 4 sequences with 3072-token prefixes, 1024-token
    chunks (4096 keys each), 32/8 heads, D = 64; sampled rows against the oracle, every row
    (O and LSE) of two (sequence, head) pairs on different KV heads, and the cache bits the
    fused append wrote."""
    c = _case((4096,) * 4, (1024,) * 4, 32, 8, 64, seed=1234, spare=0)
    o, L, kc, vc = _run(c, 0)
    got, gl = host_f64(o), host_f64(L)
    kexp = oracle.append_expected(bf16_value(c["kb"]), bf16_value(c["kn"]), c["seq"], c["pos"], c["table"], 16)
    vexp = oracle.append_expected(bf16_value(c["vb"]), bf16_value(c["vn"]), c["seq"], c["pos"], c["table"], 16)
    assert np.array_equal(host_bits(kc), _bits(kexp)) and np.array_equal(host_bits(vc), _bits(vexp))
    for b, h in ((1, 9), (2, 22)):
        sel = np.arange(c["cu"][b], c["cu"][b + 1])
        kk = oracle.gather_logical(kexp, c["table"][b], 4096, 16)
        vv = oracle.gather_logical(vexp, c["table"][b], 4096, 16)
        ro, rl = oracle.attention_head(bf16_value(c["qb"])[sel][:, h], kk[:, h // 4], vv[:, h // 4],
                                       c["scale"], 3072 + np.arange(1024), True, 0)
        assert maxabs(got[sel, h], ro) <= BF16_TOL
        assert maxabs(gl[sel, h], rl) <= LSE_TOL_BF16
    rows = np.array([0, 1, 31, 32, 63, 64, 511, 1022, 1023])
    for b in (0, 3):
        sel = c["cu"][b] + rows
        cu = np.array([0, len(rows)])
        # sampled rows: same keys, positions of the sampled rows
        q = bf16_value(c["qb"])[sel]
        kk = oracle.gather_logical(kexp, c["table"][b], 4096, 16)
        vv = oracle.gather_logical(vexp, c["table"][b], 4096, 16)
        for h in (0, 5, 31):
            ro, _ = oracle.attention_head(q[:, h], kk[:, h // 4], vv[:, h // 4], c["scale"], 3072 + rows, True, 0)
            assert maxabs(got[sel, h], ro) <= BF16_TOL


def _poison(c, window):
    """Copy of case c whose invisible cache content is NaN: slots past each context, spare
    blocks, and blocks wholly left of the window of every row of the chunk; the table entries
    of blocks no row can see (past the context, left of the window) become -1."""
    nan = np.uint16(0x7FC0)
    p = dict(c)
    kb, vb, table = c["kb"].copy(), c["vb"].copy(), c["table"].copy()
    live = np.zeros(kb.shape[0] * 16, bool)
    for b, (ctx, n) in enumerate(zip(c["ctx"], c["q_len"])):
        first = max(0, int(ctx) - int(n) - window + 1) if window > 0 and n > 0 else 0
        for t in range(first - first % 16, int(ctx)):  # blocks holding a visible key
            live[int(table[b][t // 16]) * 16 + t % 16] = t >= first
        table[b, : first // 16] = -1
        table[b, -(-int(ctx) // 16):] = -1
    for s in np.nonzero(~live)[0]:
        kb[s // 16, :, s % 16] = nan
        vb[s // 16, :, s % 16] = nan
    p.update(kb=kb, vb=vb, table=table)
    return p


@pytest.mark.parametrize("ctx,q_len,Hq,Hkv,D,window", [
    ((300, 17, 1000, 70), (300, 1, 130, 6), 8, 2, 64, 0),
    ((2000, 129, 77), (700, 129, 5), 8, 2, 128, 300),
])
def test_prefill_paged_ignores_invisible_cache_content(ctx, q_len, Hq, Hkv, D, window):
    """NaN in every cache slot no row can see, and -1 table entries for the blocks no row can
    see, leave the output unchanged (0 * NaN must never reach the PV contraction)."""
    c = _case(ctx, q_len, Hq, Hkv, D, seed=650 + D + window)
    ro, rl, _, _ = _expected(c, window)
    o, L, _, _ = _run(_poison(c, window), window)
    got = host_f64(o)
    assert np.isfinite(got).all()
    assert maxabs(got, ro) <= BF16_TOL
    assert maxabs(host_f64(L), rl) <= LSE_TOL_BF16
