"""GPU parity of attn_decode_paged_multi (q_len draft rows per sequence, causal among them)
against the oracle's chunked prefill over the paged cache (bottom-right aligned rows)."""
import numpy as np
import pytest

import oracle
from synth import DecodeWorkload, bf16_value, context_lens, int8_pool, new_tokens, paged_table, pool
from tests.gpu_util import BF16_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu


def _case(ctx, QL, Hq, Hkv, D, seed, window=0, kv="bf16", spare=3):
    ctx = np.array(ctx, np.int32)
    B = len(ctx)
    wl = DecodeWorkload("multi", seed, kv, B, Hq, Hkv, D, 1, int(ctx.max()), 16, window)
    table, nb = paged_table(ctx, 16, seed, spare, True)
    qb, qf = new_tokens(seed + 3, B * QL, Hq, D, "k")
    c = dict(wl=wl, ctx=ctx, QL=QL, table=table, nb=nb, qb=qb.reshape(B, QL, Hq, D), qf=qf)
    if kv == "bf16":
        kb, vb = pool(wl, "k", nb), pool(wl, "v", nb)
        c.update(kc=dev_bf16(kb), vc=dev_bf16(vb), ks=None, vs=None, kf=bf16_value(kb), vf=bf16_value(vb))
    else:
        (kc, ks), (vc, vs) = int8_pool(wl, "k", nb), int8_pool(wl, "v", nb)
        c.update(kc=dev(kc), vc=dev(vc), ks=dev(ks), vs=dev(vs),
                 kf=oracle.dequantize_int8(kc, ks), vf=oracle.dequantize_int8(vc, vs))
    return c


def _run(c, split=0, rows=None):
    import attention_attn_prefill_amd as A
    wl = c["wl"]
    o = A.attn_decode_paged_multi(dev_bf16(c["qb"]), c["kc"], c["vc"], dev(c["table"]), dev(c["ctx"]),
                                  int(c["ctx"].max()), k_scale=c["ks"], v_scale=c["vs"], scale=wl.scale,
                                  window=wl.window, split_tokens=split)
    torch().cuda.synchronize()
    return o


def _expected(c, seqs=None):
    B, QL = len(c["ctx"]), c["QL"]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    q = c["qf"].reshape(B, QL, *c["qf"].shape[1:])[seqs].reshape(len(seqs) * QL, *c["qf"].shape[1:])
    cu = np.arange(len(seqs) + 1) * QL
    o, _ = oracle.prefill_paged(q, cu, c["kf"], c["vf"], c["table"][seqs], c["ctx"][seqs],
                                c["wl"].scale, 16, True, c["wl"].window)
    return o.reshape(len(seqs), QL, *o.shape[1:])


CASES = [
    # ctx, QL, Hq, Hkv, D, window, kv
    ((4, 17, 100, 333, 2000), 4, 32, 8, 64, 0, "bf16"),
    ((16, 50, 700), 2, 16, 2, 128, 0, "bf16"),
    ((9, 64, 1000, 129), 8, 8, 4, 64, 0, "bf16"),
    ((300, 1500, 40), 4, 8, 2, 128, 100, "bf16"),
    ((20, 3000), 3, 20, 4, 64, 7, "bf16"),
    ((5, 800, 2100), 4, 32, 8, 128, 0, "i8"),
    ((33, 700), 2, 64, 8, 128, 64, "i8"),
    ((1, 2, 3), 1, 8, 2, 64, 0, "bf16"),
    # more than 16 query columns per KV head, bf16: virtual KV heads where two of them per cache
    # head suffice, else the paged prefill kernel
    ((9, 17, 100, 333, 2000), 8, 32, 8, 64, 0, "bf16"),   # 4 heads x 8 rows: R = 2
    ((16, 50, 700), 6, 32, 8, 128, 0, "bf16"),            # R = 2
    ((300, 1500, 40), 8, 16, 4, 64, 100, "bf16"),         # R = 2
    ((20, 3000), 5, 20, 4, 64, 7, "bf16"),                # 5 heads x 5 rows: prefill kernel
    ((13, 64, 1000, 129), 12, 16, 4, 64, 0, "bf16"),      # 4 heads x 12 rows: prefill kernel
    ((300, 1500, 40), 9, 6, 2, 128, 100, "bf16"),         # 3 heads x 9 rows: prefill kernel
    # ... and with an INT8 cache: virtual KV heads (each cache head read once per virtual head)
    ((9, 17, 100, 333, 2000), 8, 32, 8, 64, 0, "i8"),
    ((16, 50, 700), 5, 20, 4, 128, 0, "i8"),
    ((300, 1500, 40), 6, 24, 4, 128, 100, "i8"),
]


@pytest.mark.parametrize("split", [0, 32])
@pytest.mark.parametrize("ctx,QL,Hq,Hkv,D,window,kv", CASES)
def test_decode_multi_matches_oracle(ctx, QL, Hq, Hkv, D, window, kv, split):
    c = _case(ctx, QL, Hq, Hkv, D, seed=900 + QL + D + window + len(ctx), window=window, kv=kv)
    o = _run(c, split)
    assert maxabs(host_f64(o), _expected(c)) <= BF16_TOL


def test_decode_multi_one_row_equals_single_token_decode():
    """q_len = 1 is attn_decode_paged, bit for bit (same kernels, same split)."""
    import attention_attn_prefill_amd as A
    c = _case((17, 400, 1333), 1, 32, 8, 64, seed=950)
    for split in (0, 64):
        o = host_bits(_run(c, split))[:, 0]
        wl = c["wl"]
        o1 = A.attn_decode_paged(dev_bf16(c["qb"][:, 0]), c["kc"], c["vc"], dev(c["table"]), dev(c["ctx"]),
                                 int(c["ctx"].max()), scale=wl.scale, split_tokens=split)
        torch().cuda.synchronize()
        assert np.array_equal(o, host_bits(o1))


def test_decode_multi_last_row_equals_decode_and_rows_are_causal():
    """Row r only sees keys up to its own position: its output equals a single-token decode
    of a context cut to that position (same cache, same table)."""
    import attention_attn_prefill_amd as A
    c = _case((40, 513), 4, 16, 4, 128, seed=960)
    got = host_f64(_run(c))
    wl = c["wl"]
    for r in range(4):
        ctx_r = c["ctx"] - 4 + r + 1
        o1 = A.attn_decode_paged(dev_bf16(np.ascontiguousarray(c["qb"][:, r])), c["kc"], c["vc"], dev(c["table"]),
                                 dev(ctx_r), int(ctx_r.max()), scale=wl.scale)
        torch().cuda.synchronize()
        assert maxabs(got[:, r], host_f64(o1)) <= 1e-2


def test_decode_multi_rows_before_the_sequence_are_zero():
    c = _case((2, 30), 4, 8, 2, 64, seed=970)  # sequence 0 holds 2 tokens: rows 0, 1 sit at -2, -1
    got = host_f64(_run(c))
    assert (got[0, :2] == 0).all()
    exp = _expected(c, seqs=[1])
    assert maxabs(got[1], exp[0]) <= BF16_TOL


@pytest.mark.parametrize("QL", [8, 12])  # virtual KV heads (R = 2), the paged prefill kernel
def test_decode_multi_wide_rows_before_the_sequence_are_zero(QL):
    """Both wide paths keep the decode rows' meaning: with QL rows against a 3-token context,
    rows 0..QL-4 sit at negative positions and are zeros; the last three sit at 0, 1, 2."""
    c = _case((3, 40), QL, 32, 8, 64, seed=975 + QL)
    got = host_f64(_run(c))
    assert (got[0, :QL - 3] == 0).all()
    q0 = c["qf"].reshape(2, QL, *c["qf"].shape[1:])[0, QL - 3:]
    o0, _ = oracle.prefill_paged(q0, np.array([0, 3]), c["kf"], c["vf"], c["table"][:1], c["ctx"][:1],
                                 c["wl"].scale, 16, True, 0)
    assert maxabs(got[0, QL - 3:], o0) <= BF16_TOL
    assert maxabs(got[1], _expected(c, seqs=[1])[0]) <= BF16_TOL


def test_decode_multi_llama1b_eight_drafts_sampled():
    """Llama-3.2-1B-shaped verification of 8 draft tokens (4 heads x 8 rows = 32 columns per KV
    head: two virtual KV heads per cache head): sampled sequences against the oracle."""
    wl0 = DecodeWorkload("decode_llama1b_b64", 1003, "bf16", 64, 32, 8, 64, 512, 4096)
    ctx = context_lens(wl0)
    c = _case(tuple(int(x) for x in ctx), 8, 32, 8, 64, seed=1308, spare=0)
    got = host_f64(_run(c))
    seqs = [0, 5, 33, 63]
    assert maxabs(got[seqs], _expected(c, seqs)) <= BF16_TOL


def test_decode_multi_llama1b_sampled():
    """Llama-3.2-1B-shaped verification step: 64 sequences, contexts uniform in [512, 4096],
    4 draft rows each (16 MFMA columns per KV head); sampled sequences against the oracle."""
    wl0 = DecodeWorkload("decode_llama1b_b64", 1003, "bf16", 64, 32, 8, 64, 512, 4096)
    ctx = context_lens(wl0)
    c = _case(tuple(int(x) for x in ctx), 4, 32, 8, 64, seed=1303, spare=0)
    got = host_f64(_run(c))
    seqs = [0, 1, 17, 40, 63]
    assert maxabs(got[seqs], _expected(c, seqs)) <= BF16_TOL
