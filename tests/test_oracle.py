"""Pins for the fp64 oracle: each test ties it to something other than itself.

Closed forms, special cases, brute force and an independent library routine (torch's CPU
float64 scaled_dot_product_attention). Every mistake of the usual kind -- a dropped scale, a
mask off by one, a wrong GQA head map, a transposed operand, a wrong block/slot split --
fails at least one of these (test_mutants_are_caught plants such mistakes in copies).
"""
import math

import numpy as np
import pytest

import oracle
from synth import bf16_value, bf16_bits, context_lens, paged_table, WORKLOADS

RNG = np.random.default_rng(12345)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# --- P1: normalisation -------------------------------------------------------------------
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 3), (False, 0), (False, 2)])
def test_ones_v_gives_ones(causal, window):
    """V == 1 => O == 1: the softmax weights of every row sum to one."""
    q, k = _rand(2, 7, 4, 8), _rand(2, 7, 2, 8)
    v = np.ones((2, 7, 2, 8))
    o, _ = oracle.attention(q, k, v, 0.3, causal, window)
    assert np.abs(o - 1).max() < 1e-14


def test_lse_closed_form():
    """lse is log(sum exp s) of the visible scores (2 keys, hand-set scores 0 and ln 3)."""
    k = np.array([[1.0, 0.0], [0.0, 1.0]])
    q = np.array([[0.0, math.log(3.0)]])
    v = np.array([[4.0, 0.0], [0.0, 8.0]])
    o, lse = oracle.attention_head(q, k, v, 1.0, [1], causal=True)
    # weights 1/4 and 3/4
    assert np.allclose(o, [[1.0, 6.0]], atol=1e-15)
    assert abs(lse[0] - math.log(4.0)) < 1e-15


# --- P2: single visible key ---------------------------------------------------------------
def test_single_key_rows():
    """Prefill row 0 sees only key 0: O = V[0] of the mapped KV head, exactly."""
    q, k, v = _rand(1, 5, 6, 4), _rand(1, 5, 3, 4), _rand(1, 5, 3, 4)
    o, lse = oracle.attention(q, k, v, 0.5, causal=True)
    for h in range(6):
        assert np.array_equal(o[0, 0, h], v[0, 0, h // 2])
        assert lse[0, h, 0] == pytest.approx(0.5 * q[0, 0, h] @ k[0, 0, h // 2], abs=1e-15)


def test_decode_ctx1_returns_v():
    q = _rand(3, 4, 8)
    kp, vp = _rand(5, 2, 4, 8), _rand(5, 2, 4, 8)
    table = np.array([[3, -1], [0, -1], [4, -1]], np.int32)
    o, _ = oracle.decode_paged(q, kp, vp, table, np.array([1, 1, 1]), 0.1, 4)
    for b, pb in enumerate([3, 0, 4]):
        for h in range(4):
            assert np.array_equal(o[b, h], vp[pb, h // 2, 0])


# --- P3: uniform scores -> mean of the visible V rows -------------------------------------
@pytest.mark.parametrize("window", [0, 1, 3, 100])
def test_zero_query_gives_window_mean(window):
    S = 9
    v = _rand(1, S, 1, 3)
    q, k = np.zeros((1, S, 1, 3)), _rand(1, S, 1, 3)
    o, _ = oracle.attention(q, k, v, 1.0, True, window)
    for i in range(S):
        lo = 0 if window == 0 else max(0, i - window + 1)
        assert np.allclose(o[0, i, 0], v[0, lo:i + 1, 0].mean(axis=0), atol=1e-14)


# --- P4: window edge ------------------------------------------------------------------------
def test_window_one_is_identity_and_wide_window_is_causal():
    q, k, v = _rand(2, 6, 2, 5), _rand(2, 6, 2, 5), _rand(2, 6, 2, 5)
    o1, _ = oracle.attention(q, k, v, 0.7, True, 1)
    assert np.array_equal(o1, v)
    ow, _ = oracle.attention(q, k, v, 0.7, True, 6)
    oc, _ = oracle.attention(q, k, v, 0.7, True, 0)
    assert np.abs(ow - oc).max() < 1e-15


# --- P5: GQA == MHA with repeated KV heads -------------------------------------------------
def test_gqa_equals_repeated_mha():
    q, k, v = _rand(2, 7, 8, 4), _rand(2, 7, 2, 4), _rand(2, 7, 2, 4)
    og, _ = oracle.attention(q, k, v, 0.4, True, 3)
    om, _ = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.4, True, 3)
    assert np.abs(og - om).max() < 1e-15


# --- P6 / P7: paged layout ------------------------------------------------------------------
def _paged_case(seed, bs, spare, permute, B=3, Hkv=2, D=4, ctx=(5, 1, 11)):
    rng = np.random.default_rng(seed)
    ctx = np.array(ctx[:B], np.int32)
    table, nb = paged_table(ctx, bs, seed, spare, permute)
    kp, vp = rng.standard_normal((nb, Hkv, bs, D)), rng.standard_normal((nb, Hkv, bs, D))
    return ctx, table, kp, vp


def _contiguous_from_paged(pool, table, ctx, bs):
    """Inverse view built by scanning pool slots (independent of gather_logical)."""
    out = []
    for b in range(len(ctx)):
        rows = []
        for t in range(int(ctx[b])):
            hits = [(pb, off) for pb in range(pool.shape[0]) for off in range(bs)
                    if table[b][t // bs] == pb and off == t - bs * (t // bs)]
            assert len(hits) == 1
            rows.append(pool[hits[0][0], :, hits[0][1]])
        out.append(np.array(rows))
    return out


@pytest.mark.parametrize("bs", [1, 2, 3, 4])
def test_paged_equals_contiguous_any_permutation(bs):
    q = _rand(3, 4, 4)
    outs = []
    for permute, seed in ((False, 1), (True, 2), (True, 3)):
        ctx, table, kp, vp = _paged_case(seed, bs, 2, permute)
        # same logical contents under every table: write logical rows through the table
        rng = np.random.default_rng(99)
        logical_k = [rng.standard_normal((int(c), 2, 4)) for c in ctx]
        logical_v = [rng.standard_normal((int(c), 2, 4)) for c in ctx]
        for b in range(3):
            for t in range(int(ctx[b])):
                kp[table[b][t // bs], :, t % bs] = logical_k[b][t]
                vp[table[b][t // bs], :, t % bs] = logical_v[b][t]
        o, _ = oracle.decode_paged(q, kp, vp, table, ctx, 0.3, bs)
        outs.append(o)
        # contiguous reference per sequence, from the slot-scanning inverse view
        kc = _contiguous_from_paged(kp, table, ctx, bs)
        vc = _contiguous_from_paged(vp, table, ctx, bs)
        for b in range(3):
            oc, _ = oracle.attention(q[b][None, None], kc[b][None], vc[b][None], 0.3, True)
            assert np.abs(o[b] - oc[0, 0]).max() < 1e-14
    assert np.abs(outs[0] - outs[1]).max() < 1e-14
    assert np.abs(outs[0] - outs[2]).max() < 1e-14


def test_poisoned_unused_slots_never_read():
    bs = 4
    ctx, table, kp, vp = _paged_case(7, bs, 3, True)
    q = _rand(3, 4, 4)
    o_ref, _ = oracle.decode_paged(q, kp, vp, table, ctx, 0.3, bs)
    used = {(int(table[b][t // bs]), t % bs) for b in range(3) for t in range(int(ctx[b]))}
    for pb in range(kp.shape[0]):
        for off in range(bs):
            if (pb, off) not in used:
                kp[pb, :, off] = np.nan
                vp[pb, :, off] = np.nan
    o, _ = oracle.decode_paged(q, kp, vp, table, ctx, 0.3, bs)
    assert np.isfinite(o).all() and np.array_equal(o, o_ref)


def test_window_left_blocks_never_read():
    """Blocks wholly left of the window may hold anything (table entries too)."""
    bs, W = 4, 5
    ctx, table, kp, vp = _paged_case(8, bs, 0, True, ctx=(13, 9, 11))
    q = _rand(3, 4, 4)
    o_ref, _ = oracle.decode_paged(q, kp, vp, table, ctx, 0.3, bs, window=W)
    kp2, vp2 = kp.copy(), vp.copy()
    for b in range(3):
        first_visible = int(ctx[b]) - W
        for t in range(first_visible):
            kp2[table[b][t // bs], :, t % bs] = np.nan
            vp2[table[b][t // bs], :, t % bs] = np.nan
    o, _ = oracle.decode_paged(q, kp2, vp2, table, ctx, 0.3, bs, window=W)
    assert np.isfinite(o).all() and np.abs(o - o_ref).max() < 1e-14


# --- P8: brute force in pure Python -----------------------------------------------------------
def _brute(q, k, v, scale, causal, window):
    B, Sq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, Hq, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            g = h * Hkv // Hq
            for i in range(Sq):
                P = Lk - Sq + i
                keys = [j for j in range(Lk) if (not causal or j <= P) and (window == 0 or P - j < window)]
                s = [scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, g, d]) for d in range(D)) for j in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for d in range(v.shape[3]):
                    out[b, i, h, d] = math.fsum(e[n] * float(v[b, j, g, d]) for n, j in enumerate(keys)) / tot
    return out


@pytest.mark.parametrize("B,Sq,Lk,Hq,Hkv,D,causal,window", [
    (1, 1, 1, 1, 1, 1, True, 0), (2, 9, 9, 4, 2, 4, True, 0), (2, 9, 9, 4, 2, 3, True, 3),
    (1, 6, 6, 2, 2, 4, False, 0), (2, 3, 8, 4, 1, 2, True, 0), (1, 1, 7, 4, 2, 4, True, 3),
    (2, 5, 5, 3, 1, 4, True, 1), (1, 4, 9, 2, 1, 3, False, 4),
])
def test_brute_force(B, Sq, Lk, Hq, Hkv, D, causal, window):
    rng = np.random.default_rng(B * 1000 + Sq * 100 + Lk)
    q, k, v = rng.standard_normal((B, Sq, Hq, D)), rng.standard_normal((B, Lk, Hkv, D)), rng.standard_normal((B, Lk, Hkv, D))
    o, _ = oracle.attention(q, k, v, 0.6, causal, window)
    assert np.abs(o - _brute(q, k, v, 0.6, causal, window)).max() < 1e-12


@pytest.mark.parametrize("bs", [1, 2, 3])
@pytest.mark.parametrize("window", [0, 1, 3])
def test_brute_force_paged_decode(bs, window):
    rng = np.random.default_rng(bs * 10 + window)
    ctx = np.array([5, 2], np.int32)
    table, nb = paged_table(ctx, bs, 17 + bs, 1, True)
    kp, vp = rng.standard_normal((nb, 2, bs, 3)), rng.standard_normal((nb, 2, bs, 3))
    q = rng.standard_normal((2, 4, 3))
    o, _ = oracle.decode_paged(q, kp, vp, table, ctx, 0.5, bs, window)
    for b in range(2):
        n = int(ctx[b])
        kc = np.array([[kp[table[b][t // bs], g, t % bs] for g in range(2)] for t in range(n)])
        vc = np.array([[vp[table[b][t // bs], g, t % bs] for g in range(2)] for t in range(n)])
        ob = _brute(q[b][None, None], kc[None], vc[None], 0.5, True, window)
        assert np.abs(o[b] - ob[0, 0]).max() < 1e-12


# --- P9: prefill last row == decode over the same keys ---------------------------------------
def test_prefill_last_row_equals_decode():
    bs, S = 4, 10
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((1, S, 4, 8)), rng.standard_normal((1, S, 2, 8)), rng.standard_normal((1, S, 2, 8))
    op, _ = oracle.attention(q, k, v, 0.35, True, 4)
    table, nb = paged_table(np.array([S]), bs, 3, 0, True)
    kp, vp = np.zeros((nb, 2, bs, 8)), np.zeros((nb, 2, bs, 8))
    for t in range(S):
        kp[table[0][t // bs], :, t % bs] = k[0, t]
        vp[table[0][t // bs], :, t % bs] = v[0, t]
    od, _ = oracle.decode_paged(q[:, -1], kp, vp, table, np.array([S]), 0.35, bs, 4)
    assert np.abs(op[0, -1] - od[0]).max() < 1e-14


# --- P10: split + log-sum-exp merge == unsplit -------------------------------------------------
@pytest.mark.parametrize("cuts", [(3,), (1, 2, 9), (4, 8, 12)])
def test_merge_of_splits_equals_whole(cuts):
    rng = np.random.default_rng(11)
    Lk, D = 15, 6
    q, k, v = rng.standard_normal((2, D)), rng.standard_normal((Lk, D)), rng.standard_normal((Lk, D))
    o, lse = oracle.attention_head(q, k, v, 0.4, [Lk - 1, Lk - 1], causal=True)
    edges = [0, *cuts, Lk]
    outs, lses = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        if a == b:
            continue
        oo, ll = oracle.attention_head(q, k[a:b], v[a:b], 0.4, [b - a - 1] * 2, causal=True)
        outs.append(oo)
        lses.append(ll)
    # an empty split contributes weight zero
    outs.append(np.zeros_like(o))
    lses.append(np.full(2, -np.inf))
    om, lm = oracle.merge_partials(outs, lses)
    assert np.abs(om - o).max() < 1e-13 and np.abs(lm - lse).max() < 1e-13


# --- P11: an independent library routine ------------------------------------------------------
@pytest.mark.parametrize("S,Hq,Hkv,D,window", [(17, 4, 2, 8, 0), (33, 8, 2, 16, 5), (9, 2, 2, 4, 1)])
def test_matches_torch_sdpa_float64(S, Hq, Hkv, D, window):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(S)
    q, k, v = rng.standard_normal((2, S, Hq, D)), rng.standard_normal((2, S, Hkv, D)), rng.standard_normal((2, S, Hkv, D))
    o, _ = oracle.attention(q, k, v, 1 / math.sqrt(D), True, window)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    mask = j <= i
    if window:
        mask &= (i - j) < window
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ot = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=mask, scale=1 / math.sqrt(D), enable_gqa=True)
    assert np.abs(o - ot.permute(0, 2, 1, 3).numpy()).max() < 1e-12


# --- V linearity -------------------------------------------------------------------------------
def test_linear_in_v():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((1, 8, 2, 4)), rng.standard_normal((1, 8, 1, 4))
    v1, v2 = rng.standard_normal((1, 8, 1, 4)), rng.standard_normal((1, 8, 1, 4))
    o1, _ = oracle.attention(q, k, v1, 0.5, True, 3)
    o2, _ = oracle.attention(q, k, v2, 0.5, True, 3)
    o12, _ = oracle.attention(q, k, 2 * v1 - 3 * v2, 0.5, True, 3)
    assert np.abs(o12 - (2 * o1 - 3 * o2)).max() < 1e-13


# --- P12: INT8 quantizer closed forms -----------------------------------------------------------
def test_int8_hand_values():
    # absmax 1.27 -> s = fp16(0.01) = 0.01000213623046875; 1.27/s = 126.97 -> 127;
    # -0.635/s = -63.486 -> -63; 0.005/s = 0.49989 -> 0; 0.015/s = 1.4997 -> 1.
    x = np.array([[1.27, -0.635, 0.005, 0.015]], np.float32)
    codes, s = oracle.quantize_int8(x)
    assert s.dtype == np.float16 and float(s[0]) == 0.01000213623046875
    assert codes.tolist() == [[127, -63, 0, 1]]
    # exact halves round to even: s = 1 (absmax 127), 2.5 -> 2, 3.5 -> 4, -0.5 -> 0
    codes, s = oracle.quantize_int8(np.array([[127.0, 2.5, 3.5, -0.5]], np.float32))
    assert float(s[0]) == 1.0 and codes.tolist() == [[127, 2, 4, 0]]
    # the zero vector
    codes, s = oracle.quantize_int8(np.zeros((1, 4), np.float32))
    assert float(s[0]) == 0.0 and codes.tolist() == [[0, 0, 0, 0]]


def test_int8_error_bound_and_range():
    rng = np.random.default_rng(21)
    x = bf16_value(bf16_bits(rng.standard_normal((4096, 128)).astype(np.float32)))
    codes, s = oracle.quantize_int8(x)
    s64 = s.astype(np.float64)[:, None]
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(x.astype(np.float64) - codes * s64)
    assert (err <= s64 / 2 * (1 + 1e-6) + 1e-12).all()
    # the absmax element maps to +-127
    idx = np.abs(x).argmax(axis=1)
    assert (np.abs(codes[np.arange(4096), idx]) == 127).all()


# --- P13: append placement ---------------------------------------------------------------------
def test_append_writes_only_its_slots():
    bs = 3
    ctx = np.array([7, 4], np.int32)
    table, nb = paged_table(ctx, bs, 4, 2, True)
    pool = np.full((nb, 2, bs, 5), 777.0)
    seq = np.array([0, 1, 0, 1], np.int32)
    pos = np.array([6, 0, 2, 3], np.int32)
    rows = np.arange(4 * 2 * 5, dtype=np.float64).reshape(4, 2, 5)
    out = oracle.append_expected(pool, rows, seq, pos, table, bs)
    changed = {(pb, off) for pb in range(nb) for off in range(bs) if not (out[pb, :, off] == 777.0).all()}
    expect = {(int(table[0][2]), 0), (int(table[1][0]), 0), (int(table[0][0]), 2), (int(table[1][1]), 0)}
    assert changed == expect
    assert np.array_equal(out[table[0][2], :, 0], rows[0])
    assert np.array_equal(out[table[1][1], :, 0], rows[3])


# --- the pins catch planted mistakes ------------------------------------------------------------
def _mut_off_by_one(qpos, Lk, causal, window):
    qpos = np.asarray(qpos, np.int64)[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((qpos.shape[0], Lk), bool)
    if causal:
        vis &= j < qpos + (qpos == 0)  # diagonal dropped except row 0
    if window > 0:
        vis &= (qpos - j) < window
    return vis


def _mut_window_wide(qpos, Lk, causal, window):
    qpos = np.asarray(qpos, np.int64)[:, None]
    j = np.arange(Lk)[None, :]
    vis = np.ones((qpos.shape[0], Lk), bool)
    if causal:
        vis &= j <= qpos
    if window > 0:
        vis &= (qpos - j) <= window
    return vis


@pytest.mark.parametrize("mutant", [_mut_off_by_one, _mut_window_wide])
def test_mutants_are_caught(monkeypatch, mutant):
    import oracle.attn_fp64 as oa
    monkeypatch.setattr(oa, "visible_mask", mutant)
    with pytest.raises(AssertionError):
        test_brute_force(2, 9, 9, 4, 2, 3, True, 3)


def test_gqa_head_map_mutant_is_caught(monkeypatch):
    import oracle.attn_fp64 as oa
    orig = oa.attention_head

    def attention_mod(q, k, v, scale, causal=True, window=0):
        B, Sq, Hq, D = q.shape
        Hkv = k.shape[2]
        o = np.empty((B, Sq, Hq, v.shape[3]))
        lse = np.empty((B, Hq, Sq))
        for b in range(B):
            for h in range(Hq):
                g = h % Hkv  # wrong grouping
                o[b, :, h], lse[b, h] = orig(q[b, :, h], k[b, :, g], v[b, :, g], scale,
                                             np.arange(Sq) + k.shape[1] - Sq, causal, window)
        return o, lse
    monkeypatch.setattr(oracle, "attention", attention_mod)
    with pytest.raises(AssertionError):
        test_gqa_equals_repeated_mha()


# --- workload recipe sanity ---------------------------------------------------------------------
def test_workload_recipe():
    wl = WORKLOADS["decode_llama1b_b64"]
    ctx = context_lens(wl)
    assert ctx.min() >= 512 and ctx.max() <= 4096 and len(ctx) == 64
    table, nb = paged_table(ctx, 16, wl.seed)
    live = np.concatenate([table[b][: -(-int(c) // 16)] for b, c in enumerate(ctx)])
    assert sorted(live.tolist()) == list(range(nb))


def test_gather_mutants_are_caught(monkeypatch):
    import oracle.attn_fp64 as oa

    def swapped(pool, table_row, n_tokens, block_size):  # slot and block index exchanged
        t = np.arange(n_tokens)
        return pool[np.asarray(table_row)[t % block_size], :, t // block_size]
    monkeypatch.setattr(oa, "gather_logical", swapped)
    with pytest.raises((AssertionError, IndexError)):
        test_brute_force_paged_decode(2, 0)


def test_quantizer_rounding_mutant_is_caught(monkeypatch):
    import oracle.attn_fp64 as oa
    monkeypatch.setattr(oa.np, "rint", lambda x: np.floor(np.asarray(x) + 0.5))  # half away-ish
    try:
        with pytest.raises(AssertionError):
            test_int8_hand_values()
    finally:
        monkeypatch.undo()


def test_golden_regression():
    """Oracle outputs on a small seeded case, written by tests/golden/make_golden.py."""
    import json
    import os
    from tests.golden.make_golden import compute
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    with open(path) as f:
        stored = json.load(f)
    now = compute()
    for key, val in stored.items():
        assert np.abs(np.asarray(val) - np.asarray(now[key])).max() < 1e-12, key


# --- chunked prefill over the paged cache ---------------------------------------------------------
def _scatter(pool, table, rows_per_seq, bs):
    """Test-side placement of logical rows into a pool (independent of the oracle)."""
    for b, rows in enumerate(rows_per_seq):
        for t in range(len(rows)):
            pool[table[b][t // bs], :, t % bs] = rows[t]


@pytest.mark.parametrize("window", [0, 3, 50])
def test_prefill_paged_chunks_equal_full_prefill(window):
    """Each chunk of a sequence's queries against its paged prefix equals the full prefill rows."""
    rng = np.random.default_rng(31 + window)
    bs, Hq, Hkv, D = 4, 4, 2, 8
    S = np.array([13, 6, 20])
    table, nb = paged_table(S, bs, 9, 2, True)
    q = [rng.standard_normal((n, Hq, D)) for n in S]
    k = [rng.standard_normal((n, Hkv, D)) for n in S]
    v = [rng.standard_normal((n, Hkv, D)) for n in S]
    kp, vp = np.full((nb, Hkv, bs, D), np.nan), np.full((nb, Hkv, bs, D), np.nan)
    _scatter(kp, table, k, bs)
    _scatter(vp, table, v, bs)
    full = [oracle.attention(q[b][None], k[b][None], v[b][None], 0.4, True, window)[0][0] for b in range(3)]
    # three chunk rounds with ragged chunk sizes (0 allowed)
    cuts = [np.array([0, 5, 13]), np.array([0, 1, 6]), np.array([7, 20, 20])]
    done = np.zeros(3, int)
    for r in range(3):
        new = [min(int(cuts[r][b]), int(S[b])) - done[b] if r < 2 else int(S[b]) - done[b] for b in range(3)]
        new = [max(0, x) for x in new]
        ctx = done + np.array(new)
        cu = np.concatenate([[0], np.cumsum(new)])
        qc = np.concatenate([q[b][done[b]:ctx[b]] for b in range(3)])
        o, _ = oracle.prefill_paged(qc, cu, kp, vp, table, ctx, 0.4, bs, True, window)
        for b in range(3):
            assert np.abs(o[cu[b]:cu[b + 1]] - full[b][done[b]:ctx[b]]).max(initial=0) < 1e-13
        done = ctx


def test_prefill_paged_single_row_is_decode():
    rng = np.random.default_rng(77)
    bs = 3
    ctx = np.array([7, 1, 11], np.int32)
    table, nb = paged_table(ctx, bs, 5, 1, True)
    kp, vp = rng.standard_normal((nb, 2, bs, 4)), rng.standard_normal((nb, 2, bs, 4))
    q = rng.standard_normal((3, 4, 4))
    od, _ = oracle.decode_paged(q, kp, vp, table, ctx, 0.3, bs, 2)
    op, _ = oracle.prefill_paged(q, np.arange(4), kp, vp, table, ctx, 0.3, bs, True, 2)
    assert np.abs(od - op).max() < 1e-14


# ---- RoPE (rotary position embedding; Llama pairing (i, i + D/2), theta_i = base^(-2i/D)) ----
def test_rope_identity_at_position_zero():
    x = np.random.default_rng(0).standard_normal((3, 2, 64))
    assert np.array_equal(oracle.rope(x, [0, 0, 0]), x)


@pytest.mark.parametrize("D", [64, 128])
def test_rope_basis_vectors_closed_form(D):
    """Hand-computed rotations pin the pairing and the frequency schedule: e_0 turns by the
    angle pos (theta_0 = 1) into e_{D/2}; e_{D/4} has theta = base^(-1/2), so with base 10^4 it
    turns by 1 rad at pos 100, into e_{3D/4}; e_{D/2} turns back towards -e_0."""
    e = np.eye(D)
    out = oracle.rope(e[None, [0]], [3], 10000.0)[0, 0]
    want = np.zeros(D)
    want[0], want[D // 2] = math.cos(3.0), math.sin(3.0)
    assert np.allclose(out, want, atol=1e-15)
    out = oracle.rope(e[None, [D // 4]], [100], 10000.0)[0, 0]
    want = np.zeros(D)
    want[D // 4], want[3 * D // 4] = math.cos(1.0), math.sin(1.0)
    assert np.allclose(out, want, atol=1e-12)
    out = oracle.rope(e[None, [D // 2]], [3], 10000.0)[0, 0]
    want = np.zeros(D)
    want[0], want[D // 2] = -math.sin(3.0), math.cos(3.0)
    assert np.allclose(out, want, atol=1e-15)


def test_rope_group_norm_and_relative_position():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 3, 64))
    a, b = np.array([0, 5, 77, 4000]), np.array([1, 9, 300, 12345])
    # composition: turning by a then by b is turning by a + b
    assert np.allclose(oracle.rope(oracle.rope(x, a), b), oracle.rope(x, a + b), atol=1e-9)
    # each (i, i + D/2) pair keeps its length
    r = oracle.rope(x, b)
    n0 = x[..., :32] ** 2 + x[..., 32:] ** 2
    n1 = r[..., :32] ** 2 + r[..., 32:] ** 2
    assert np.allclose(n0, n1, atol=1e-12)
    # q.k after rotation depends only on the position difference
    q, k = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    d1 = (oracle.rope(q, [50]) * oracle.rope(k, [20])).sum()
    d2 = (oracle.rope(q, [1030]) * oracle.rope(k, [1000])).sum()
    assert abs(d1 - d2) < 1e-9


def test_bf16_round_hand_values():
    ulp = 2.0 ** -7  # bf16 spacing in [1, 2)
    vals = np.array([1.0, 1 + ulp / 2, 1 + 1.5 * ulp, 1 + ulp / 2 + 2.0 ** -20, -3.0, 0.0])
    want = np.array([1.0, 1.0, 1 + 2 * ulp, 1 + ulp, -3.0, 0.0])
    assert np.array_equal(oracle.bf16_round(vals), want)
    # the rounding agrees with the bit-level generator's on random fp32 values
    x = np.random.default_rng(2).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.bf16_round(x), bf16_value(bf16_bits(x)))


# ---- FP8 E4M3 (OCP format: bias 7, 3 mantissa bits, max 448, S.1111.111 NaN) --------------
def test_fp8_decode_hand_values():
    vals = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
            0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5}
    for code, v in vals.items():
        assert oracle.fp8_e4m3_decode(np.uint8(code)) == v, hex(code)
    assert np.isnan(oracle.fp8_e4m3_decode(np.uint8(0x7F))) and np.isnan(oracle.fp8_e4m3_decode(np.uint8(0xFF)))


def test_fp8_encode_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_decode(codes)), codes)
    # ties go to the even code; just above / below a tie go to the nearer code
    assert oracle.fp8_e4m3_encode(1.0625) == 0x38      # between 1 (even) and 1.125
    assert oracle.fp8_e4m3_encode(1.1875) == 0x3A      # between 1.125 and 1.25 (even)
    assert oracle.fp8_e4m3_encode(1.0625 + 1e-9) == 0x39
    assert oracle.fp8_e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal: to 0 (even)
    assert oracle.fp8_e4m3_encode(1.5 * 2.0 ** -9) == 0x02
    assert oracle.fp8_e4m3_encode(-3.0) == 0xC4 and oracle.fp8_e4m3_encode(440.0) == 0x7E
    assert oracle.fp8_e4m3_encode(-2.0 ** -11) == 0x80  # rounds to -0
    with pytest.raises(ValueError):
        oracle.fp8_e4m3_encode(449.0)


def test_fp8_quantizer_bounds():
    x = np.random.default_rng(3).standard_normal((50, 128)).astype(np.float32)
    codes, s = oracle.quantize_fp8(x)
    y = oracle.dequantize_fp8(codes, s)
    s64 = s.astype(np.float64)[:, None]
    # relative error of E4M3 is at most 2^-4 of the value, or half a subnormal step (2^-10 s)
    assert (np.abs(y - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s64) * 1.0001).all()
    # the absmax element maps to (nearly) +-448: its code is 0x7E / 0xFE or one step below
    amax = np.abs(oracle.fp8_e4m3_decode(codes)).max(axis=1)
    assert (amax >= 416).all() and (amax <= 448).all()
    z, sz = oracle.quantize_fp8(np.zeros((2, 64), np.float32))
    assert (z == 0).all() and (sz == 0).all()


# ---- scale rules of the byte caches, pinned by hand values --------------------------------------
def test_fp8_quantizer_hand_values():
    # absmax 1.0: fp32 1/448 = 0.00223214... is not an fp16 value; to nearest-even fp16 it is
    # 2^-9 * (1 + 146/1024) = 0.0022315979 (bits 0x1892). 1.0 / s = 448.11, clamped to 448 -> 0x7E.
    # x1 = 1.1875 * s exactly (11 + 5 significant bits), so x1 / s = 1.1875, the midpoint of
    # 1.125 (0x39) and 1.25 (0x3A): the tie goes to the even code 0x3A. Divided by the unrounded
    # fp32 1/448 instead it would be 1.18721 -> 0x39; a divisor other than 448 changes the scale.
    # -0.5 / s = -224.05 -> -224 = -(1 + 6/8) * 2^7 -> 0xF6; 0 -> 0x00.
    s_bits = 0x1892
    s = float(np.uint16(s_bits).view(np.float16))
    assert s == 2.0 ** -9 * (1 + 146 / 1024)
    x = np.array([[1.0, 1.1875 * s, -0.5, 0.0]], np.float32)
    codes, sc = oracle.quantize_fp8(x)
    assert int(sc.view(np.uint16)[0]) == s_bits
    assert codes.tolist() == [[0x7E, 0x3A, 0xF6, 0x00]]
    # absmax 448 gives the scale 1 exactly, and then every code is the E4M3 value of x itself
    codes, sc = oracle.quantize_fp8(np.array([[448.0, -3.0, 1.0625, 2.0 ** -9]], np.float32))
    assert float(sc[0]) == 1.0 and codes.tolist() == [[0x7E, 0xC4, 0x38, 0x01]]


def test_fp8_quantizer_scale_mutants_are_caught(monkeypatch):
    import oracle.attn_fp64 as oa

    def unrounded(x):  # divides by fp32 a / 448 instead of the stored fp16 scale
        x = np.asarray(x, np.float32)
        a = np.abs(x).max(axis=-1)
        s32 = a / np.float32(448.0)
        y = np.clip(x / s32[..., None], np.float32(-448.0), np.float32(448.0))
        return oa.fp8_e4m3_encode(y.astype(np.float64)), s32.astype(np.float16)

    def divisor_440(x):  # the rule with 440 in place of 448
        x = np.asarray(x, np.float32)
        s16 = (np.abs(x).max(axis=-1) / np.float32(440.0)).astype(np.float16)
        y = np.clip(x / s16.astype(np.float32)[..., None], np.float32(-448.0), np.float32(448.0))
        return oa.fp8_e4m3_encode(y.astype(np.float64)), s16

    for mutant in (unrounded, divisor_440):
        monkeypatch.setattr(oracle, "quantize_fp8", mutant)
        with pytest.raises(AssertionError):
            test_fp8_quantizer_hand_values()
        monkeypatch.undo()


def test_dequantize_hand_values():
    # INT8: code * scale, exactly
    codes = np.array([[127, -3, 0, 1]], np.int8)
    assert oracle.dequantize_int8(codes, np.array([0.5], np.float16)).tolist() == [[63.5, -1.5, 0.0, 0.5]]
    assert oracle.dequantize_int8(codes, np.array([2.0 ** -20], np.float16)).tolist() == \
        [[127 * 2.0 ** -20, -3 * 2.0 ** -20, 0.0, 2.0 ** -20]]
    # FP8: E4M3 value * scale (0x38 = 1, 0xC4 = -3, 0x01 = 2^-9, 0x7E = 448)
    c8 = np.array([[0x38, 0xC4, 0x01, 0x7E]], np.uint8)
    assert oracle.dequantize_fp8(c8, np.array([0.25], np.float16)).tolist() == [[0.25, -0.75, 2.0 ** -11, 112.0]]


def _scaled_cache_case(bs=2, seed=31):
    """A tiny INT8 paged cache with distinct fp16 scales per (block, head, slot) for K and V."""
    rng = np.random.default_rng(seed)
    ctx = np.array([5, 3, 1], np.int32)
    table, nb = paged_table(ctx, bs, seed, 1, True)
    Hkv, D = 2, 3
    kc = rng.integers(-127, 128, (nb, Hkv, bs, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (nb, Hkv, bs, D)).astype(np.int8)
    ks = (rng.uniform(0.5, 1.5, (nb, Hkv, bs)) / 100).astype(np.float16)
    vs = (rng.uniform(0.5, 1.5, (nb, Hkv, bs)) / 50).astype(np.float16)
    q = rng.standard_normal((3, 4, D))
    return ctx, table, kc, vc, ks, vs, q


@pytest.mark.parametrize("window", [0, 2])
def test_decode_paged_scaled_branch_brute(window):
    bs = 2
    ctx, table, kc, vc, ks, vs, q = _scaled_cache_case(bs)
    o, _ = oracle.decode_paged(q, kc, vc, table, ctx, 0.7, bs, window, k_scale=ks, v_scale=vs)
    for b in range(len(ctx)):
        n = int(ctx[b])
        # the cache the attention sees, built here token by token: code * scale of its slot
        kk = np.zeros((n, 2, 3))
        vv = np.zeros((n, 2, 3))
        for t in range(n):
            pb, slot = int(table[b][t // bs]), t % bs
            for g in range(2):
                for d in range(3):
                    kk[t, g, d] = float(kc[pb, g, slot, d]) * float(ks[pb, g, slot])
                    vv[t, g, d] = float(vc[pb, g, slot, d]) * float(vs[pb, g, slot])
        ob = _brute(q[b][None, None], kk[None], vv[None], 0.7, True, window)
        assert np.abs(o[b] - ob[0, 0]).max() < 1e-12


def test_decode_paged_scale_mutants_are_caught(monkeypatch):
    orig = oracle.decode_paged

    def k_scale_on_v(*a, k_scale=None, v_scale=None, **kw):
        return orig(*a, k_scale=k_scale, v_scale=k_scale, **kw)

    def v_scale_dropped(*a, k_scale=None, v_scale=None, **kw):
        return orig(*a, k_scale=k_scale, v_scale=np.ones_like(v_scale), **kw)

    def k_scale_dropped(*a, k_scale=None, v_scale=None, **kw):
        return orig(*a, k_scale=np.ones_like(k_scale), v_scale=v_scale, **kw)

    for mutant in (k_scale_on_v, v_scale_dropped, k_scale_dropped):
        monkeypatch.setattr(oracle, "decode_paged", mutant)
        with pytest.raises(AssertionError):
            test_decode_paged_scaled_branch_brute(0)
        monkeypatch.undo()
