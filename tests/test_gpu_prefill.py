"""GPU parity of attn_prefill (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from synth import PrefillWorkload, WORKLOADS, prefill_inputs, prefill_slab
from tests.gpu_util import BF16_TOL, F32_TOL, dev, dev_bf16, host_bits, host_f64, maxabs, torch

pytestmark = pytest.mark.gpu

# bf16 prefill normalises by l = sum of the bf16-rounded probabilities (the values the PV
# contraction uses), each within a relative 2^-9 of the exact exp, so ln l -- and the reported
# LSE -- is within 2^-9 (~0.00195) of the exact log-sum-exp; fp32 accumulation adds ~1e-6.
LSE_TOL_BF16 = 4e-3


def _run(wl, x, causal=None, window=None, lse=True):
    import attention_attn_prefill_amd as A
    t = torch()
    if wl.dtype == "bf16":
        q, k, v = (dev_bf16(x[n + "_bits"]) for n in "qkv")
    else:
        q, k, v = (dev(x[n]) for n in "qkv")
    L = t.empty((wl.B, wl.Hq, wl.S), dtype=t.float32, device="cuda") if lse else None
    o = A.attn_prefill(q, k, v, scale=wl.scale, causal=wl.causal if causal is None else causal,
                       window=wl.window if window is None else window, lse=L)
    t.cuda.synchronize()
    return o, L


def test_prefill_f32_s128():
    wl = WORKLOADS["prefill_f32_s128"]
    x = prefill_inputs(wl)
    o, L = _run(wl, x)
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], wl.scale, True, 0)
    assert maxabs(host_f64(o), ro) <= F32_TOL
    assert maxabs(host_f64(L), rl) <= F32_TOL


SMALL = [
    # B, S, Hq, Hkv, D, causal, window
    (1, 200, 4, 4, 64, True, 0),
    (2, 333, 8, 2, 64, True, 0),
    (1, 257, 8, 1, 128, True, 50),
    (1, 130, 6, 3, 128, True, 0),
    (2, 190, 4, 4, 128, False, 0),
    (1, 300, 8, 2, 64, True, 1),
    (1, 300, 4, 2, 64, False, 64),
    (1, 1, 4, 1, 64, True, 0),
    (1, 64, 2, 1, 128, True, 0),
    (1, 129, 12, 4, 64, True, 100),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal,window", SMALL)
def test_prefill_bf16_small(B, S, Hq, Hkv, D, causal, window):
    wl = PrefillWorkload("small", 7000 + S, "bf16", B, S, Hq, Hkv, D, causal, window)
    x = prefill_inputs(wl)
    o, L = _run(wl, x)
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], wl.scale, causal, window)
    assert maxabs(host_f64(o), ro) <= BF16_TOL
    assert maxabs(host_f64(L), rl) <= LSE_TOL_BF16


@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 100, 4, 4, 64), (1, 77, 8, 2, 128), (2, 1000, 32, 8, 64)])
def test_prefill_f32_small(B, S, Hq, Hkv, D):
    wl = PrefillWorkload("small32", 8000 + S, "f32", B, S, Hq, Hkv, D, True, 0)
    x = prefill_inputs(wl)
    o, L = _run(wl, x)
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], wl.scale, True, 0)
    assert maxabs(host_f64(o), ro) <= F32_TOL
    assert maxabs(host_f64(L), rl) <= F32_TOL


def test_single_key_row_is_exact():
    """Row 0 sees only key 0, so its output is V[0] bit for bit (P = 1, l = 1)."""
    wl = PrefillWorkload("row0", 9001, "bf16", 2, 150, 8, 2, 128, True, 0)
    x = prefill_inputs(wl)
    o, _ = _run(wl, x, lse=False)
    got = host_bits(o)[:, 0]  # [B][Hq][D]
    want = np.repeat(x["v_bits"][:, 0], 4, axis=1)
    assert np.array_equal(got, want)


def test_window_one_is_v():
    wl = PrefillWorkload("w1", 9002, "bf16", 1, 200, 4, 2, 64, True, 1)
    x = prefill_inputs(wl)
    o, _ = _run(wl, x, lse=False)
    assert np.array_equal(host_bits(o), np.repeat(x["v_bits"], 2, axis=2))


def test_prefill_deterministic():
    wl = PrefillWorkload("det", 9003, "bf16", 1, 1000, 8, 2, 128, True, 300)
    x = prefill_inputs(wl)
    a, _ = _run(wl, x)
    b, _ = _run(wl, x)
    assert np.array_equal(host_bits(a), host_bits(b))


def _sampled_check(wl, rows, heads, full_pairs=()):
    """Rows `rows` of heads `heads` in every batch, and every row of the (batch, head) pairs
    `full_pairs`, against the oracle (O and LSE)."""
    x = prefill_inputs(wl)
    o, L = _run(wl, x)
    got, gl = host_f64(o), host_f64(L)
    G = wl.Hq // wl.Hkv
    worst = 0.0
    checks = [(b, h, rows) for b in range(wl.B) for h in heads]
    checks += [(b, h, list(range(wl.S))) for b, h in full_pairs]
    for b, h, rr in checks:
        q = prefill_slab(wl, "q", b, h)[rr]
        k = prefill_slab(wl, "k", b, h // G)
        v = prefill_slab(wl, "v", b, h // G)
        ro, rl = oracle.attention_head(q, k, v, wl.scale, rr, wl.causal, wl.window)
        worst = max(worst, maxabs(got[b, rr, h], ro))
        assert maxabs(gl[b, h, rr], rl) <= LSE_TOL_BF16
    assert worst <= BF16_TOL, worst
    return o


def test_prefill_llama1b_s4096_sampled():
    wl = WORKLOADS["prefill_llama1b_s4096"]
    rows = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 1000, 2047, 2048, 3071, 4094, 4095]
    _sampled_check(wl, rows, [0, 3, 4, 17, 31], full_pairs=[(0, 9), (0, 26)])


def test_prefill_swa_s16384_sampled():
    """The long-context sliding-window prefill at full size: sampled rows (first / last rows,
    tile and window edges) of three heads per batch, and every one of the 16384 rows of one
    (batch, head) pair per batch, on different KV heads."""
    wl = WORKLOADS["prefill_swa_s16384"]
    rows = [0, 1, 63, 64, 4094, 4095, 4096, 4097, 8191, 12000, 16383]
    _sampled_check(wl, rows, [0, 5, 30], full_pairs=[(0, 5), (1, 22)])
