"""GPU check that the decode entry points write only inside the buffers they are given: the
workspace is exactly the size attn_decode_(multi_)workspace_size reports and the output exactly
its shape, both carved out of larger buffers filled with a sentinel byte, which must be intact
afterwards. Covers the balanced shape, fixed splits (window and explicit split_tokens),
multi-row decode, virtual KV heads (INT8 and bf16) and the paged prefill kernel's path, and the
contiguous prefill's O and LSE with ragged query tails, and kv_cache_append with table entries
past the pool."""
import numpy as np
import pytest

from synth import DecodeWorkload, context_lens, int8_pool, new_tokens, paged_table, pool
from tests.gpu_util import dev, dev_bf16, torch

pytestmark = pytest.mark.gpu
SENTINEL = 0xA5
PAD = 1 << 16  # guard bytes after each buffer


def _guarded(nbytes):
    t = torch()
    return t.full((nbytes + PAD,), SENTINEL, dtype=t.uint8, device="cuda")


CASES = [
    # B, q_len, Hq, Hkv, D, kv, window, split, (lo, hi) context range
    (48, 1, 32, 8, 64, "bf16", 0, 0, (1, 3000)),      # balanced shape
    (5, 1, 16, 2, 128, "bf16", 100, 0, (200, 900)),   # fixed splits chosen for the window
    (7, 1, 8, 2, 64, "bf16", 0, 48, (1, 2000)),       # explicit split_tokens
    (9, 4, 32, 8, 64, "bf16", 0, 0, (4, 1500)),       # multi-row, 16 columns
    (6, 8, 32, 8, 64, "bf16", 0, 0, (8, 1500)),       # 8 drafts: two virtual KV heads (bf16)
    (6, 12, 32, 8, 64, "bf16", 0, 0, (12, 1500)),     # 12 drafts: the paged prefill kernel
    (6, 1, 64, 2, 64, "i8", 0, 0, (1, 2000)),         # INT8, 32 heads per KV head: virtual heads
    (4, 5, 20, 4, 128, "i8", 64, 0, (5, 900)),        # INT8, 5 x 5 columns, window: fixed splits
]


@pytest.mark.parametrize("B,QL,Hq,Hkv,D,kv,window,split,rng", CASES)
def test_decode_writes_stay_inside_the_given_buffers(B, QL, Hq, Hkv, D, kv, window, split, rng):
    import attention_attn_prefill_amd as A
    t = torch()
    seed = 8100 + B + QL + Hq + D + window + split
    wl = DecodeWorkload("bounds", seed, kv, B, Hq, Hkv, D, rng[0], rng[1], 16, window)
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, 16, seed, 2, True)
    if kv == "bf16":
        kc, vc, ks, vs = dev_bf16(pool(wl, "k", nb)), dev_bf16(pool(wl, "v", nb)), None, None
    else:
        (k8, k_s), (v8, v_s) = int8_pool(wl, "k", nb), int8_pool(wl, "v", nb)
        kc, vc, ks, vs = dev(k8), dev(v8), dev(k_s), dev(v_s)
    qb, _ = new_tokens(seed + 1, B * QL, Hq, D, "k")
    shape = (B, QL, Hq, D) if QL > 1 else (B, Hq, D)
    q = dev_bf16(qb).view(*shape)
    mx = int(ctx.max())
    need = (A.attn_decode_multi_workspace_size(B, QL, Hq, Hkv, D, mx, window, split) if QL > 1
            else A.attn_decode_workspace_size(B, Hq, Hkv, D, mx, window, split))
    ws_buf = _guarded(need)
    out_bytes = B * QL * Hq * D * 2
    out_buf = _guarded(out_bytes)
    out = out_buf[:out_bytes].view(t.bfloat16).view(*shape)
    ws = ws_buf[:need] if need > 0 else None
    kw = dict(k_scale=ks, v_scale=vs, scale=wl.scale, window=window, split_tokens=split, out=out,
              workspace=ws)
    if QL > 1:
        A.attn_decode_paged_multi(q, kc, vc, dev(table), dev(ctx), mx, **kw)
    else:
        A.attn_decode_paged(q, kc, vc, dev(table), dev(ctx), mx, **kw)
    t.cuda.synchronize()
    assert (ws_buf[need:] == SENTINEL).all().item(), "write past the workspace"
    assert (out_buf[out_bytes:] == SENTINEL).all().item(), "write past the output"
    assert t.isfinite(out.float()).all().item()


@pytest.mark.parametrize("B,S,Hq,Hkv,D,window", [(2, 1000, 8, 2, 64, 0), (1, 777, 16, 4, 128, 100),
                                                (3, 33, 12, 4, 64, 0)])
def test_prefill_writes_stay_inside_out_and_lse(B, S, Hq, Hkv, D, window):
    """Ragged query tails (S not a multiple of the 32-row blocks): no write past O or the LSE."""
    import attention_attn_prefill_amd as A
    t = torch()
    gen = t.Generator(device="cuda").manual_seed(8200 + S)
    q = t.randn((B, S, Hq, D), device="cuda", generator=gen).to(t.bfloat16)
    k = t.randn((B, S, Hkv, D), device="cuda", generator=gen).to(t.bfloat16)
    v = t.randn((B, S, Hkv, D), device="cuda", generator=gen).to(t.bfloat16)
    ob, lb = B * S * Hq * D * 2, B * Hq * S * 4
    o_buf, l_buf = _guarded(ob), _guarded(lb)
    out = o_buf[:ob].view(t.bfloat16).view(B, S, Hq, D)
    lse = l_buf[:lb].view(t.float32).view(B, Hq, S)
    A.attn_prefill(q, k, v, causal=True, window=window, out=out, lse=lse)
    t.cuda.synchronize()
    assert (o_buf[ob:] == SENTINEL).all().item() and (l_buf[lb:] == SENTINEL).all().item()
    assert t.isfinite(out.float()).all().item() and t.isfinite(lse).all().item()


@pytest.mark.parametrize("int8", [False, True])
def test_append_writes_stay_inside_the_pool(int8):
    """Rows whose table entry is past the pool (num_blocks, or any larger id), negative, or whose
    position is past the table are skipped: nothing lands after the pool or its scales."""
    import attention_attn_prefill_amd as A
    t = torch()
    Hkv, D, bs, nb = 2, 64, 16, 6
    table = np.array([[0, 1, 2], [3, nb, 4], [5, nb + 7, -1]], np.int32)
    seq = np.array([0, 0, 1, 1, 1, 2, 2, 2, 0], np.int32)
    pos = np.array([0, 47, 5, 20, 40, 3, 17, 33, 48], np.int32)  # rows 3, 6, 7, 8 are skipped
    kn, _ = new_tokens(8300 + int8, len(seq), Hkv, D, "k")
    vn, _ = new_tokens(8310 + int8, len(seq), Hkv, D, "v")
    esize = 1 if int8 else 2
    cb = nb * Hkv * bs * D * esize
    bufs = [_guarded(cb), _guarded(cb)]
    dt = t.int8 if int8 else t.bfloat16
    kc, vc = (b[:cb].view(dt).view(nb, Hkv, bs, D) for b in bufs)
    kw = {}
    if int8:
        sb = nb * Hkv * bs * 2
        sbufs = [_guarded(sb), _guarded(sb)]
        kw = dict(k_scale=sbufs[0][:sb].view(t.float16).view(nb, Hkv, bs),
                  v_scale=sbufs[1][:sb].view(t.float16).view(nb, Hkv, bs))
        bufs += sbufs
    A.kv_cache_append(dev_bf16(kn), dev_bf16(vn), dev(seq), dev(pos), dev(table), kc, vc, **kw)
    t.cuda.synchronize()
    sizes = [cb, cb] + ([sb, sb] if int8 else [])
    for b, n in zip(bufs, sizes):
        assert (b[n:] == SENTINEL).all().item()
