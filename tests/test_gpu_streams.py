"""GPU checks of the stream argument: the entry points queue their kernels on the caller's stream
(here a side stream that must wait for another stream's work before its inputs are ready), and
the allocation-free decode can be captured in a HIP graph and replayed with new queries."""
import numpy as np
import pytest

from synth import DecodeWorkload, context_lens, decode_query, new_tokens, paged_table, pool
from tests.gpu_util import dev, dev_bf16, host_bits, torch

pytestmark = pytest.mark.gpu


def _decode_case(seed):
    wl = DecodeWorkload("streams", seed, "bf16", 24, 32, 8, 64, 100, 3000)
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, 16, wl.seed, 2, True)
    qbits, _ = decode_query(wl)
    return wl, dict(q=dev_bf16(qbits), kc=dev_bf16(pool(wl, "k", nb)), vc=dev_bf16(pool(wl, "v", nb)),
                    table=dev(table), ctx=dev(ctx), mx=int(ctx.max()))


def test_kernels_run_on_the_callers_stream():
    """The queries only become valid on a side stream after a long chain of kernels on a third
    stream; decode and prefill issued on the side stream behind an event wait must see them.
    A launch on any other stream would read the zeros the buffers hold before the copy."""
    import attention_attn_prefill_amd as A
    t = torch()
    wl, c = _decode_case(7100)
    gen = t.Generator(device="cuda").manual_seed(7101)
    qp, kp, vp = (t.randn((1, 1000, 8, 64), device="cuda", generator=gen, dtype=t.bfloat16)
                  for _ in range(3))
    ref_d = A.attn_decode_paged(c["q"], c["kc"], c["vc"], c["table"], c["ctx"], c["mx"], scale=wl.scale)
    ref_p = A.attn_prefill(qp, kp, vp)
    t.cuda.synchronize()

    q_d, q_p = t.zeros_like(c["q"]), t.zeros_like(qp)
    producer, consumer = t.cuda.Stream(), t.cuda.Stream()
    ready = t.cuda.Event()
    with t.cuda.stream(producer):
        busy = t.ones(64 << 20, device="cuda")
        for _ in range(40):
            busy.mul_(1.0001)
        q_d.copy_(c["q"])
        q_p.copy_(qp)
        ready.record(producer)
    with t.cuda.stream(consumer):
        consumer.wait_event(ready)
        got_d = A.attn_decode_paged(q_d, c["kc"], c["vc"], c["table"], c["ctx"], c["mx"], scale=wl.scale)
        got_p = A.attn_prefill(q_p, kp, vp)
    consumer.synchronize()
    t.cuda.synchronize()
    assert np.array_equal(host_bits(got_d), host_bits(ref_d))
    assert np.array_equal(host_bits(got_p), host_bits(ref_p))


def test_noalloc_decode_replays_in_a_hip_graph():
    """attn_decode_paged_noalloc captured once, then replayed three times with new queries
    written into the captured buffer between replays: every replay equals an eager
    attn_decode_paged on the same queries, bit for bit."""
    import attention_attn_prefill_amd as A
    t = torch()
    wl, c = _decode_case(7200)
    q_static = c["q"].clone()
    out_static = t.empty_like(q_static)
    args = (c["kc"], c["vc"], c["table"], c["ctx"], c["mx"])
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):  # first call outside the capture (per-device set-up)
        A.attn_decode_paged_noalloc(q_static, *args, scale=wl.scale, out=out_static)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        A.attn_decode_paged_noalloc(q_static, *args, scale=wl.scale, out=out_static)
    B, Hq, D = q_static.shape
    for i in range(3):
        qb, _ = new_tokens(7201 + i, B, Hq, D, "k")
        q_static.copy_(dev_bf16(qb).view(B, Hq, D))
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        ref = A.attn_decode_paged(q_static, *args, scale=wl.scale)
        t.cuda.synchronize()
        assert np.array_equal(host_bits(out_static), host_bits(ref)), i
