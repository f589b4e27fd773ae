"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over the configurations the targets are set on
(default `--workload target`):
  * for each decode workload -- INT8-KV paged decode on a 70B-shaped layer (B = 16, 64/8
    heads, D = 128, context 32768), sliding-window paged decode (B = 32, 32/8 heads, D = 128,
    context 16384, window 4096) and the Llama-3.2-1B-shaped paged decode (B = 64, 32/8 heads,
    D = 64, contexts uniform in [512, 4096]): kv_cache_append of each sequence's newest token,
    a 512 MiB scratch read that evicts L2 and the Infinity Cache with clean lines (so the
    decode reads its cache from HBM and no dirty write-back overlaps it), attn_decode_paged
    (split KV + log-sum-exp merge);
  * attn_prefill on the long-context sliding-window prefill (B = 2, S = 16384, 32/8 heads,
    D = 128, window 4096) and on the Llama-3.2-1B-shaped causal prefill (B = 1, S = 4096,
    32/8 heads, D = 64).
Each call is bracketed by HIP events on the stream the library launches on. `value` and
`roofline` are the long-context prefill's TFLOP/s (algorithmic flops: visible (query, key) pairs
x 4D); `roofline_decode` is the INT8 decode's HBM GB/s (algorithmic bytes: each visible K/V
byte and scale once, plus Q and O); every other workload carries its own roofline object
(`roofline_decode_swa`, `roofline_decode_llama1b`, `roofline_prefill_llama1b`) and its
per-call entry under `prefill` / `decode`. `--workload llama1b | swa | int8_70b | fp8_70b` run
subsets (for profiling). Outside the timed steps, the default run also times
attn_prefill_paged (chunked prefill over the paged cache with fused append: 4 sequences,
1024-token chunks after 3072-token prefixes), attn_decode_paged_multi (4 and 8 draft rows per
sequence on the Llama-shaped cache; 8 rows run as two virtual KV heads per cache head), kv_cache_append_rope
(a 64k-token prompt written into a
paged cache with RoPE on K) and attn_decode_paged over an FP8 E4M3 copy of the Llama-shaped
cache.

Before touching the GPU, bench.py runs attention_attn_prefill_amd/attn_peaks (built with the
library) as a child process: a bf16 MFMA-only loop (with the shader clock it ran at), an HBM
streaming read and a random 2 KB-block gather; the JSON line carries them as
`measured_peaks`, and each roofline object adds `frac_of_measured` beside the fraction of the
published peak. Per-call times also come as p10 / p50 / p90 over the timed steps.

The cpu_baseline leg times the fp64 oracle on whole (batch, head) pairs of the headline
prefill and compares every row of each with the timed run's output (untimed).

Prints one JSON line. Inputs are seeded synthetic tensors (synth/) resident in HBM before the
timed region starts.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_CALIBRATION_BYTES = 256 * 1024 * 1024  # each direction of the calibration copy
KERNEL_SOURCES = {  # the source each measured call's kernels come from
    "prefill": "attention_attn_prefill_amd/csrc/prefill_bf16.hip",
    "decode": "attention_attn_prefill_amd/csrc/decode.hip",
}


def source_hash(kernel: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or
    None when there is none or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith(" "):
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def prefill_pairs(S: int, causal: bool, window: int) -> int:
    """Visible (query, key) pairs of one head."""
    if not causal:
        return S * (S if window == 0 else min(S, window))  # not used by the workloads here
    if window == 0 or window >= S:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window


def prefill_flops(wl) -> float:
    return 4.0 * wl.D * wl.Hq * wl.B * prefill_pairs(wl.S, wl.causal, wl.window)


def decode_bytes(wl, ctx) -> float:
    vis = np.minimum(ctx, wl.window) if wl.window > 0 else ctx
    per_tok = 2 * wl.Hkv * wl.D * (1 if wl.kv_dtype in ("i8", "fp8") else 2)
    if wl.kv_dtype in ("i8", "fp8"):
        per_tok += 2 * wl.Hkv * 2  # fp16 scales of K and V
    return float(vis.sum()) * per_tok + 2.0 * wl.B * wl.Hq * wl.D * 2


def _bf16(t, bits):
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).cuda()


def setup_prefill(t, wl):
    from synth import prefill_inputs
    x = prefill_inputs(wl)
    q, k, v = (_bf16(t, x[n + "_bits"]) for n in "qkv")
    o = t.empty_like(q)
    return dict(q=q, k=k, v=v, o=o)


def setup_decode(t, wl):
    """Paged cache, table, queries and the newest token's K/V for each sequence."""
    import attention_attn_prefill_amd as A
    from synth import context_lens, decode_query, new_tokens, paged_table, pool
    ctx = context_lens(wl)
    table, nb = paged_table(ctx, wl.block_size, wl.seed)
    qbits, _ = decode_query(wl)
    d = dict(ctx_np=ctx, table=t.from_numpy(table).cuda(), ctx=t.from_numpy(ctx).cuda(),
             q=_bf16(t, qbits), nb=nb)
    if wl.kv_dtype == "bf16":
        d["kc"] = _bf16(t, pool(wl, "k", nb))
        d["vc"] = _bf16(t, pool(wl, "v", nb))
        d["ks"] = d["vs"] = None
    else:  # quantize a bf16 pool in physical order with the library's append kernel
        T = nb * wl.block_size
        ident = t.arange(nb, dtype=t.int32, device="cuda")[None]
        seq = t.zeros(T, dtype=t.int32, device="cuda")
        pos = t.arange(T, dtype=t.int32, device="cuda")
        for which in ("k", "v"):
            src = pool(wl, which, nb)
            rows = _bf16(t, np.ascontiguousarray(src.transpose(0, 2, 1, 3)).reshape(T, wl.Hkv, wl.D))
            del src
            c = t.empty((nb, wl.Hkv, wl.block_size, wl.D), dtype=t.int8 if wl.kv_dtype == "i8" else t.uint8,
                        device="cuda")
            s = t.empty((nb, wl.Hkv, wl.block_size), dtype=t.float16, device="cuda")
            A.kv_cache_append(rows, rows, seq, pos, ident, c, c, k_scale=s, v_scale=s)
            t.cuda.synchronize()
            del rows
            d[which + "c"], d[which + "s"] = c, s
    kn, _ = new_tokens(wl.seed + 77, wl.B, wl.Hkv, wl.D, "k")
    vn, _ = new_tokens(wl.seed + 78, wl.B, wl.Hkv, wl.D, "v")
    d["kn"], d["vn"] = _bf16(t, kn), _bf16(t, vn)
    d["seq"] = t.arange(wl.B, dtype=t.int32, device="cuda")
    d["pos"] = (d["ctx"] - 1).to(t.int32)
    d["o"] = t.empty_like(d["q"])
    need = A.attn_decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.D, wl.ctx_hi, wl.window, 0)
    d["ws"] = t.empty(max(need, 1), dtype=t.uint8, device="cuda")
    return d


CHUNK = dict(B=4, ctx=4096, q_len=1024, Hq=32, Hkv=8, D=64, seed=1202)


def setup_chunked(t):
    """Chunked prefill over the paged cache (Llama-3.2-1B heads): 4 sequences whose 3072-token
    prefixes sit in a permuted bf16 pool; each call appends and attends a 1024-token chunk."""
    from synth import DecodeWorkload, new_tokens, paged_table, pool
    c = CHUNK
    ctx = np.full(c["B"], c["ctx"], np.int32)
    wl = DecodeWorkload("chunk_llama1b", c["seed"], "bf16", c["B"], c["Hq"], c["Hkv"], c["D"], c["ctx"], c["ctx"])
    table, nb = paged_table(ctx, 16, c["seed"])
    T = c["B"] * c["q_len"]
    kn, _ = new_tokens(c["seed"] + 1, T, c["Hkv"], c["D"], "k")
    vn, _ = new_tokens(c["seed"] + 2, T, c["Hkv"], c["D"], "v")
    qb, _ = new_tokens(c["seed"] + 3, T, c["Hq"], c["D"], "k")
    cu = np.arange(c["B"] + 1, dtype=np.int32) * c["q_len"]
    return dict(q=_bf16(t, qb), kn=_bf16(t, kn), vn=_bf16(t, vn), kc=_bf16(t, pool(wl, "k", nb)),
                vc=_bf16(t, pool(wl, "v", nb)), table=t.from_numpy(table).cuda(),
                cu=t.from_numpy(cu).cuda(), ctx=t.from_numpy(ctx).cuda(),
                o=t.empty((T, c["Hq"], c["D"]), dtype=t.bfloat16, device="cuda"))


def chunked_flops() -> float:
    c = CHUNK
    prefix = c["ctx"] - c["q_len"]
    pairs = c["q_len"] * prefix + c["q_len"] * (c["q_len"] + 1) // 2
    return 4.0 * c["D"] * c["Hq"] * c["B"] * pairs


def _pct(x) -> dict:
    """p10 / p50 / p90 of per-call times (ms)."""
    return {f"p{q}": float(np.percentile(x, q)) for q in (10, 50, 90)}


def time_chunked(t, A, reps: int):
    """attn_prefill_paged with fused append, timed per call with events (outside the step)."""
    C = setup_chunked(t)
    c = CHUNK

    def call():
        A.attn_prefill_paged(C["q"], C["kc"], C["vc"], C["table"], C["cu"], C["ctx"], c["q_len"],
                             k_new=C["kn"], v_new=C["vn"], causal=True, out=C["o"])
    for _ in range(3):
        call()
    ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    t.cuda.synchronize()
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms = float(np.mean(per))
    fl = chunked_flops()
    tf = fl / (ms * 1e-3) / 1e12
    return {"kernel": "attn_prefill_paged (paged bf16 MFMA prefill, append in the same launch)",
            "ms": ms, "ms_percentiles": _pct(per),
            "TFLOP/s": tf, "frac_mfma_peak": tf / BF16_PEAK_TFLOPS, "algorithmic_flops": fl,
            "tokens_per_s": c["B"] * c["q_len"] / (ms * 1e-3), "calls": reps,
            "workload": f"B={c['B']} chunks of {c['q_len']} rows after {c['ctx'] - c['q_len']}-token "
                        f"prefixes, Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} causal, block 16, "
                        "permuted pool"}


def time_decode_multi(t, A, dwl, Dd, reps: int, q_len: int = 4):
    """attn_decode_paged_multi (speculative verification, q_len draft rows per sequence) on the
    decode workload's cache, timed per call with events after a cache-evicting read."""
    from synth import new_tokens
    qb, _ = new_tokens(dwl.seed + 91, dwl.B * q_len, dwl.Hq, dwl.D, "k")
    q = _bf16(t, qb).view(dwl.B, q_len, dwl.Hq, dwl.D)
    o = t.empty_like(q)
    need = A.attn_decode_multi_workspace_size(dwl.B, q_len, dwl.Hq, dwl.Hkv, dwl.D, dwl.ctx_hi, dwl.window, 0)
    ws = t.empty(max(need, 1), dtype=t.uint8, device="cuda")
    flush = t.ones(512 * 1024 * 1024 // 4, dtype=t.float32, device="cuda")

    def call():
        A.attn_decode_paged_multi(q, Dd["kc"], Dd["vc"], Dd["table"], Dd["ctx"], dwl.ctx_hi,
                                  k_scale=Dd["ks"], v_scale=Dd["vs"], scale=dwl.scale, window=dwl.window,
                                  out=o, workspace=ws)
    call()
    ms = []
    for _ in range(reps):
        flush.sum()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        t.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    per, ms = ms, float(np.mean(ms))
    # algorithmic bytes: the visible K/V once (as single-token decode) plus q_len x Q and O
    byts = decode_bytes(dwl, Dd["ctx_np"]) + 2.0 * dwl.B * (q_len - 1) * dwl.Hq * dwl.D * 2
    gbs = byts / (ms * 1e-3) / 1e9
    G = dwl.Hq // dwl.Hkv
    if q_len * G <= 16:
        path = "decode kernels"
    else:  # the library's routing: two virtual KV heads per cache head when that suffices
        R = next((r for r in range(1, G + 1) if G % r == 0 and (G // r) * q_len <= 16), 0)
        path = "decode kernels, 2 virtual KV heads per cache head" if R == 2 else "paged prefill kernel"
    return {"kernel": f"attn_decode_paged_multi ({path})", "q_len": q_len, "ms": ms,
            "ms_percentiles": _pct(per),
            "GB/s": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "algorithmic_bytes": byts,
            "tokens_per_s": dwl.B * q_len / (ms * 1e-3), "calls": reps,
            "workload": f"{dwl.name} cache, {q_len} draft rows per sequence, causal among them"}


def time_append_rope(t, A, reps: int):
    """kv_cache_append_rope filling a permuted bf16 cache with 16 x 4096 prompt tokens (8 KV
    heads, D = 128): HBM GB/s of the rows read and written."""
    from synth import paged_table
    B, S, Hkv, D = 16, 4096, 8, 128
    ctx = np.full(B, S, np.int32)
    table, nb = paged_table(ctx, 16, 1404)
    T = B * S
    gen = t.Generator(device="cuda").manual_seed(1404)
    kn = t.randn((T, Hkv, D), device="cuda", generator=gen).to(t.bfloat16)
    vn = t.randn((T, Hkv, D), device="cuda", generator=gen).to(t.bfloat16)
    seq = t.arange(B, dtype=t.int32, device="cuda").repeat_interleave(S)
    pos = t.arange(S, dtype=t.int32, device="cuda").repeat(B)
    kc = t.empty((nb, Hkv, 16, D), dtype=t.bfloat16, device="cuda")
    vc = t.empty_like(kc)
    tt = t.from_numpy(table).cuda()

    def call():
        A.kv_cache_append_rope(kn, vn, seq, pos, tt, kc, vc, rope_base=500000.0)
    call()
    ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    t.cuda.synchronize()
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    ms = float(np.mean(per))
    byts = 4.0 * T * Hkv * D * 2 + 2.0 * T * 4  # K, V read and written; seq, pos read
    gbs = byts / (ms * 1e-3) / 1e9
    return {"kernel": "kv_cache_append_rope", "ms": ms, "ms_percentiles": _pct(per), "GB/s": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "algorithmic_bytes": byts, "calls": reps,
            "workload": f"{T} tokens ({B} x {S}), Hkv={Hkv} D={D} bf16, RoPE base 500000, permuted pool"}


def time_decode_fp8(t, A, dwl, Dd, reps: int):
    """attn_decode_paged over an FP8 E4M3 copy of the decode workload's bf16 cache (quantized
    on the GPU by kv_cache_append), timed per call after a cache-evicting read."""
    import dataclasses
    nb = Dd["nb"]
    T = nb * dwl.block_size
    ident = t.arange(nb, dtype=t.int32, device="cuda")[None]
    seq = t.zeros(T, dtype=t.int32, device="cuda")
    pos = t.arange(T, dtype=t.int32, device="cuda")
    q8 = {}
    for which in ("k", "v"):
        rows = Dd[which + "c"].permute(0, 2, 1, 3).contiguous().view(T, dwl.Hkv, dwl.D)
        c = t.empty((nb, dwl.Hkv, dwl.block_size, dwl.D), dtype=t.uint8, device="cuda")
        s = t.empty((nb, dwl.Hkv, dwl.block_size), dtype=t.float16, device="cuda")
        A.kv_cache_append(rows, rows, seq, pos, ident, c, c, k_scale=s, v_scale=s)
        del rows
        q8[which] = (c, s)
    flush = t.ones(512 * 1024 * 1024 // 4, dtype=t.float32, device="cuda")
    o = t.empty_like(Dd["q"])

    def call():
        A.attn_decode_paged(Dd["q"], q8["k"][0], q8["v"][0], Dd["table"], Dd["ctx"], dwl.ctx_hi,
                            k_scale=q8["k"][1], v_scale=q8["v"][1], scale=dwl.scale, window=dwl.window,
                            out=o)
    call()
    ms = []
    for _ in range(reps):
        flush.sum()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        t.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    per, ms = ms, float(np.mean(ms))
    byts = decode_bytes(dataclasses.replace(dwl, kv_dtype="fp8"), Dd["ctx_np"])
    gbs = byts / (ms * 1e-3) / 1e9
    return {"kernel": "attn_decode_paged (FP8 E4M3 cache)", "ms": ms, "ms_percentiles": _pct(per),
            "GB/s": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "algorithmic_bytes": byts, "calls": reps,
            "tokens_per_s": dwl.B / (ms * 1e-3),
            "workload": f"{dwl.name} shapes with the cache quantized to FP8 E4M3 + fp16 per-token scales"}


def cpu_baseline(pwl, budget_s: float, o_dev=None):
    """The oracle, untuned, on a time-bounded sample of the same workload: whole (batch, head)
    pairs, every query row of each, taken in an order that alternates batches and walks the
    heads by 13 (so several KV heads are covered). With o_dev (the timed prefill's output, on
    the device) every row of each sampled pair is also compared with the oracle (untimed):
    `prefill_max_abs_err`, the largest |GPU - oracle| over them."""
    import oracle
    from synth import prefill_slab
    cores, blas = 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            cores = max(i.get("num_threads", 1) for i in libs)
            blas = ",".join(sorted({str(i.get("internal_api")) for i in libs}))
    except Exception:  # pragma: no cover
        pass
    G = pwl.Hq // pwl.Hkv
    pos = np.arange(pwl.S)
    n_pairs = pwl.Hq * pwl.B
    order = [(i % pwl.B, (i // pwl.B * 13) % pwl.Hq) for i in range(n_pairs)]
    pairs, flops, el, err, rows = [], 0.0, 0.0, 0.0, 0
    for b, h in order:
        if el >= budget_s:
            break
        q = prefill_slab(pwl, "q", b, h)
        k = prefill_slab(pwl, "k", b, h // G)
        v = prefill_slab(pwl, "v", b, h // G)
        t0 = time.perf_counter()
        ro, _ = oracle.attention_head(q, k, v, pwl.scale, pos, pwl.causal, pwl.window)
        el += time.perf_counter() - t0
        if o_dev is not None:
            got = o_dev[b, :, h, :].float().cpu().numpy().astype(np.float64)
            err = max(err, float(np.max(np.abs(got - ro))))
            rows += got.shape[0]
        pairs.append((b, h))
        flops += 4.0 * pwl.D * prefill_pairs(pwl.S, pwl.causal, pwl.window)
    out = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"fp64 NumPy oracle prefill of {len(pairs)} of {n_pairs} (batch, head) pairs of "
                     f"{pwl.name} ({', '.join(f'b{b}h{h}' for b, h in pairs)}), all {pwl.S} rows each, "
                     f"{el:.1f} s; BLAS ({blas}) threads = cores"}
    if o_dev is not None:
        out["prefill_max_abs_err"] = err  # the timed run's output, bf16, against the fp64 oracle
        out["rows_checked"] = rows
    return out


def measured_peaks() -> dict | None:
    """Run the measured-ceiling program built next to the library (bf16 MFMA loop, shader
    clock, HBM streaming read, random 2 KB gather) as a child process; None if not built."""
    import subprocess
    exe = os.path.join(ROOT, "attention_attn_prefill_amd", "attn_peaks")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    except subprocess.TimeoutExpired:
        return {"error": "timed out"}
    if r.returncode != 0:
        return {"error": r.stderr.strip()[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


# Which calls one step runs. The first prefill workload gives `value` and `roofline`, the first
# decode workload `roofline_decode`; every other workload gets a roofline object of its own.
WORKLOAD_SETS = {
    # the configurations the targets are set on (long-context sliding-window prefill; INT8 and
    # sliding-window paged decode), with the Llama-3.2-1B-shaped prefill and decode beside them
    "target": (["prefill_swa_s16384", "prefill_llama1b_s4096"],
               ["decode_int8_70b_b16", "decode_swa_b32", "decode_llama1b_b64"]),
    "llama1b": (["prefill_llama1b_s4096"], ["decode_llama1b_b64"]),
    "swa": (["prefill_swa_s16384"], ["decode_swa_b32"]),
    "int8_70b": ([], ["decode_int8_70b_b16"]),
    "fp8_70b": ([], ["decode_fp8_70b_b16"]),
}
ROOFLINE_KEY = {  # JSON key of each workload's roofline object
    "decode_swa_b32": "roofline_decode_swa", "decode_llama1b_b64": "roofline_decode_llama1b",
    "prefill_llama1b_s4096": "roofline_prefill_llama1b", "prefill_swa_s16384": "roofline_prefill_swa",
    "decode_int8_70b_b16": "roofline_decode_int8", "decode_fp8_70b_b16": "roofline_decode_fp8",
}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="target", choices=sorted(WORKLOAD_SETS))
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache-evicting scratch read")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-prefill, multi-row, RoPE-append and FP8 timings beside the step")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-ceiling program (MFMA loop, HBM read and gather)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 3 times (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the attention "
              "path in this repository runs on a single GPU", file=sys.stderr)
        return 2

    # measured ceilings first, in a child process, before this process touches the GPU
    peaks = None if (args.no_peaks or args.copy_calibration) else measured_peaks()

    import torch as t
    import attention_attn_prefill_amd as A
    from synth import WORKLOADS
    A.lib()  # fail loudly if the HIP library is missing
    assert t.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        src = t.ones(COPY_CALIBRATION_BYTES // 4, dtype=t.float32, device="cuda")
        dst = t.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        t.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_CALIBRATION_BYTES, "launches": 3}))
        return 0

    import dataclasses
    c5 = WORKLOADS["decode_int8_70b_b16"]
    wls = dict(WORKLOADS)
    wls["decode_fp8_70b_b16"] = dataclasses.replace(c5, name="decode_fp8_70b_b16", kv_dtype="fp8")
    pnames, dnames = WORKLOAD_SETS[args.workload]
    pwls = [wls[n] for n in pnames]
    dwls = [wls[n] for n in dnames]
    print(f"bench: setting up {', '.join(pnames + dnames)}", file=sys.stderr, flush=True)
    P, Dd = {}, {}
    for w in pwls:
        P[w.name] = setup_prefill(t, w)
        print(f"bench: {w.name} ready", file=sys.stderr, flush=True)
    for w in dwls:
        Dd[w.name] = setup_decode(t, w)
        print(f"bench: {w.name} ready", file=sys.stderr, flush=True)
    flush = t.ones(512 * 1024 * 1024 // 4, dtype=t.float32, device="cuda")
    t.cuda.synchronize()

    def step(ev=None):
        e = ev or {}

        def rec(key):
            if key in e:
                e[key].record()
        for w in dwls:
            d = Dd[w.name]
            rec(("a0", w.name))
            A.kv_cache_append(d["kn"], d["vn"], d["seq"], d["pos"], d["table"], d["kc"], d["vc"],
                              k_scale=d["ks"], v_scale=d["vs"])
            rec(("a1", w.name))
            if not args.no_flush:
                flush.sum()
            rec(("d0", w.name))
            A.attn_decode_paged(d["q"], d["kc"], d["vc"], d["table"], d["ctx"], w.ctx_hi,
                                k_scale=d["ks"], v_scale=d["vs"], scale=w.scale, window=w.window,
                                out=d["o"], workspace=d["ws"])
            rec(("d1", w.name))
        for w in pwls:
            p = P[w.name]
            rec(("p0", w.name))
            A.attn_prefill(p["q"], p["k"], p["v"], scale=w.scale, causal=w.causal, window=w.window,
                           out=p["o"])
            rec(("p1", w.name))

    for _ in range(args.warmup):
        step()
    t.cuda.synchronize()
    keys = [(k, w.name) for w in dwls for k in ("a0", "a1", "d0", "d1")] + \
           [(k, w.name) for w in pwls for k in ("p0", "p1")]
    evs = [{k: t.cuda.Event(enable_timing=True) for k in keys} for _ in range(args.steps)]
    t.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    t.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def times(a, b):  # per-step times (ms) between two events
        return np.array([e[a].elapsed_time(e[b]) for e in evs])

    out = {"metric": "paged decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% MFMA peak)",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) tensors, bf16; INT8 cache quantized on the GPU from them; no dataset)"}
    mfma_meas = (peaks or {}).get("mfma_bf16_tflops")
    gather_meas = (peaks or {}).get("hbm_gather_2k_gbs")
    decodes, prefills = {}, {}
    for w in dwls:
        d = Dd[w.name]
        x = times(("d0", w.name), ("d1", w.name))
        ms = float(x.mean())
        byts = decode_bytes(w, d["ctx_np"])
        gbs = byts / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode", w.name)}
        if gather_meas:
            roof["frac_of_measured"] = gbs / gather_meas  # the random 2 KB gather ceiling
        decodes[w.name] = {
            "kernel": "attn_decode_paged (split KV + log-sum-exp merge; time per call, both kernels)",
            "ms": ms, "ms_percentiles": _pct(x), "GB/s": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "algorithmic_bytes": byts, "tokens_per_s": w.B / (ms * 1e-3),
            "append_ms": float(times(("a0", w.name), ("a1", w.name)).mean()), "roofline": roof,
            "workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} kv={w.kv_dtype} "
                        f"ctx=[{w.ctx_lo},{w.ctx_hi}] window={w.window} block=16"}
    for w in pwls:
        x = times(("p0", w.name), ("p1", w.name))
        ms = float(x.mean())
        fl = prefill_flops(w)
        tf = fl / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / BF16_PEAK_TFLOPS, "traffic": measured_traffic("prefill", w.name)}
        if mfma_meas:
            roof["frac_of_measured"] = tf / mfma_meas
        prefills[w.name] = {
            "kernel": "attn_prefill (bf16 MFMA)", "ms": ms, "ms_percentiles": _pct(x), "TFLOP/s": tf,
            "algorithmic_flops": fl, "tokens_per_s": w.B * w.S / (ms * 1e-3), "roofline": roof,
            "workload": f"{w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
                        f"causal={w.causal} window={w.window}"}
    if pwls:
        head = prefills[pwls[0].name]
        out.update(value=head["TFLOP/s"], unit="TFLOP/s")
        out["roofline"] = head["roofline"]
    else:
        head = decodes[dwls[0].name]
        out.update(value=head["GB/s"], unit="GB/s")
        out["roofline"] = head["roofline"]
    if dwls:
        out["roofline_decode"] = decodes[dwls[0].name]["roofline"]
    for name, entry in list(decodes.items()) + list(prefills.items()):
        if entry["roofline"] is not out["roofline"] and entry["roofline"] is not out.get("roofline_decode"):
            out[ROOFLINE_KEY[name]] = entry["roofline"]
    out["prefill"] = prefills
    out["decode"] = decodes
    if peaks is not None:
        out["measured_peaks"] = peaks
    out["config"] = {"workload": " + ".join(pnames + dnames),
                     "headline": {"value": pnames[0] if pnames else dnames[0],
                                  "roofline_decode": dnames[0] if dnames else None},
                     "step": "per decode workload: kv_cache_append -> cache flush -> attn_decode_paged; "
                             "then attn_prefill per prefill workload"}
    if "decode_llama1b_b64" in Dd and not args.no_chunked:
        dwl, d3 = wls["decode_llama1b_b64"], Dd["decode_llama1b_b64"]
        out["prefill_paged"] = time_chunked(t, A, max(5, args.steps))
        out["decode_multi"] = time_decode_multi(t, A, dwl, d3, max(5, args.steps))
        # 8 drafts: 32 query columns per KV head, two virtual KV heads of 16 columns each
        out["decode_multi_8"] = time_decode_multi(t, A, dwl, d3, max(5, args.steps), q_len=8)
        out["append_rope"] = time_append_rope(t, A, max(5, args.steps))
        out["decode_fp8"] = time_decode_fp8(t, A, dwl, d3, max(5, args.steps))
    if args.cpu_budget > 0 and pwls:
        w = pwls[0]
        o_host = P[w.name]["o"]
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, o_host)
        prefills[w.name]["max_abs_err_vs_oracle"] = out["cpu_baseline"]["prefill_max_abs_err"]
        prefills[w.name]["rows_checked_vs_oracle"] = out["cpu_baseline"]["rows_checked"]
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
