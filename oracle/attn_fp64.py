"""Plain fp64 CPU oracle for causal/sliding-window prefill attention and paged-KV decode attention.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py
may import this package. The library in attention_attn_prefill_amd/ never does, and nothing
here imports that library. Both sides take their inputs from synth/ only.

What the pages fix, and where (page title, section):
  [TI] "从零构建CUDA推理引擎：Tiny-Infer项目的技术深度解析" (Tiny-Infer, a CUDA/C++ inference engine)
       - 技术架构与模块设计: naive multi-head attention (week 1); a static KV cache preallocated
         to the maximum context, with attention changed to run incrementally for decode (week 2).
       - Flash Attention：内存与计算的重平衡: block-wise attention with an online softmax yields
         the ordinary softmax result without ever storing the full score matrix; therefore the
         oracle is the ordinary definition, not the tiled algorithm.
       - 分页KV缓存：借鉴操作系统的内存管理: the cache is split into fixed-size blocks and a
         mapping table turns a logical position into a physical block.
       - 推测性解码与INT8量化: the KV cache is stored as INT8 instead of FP16.
  [IL] "从零开始的LLM推理优化实验室：从PyTorch基线到Triton内核的完整实践", KV缓存实验与长上下文优化:
       static, growing and sliding-window KV caches.
  [TF] "Triton融合算子优化：LLM推理性能提升3倍的工程实践", 3.3 FP8量化支持: FP8 E4M3 with a
       dynamic per-token scale; 3.1 RMSNorm + RoPE 融合: rotary
       position embedding applied to rows at their position ids, fused with the neighbouring
       elementwise step so the rows cross HBM once; [TI] 技术架构与模块设计 lists RoPE among the
       Llama 3.2 1B operators.

Readings where the pages are silent (the same list is kept in the design notes):
  * query i of Sq queries against Lk keys sits at absolute position P(i) = Lk - Sq + i
    (prefill: P(i) = i; single-token decode: P = ctx - 1);
  * causal: key j is visible iff j <= P(i); sliding window W > 0: additionally P(i) - j < W,
    i.e. exactly W keys including the query's own position; W = 0 means no window;
  * grouped-query attention: query head h reads KV head h // (Hq // Hkv);
  * paged layout: pools [num_blocks][Hkv][block_size][D]; logical token t of sequence b is
    slot t % block_size of physical block table[b][t // block_size];
  * INT8 KV: per token and KV head, a = max|x|, s = fp16(fp32(a) / 127) (both roundings to
    nearest-even), code = clamp(rint(fp32(x) / fp32(s)), -127, 127) with rint ties-to-even;
    s == 0 (a == 0, or a / 127 below half the smallest fp16 subnormal) gives code 0; the
    dequantized value the attention sees is code * s, exactly;
  * FP8 KV: E4M3 as defined by the OCP 8-bit floating point format (1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals, largest finite 448, S.1111.111 = NaN, no infinities);
    per token and KV head a = max|x|, s = fp16(fp32(a) / 448), code = E4M3 of
    clamp(fp32(x) / fp32(s), -448, 448) rounded to nearest-even, sign kept (so -0 is 0x80);
    s == 0 gives code 0; the value attention sees is decode(code) * s;
  * RoPE (the pages name it, give no formula): the Llama convention -- dimension i < D/2 is
    paired with i + D/2 and the pair is rotated by the angle pos * base^(-2i/D); the rotated
    fp64 value is rounded to fp32 and then to bf16 (both to nearest-even) when stored as bf16.

Every function computes in float64 from the exact values the GPU receives.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible_mask", "attention_head", "attention", "gather_logical", "decode_paged", "rope",
    "bf16_round",
    "prefill_paged", "quantize_int8", "dequantize_int8", "append_expected", "merge_partials",
    "fp8_e4m3_decode", "fp8_e4m3_encode", "quantize_fp8", "dequantize_fp8",
]


def visible_mask(qpos, Lk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [len(qpos)][Lk]: which keys each query position may attend to."""
    qpos = np.asarray(qpos, np.int64)[:, None]
    j = np.arange(Lk, dtype=np.int64)[None, :]
    vis = np.ones((qpos.shape[0], Lk), bool)
    if causal:
        vis &= j <= qpos
    if window > 0:
        vis &= (qpos - j) < window
    return vis


def attention_head(q, k, v, scale: float, qpos, causal: bool = True, window: int = 0,
                   row_block: int = 1024):
    """Softmax attention of one query head against one KV head.

    q: [n][D] query rows at absolute positions qpos [n]; k, v: [Lk][D].
    Returns (o [n][D], lse [n]) in float64, lse = natural log of sum_j exp(s_j).

    Rows are independent, so they are processed in groups of `row_block` only to bound
    memory; each group's scores are restricted to the key range any of its rows can see,
    and the exact per-row mask is applied inside it.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    qpos = np.asarray(qpos, np.int64)
    n, Lk = q.shape[0], k.shape[0]
    o = np.empty((n, v.shape[1]), np.float64)
    lse = np.empty(n, np.float64)
    for r0 in range(0, n, row_block):
        rows = slice(r0, min(n, r0 + row_block))
        pos = qpos[rows]
        lo = 0
        hi = Lk
        if causal:
            hi = min(Lk, int(pos.max()) + 1)
        if window > 0:
            lo = max(0, int(pos.min()) - window + 1)
        s = scale * (q[rows] @ k[lo:hi].T)
        vis = visible_mask(pos, Lk, causal, window)[:, lo:hi]
        if not vis.any(axis=1).all():
            raise ValueError("a query row has no visible key")
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        o[rows] = (p / l) @ v[lo:hi]
        lse[rows] = (m + np.log(l))[:, 0]
    return o, lse


def attention(q, k, v, scale: float, causal: bool = True, window: int = 0):
    """Multi-head / grouped-query attention over contiguous tensors.

    q: [B][Sq][Hq][D]; k, v: [B][Lk][Hkv][D]. Returns (o [B][Sq][Hq][D], lse [B][Hq][Sq]).
    """
    B, Sq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    qpos = np.arange(Sq, dtype=np.int64) + (Lk - Sq)
    o = np.empty((B, Sq, Hq, v.shape[3]), np.float64)
    lse = np.empty((B, Hq, Sq), np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            o[b, :, h, :], lse[b, h, :] = attention_head(
                q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], scale, qpos, causal, window)
    return o, lse


def gather_logical(pool, table_row, n_tokens: int, block_size: int):
    """Logical rows [n_tokens][...] of one sequence from a paged pool [num_blocks][Hkv][bs][...]."""
    t = np.arange(n_tokens, dtype=np.int64)
    phys = np.asarray(table_row, np.int64)[t // block_size]
    if (phys < 0).any() or (phys >= pool.shape[0]).any():
        raise ValueError("block table entry out of range for a live token")
    return pool[phys, :, t % block_size]  # [n_tokens][Hkv][...]


def dequantize_int8(codes, scales):
    """Exact value code * scale in float64; codes [...][D] int8, scales [...] fp16."""
    return np.asarray(codes, np.float64) * np.asarray(scales, np.float64)[..., None]


def decode_paged(q, k_pool, v_pool, table, ctx, scale: float, block_size: int, window: int = 0,
                 k_scale=None, v_scale=None, heads=None):
    """Single-token decode over a paged cache.

    q: [B][Hq][D] (the query of each sequence sits at position ctx[b] - 1);
    pools: [num_blocks][Hkv][bs][D] (float values, or int8 codes with fp16 scales
    [num_blocks][Hkv][bs]); table: int32 [B][max_blocks]; ctx: int32 [B].
    `heads` optionally restricts the computed query heads (others are left NaN).
    Returns (o [B][Hq][D], lse [B][Hq]).
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.full((B, Hq, v_pool.shape[3]), np.nan)
    lse = np.full((B, Hq), np.nan)
    heads = range(Hq) if heads is None else heads
    for b in range(B):
        n = int(ctx[b])
        kk = gather_logical(k_pool, table[b], n, block_size)
        vv = gather_logical(v_pool, table[b], n, block_size)
        if k_scale is not None:
            kk = dequantize_int8(kk, gather_logical(k_scale, table[b], n, block_size))
            vv = dequantize_int8(vv, gather_logical(v_scale, table[b], n, block_size))
        for h in heads:
            g = h // G
            ob, lb = attention_head(q[b, h][None, :], kk[:, g, :], vv[:, g, :], scale,
                                    [n - 1], True, window)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def prefill_paged(q, cu_q, k_pool, v_pool, table, ctx, scale: float, block_size: int,
                  causal: bool = True, window: int = 0):
    """Chunked prefill against a paged cache that already holds every key of the chunk.

    q: [total_q][Hq][D] packed rows; sequence b owns rows cu_q[b] .. cu_q[b+1]-1, the last
    q_len_b = cu_q[b+1] - cu_q[b] positions of its ctx[b] keys, so row i of b sits at position
    ctx[b] - q_len_b + i (bottom-right alignment). Pools [num_blocks][Hkv][bs][D].
    Returns (o [total_q][Hq][D], lse [total_q][Hq]).
    """
    total, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    o = np.zeros((total, Hq, v_pool.shape[3]))
    lse = np.zeros((total, Hq))
    for b in range(len(ctx)):
        r0, r1 = int(cu_q[b]), int(cu_q[b + 1])
        if r1 == r0:
            continue
        n = int(ctx[b])
        kk = gather_logical(k_pool, table[b], n, block_size)
        vv = gather_logical(v_pool, table[b], n, block_size)
        qpos = np.arange(r1 - r0) + (n - (r1 - r0))
        for h in range(Hq):
            o[r0:r1, h], lse[r0:r1, h] = attention_head(q[r0:r1, h], kk[:, h // G], vv[:, h // G],
                                                        scale, qpos, causal, window)
    return o, lse


def quantize_int8(x):
    """Symmetric per-row INT8 quantization of the last axis, in fp32 as the kernel does it.

    x: float32 [...][D]. Returns (codes int8 [...][D], scales float16 [...]).
    """
    x = np.asarray(x, np.float32)
    a = np.abs(x).max(axis=-1)
    s16 = (a / np.float32(127.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    q = np.rint(x / safe[..., None])
    q = np.clip(q, -127, 127)
    q = np.where((s32 == 0)[..., None], 0, q)
    return q.astype(np.int8), s16


def fp8_e4m3_decode(codes):
    """Value of E4M3 codes (uint8) in float64: sign * 2^(e-7) * (1 + m/8), or for e == 0 the
    subnormal sign * 2^-6 * m/8; code 0x7f / 0xff is NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def fp8_e4m3_encode(x):
    """Nearest E4M3 code (ties to the even code) of float values |x| <= 448, by comparing with
    the decoded values of all 127 non-negative finite codes; the sign bit is x's (so negative
    values that round to zero give 0x80, -0)."""
    x = np.asarray(x, np.float64)
    if np.any(np.abs(x) > 448) or np.any(np.isnan(x)):
        raise ValueError("fp8_e4m3_encode expects |x| <= 448")
    grid = fp8_e4m3_decode(np.arange(127, dtype=np.uint8))  # 0 .. 448, increasing
    a = np.abs(x)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 126)  # first grid value >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == grid[hi], hi, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)  # -0 keeps its sign


def quantize_fp8(x):
    """Per-row FP8 E4M3 quantization of the last axis, in fp32 as the kernel does it.

    x: float32 [...][D]. Returns (codes uint8 [...][D], scales float16 [...]).
    """
    x = np.asarray(x, np.float32)
    a = np.abs(x).max(axis=-1)
    s16 = (a / np.float32(448.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    y = np.clip(x / safe[..., None], np.float32(-448.0), np.float32(448.0))
    codes = fp8_e4m3_encode(y.astype(np.float64))
    return np.where((s32 == 0)[..., None], 0, codes).astype(np.uint8), s16


def dequantize_fp8(codes, scales):
    """Exact value decode(code) * scale in float64; codes [...][D] uint8, scales [...] fp16."""
    return fp8_e4m3_decode(codes) * np.asarray(scales, np.float64)[..., None]


def append_expected(pool, rows, seq_idx, pos, table, block_size: int):
    """The pool after writing rows[t] ([T][Hkv][...]) at logical position pos[t] of seq_idx[t]."""
    out = np.array(pool, copy=True)
    for t in range(len(seq_idx)):
        b, p = int(seq_idx[t]), int(pos[t])
        pb = int(table[b][p // block_size])
        out[pb, :, p % block_size] = rows[t]
    return out


def rope(x, pos, base: float = 10000.0):
    """Rotary position embedding of rows x [T][H][D] (any float) at positions pos [T], fp64.

    Pair (i, i + D/2) of row t is rotated by angle pos[t] * base ** (-2 i / D):
    out_i = x_i cos - x_{i+D/2} sin, out_{i+D/2} = x_i sin + x_{i+D/2} cos.
    """
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    half = D // 2
    inv_freq = base ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(pos, np.float64)[:, None] * inv_freq[None, :]  # [T][D/2]
    c, s_ = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s_, a * s_ + b * c], axis=-1)


def bf16_round(x):
    """fp64 -> fp32 -> bf16 (each to nearest-even), returned as the bf16 values in float64."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def merge_partials(outs, lses):
    """Combine attention over disjoint key subsets: outs [n][..][D], lses [n][..] -> (o, lse).

    With M = max lse_s and w_s = exp(lse_s - M): o = sum w_s o_s / sum w_s,
    lse = M + ln sum w_s. Subsets with lse = -inf get weight 0.
    """
    outs = np.asarray(outs, np.float64)
    lses = np.asarray(lses, np.float64)
    M = lses.max(axis=0)
    w = np.exp(lses - M)
    tot = w.sum(axis=0)
    o = (w[..., None] * outs).sum(axis=0) / tot[..., None]
    return o, M + np.log(tot)
