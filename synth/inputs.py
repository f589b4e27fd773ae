"""Seeded synthetic workloads for prefill and paged-decode attention.

This module is the only code shared by the oracle side and the HIP side. It draws random
numbers and rounds the drawn fp32 samples to the storage type (bf16 by round-to-nearest-even,
fp16 by numpy's RNE cast). It holds no attention arithmetic: no scores, no softmax, no
position-to-slot index math and no quantization.

Recipe (the pages name no dataset; these tensors are the workload):
  * every tensor is N(0,1) fp32 from numpy PCG64, seeded per (workload seed, tensor id,
    sub-index...), then rounded to bf16 unless the workload is fp32;
  * prefill Q/K/V are drawn per (batch, head) as [S][D] slabs and stacked to [B][S][H][D];
  * decode context lengths are integers uniform in [ctx_lo, ctx_hi] (inclusive);
  * the physical block pool holds sum(ceil(ctx/bs)) blocks plus optional spare blocks; a
    seeded permutation of the pool is dealt out in order to (sequence, logical block);
    table entries past a sequence's last block are -1;
  * pool contents are drawn per physical block in chunks of 64 blocks, so a test can
    regenerate exactly the blocks it samples.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "PrefillWorkload", "DecodeWorkload", "WORKLOADS",
    "bf16_bits", "bf16_value", "prefill_slab", "prefill_inputs", "decode_query",
    "context_lens", "paged_table", "pool_blocks", "pool", "int8_pool_blocks", "int8_pool",
    "fp8_pool", "new_tokens",
]

# tensor ids for seeding sub-streams
_Q, _K, _V, _CTX, _PERM, _KNEW, _VNEW, _KI8, _VI8, _KF8, _VF8 = range(1, 12)
_POOL_CHUNK = 64


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    seed: int
    dtype: str  # "f32" or "bf16"
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    causal: bool = True
    window: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    kv_dtype: str  # "bf16" or "i8"
    B: int
    Hq: int
    Hkv: int
    D: int
    ctx_lo: int
    ctx_hi: int
    block_size: int = 16
    window: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    # causal prefill, contiguous, fp32: 1 x 1 head x 128 x 64
    "prefill_f32_s128": PrefillWorkload("prefill_f32_s128", 1001, "f32", 1, 128, 1, 1, 64),
    # Llama-3.2-1B-shaped causal GQA prefill, bf16
    "prefill_llama1b_s4096": PrefillWorkload("prefill_llama1b_s4096", 1002, "bf16", 1, 4096, 32, 8, 64),
    # Llama-3.2-1B-shaped paged decode, bf16 KV, ragged contexts
    "decode_llama1b_b64": DecodeWorkload("decode_llama1b_b64", 1003, "bf16", 64, 32, 8, 64, 512, 4096),
    # sliding-window prefill then decode, head_dim 128
    "prefill_swa_s16384": PrefillWorkload("prefill_swa_s16384", 1004, "bf16", 2, 16384, 32, 8, 128,
                                          True, 4096),
    "decode_swa_b32": DecodeWorkload("decode_swa_b32", 2004, "bf16", 32, 32, 8, 128, 16384, 16384,
                                     16, 4096),
    # INT8-KV paged decode on one GPU's share of a 70B-shaped layer
    "decode_int8_70b_b16": DecodeWorkload("decode_int8_70b_b16", 1005, "i8", 16, 64, 8, 128,
                                          32768, 32768),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(k) for k in key]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs: the largest sum, 0xFF7FFFFF + 0x8000, still fits in 32 bits
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(shape, *key: int) -> np.ndarray:
    return _rng(*key).standard_normal(shape, dtype=np.float32)


def prefill_slab(wl: PrefillWorkload, which: str, b: int, h: int) -> np.ndarray:
    """[S][D] fp32 values of tensor `which` in {"q","k","v"} for batch b, head h (bf16-exact if bf16)."""
    tid = {"q": _Q, "k": _K, "v": _V}[which]
    x = _normal((wl.S, wl.D), wl.seed, tid, b, h)
    if wl.dtype == "bf16":
        x = bf16_value(bf16_bits(x))
    return x


def prefill_inputs(wl: PrefillWorkload) -> dict:
    """Full Q [B][S][Hq][D], K/V [B][S][Hkv][D] as fp32 values (and uint16 bits when bf16)."""
    out = {}
    for which, H in (("q", wl.Hq), ("k", wl.Hkv), ("v", wl.Hkv)):
        t = np.empty((wl.B, wl.S, H, wl.D), np.float32)
        for b in range(wl.B):
            for h in range(H):
                t[b, :, h, :] = prefill_slab(wl, which, b, h)
        out[which] = t
        if wl.dtype == "bf16":
            out[which + "_bits"] = bf16_bits(t)
    return out


def decode_query(wl: DecodeWorkload) -> tuple[np.ndarray, np.ndarray]:
    """Decode queries [B][Hq][D]: (bf16 bits, fp32 values)."""
    bits = bf16_bits(_normal((wl.B, wl.Hq, wl.D), wl.seed, _Q))
    return bits, bf16_value(bits)


def context_lens(wl: DecodeWorkload) -> np.ndarray:
    if wl.ctx_lo == wl.ctx_hi:
        return np.full(wl.B, wl.ctx_lo, np.int32)
    return _rng(wl.seed, _CTX).integers(wl.ctx_lo, wl.ctx_hi + 1, size=wl.B).astype(np.int32)


def paged_table(ctx: np.ndarray, block_size: int, seed: int, spare_blocks: int = 0,
                permute: bool = True, max_blocks_per_seq: int | None = None):
    """Block table for the given context lengths.

    Returns (table int32 [B][max_blocks_per_seq], num_blocks). Sequence b owns
    ceil(ctx[b]/block_size) physical blocks, taken in order from a seeded permutation of
    range(num_blocks) (identity when permute is False); entries past them are -1.
    """
    per_seq = [-(-int(c) // block_size) for c in ctx]
    num_blocks = sum(per_seq) + spare_blocks
    order = _rng(seed, _PERM).permutation(num_blocks) if permute else np.arange(num_blocks)
    mb = max(per_seq) if max_blocks_per_seq is None else max_blocks_per_seq
    table = np.full((len(ctx), mb), -1, np.int32)
    cursor = 0
    for b, n in enumerate(per_seq):
        table[b, :n] = order[cursor:cursor + n]
        cursor += n
    return table, num_blocks


def pool_blocks(wl: DecodeWorkload, which: str, blocks) -> np.ndarray:
    """fp32 (bf16-exact) contents [len(blocks)][Hkv][bs][D] of physical blocks of pool `which`."""
    tid = {"k": _K, "v": _V}[which]
    blocks = np.asarray(blocks, np.int64)
    out = np.empty((len(blocks), wl.Hkv, wl.block_size, wl.D), np.float32)
    per_block = (wl.Hkv, wl.block_size, wl.D)
    cache = {}
    for i, pb in enumerate(blocks):
        c = int(pb) // _POOL_CHUNK
        if c not in cache:
            cache[c] = _normal((_POOL_CHUNK,) + per_block, wl.seed, tid, c)
        out[i] = cache[c][int(pb) % _POOL_CHUNK]
    return bf16_value(bf16_bits(out))


def pool(wl: DecodeWorkload, which: str, num_blocks: int) -> np.ndarray:
    """Whole pool as bf16 bits [num_blocks][Hkv][bs][D]."""
    per_block = (wl.Hkv, wl.block_size, wl.D)
    tid = {"k": _K, "v": _V}[which]
    out = np.empty((num_blocks,) + per_block, np.uint16)
    for c in range(-(-num_blocks // _POOL_CHUNK)):
        lo, hi = c * _POOL_CHUNK, min(num_blocks, (c + 1) * _POOL_CHUNK)
        out[lo:hi] = bf16_bits(_normal((_POOL_CHUNK,) + per_block, wl.seed, tid, c)[: hi - lo])
    return out


def int8_pool_blocks(wl: DecodeWorkload, which: str, blocks):
    """Directly drawn int8 codes [n][Hkv][bs][D] (uniform in [-127,127]) and fp16 scales
    [n][Hkv][bs] (uniform in [0.5, 1.5) * 3/127), for decode tests that bypass quantization."""
    tid = {"k": _KI8, "v": _VI8}[which]
    blocks = np.asarray(blocks, np.int64)
    codes = np.empty((len(blocks), wl.Hkv, wl.block_size, wl.D), np.int8)
    scales = np.empty((len(blocks), wl.Hkv, wl.block_size), np.float16)
    cache = {}
    for i, pb in enumerate(blocks):
        c = int(pb) // _POOL_CHUNK
        if c not in cache:
            r = _rng(wl.seed, tid, c)
            cc = r.integers(-127, 128, size=(_POOL_CHUNK, wl.Hkv, wl.block_size, wl.D), dtype=np.int8)
            ss = ((0.5 + r.random((_POOL_CHUNK, wl.Hkv, wl.block_size), dtype=np.float32))
                  * np.float32(3.0 / 127.0)).astype(np.float16)
            cache[c] = (cc, ss)
        codes[i] = cache[c][0][int(pb) % _POOL_CHUNK]
        scales[i] = cache[c][1][int(pb) % _POOL_CHUNK]
    return codes, scales


def int8_pool(wl: DecodeWorkload, which: str, num_blocks: int):
    return int8_pool_blocks(wl, which, np.arange(num_blocks))


def fp8_pool(wl: DecodeWorkload, which: str, num_blocks: int):
    """Directly drawn FP8 E4M3 codes [n][Hkv][bs][D] and fp16 scales [n][Hkv][bs] (uniform in
    [0.5, 1.5) / 64), for decode tests that bypass quantization. Codes are uniform over the
    bytes 0x00-0x67 and 0x80-0xE7 (exponent field at most 12: magnitudes up to 60, so values
    times scales stay within about +-1.4, the range of N(0,1) data). Byte values only: no
    format arithmetic happens here."""
    tid = {"k": _KF8, "v": _VF8}[which]
    r = _rng(wl.seed, tid, 0)
    b = r.integers(0, 2 * 0x68, size=(num_blocks, wl.Hkv, wl.block_size, wl.D), dtype=np.int64)
    codes = np.where(b >= 0x68, b - 0x68 + 0x80, b).astype(np.uint8)
    scales = ((0.5 + r.random((num_blocks, wl.Hkv, wl.block_size), dtype=np.float32))
              * np.float32(1.0 / 64.0)).astype(np.float16)
    return codes, scales


def new_tokens(seed: int, T: int, Hkv: int, D: int, which: str) -> tuple[np.ndarray, np.ndarray]:
    """K or V rows [T][Hkv][D] to append: (bf16 bits, fp32 values)."""
    tid = {"k": _KNEW, "v": _VNEW}[which]
    bits = bf16_bits(_normal((T, Hkv, D), seed, tid))
    return bits, bf16_value(bits)
