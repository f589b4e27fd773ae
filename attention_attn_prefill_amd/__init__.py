"""Python binding of libattn (argument marshalling only).

Every computation runs in the HIP kernels of libattn.so; torch supplies device memory and the
current stream. The names follow the C ABI in include/attn.h: attn_prefill,
attn_prefill_paged, attn_decode_paged, attn_decode_paged_multi, kv_cache_append,
attn_decode_workspace_size, attn_decode_multi_workspace_size, kv_cache_append_rope,
attn_rope_inplace.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_DTYPE, ATTN_ERR_UNSUPPORTED, \
    ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(7)
ATTN_F32, ATTN_BF16, ATTN_I8, ATTN_FP8 = 0, 1, 2, 3

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "attn_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _I, _P]),
    "attn_decode_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_prefill_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                _I, _I, ctypes.c_float, _I, _I, _P]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                               ctypes.c_float, _I, _I, _P, ctypes.c_size_t, _P]),
    "attn_decode_multi_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "attn_decode_paged_multi": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                     _I, _I, ctypes.c_float, _I, _I, _P, ctypes.c_size_t, _P]),
    "kv_cache_append": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "kv_cache_append_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                  ctypes.c_float, _P]),
    "attn_rope_inplace": (_I, [_P, _P, _I, _I, _I, ctypes.c_float, _P]),
    "attn_status_str": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
}


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libattn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m attention_attn_prefill_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != ATTN_OK:
        L = lib()
        raise AttnError(status, f"{L.attn_status_str(status).decode()}: {L.attn_last_error().decode()}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.int8:
        return ATTN_I8
    if t.dtype == torch.uint8 or t.dtype == getattr(torch, "float8_e4m3fn", None):
        return ATTN_FP8  # FP8 E4M3 codes, one per byte
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def attn_prefill(q, k, v, *, scale: float | None = None, causal: bool = True, window: int = 0,
                 out=None, lse=None):
    """Prefill attention. q [B][S][Hq][D], k/v [B][S][Hkv][D] (float32 or bfloat16).

    Returns out (same shape/dtype as q); fills `lse` ([B][Hq][S] float32) when given.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = D ** -0.5
    _check(lib().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q),
                              B, S, Hq, Hkv, D, float(scale), int(bool(causal)), int(window),
                              _stream(q)))
    return out


def attn_prefill_paged(q, k_cache, v_cache, block_table, cu_q, context_lens, max_q_len: int, *,
                       k_new=None, v_new=None, scale: float | None = None, causal: bool = True,
                       window: int = 0, out=None, lse=None):
    """Chunked prefill over a paged cache (bf16). q [total_q][Hq][D] packed by cu_q [B+1];
    k_new/v_new [total_q][Hkv][D], when given, are written into the cache by the same launch."""
    import torch
    total_q, Hq, D = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    B = cu_q.shape[0] - 1
    if out is None:
        out = torch.empty_like(q)
    _check(lib().attn_prefill_paged(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(cu_q), _ptr(context_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, D, bs,
        block_table.shape[1], num_blocks, int(max_q_len), total_q,
        float(D ** -0.5 if scale is None else scale), int(bool(causal)), int(window), _stream(q)))
    return out


def attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, window=0, split_tokens=0) -> int:
    return int(lib().attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, window, split_tokens))


def attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, max_context_len: int, *,
                      k_scale=None, v_scale=None, scale: float | None = None, window: int = 0,
                      split_tokens: int = 0, out=None, workspace=None):
    """Single-token decode over a paged cache.

    q [B][Hq][D] bf16; caches [num_blocks][Hkv][block_size][D] bf16, int8, or uint8 /
    float8_e4m3fn holding FP8 E4M3 codes (+ fp16 scales [num_blocks][Hkv][block_size]); block_table int32 [B][max_blocks]; context_lens int32 [B].
    A workspace of attn_decode_workspace_size(...) bytes is allocated when not given.
    """
    import torch
    B, Hq, D = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    need = attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, window, split_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(out), _dtype_code(k_cache), B, Hq, Hkv, D, bs,
        block_table.shape[1], num_blocks, int(max_context_len),
        float(D ** -0.5 if scale is None else scale), int(window), int(split_tokens),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def attn_decode_multi_workspace_size(B, q_len, Hq, Hkv, D, max_context_len, window=0,
                                     split_tokens=0) -> int:
    return int(lib().attn_decode_multi_workspace_size(B, q_len, Hq, Hkv, D, max_context_len, window,
                                                      split_tokens))


def attn_decode_paged_multi(q, k_cache, v_cache, block_table, context_lens, max_context_len: int, *,
                            k_scale=None, v_scale=None, scale: float | None = None, window: int = 0,
                            split_tokens: int = 0, out=None, workspace=None):
    """q_len query rows per sequence (speculative verification): q [B][q_len][Hq][D] bf16, row r at
    position context_lens[b] - q_len + r, causal; caches and table as in attn_decode_paged."""
    import torch
    B, QL, Hq, D = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    need = attn_decode_multi_workspace_size(B, QL, Hq, Hkv, D, max_context_len, window, split_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_decode_paged_multi(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(out), _dtype_code(k_cache), B, QL, Hq, Hkv, D, bs,
        block_table.shape[1], num_blocks, int(max_context_len),
        float(D ** -0.5 if scale is None else scale), int(window), int(split_tokens),
        _ptr(workspace), ws_bytes, _stream(q)))
    return out


def kv_cache_append(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, *,
                    k_scale=None, v_scale=None):
    """Write rows k_new/v_new [T][Hkv][D] (bf16) at (seq_idx[t], pos[t]) of the paged cache."""
    T, Hkv, D = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    _check(lib().kv_cache_append(
        _ptr(k_new), _ptr(v_new), _ptr(seq_idx), _ptr(pos), _ptr(block_table), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _dtype_code(k_cache), T, Hkv, D, bs,
        block_table.shape[0], block_table.shape[1], num_blocks, _stream(k_new)))


def kv_cache_append_rope(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, *,
                         rope_base: float = 10000.0, k_scale=None, v_scale=None):
    """kv_cache_append with each K row rotated (RoPE) at its position before it is stored."""
    T, Hkv, D = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    _check(lib().kv_cache_append_rope(
        _ptr(k_new), _ptr(v_new), _ptr(seq_idx), _ptr(pos), _ptr(block_table), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _dtype_code(k_cache), T, Hkv, D, bs,
        block_table.shape[0], block_table.shape[1], num_blocks, float(rope_base), _stream(k_new)))


def attn_rope_inplace(x, pos, *, rope_base: float = 10000.0):
    """Rotate bf16 rows x [T][H][D] in place at positions pos [T] (int32)."""
    _need(x, "x")
    T, H, D = x.shape
    _check(lib().attn_rope_inplace(_ptr(x), _ptr(pos), T, H, D, float(rope_base), _stream(x)))
    return x
