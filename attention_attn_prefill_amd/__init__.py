"""Python binding of libattn (argument marshalling only).

Every computation runs in the HIP kernels of libattn.so; torch supplies device memory and the
current stream. The names follow the C ABI in include/attn.h: attn_prefill,
attn_prefill_paged, attn_decode_paged, attn_decode_paged_multi, kv_cache_append,
attn_decode_workspace_size, attn_decode_multi_workspace_size, attn_decode_paged_noalloc,
kv_cache_append_rope, attn_rope_inplace.
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
    "attn_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                                       ctypes.c_float, _I, _I, _P]),
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


def _byte_cache_dtypes():
    import torch
    return tuple(d for d in (torch.int8, torch.uint8, getattr(torch, "float8_e4m3fn", None)) if d is not None)


def _need(t, name, dtypes=None, shape=None, ndim=None):
    """Reject what the C ABI cannot see: a wrong dtype or shape (the library reads raw memory
    with the layout its sizes imply) or a non-contiguous view; raises ValueError. Devices are
    checked once all arguments passed these checks (_on_device)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: {t.dim()} dimensions, expected {ndim}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    """Every given tensor must live on the device of the first one (a GPU)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call runs on {dev}")


def _need_scales(k_cache, k_scale, v_scale):
    """fp16 scales [num_blocks][Hkv][block_size] for byte caches; none for a bf16 cache."""
    import torch
    if k_cache.dtype == torch.bfloat16:
        if k_scale is not None or v_scale is not None:
            raise ValueError("k_scale / v_scale are only for int8 / fp8 caches")
        return
    shape = tuple(k_cache.shape[:3])
    _need(k_scale, "k_scale", (torch.float16,), shape)
    _need(v_scale, "v_scale", (torch.float16,), shape)


def _need_cache(k_cache, v_cache, bf16_only=False):
    import torch
    dts = (torch.bfloat16,) if bf16_only else (torch.bfloat16,) + _byte_cache_dtypes()
    _need(k_cache, "k_cache", dts, ndim=4)
    _need(v_cache, "v_cache", (k_cache.dtype,), tuple(k_cache.shape))


def attn_prefill(q, k, v, *, scale: float | None = None, causal: bool = True, window: int = 0,
                 out=None, lse=None):
    """Prefill attention. q [B][S][Hq][D], k/v [B][S][Hkv][D] (float32 or bfloat16).

    Returns out (same shape/dtype as q); fills `lse` ([B][Hq][S] float32) when given.
    """
    import torch
    _need(q, "q", (torch.float32, torch.bfloat16), ndim=4)
    B, S, Hq, D = q.shape
    _need(k, "k", (q.dtype,), ndim=4)
    Hkv = k.shape[2]
    _need(k, "k", shape=(B, S, Hkv, D))
    _need(v, "v", (q.dtype,), tuple(k.shape))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (q.dtype,), tuple(q.shape))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (B, Hq, S))
    _on_device(q=q, k=k, v=v, out=out, lse=lse)
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
    _need(q, "q", (torch.bfloat16,), ndim=3)
    total_q, Hq, D = q.shape
    _need_cache(k_cache, v_cache, bf16_only=True)
    num_blocks, Hkv, bs, Dc = k_cache.shape
    if Dc != D:
        raise ValueError(f"k_cache head_dim {Dc} != q head_dim {D}")
    _need(cu_q, "cu_q", (torch.int32,), ndim=1)
    B = cu_q.shape[0] - 1
    _need(block_table, "block_table", (torch.int32,), ndim=2)
    if block_table.shape[0] != B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows, cu_q describes {B} sequences")
    _need(context_lens, "context_lens", (torch.int32,), (B,))
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must be given together")
    if k_new is not None:
        _need(k_new, "k_new", (torch.bfloat16,), (total_q, Hkv, D))
        _need(v_new, "v_new", (torch.bfloat16,), (total_q, Hkv, D))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (torch.bfloat16,), tuple(q.shape))
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (total_q, Hq))
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, cu_q=cu_q,
               context_lens=context_lens, k_new=k_new, v_new=v_new, out=out, lse=lse)
    _check(lib().attn_prefill_paged(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(cu_q), _ptr(context_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, D, bs,
        block_table.shape[1], num_blocks, int(max_q_len), total_q,
        float(D ** -0.5 if scale is None else scale), int(bool(causal)), int(window), _stream(q)))
    return out


def attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, window=0, split_tokens=0) -> int:
    return int(lib().attn_decode_workspace_size(B, Hq, Hkv, D, max_context_len, window, split_tokens))


def _decode_args(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, out, workspace,
                 multi):
    """Checks shared by the decode wrappers; q is [B][Hq][D], or [B][q_len][Hq][D] (multi)."""
    import torch
    _need(q, "q", (torch.bfloat16,))
    if multi and q.dim() != 4:
        raise ValueError("q must be [B][q_len][Hq][D]")
    if not multi and q.dim() != 3:
        raise ValueError("q must be [B][Hq][D]; attn_decode_paged_multi takes [B][q_len][Hq][D]")
    _need_cache(k_cache, v_cache)
    if k_cache.shape[3] != q.shape[-1]:
        raise ValueError(f"k_cache head_dim {k_cache.shape[3]} != q head_dim {q.shape[-1]}")
    _need_scales(k_cache, k_scale, v_scale)
    B = q.shape[0]
    _need(block_table, "block_table", (torch.int32,), ndim=2)
    if block_table.shape[0] != B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows for a batch of {B}")
    _need(context_lens, "context_lens", (torch.int32,), (B,))
    if out is not None:
        _need(out, "out", (torch.bfloat16,), tuple(q.shape))
    if workspace is not None:
        _need(workspace, "workspace")
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
               block_table=block_table, context_lens=context_lens, out=out, workspace=workspace)


def attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, max_context_len: int, *,
                      k_scale=None, v_scale=None, scale: float | None = None, window: int = 0,
                      split_tokens: int = 0, out=None, workspace=None):
    """Single-token decode over a paged cache.

    q [B][Hq][D] bf16; caches [num_blocks][Hkv][block_size][D] bf16, int8, or uint8 /
    float8_e4m3fn holding FP8 E4M3 codes (+ fp16 scales [num_blocks][Hkv][block_size]);
    block_table int32 [B][max_blocks]; context_lens int32 [B]. A workspace of
    attn_decode_workspace_size(...) bytes is allocated when not given.
    """
    import torch
    _decode_args(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, out, workspace,
                 False)
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


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, context_lens, max_context_len: int, *,
                              k_scale=None, v_scale=None, scale: float | None = None, window: int = 0,
                              split_tokens: int = 0, out=None):
    """attn_decode_paged without a workspace: the library keeps the partials in a static
    per-GPU device array (32 MiB). Calls that may overlap on one GPU must not be issued."""
    import torch
    _decode_args(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, out, None,
                 False)
    B, Hq, D = q.shape
    num_blocks, Hkv, bs, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    _check(lib().attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        _ptr(context_lens), _ptr(out), _dtype_code(k_cache), B, Hq, Hkv, D, bs,
        block_table.shape[1], num_blocks, int(max_context_len),
        float(D ** -0.5 if scale is None else scale), int(window), int(split_tokens), _stream(q)))
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
    _decode_args(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, out, workspace,
                 True)
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


def _append_args(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, k_scale, v_scale):
    import torch
    _need(k_new, "k_new", (torch.bfloat16,), ndim=3)
    T, Hkv, D = k_new.shape
    _need(v_new, "v_new", (torch.bfloat16,), (T, Hkv, D))
    _need(seq_idx, "seq_idx", (torch.int32,), (T,))
    _need(pos, "pos", (torch.int32,), (T,))
    _need(block_table, "block_table", (torch.int32,), ndim=2)
    _need_cache(k_cache, v_cache)
    if tuple(k_cache.shape[1:2]) + tuple(k_cache.shape[3:]) != (Hkv, D):
        raise ValueError(f"k_cache {tuple(k_cache.shape)} does not hold rows of {Hkv} heads x {D}")
    _need_scales(k_cache, k_scale, v_scale)
    _on_device(k_new=k_new, v_new=v_new, seq_idx=seq_idx, pos=pos, block_table=block_table,
               k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale)


def kv_cache_append(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, *,
                    k_scale=None, v_scale=None):
    """Write rows k_new/v_new [T][Hkv][D] (bf16) at (seq_idx[t], pos[t]) of the paged cache."""
    _append_args(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, k_scale, v_scale)
    T, Hkv, D = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    _check(lib().kv_cache_append(
        _ptr(k_new), _ptr(v_new), _ptr(seq_idx), _ptr(pos), _ptr(block_table), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _dtype_code(k_cache), T, Hkv, D, bs,
        block_table.shape[0], block_table.shape[1], num_blocks, _stream(k_new)))


def kv_cache_append_rope(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, *,
                         rope_base: float = 10000.0, k_scale=None, v_scale=None):
    """kv_cache_append with each K row rotated (RoPE) at its position before it is stored."""
    _append_args(k_new, v_new, seq_idx, pos, block_table, k_cache, v_cache, k_scale, v_scale)
    T, Hkv, D = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    _check(lib().kv_cache_append_rope(
        _ptr(k_new), _ptr(v_new), _ptr(seq_idx), _ptr(pos), _ptr(block_table), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _dtype_code(k_cache), T, Hkv, D, bs,
        block_table.shape[0], block_table.shape[1], num_blocks, float(rope_base), _stream(k_new)))


def attn_rope_inplace(x, pos, *, rope_base: float = 10000.0):
    """Rotate bf16 rows x [T][H][D] in place at positions pos [T] (int32)."""
    import torch
    _need(x, "x", (torch.bfloat16,), ndim=3)
    T, H, D = x.shape
    _need(pos, "pos", (torch.int32,), (T,))
    _on_device(x=x, pos=pos)
    _check(lib().attn_rope_inplace(_ptr(x), _ptr(pos), T, H, D, float(rope_base), _stream(x)))
    return x
