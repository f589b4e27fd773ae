"""CPU checks of the Python binding's argument validation: every tensor crosses the C ABI as a
raw pointer, so the binding rejects dtypes, shapes, strides and devices the library would
misread, before anything reaches the library. Host tensors are used throughout; the checks
that precede the device check name the faulty argument, and otherwise-valid host tensors are
rejected as not being on the device."""
import pytest
import torch

import attention_attn_prefill_amd as A

bf, f32, i32, i64, f16 = torch.bfloat16, torch.float32, torch.int32, torch.int64, torch.float16


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _decode_kw(**over):
    kw = dict(q=z(2, 8, 64), k_cache=z(5, 2, 16, 64), v_cache=z(5, 2, 16, 64),
              block_table=z(2, 3, dtype=i32), context_lens=z(2, dtype=i32))
    kw.update(over)
    return kw


def _call_decode(kw, **opts):
    return A.attn_decode_paged(kw["q"], kw["k_cache"], kw["v_cache"], kw["block_table"],
                               kw["context_lens"], 40, **opts)


@pytest.mark.parametrize("over,opts,msg", [
    (dict(q=z(2, 8, 64, dtype=f32)), {}, "q: dtype"),
    (dict(v_cache=z(5, 2, 16, 64, dtype=torch.int8)), {}, "v_cache: dtype"),  # mixed cache kinds
    (dict(v_cache=z(5, 2, 16, 128)), {}, "v_cache: shape"),
    (dict(k_cache=z(5, 2, 16, 128), v_cache=z(5, 2, 16, 128)), {}, "head_dim"),
    (dict(block_table=z(2, 3, dtype=i64)), {}, "block_table: dtype"),
    (dict(context_lens=z(2, dtype=i64)), {}, "context_lens: dtype"),
    (dict(context_lens=z(3, dtype=i32)), {}, "context_lens: shape"),
    (dict(block_table=z(3, 3, dtype=i32)), {}, "block_table has 3 rows"),
    (dict(q=z(2, 64, 8).transpose(1, 2)), {}, "q must be contiguous"),
    ({}, dict(out=z(2, 8, 64, dtype=f32)), "out: dtype"),
    ({}, dict(out=z(2, 8, 32)), "out: shape"),
    ({}, dict(k_scale=z(5, 2, 16, dtype=f16)), "only for int8"),
    (dict(k_cache=z(5, 2, 16, 64, dtype=torch.int8), v_cache=z(5, 2, 16, 64, dtype=torch.int8)), {},
     "k_scale is required"),
    (dict(k_cache=z(5, 2, 16, 64, dtype=torch.int8), v_cache=z(5, 2, 16, 64, dtype=torch.int8)),
     dict(k_scale=z(5, 2, 16, dtype=f32), v_scale=z(5, 2, 16, dtype=f16)), "k_scale: dtype"),
    (dict(k_cache=z(5, 2, 16, 64, dtype=torch.uint8), v_cache=z(5, 2, 16, 64, dtype=torch.uint8)),
     dict(k_scale=z(5, 2, 16, dtype=f16), v_scale=z(5, 2, 8, dtype=f16)), "v_scale: shape"),
    ({}, {}, "must be a device tensor"),
])
def test_decode_rejects(over, opts, msg):
    with pytest.raises(ValueError, match=msg):
        _call_decode(_decode_kw(**over), **opts)


def test_decode_multi_rejects():
    kw = _decode_kw(q=z(2, 3, 8, 64))
    with pytest.raises(ValueError, match="must be a device tensor"):
        A.attn_decode_paged_multi(kw["q"], kw["k_cache"], kw["v_cache"], kw["block_table"], kw["context_lens"], 40)
    with pytest.raises(ValueError, match=r"q must be \[B\]\[q_len\]"):
        A.attn_decode_paged_multi(z(2, 8, 64), kw["k_cache"], kw["v_cache"], kw["block_table"], kw["context_lens"], 40)
    with pytest.raises(ValueError, match="out: shape"):
        A.attn_decode_paged_multi(kw["q"], kw["k_cache"], kw["v_cache"], kw["block_table"], kw["context_lens"], 40,
                                  out=z(2, 8, 64))


@pytest.mark.parametrize("args,opts,msg", [
    ((z(1, 8, 4, 64, dtype=f32), z(1, 8, 2, 64), z(1, 8, 2, 64)), {}, "k: dtype"),
    ((z(1, 8, 4, 64), z(1, 7, 2, 64), z(1, 7, 2, 64)), {}, "k: shape"),
    ((z(1, 8, 4, 64), z(1, 8, 2, 64), z(1, 8, 1, 64)), {}, "v: shape"),
    ((z(1, 8, 4, 64), z(1, 8, 2, 64), z(1, 8, 2, 64)), dict(out=z(1, 8, 4, 64, dtype=f32)), "out: dtype"),
    ((z(1, 8, 4, 64), z(1, 8, 2, 64), z(1, 8, 2, 64)), dict(lse=z(1, 8, 4, dtype=f32)), "lse: shape"),
    ((z(1, 8, 4, 64), z(1, 8, 2, 64), z(1, 8, 2, 64)), dict(lse=z(1, 4, 8, dtype=bf)), "lse: dtype"),
    ((z(8, 4, 64), z(1, 8, 2, 64), z(1, 8, 2, 64)), {}, "q: 3 dimensions"),
    ((z(1, 8, 4, 64), z(1, 8, 2, 64), z(1, 8, 2, 64)), {}, "must be a device tensor"),
])
def test_prefill_rejects(args, opts, msg):
    with pytest.raises(ValueError, match=msg):
        A.attn_prefill(*args, **opts)


def _paged(**over):
    kw = dict(q=z(10, 8, 64), k_cache=z(6, 2, 16, 64), v_cache=z(6, 2, 16, 64),
              block_table=z(2, 3, dtype=i32), cu_q=z(3, dtype=i32), context_lens=z(2, dtype=i32))
    opts = {k: over.pop(k) for k in list(over) if k in ("k_new", "v_new", "out", "lse")}
    kw.update(over)
    return A.attn_prefill_paged(kw["q"], kw["k_cache"], kw["v_cache"], kw["block_table"], kw["cu_q"],
                                kw["context_lens"], 5, **opts)


@pytest.mark.parametrize("over,msg", [
    (dict(k_cache=z(6, 2, 16, 64, dtype=torch.int8)), "k_cache: dtype"),
    (dict(cu_q=z(3, dtype=i64)), "cu_q: dtype"),
    (dict(block_table=z(3, 3, dtype=i32)), "block_table has 3 rows"),
    (dict(context_lens=z(2, dtype=i64)), "context_lens: dtype"),
    (dict(k_new=z(10, 2, 64)), "given together"),
    (dict(k_new=z(10, 2, 64), v_new=z(10, 2, 32)), "v_new: shape"),
    (dict(lse=z(10, 4, dtype=f32)), "lse: shape"),
    ({}, "must be a device tensor"),
])
def test_prefill_paged_rejects(over, msg):
    with pytest.raises(ValueError, match=msg):
        _paged(**over)


def _append(rope=False, **over):
    kw = dict(k_new=z(4, 2, 64), v_new=z(4, 2, 64), seq_idx=z(4, dtype=i32), pos=z(4, dtype=i32),
              block_table=z(2, 3, dtype=i32), k_cache=z(6, 2, 16, 64), v_cache=z(6, 2, 16, 64))
    opts = {k: over.pop(k) for k in list(over) if k in ("k_scale", "v_scale")}
    kw.update(over)
    fn = A.kv_cache_append_rope if rope else A.kv_cache_append
    return fn(kw["k_new"], kw["v_new"], kw["seq_idx"], kw["pos"], kw["block_table"], kw["k_cache"],
              kw["v_cache"], **opts)


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("over,msg", [
    (dict(seq_idx=z(4, dtype=i64)), "seq_idx: dtype"),
    (dict(pos=z(3, dtype=i32)), "pos: shape"),
    (dict(v_new=z(4, 2, 64, dtype=f32)), "v_new: dtype"),
    (dict(v_cache=z(6, 2, 16, 64, dtype=torch.int8)), "v_cache: dtype"),
    (dict(k_cache=z(6, 4, 16, 64), v_cache=z(6, 4, 16, 64)), "does not hold rows"),
    (dict(k_cache=z(6, 2, 16, 64, dtype=torch.int8), v_cache=z(6, 2, 16, 64, dtype=torch.int8),
          k_scale=z(6, 2, 16, dtype=f16)), "v_scale is required"),
    ({}, "must be a device tensor"),
])
def test_append_rejects(rope, over, msg):
    with pytest.raises(ValueError, match=msg):
        _append(rope, **over)


def test_rope_inplace_rejects():
    with pytest.raises(ValueError, match="x: dtype"):
        A.attn_rope_inplace(z(4, 2, 64, dtype=f32), z(4, dtype=i32))
    with pytest.raises(ValueError, match="must be a device tensor"):
        A.attn_rope_inplace(z(4, 2, 64), z(4, dtype=i32))
    with pytest.raises(ValueError, match="pos: dtype"):
        A.attn_rope_inplace(z(4, 2, 64), z(4, dtype=i64))


@pytest.mark.parametrize("multi", [False, True])
def test_auto_workspace_is_allocated_on_the_call_device(monkeypatch, multi):
    """When no workspace is given, the binding allocates it on q's device (a host buffer passed
    as the device workspace makes the kernel write to a host address). Host tensors stand in
    for device ones: the device check and the library call are replaced by recorders."""
    calls = []
    real_empty = torch.empty

    def empty(*a, **kw):
        calls.append(kw.get("device"))
        kw.pop("device", None)
        return real_empty(*a, **kw)

    class FakeLib:
        def __getattr__(self, name):
            if name.endswith("workspace_size"):
                return lambda *a: 4096
            return lambda *a: A.ATTN_OK

    monkeypatch.setattr(A, "_on_device", lambda **kw: None)
    monkeypatch.setattr(A, "_stream", lambda t: None)
    monkeypatch.setattr(A, "lib", lambda: FakeLib())
    monkeypatch.setattr(torch, "empty", empty)
    q = z(2, 3, 8, 64) if multi else z(2, 8, 64)
    kw = _decode_kw(q=q)
    fn = A.attn_decode_paged_multi if multi else A.attn_decode_paged
    fn(kw["q"], kw["k_cache"], kw["v_cache"], kw["block_table"], kw["context_lens"], 40,
       out=torch.zeros(q.shape, dtype=bf))
    assert calls == [q.device], calls  # the workspace, on q's device
