"""Python entry points with the C ABI's names: argument marshalling only.

Every step of the hot path runs in the HIP kernels behind ``libpagedkv.so``;
these wrappers read shapes, device pointers and the current stream from torch
tensors and pass them through.  torch supplies device memory and streams only.
"""

import torch

from ._lib import (BLOCK_SIZE, PKV_BF16, PKV_F32, check, lib)

_DTYPES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}


def _dt(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _temp_workspace(nbytes_fn, device, stream):
    """A workspace owned by one call (None if 0 bytes).  When the call runs on
    a stream other than torch's current one, the buffer is marked as used there,
    so torch's caching allocator does not hand it out again before that
    stream's work has run."""
    ws = nbytes_fn(device)
    if ws is not None and stream is not None:
        st = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream))
        ws.record_stream(st)
    return ws


def _need_workspace(workspace, cname):
    """The split forms share the plan's work list through the workspace: a fresh
    buffer would hold no plan, so it must be the caller's."""
    if workspace is None:
        raise ValueError(f"{cname}: workspace is required (the one the plan launch filled)")


def pkv_write(key_cache, value_cache, k, v, slot_mapping, stream=None):
    """Scatter new tokens' K/V rows ``[T, Hkv, D]`` into their slots (bit copy)."""
    nb, bs, hkv, d = key_cache.shape
    if value_cache.shape != key_cache.shape or k.shape != v.shape or k.shape[1:] != (hkv, d):
        raise ValueError("shape mismatch between caches and k/v")
    if k.dtype != key_cache.dtype or v.dtype != key_cache.dtype or value_cache.dtype != key_cache.dtype:
        raise TypeError("caches and k/v must share one dtype")
    t = k.shape[0]
    if slot_mapping.shape != (t,):
        raise ValueError("slot_mapping must be [num_tokens]")
    check("pkv_write", lib().pkv_write(
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), _dev(k, "k"), _dev(v, "v"),
        _dev(slot_mapping, "slot_mapping", torch.int32), t, nb, bs, hkv, d, _dt(key_cache),
        _stream(stream)))


def pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len):
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len))


def decode_workspace(num_seqs, num_q_heads, head_dim, max_context_len, device="cuda"):
    """A device buffer of the size ``pkv_attention_decode`` needs (None if 0 bytes).

    torch's allocator returns blocks aligned to at least 256 bytes, as the call
    requires."""
    n = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _decode_call(cname, out, q, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, workspace, stream, own_workspace=False):
    if not own_workspace:
        _need_workspace(workspace, cname)
    s, hq, d = q.shape
    nb, bs, hkv, dk = key_cache.shape
    if out.shape != q.shape or dk != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if out.dtype != q.dtype or key_cache.dtype != q.dtype or value_cache.dtype != q.dtype:
        raise TypeError("q, caches and out must share one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    mb = block_tables.shape[1]
    if workspace is None:
        workspace = _temp_workspace(lambda dv: decode_workspace(s, hq, d, max_context_len, dv), q.device, stream)
    ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(cname, getattr(lib(), cname)(
        _dev(out, "out"), _dev(q, "q"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        float(scale), bs, hq, hkv, d, s, mb, nb, int(max_context_len), _dt(q), ws_ptr, ws_bytes,
        _stream(stream)))
    return out


def pkv_attention_decode(out, q, key_cache, value_cache, block_tables, context_lens, scale,
                         max_context_len, workspace=None, stream=None):
    """Paged decode attention for one new token per sequence; writes ``out`` [S, Hq, D].
    Without ``workspace``, the call uses a buffer of its own."""
    return _decode_call("pkv_attention_decode", out, q, key_cache, value_cache, block_tables,
                        context_lens, scale, max_context_len, workspace, stream, own_workspace=True)


def pkv_attention_decode_plan(out, q, key_cache, value_cache, block_tables, context_lens,
                              scale, max_context_len, workspace=None, stream=None):
    """First launch of ``pkv_attention_decode`` alone (work list from context_lens).
    ``workspace`` is required: the later launches read the plan from it."""
    return _decode_call("pkv_attention_decode_plan", out, q, key_cache, value_cache,
                        block_tables, context_lens, scale, max_context_len, workspace, stream)


def pkv_attention_decode_plan_upload(out, q, key_cache, value_cache, block_tables, context_lens, scale,
                                     max_context_len, host_context_lens, upload_src, upload_dst,
                                     workspace=None, merge_out=None, merge_workspace=None,
                                     host_block_tables=None, stream=None):
    """``_plan`` from a pinned host copy of the lengths, fused with the copy of the
    pinned ``upload_src`` into the device tensor ``upload_dst`` (same byte size),
    in one launch.  ``block_tables`` / ``context_lens`` are the device tensors the
    later launches read (usually views of ``upload_dst``).  With ``merge_out`` and
    ``merge_workspace``, the launch also merges the previous step's partials
    (same shapes, another workspace) into ``merge_out``.  With
    ``host_block_tables`` (pinned, [S, MB]), it also copies each row's used
    entries into ``block_tables``.  ``workspace`` is required (the later launches
    read the plan from it)."""
    _need_workspace(workspace, "pkv_attention_decode_plan_upload")
    if host_block_tables is not None:
        if host_block_tables.is_cuda or not host_block_tables.is_pinned() or not host_block_tables.is_contiguous():
            raise TypeError("host_block_tables must be a contiguous pinned host tensor")
        if host_block_tables.dtype != torch.int32 or tuple(host_block_tables.shape) != tuple(block_tables.shape):
            raise ValueError("host_block_tables must be int32 of block_tables' shape")
    if (merge_out is None) != (merge_workspace is None):
        raise ValueError("give both merge_out and merge_workspace, or neither")
    for name, t in (("host_context_lens", host_context_lens), ("upload_src", upload_src)):
        if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned() or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous pinned host tensor")
    if host_context_lens.dtype != torch.int32 or host_context_lens.shape != (q.shape[0],):
        raise ValueError("host_context_lens must be int32 [num_seqs]")
    nbytes = upload_src.numel() * upload_src.element_size()
    if upload_dst.numel() * upload_dst.element_size() != nbytes:
        raise ValueError("upload_src and upload_dst must have the same byte size")
    s, hq, d = q.shape
    nb, bs, hkv, dk = key_cache.shape
    if out.shape != q.shape or dk != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    ws_ptr = _dev(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    check("pkv_attention_decode_plan_upload", lib().pkv_attention_decode_plan_upload(
        _dev(out, "out"), _dev(q, "q"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        float(scale), bs, hq, hkv, d, s, block_tables.shape[1], nb, int(max_context_len), _dt(q), ws_ptr,
        ws_bytes, host_context_lens.data_ptr(), upload_src.data_ptr(), _dev(upload_dst, "upload_dst"), nbytes,
        None if host_block_tables is None else host_block_tables.data_ptr(),
        None if merge_out is None else _dev(merge_out, "merge_out"),
        None if merge_workspace is None else _dev(merge_workspace, "merge_workspace"), _stream(stream)))
    return out


def pkv_attention_decode_partitions(out, q, key_cache, value_cache, block_tables, context_lens,
                                    scale, max_context_len, workspace=None, stream=None):
    """Second launch of ``pkv_attention_decode`` alone (partition kernel); ``workspace``
    is required (the one the plan launch filled)."""
    return _decode_call("pkv_attention_decode_partitions", out, q, key_cache, value_cache,
                        block_tables, context_lens, scale, max_context_len, workspace, stream)


def pkv_attention_decode_merge(out, q, key_cache, value_cache, block_tables, context_lens, scale,
                               max_context_len, workspace=None, stream=None):
    """Third launch of ``pkv_attention_decode`` alone (log-sum-exp merge); ``workspace``
    is required (the one the partitions wrote)."""
    return _decode_call("pkv_attention_decode_merge", out, q, key_cache, value_cache, block_tables,
                        context_lens, scale, max_context_len, workspace, stream)


def _append_call(cname, out, q, k_new, v_new, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, workspace, stream):
    s, hq, d = q.shape
    nb, bs, hkv, dk = key_cache.shape
    if out.shape != q.shape or dk != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if k_new.shape != (s, hkv, d) or v_new.shape != (s, hkv, d):
        raise ValueError("k_new / v_new must be [num_seqs, num_kv_heads, head_dim]")
    for t in (out, k_new, v_new, key_cache, value_cache):
        if t.dtype != q.dtype:
            raise TypeError("q, k_new, v_new, caches and out must share one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    mb = block_tables.shape[1]
    if workspace is None:
        workspace = _temp_workspace(lambda dv: decode_workspace(s, hq, d, max_context_len, dv), q.device, stream)
    ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(cname, getattr(lib(), cname)(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        float(scale), bs, hq, hkv, d, s, mb, nb, int(max_context_len), _dt(q), ws_ptr, ws_bytes,
        _stream(stream)))
    return out


def pkv_attention_decode_append(out, q, k_new, v_new, key_cache, value_cache, block_tables, context_lens,
                                scale, max_context_len, workspace=None, stream=None):
    """Decode step with each sequence's new token (position ctx - 1) appended to the cache
    in the same launch: equals pkv_write of k_new / v_new at that slot, then decode (bf16)."""
    return _append_call("pkv_attention_decode_append", out, q, k_new, v_new, key_cache, value_cache,
                        block_tables, context_lens, scale, max_context_len, workspace, stream)


def pkv_attention_decode_partitions_append(out, q, k_new, v_new, key_cache, value_cache, block_tables,
                                           context_lens, scale, max_context_len, workspace=None,
                                           stream=None):
    """Partition launch of the append form (after the plan, before the merge);
    ``workspace`` is required (the one the plan launch filled)."""
    _need_workspace(workspace, "pkv_attention_decode_partitions_append")
    return _append_call("pkv_attention_decode_partitions_append", out, q, k_new, v_new, key_cache,
                        value_cache, block_tables, context_lens, scale, max_context_len, workspace, stream)


class DecodeGraph:
    """One decode step as a HIP graph (``pkv_decode_graph_create`` / ``_launch`` /
    ``_destroy``).

    With ``slot_mapping`` the step is ``pkv_write(k_new, v_new, slot_mapping)`` +
    ``pkv_attention_decode``; without it, the bf16 append form (``k_new``/``v_new``
    are [S, Hkv, D], one new row per sequence).  Every tensor's address is fixed
    into the graph, so this object keeps them alive: update their contents in
    place between launches.  ``max_context_len`` bounds every later context.
    """

    def __init__(self, out, q, k_new, v_new, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, slot_mapping=None, workspace=None):
        import ctypes
        s, hq, d = q.shape
        nb, bs, hkv, dk = key_cache.shape
        if out.shape != q.shape or dk != d or value_cache.shape != key_cache.shape:
            raise ValueError("shape mismatch")
        for t in (out, k_new, v_new, key_cache, value_cache):
            if t.dtype != q.dtype:
                raise TypeError("q, k_new, v_new, caches and out must share one dtype")
        if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
            raise ValueError("block_tables must be [S, MB] and context_lens [S]")
        if slot_mapping is None:
            if k_new.shape != (s, hkv, d) or v_new.shape != (s, hkv, d):
                raise ValueError("k_new / v_new must be [num_seqs, num_kv_heads, head_dim]")
            slots_ptr, t = None, 0
        else:
            t = k_new.shape[0]
            if k_new.shape != v_new.shape or k_new.shape[1:] != (hkv, d) or slot_mapping.shape != (t,):
                raise ValueError("k_new / v_new must be [T, Hkv, D] and slot_mapping [T]")
            slots_ptr = _dev(slot_mapping, "slot_mapping", torch.int32)
        if workspace is None:
            workspace = decode_workspace(s, hq, d, max_context_len, q.device)
        ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._keep = (out, q, k_new, v_new, key_cache, value_cache, block_tables, context_lens, slot_mapping,
                      workspace)
        h = ctypes.c_void_p(0)
        check("pkv_decode_graph_create", lib().pkv_decode_graph_create(
            ctypes.addressof(h), _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
            slots_ptr, t, _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
            float(scale), bs, hq, hkv, d, s, block_tables.shape[1], nb, int(max_context_len), _dt(q), ws_ptr,
            ws_bytes))
        self._h = h.value

    def launch(self, stream=None):
        if not self._h:
            raise RuntimeError("graph destroyed")
        check("pkv_decode_graph_launch", lib().pkv_decode_graph_launch(self._h, _stream(stream)))

    def close(self):
        if getattr(self, "_h", None):
            lib().pkv_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pkv_varlen_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                               max_query_len, max_context_len):
    return int(lib().pkv_varlen_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads,
                                                head_dim, max_query_len, max_context_len))


def varlen_workspace(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len,
                     max_context_len, device="cuda"):
    """A device buffer of the size ``pkv_attention_varlen`` needs (None if 0 bytes)."""
    n = pkv_varlen_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                   max_query_len, max_context_len)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def pkv_attention_varlen(out, q, key_cache, value_cache, block_tables, context_lens,
                         query_start_loc, scale, max_query_len, max_context_len, workspace=None,
                         stream=None):
    """Causal attention for variable query lengths (decode rows and prefill chunks), bf16.

    ``q``/``out`` [T, Hq, D]; ``query_start_loc`` int32 [S+1] on the device.
    """
    t, hq, d = q.shape
    nb, bs, hkv, dk = key_cache.shape
    if out.shape != q.shape or dk != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if out.dtype != q.dtype or key_cache.dtype != q.dtype or value_cache.dtype != q.dtype:
        raise TypeError("q, caches and out must share one dtype")
    s = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != s or query_start_loc.shape != (s + 1,):
        raise ValueError("block_tables must be [S, MB] and query_start_loc [S+1]")
    mb = block_tables.shape[1]
    if workspace is None:
        workspace = _temp_workspace(
            lambda dv: varlen_workspace(s, t, hq, hkv, d, max_query_len, max_context_len, dv), q.device, stream)
    ws_ptr = 0 if workspace is None else _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("pkv_attention_varlen", lib().pkv_attention_varlen(
        _dev(out, "out"), _dev(q, "q"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start_loc, "query_start_loc", torch.int32), t, int(max_query_len), float(scale), bs,
        hq, hkv, d, s, mb, nb, int(max_context_len), _dt(q), ws_ptr, ws_bytes, _stream(stream)))
    return out


def _varlen_args(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc, scale,
                 max_query_len, max_context_len, workspace):
    t, hq, d = q.shape
    nb, bs, hkv, dk = key_cache.shape
    if out.shape != q.shape or dk != d or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if out.dtype != q.dtype or key_cache.dtype != q.dtype or value_cache.dtype != q.dtype:
        raise TypeError("q, caches and out must share one dtype")
    s = context_lens.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != s or query_start_loc.shape != (s + 1,):
        raise ValueError("block_tables must be [S, MB] and query_start_loc [S+1]")
    return (_dev(out, "out"), _dev(q, "q"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
            _dev(query_start_loc, "query_start_loc", torch.int32), t, int(max_query_len), float(scale), bs, hq,
            hkv, d, s, block_tables.shape[1], nb, int(max_context_len), _dt(q), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size())


def pkv_attention_varlen_plan_upload(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                                     scale, max_query_len, max_context_len, host_context_lens, upload_src,
                                     upload_dst, workspace=None, host_block_tables=None, stream=None):
    """Plan of ``pkv_attention_varlen`` from pinned host lengths, fused with the
    upload of the pinned ``upload_src`` into ``upload_dst`` (and, with
    ``host_block_tables``, of each table row's used entries into
    ``block_tables``); ``workspace`` is required (``_partitions`` reads the plan)."""
    _need_workspace(workspace, "pkv_attention_varlen_plan_upload")
    for name, t in (("host_context_lens", host_context_lens), ("upload_src", upload_src)):
        if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_pinned() or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous pinned host tensor")
    if host_block_tables is not None:
        if host_block_tables.is_cuda or not host_block_tables.is_pinned() or not host_block_tables.is_contiguous():
            raise TypeError("host_block_tables must be a contiguous pinned host tensor")
        if host_block_tables.dtype != torch.int32 or tuple(host_block_tables.shape) != tuple(block_tables.shape):
            raise ValueError("host_block_tables must be int32 of block_tables' shape")
    if host_context_lens.dtype != torch.int32 or host_context_lens.shape != (context_lens.shape[0],):
        raise ValueError("host_context_lens must be int32 [num_seqs]")
    nbytes = upload_src.numel() * upload_src.element_size()
    if upload_dst.numel() * upload_dst.element_size() != nbytes:
        raise ValueError("upload_src and upload_dst must have the same byte size")
    a = _varlen_args(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc, scale,
                     max_query_len, max_context_len, workspace)
    check("pkv_attention_varlen_plan_upload", lib().pkv_attention_varlen_plan_upload(
        *a, host_context_lens.data_ptr(), upload_src.data_ptr(), _dev(upload_dst, "upload_dst"), nbytes,
        None if host_block_tables is None else host_block_tables.data_ptr(), _stream(stream)))
    return out


def pkv_attention_varlen_partitions(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                                    scale, max_query_len, max_context_len, workspace=None, stream=None):
    """The launches of ``pkv_attention_varlen`` after its plan (decode partitions,
    prefill tiles, merge); ``workspace`` is required (the planned one)."""
    _need_workspace(workspace, "pkv_attention_varlen_partitions")
    a = _varlen_args(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc, scale,
                     max_query_len, max_context_len, workspace)
    check("pkv_attention_varlen_partitions", lib().pkv_attention_varlen_partitions(*a, _stream(stream)))
    return out


def _varlen_launch(cname, out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc, scale,
                   max_query_len, max_context_len, workspace, stream):
    _need_workspace(workspace, cname)
    a = _varlen_args(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc, scale,
                     max_query_len, max_context_len, workspace)
    check(cname, getattr(lib(), cname)(*a, _stream(stream)))
    return out


def pkv_attention_varlen_plan(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                              scale, max_query_len, max_context_len, workspace=None, stream=None):
    """First launch of ``pkv_attention_varlen`` alone (work lists, ticket counters reset);
    ``workspace`` is required: the later launches read the plan from it."""
    return _varlen_launch("pkv_attention_varlen_plan", out, q, key_cache, value_cache, block_tables, context_lens,
                          query_start_loc, scale, max_query_len, max_context_len, workspace, stream)


def pkv_attention_varlen_decode_partitions(out, q, key_cache, value_cache, block_tables, context_lens,
                                           query_start_loc, scale, max_query_len, max_context_len, workspace=None,
                                           stream=None):
    """The one-row sequences' partitions of a planned varlen step."""
    return _varlen_launch("pkv_attention_varlen_decode_partitions", out, q, key_cache, value_cache, block_tables,
                          context_lens, query_start_loc, scale, max_query_len, max_context_len, workspace, stream)


def pkv_attention_varlen_prefill_tiles(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                                       scale, max_query_len, max_context_len, workspace=None, stream=None):
    """The chunk rows' matrix-core tiles of a planned varlen step."""
    return _varlen_launch("pkv_attention_varlen_prefill_tiles", out, q, key_cache, value_cache, block_tables,
                          context_lens, query_start_loc, scale, max_query_len, max_context_len, workspace, stream)


def pkv_attention_varlen_merge(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                               scale, max_query_len, max_context_len, workspace=None, stream=None):
    """The log-sum-exp merge of a planned varlen step (after both kinds of tiles)."""
    return _varlen_launch("pkv_attention_varlen_merge", out, q, key_cache, value_cache, block_tables, context_lens,
                          query_start_loc, scale, max_query_len, max_context_len, workspace, stream)


def pkv_lse_merge(out, part_m, part_l, part_o, num_parts, stream=None):
    """Merge partial softmax results (base-2 maxima); ``out`` [rows, D]."""
    rows, maxp, d = part_o.shape
    if part_m.shape != (rows, maxp) or part_l.shape != (rows, maxp) or num_parts.shape != (rows,):
        raise ValueError("shape mismatch")
    if out.shape != (rows, d):
        raise ValueError("out must be [rows, head_dim]")
    check("pkv_lse_merge", lib().pkv_lse_merge(
        _dev(out, "out"), _dev(part_m, "part_m", torch.float32), _dev(part_l, "part_l", torch.float32),
        _dev(part_o, "part_o", torch.float32), _dev(num_parts, "num_parts", torch.int32), rows, maxp, d,
        _dt(out), _stream(stream)))
    return out


def pkv_copy_blocks(key_cache, value_cache, pairs, stream=None):
    """Copy-on-write block copies; ``pairs`` is a device int32 [n, 2] of (src, dst)."""
    nb, bs, hkv, d = key_cache.shape
    n = pairs.shape[0] if pairs.numel() else 0
    if n and tuple(pairs.shape) != (n, 2):
        raise ValueError("pairs must be [n, 2]")
    if n == 0:
        return
    check("pkv_copy_blocks", lib().pkv_copy_blocks(
        _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"), _dev(pairs, "pairs", torch.int32),
        n, nb, bs, hkv, d, _dt(key_cache), _stream(stream)))


def _pool_ptr(t, name):
    """Address of a pool: a device tensor, or a page-locked host tensor (the
    library maps it for the device and rejects anything else)."""
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or t.is_pinned()):
        raise TypeError(f"{name} must be a device tensor or a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def pkv_swap_blocks(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache, pairs, stream=None):
    """Block copies between two pools (device and pinned host, either way round);
    ``pairs`` is a device int32 [n, 2] of (src block, dst block)."""
    snb, bs, hkv, d = src_key_cache.shape
    dnb = dst_key_cache.shape[0]
    for name, t, nb in (("dst_key_cache", dst_key_cache, dnb), ("dst_value_cache", dst_value_cache, dnb),
                        ("src_value_cache", src_value_cache, snb)):
        if tuple(t.shape) != (nb, bs, hkv, d):
            raise ValueError(f"{name} must be [{nb}, {bs}, {hkv}, {d}]")
        if t.dtype != src_key_cache.dtype:
            raise TypeError("all four pools must share one dtype")
    n = pairs.shape[0] if pairs.numel() else 0
    if n and tuple(pairs.shape) != (n, 2):
        raise ValueError("pairs must be [n, 2]")
    if n == 0:
        return
    check("pkv_swap_blocks", lib().pkv_swap_blocks(
        _pool_ptr(dst_key_cache, "dst_key_cache"), _pool_ptr(dst_value_cache, "dst_value_cache"),
        _pool_ptr(src_key_cache, "src_key_cache"), _pool_ptr(src_value_cache, "src_value_cache"),
        _dev(pairs, "pairs", torch.int32), n, snb, dnb, bs, hkv, d, _dt(src_key_cache), _stream(stream)))


def pkv_check_tables(block_tables, context_lens, num_blocks):
    """Host-side table validation (numpy int32 arrays).  Raises PagedKVError on a bad entry."""
    import numpy as np
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    c = np.ascontiguousarray(context_lens, dtype=np.int32)
    check("pkv_check_tables", lib().pkv_check_tables(
        t.ctypes.data, c.ctypes.data, t.shape[0], t.shape[1], int(num_blocks)))


def pkv_check_slots(slot_mapping, num_blocks):
    """Host-side slot validation: in range and no duplicates (numpy int32)."""
    import numpy as np
    s = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    check("pkv_check_slots", lib().pkv_check_slots(s.ctypes.data, s.shape[0], int(num_blocks),
                                                   BLOCK_SIZE))
