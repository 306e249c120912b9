"""Python binding of libpkv with the same call names as the C ABI.

Argument marshalling only: tensors are checked for device, dtype and contiguity, turned into
pointers, and handed to the library together with the current HIP stream. Every step of the
computation runs in the library's kernels (or, for the allocator, its C++ code).
"""

import ctypes
import math

import numpy as np
import torch

from ._lib import BF16, F16, F32, check, lib

BLOCK_SIZE = 16
_TORCH_TO_PKV = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}


def pkv_dtype(t):
    try:
        return _TORCH_TO_PKV[t.dtype if isinstance(t, torch.Tensor) else t]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype if isinstance(t, torch.Tensor) else t}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# The current stream's raw handle, without building a torch Stream object per call (a few
# microseconds each, which a host-bound decode loop pays several times per step).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    if _raw_stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return ctypes.c_void_p(_raw_stream(idx))


def _need(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _as_c(a, dtype):
    """A C-contiguous NumPy array of ``dtype`` (no copy when ``a`` already is one)."""
    if isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous:
        return a
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def cache_shapes(num_blocks, num_kv_heads, head_dim, dtype):
    """Shapes of the K and V caches in the library's layout (see include/pkv.h)."""
    x = 16 // _ELEM_BYTES[pkv_dtype(dtype)]
    return ((num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x),
            (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE))


def alloc_caches(num_blocks, num_kv_heads, head_dim, dtype, device="cuda", fill=None):
    ks, vs = cache_shapes(num_blocks, num_kv_heads, head_dim, dtype)
    k = torch.empty(ks, dtype=dtype, device=device)
    v = torch.empty(vs, dtype=dtype, device=device)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


def cache_bytes(num_blocks, num_kv_heads, head_dim, dtype):
    return int(lib.pkv_cache_bytes(num_blocks, num_kv_heads, head_dim, BLOCK_SIZE,
                                   pkv_dtype(dtype)))


def _num_blocks(k_cache, num_kv_heads, head_dim):
    per = num_kv_heads * head_dim * BLOCK_SIZE
    if k_cache.numel() % per:
        raise ValueError("k_cache size is not a whole number of blocks")
    return k_cache.numel() // per


def pkv_write(k, v, k_cache, v_cache, slot_mapping):
    """Scatter k, v [T, Hkv, hd] into the caches at slot_mapping [T] (int32)."""
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, dtype=k.dtype, device=k.device)
    _need(slot_mapping, "slot_mapping", dtype=torch.int32, device=k.device)
    T, hkv, hd = k.shape
    if v.shape != k.shape or slot_mapping.numel() != T:
        raise ValueError("k, v and slot_mapping shapes disagree")
    nb = _num_blocks(k_cache, hkv, hd)
    check(lib.pkv_write(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T,
                        hkv, hd, BLOCK_SIZE, nb, pkv_dtype(k), _stream(k.device)), "pkv_write")


def pkv_copy_blocks(k_cache, v_cache, src, dst, *, num_kv_heads, head_dim):
    """Copy block src[i] to block dst[i] in both caches (every kv head), for each pair i.

    src, dst: int32 device tensors of one length (the copy-on-write pairs that
    BlockAllocator.append reports, uploaded)."""
    _need(k_cache, "k_cache", device=k_cache.device)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=k_cache.device)
    _need(src, "src", dtype=torch.int32, device=k_cache.device)
    _need(dst, "dst", dtype=torch.int32, device=k_cache.device)
    if src.numel() != dst.numel():
        raise ValueError("src and dst lengths differ")
    nb = _num_blocks(k_cache, num_kv_heads, head_dim)
    if v_cache.numel() != k_cache.numel():
        raise ValueError("k_cache and v_cache sizes differ")
    check(lib.pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src), _ptr(dst), src.numel(),
                              num_kv_heads, head_dim, BLOCK_SIZE, nb, pkv_dtype(k_cache),
                              _stream(k_cache.device)), "pkv_copy_blocks")


def pkv_probe_read(base, tile_ids, *, num_workers, sink=None):
    """Read-bandwidth probe (see include/pkv.h): wave w reads the 4096-byte tiles
    tile_ids[w*per ..] of base with the stream pass's loads and writes the XOR of what each lane
    read to sink[w*64 + lane]. Returns sink (uint32 values in an int32 tensor [W*64])."""
    _need(base, "base", device=base.device)
    _need(tile_ids, "tile_ids", dtype=torch.int32, device=base.device)
    if sink is None:
        sink = torch.empty(num_workers * 64, dtype=torch.int32, device=base.device)
    _need(sink, "sink", dtype=torch.int32, device=base.device)
    if sink.numel() < num_workers * 64:
        raise ValueError("sink must hold num_workers * 64 words")
    check(lib.pkv_probe_read(_ptr(base), base.numel() * base.element_size(), _ptr(tile_ids),
                             tile_ids.numel(), num_workers, _ptr(sink), _stream(base.device)),
          "pkv_probe_read")
    return sink


def pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_context_len,
                               dtype):
    return int(lib.pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                              max_context_len, pkv_dtype(dtype)))


def pkv_decode_kernel(num_q_heads, num_kv_heads, dtype):
    """1 if the stream pass runs the vector kernel for this shape, 2 the matrix-core one."""
    return int(lib.pkv_decode_kernel(num_q_heads, num_kv_heads, pkv_dtype(dtype)))


def pkv_decode_num_workers(num_q_heads, num_kv_heads, head_dim, dtype):
    """Waves of the stream pass that fill the current device once (a multiple of 4)."""
    return int(lib.pkv_decode_num_workers(num_q_heads, num_kv_heads, head_dim, pkv_dtype(dtype)))


def pkv_decode_stream_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, dtype,
                                      num_workers):
    return int(lib.pkv_decode_stream_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                     pkv_dtype(dtype), num_workers))


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads, out):
    _need(q, "q")
    dev = q.device
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, dtype=q.dtype, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, device=dev)
    B, hq, hd = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    nb = _num_blocks(k_cache, num_kv_heads, hd)
    return out, B, hq, hd, nb, block_tables.shape[1]


def pkv_decode_attn(q, k_cache, v_cache, block_tables, context_lens, *, num_kv_heads, scale,
                    max_context_len, out=None, workspace=None):
    """out [B, Hq, hd] = paged decode attention. Allocates the workspace if none is given."""
    out, B, hq, hd, nb, mb = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                          num_kv_heads, out)
    need = pkv_decode_workspace_bytes(B, hq, num_kv_heads, hd, max_context_len, q.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.pkv_decode_attn(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_tables), _ptr(context_lens), B, hq, num_kv_heads, hd,
                              BLOCK_SIZE, nb, mb, max_context_len, float(scale), pkv_dtype(q),
                              _ptr(workspace), ws_bytes, _stream(q.device)), "pkv_decode_attn")
    return out


def _new_args(q, k_new, v_new, num_kv_heads):
    B, _, hd = q.shape
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, dtype=q.dtype, device=q.device)
        if tuple(t.shape) != (B, num_kv_heads, hd):
            raise ValueError(f"{n} must be [B, num_kv_heads, head_dim]")


def pkv_decode_append_attn(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, *,
                           num_kv_heads, scale, max_context_len, out=None, workspace=None):
    """Write each sequence's newest token (k_new, v_new [B, Hkv, hd]) into its slot, then
    decode attention: pkv_write followed by pkv_decode_attn in one pass."""
    out, B, hq, hd, nb, mb = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                          num_kv_heads, out)
    _new_args(q, k_new, v_new, num_kv_heads)
    need = pkv_decode_workspace_bytes(B, hq, num_kv_heads, hd, max_context_len, q.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.pkv_decode_append_attn(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), B, hq,
                                     num_kv_heads, hd, BLOCK_SIZE, nb, mb, max_context_len,
                                     float(scale), pkv_dtype(q), _ptr(workspace), ws_bytes,
                                     _stream(q.device)), "pkv_decode_append_attn")
    return out


def pkv_decode_append_attn_noalloc(q, k_new, v_new, k_cache, v_cache, block_tables,
                                   context_lens, *, num_kv_heads, scale, max_context_len, out):
    """pkv_decode_append_attn on the library's own per-device scratch: no workspace, and
    nothing is allocated here either (out is required). Calls that overlap on one GPU race."""
    _need(out, "out", dtype=q.dtype, device=q.device)
    out, B, hq, hd, nb, mb = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                          num_kv_heads, out)
    _new_args(q, k_new, v_new, num_kv_heads)
    check(lib.pkv_decode_append_attn_noalloc(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                             _ptr(context_lens), B, hq, num_kv_heads, hd,
                                             BLOCK_SIZE, nb, mb, max_context_len, float(scale),
                                             pkv_dtype(q), _stream(q.device)),
          "pkv_decode_append_attn_noalloc")
    return out


def pkv_decode_append_stream(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, *,
                             num_kv_heads, scale, max_context_len, num_workers, workspace,
                             out=None):
    """Pass 1 of pkv_decode_append_attn (see include/pkv.h). Returns out."""
    out, B, hq, hd, nb, mb = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                          num_kv_heads, out)
    _new_args(q, k_new, v_new, num_kv_heads)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.pkv_decode_append_stream(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                       _ptr(context_lens), B, hq, num_kv_heads, hd, BLOCK_SIZE,
                                       nb, mb, max_context_len, float(scale), pkv_dtype(q),
                                       num_workers, _ptr(workspace), ws_bytes,
                                       _stream(q.device)), "pkv_decode_append_stream")
    return out


def pkv_decode_stream(q, k_cache, v_cache, block_tables, context_lens, *, num_kv_heads, scale,
                      max_context_len, num_workers, workspace, out=None):
    """Pass 1 of decode attention (see include/pkv.h). Returns out."""
    out, B, hq, hd, nb, mb = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                          num_kv_heads, out)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.pkv_decode_stream(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                _ptr(block_tables), _ptr(context_lens), B, hq, num_kv_heads, hd,
                                BLOCK_SIZE, nb, mb, max_context_len, float(scale), pkv_dtype(q),
                                num_workers, _ptr(workspace), ws_bytes, _stream(q.device)),
          "pkv_decode_stream")
    return out


def pkv_decode_merge(out, workspace, *, num_kv_heads, num_workers):
    """Pass 2 of decode attention: log-sum-exp merge of the cut segments' pieces into out."""
    _need(out, "out")
    _need(workspace, "workspace", device=out.device)
    B, hq, hd = out.shape
    check(lib.pkv_decode_merge(_ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), B, hq, num_kv_heads,
                               hd, pkv_dtype(out), num_workers, _stream(out.device)),
          "pkv_decode_merge")
    return out


def pkv_decode_append_merge(out, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                            workspace, *, num_kv_heads, max_context_len, num_workers):
    """Pass 2 of pkv_decode_append_attn: the merge, plus the stores of the newest tokens' K/V
    into their slots."""
    _need(out, "out")
    dev = out.device
    B, hq, hd = out.shape
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, dtype=out.dtype, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, device=dev)
    _need(workspace, "workspace", device=dev)
    nb = _num_blocks(k_cache, num_kv_heads, hd)
    check(lib.pkv_decode_append_merge(_ptr(out), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                      _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), nb,
                                      block_tables.shape[1], max_context_len, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), B, hq,
                                      num_kv_heads, hd, pkv_dtype(out), num_workers,
                                      _stream(dev)), "pkv_decode_append_merge")
    return out


def pkv_decode_plan(block_tables, context_lens, *, num_q_heads, num_kv_heads, num_blocks,
                    max_context_len, dtype, out=None, max_group=0):
    """Shared-prefix plan of a batch from HOST copies of its tables [B, max_blocks] and lengths
    [B] (int32; table entries may carry BLOCK_SHARED). Returns an int32 NumPy array (a view of
    ``out`` when that is large enough). max_group: largest Hq/Hkv that gets runs (0: the
    library's default)."""
    t = _as_c(block_tables, np.int32)
    lens = _as_c(context_lens, np.int32)
    if t.ndim != 2 or lens.shape != (t.shape[0],):
        raise ValueError("block_tables must be [B, max_blocks] and context_lens [B]")
    B, mb = t.shape
    n = ctypes.c_size_t(0)
    for _ in range(2):
        cap = 0 if out is None else int(out.size)
        st = lib.pkv_decode_plan(t.ctypes.data, lens.ctypes.data, B, mb, int(max_context_len),
                                 num_q_heads, num_kv_heads, int(num_blocks), pkv_dtype(dtype),
                                 int(max_group), out.ctypes.data if out is not None else None,
                                 cap, ctypes.byref(n))
        if st == 0:
            return out[:n.value]
        if st != 6:  # anything but a too-small buffer
            check(st, "pkv_decode_plan")
        out = np.empty(n.value, np.int32)
    raise RuntimeError("pkv_decode_plan: plan size changed between calls")


def pkv_decode_planned_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, dtype,
                                       num_workers, plan):
    p = _as_c(plan, np.int32)
    return int(lib.pkv_decode_planned_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                      pkv_dtype(dtype), num_workers,
                                                      p.ctypes.data, p.size))


def pkv_decode_planned(q, k_cache, v_cache, block_tables, context_lens, plan, plan_dev, *,
                       num_kv_heads, scale, max_context_len, num_workers, workspace,
                       k_new=None, v_new=None, out=None, passes=0, events=None,
                       shared_launch="auto"):
    """Decode step with a shared-prefix plan (see include/pkv.h). plan: the host plan (NumPy
    int32), plan_dev: the same ints on the device (int32 tensor). With k_new / v_new it is the
    fused newest-token step. passes: 0 all, 1 shared pass, 2 stream pass, 3 merge, 4 shared
    and stream pass as the library chooses, 5 those two in one launch. events: three
    torch.cuda.Events to record after the shared pass, the stream pass and the merge; the
    passes then run as separate calls, the shared and stream passes as shared_launch says:
    "auto" (pass 4) or "one" (pass 5), the first event recorded before them, or "two" (passes
    1 and 2)."""
    if shared_launch not in ("auto", "one", "two"):
        raise ValueError("shared_launch is 'auto', 'one' or 'two'")
    out, B, hq, hd, nb, mb = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                          num_kv_heads, out)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        _new_args(q, k_new, v_new, num_kv_heads)
    p = _as_c(plan, np.int32)
    _need(plan_dev, "plan_dev", dtype=torch.int32, device=q.device)
    if plan_dev.numel() < p.size:
        raise ValueError("plan_dev is shorter than the plan")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), _ptr(context_lens), B, hq, num_kv_heads, hd, BLOCK_SIZE, nb, mb,
            max_context_len, float(scale), pkv_dtype(q), p.ctypes.data, _ptr(plan_dev), p.size,
            num_workers, _ptr(workspace), ws_bytes, _stream(q.device))
    if events is None:
        check(lib.pkv_decode_planned(int(passes), *args), "pkv_decode_planned")
    elif shared_launch == "two":
        for ps, ev in zip((1, 2, 3), events):
            check(lib.pkv_decode_planned(ps, *args), "pkv_decode_planned")
            ev.record()
    else:
        events[0].record()
        for ps, ev in zip((4 if shared_launch == "auto" else 5, 3), events[1:]):
            check(lib.pkv_decode_planned(ps, *args), "pkv_decode_planned")
            ev.record()
    return out


def pkv_decode_planned_launches(plan, *, batch, num_q_heads, num_kv_heads, max_blocks, dtype,
                                num_workers):
    """Launches (1 or 2) of the shared and stream passes that pkv_decode_planned's automatic
    choice gives this plan (host only; 0 for a plan that fails validation)."""
    p = _as_c(plan, np.int32)
    return int(lib.pkv_decode_planned_launches(p.ctypes.data, p.size, batch, num_q_heads,
                                               num_kv_heads, max_blocks, pkv_dtype(dtype),
                                               num_workers))


PREFILL_MAX_BLOCKS = 512  # blocks of one prefill unit (longer rows are split and merged)


def pkv_prefill_plan(query_start, context_lens, *, num_q_heads, num_kv_heads, max_blocks,
                     max_context_len, dtype, out=None):
    """Prefill plan from HOST copies of query_start [S+1] and context_lens [S] (int32): the new
    tokens of sequence s are the last query_start[s+1] - query_start[s] of its context_lens[s].
    Returns an int32 NumPy array (a view of ``out`` when that is large enough)."""
    qs = _as_c(query_start, np.int32)
    lens = _as_c(context_lens, np.int32)
    if qs.ndim != 1 or lens.shape != (qs.size - 1,):
        raise ValueError("query_start must be [S+1] and context_lens [S]")
    S = lens.size
    n = ctypes.c_size_t(0)
    for _ in range(2):
        cap = 0 if out is None else int(out.size)
        st = lib.pkv_prefill_plan(qs.ctypes.data, lens.ctypes.data, S, int(max_blocks),
                                  int(max_context_len), num_q_heads, num_kv_heads,
                                  pkv_dtype(dtype), out.ctypes.data if out is not None else None,
                                  cap, ctypes.byref(n))
        if st == 0:
            return out[:n.value]
        if st != 6:  # anything but a too-small buffer
            check(st, "pkv_prefill_plan")
        out = np.empty(n.value, np.int32)
    raise RuntimeError("pkv_prefill_plan: plan size changed between calls")


def pkv_prefill_workspace_bytes(num_q_heads, num_kv_heads, head_dim, plan):
    p = _as_c(plan, np.int32)
    n = int(lib.pkv_prefill_workspace_bytes(num_q_heads, num_kv_heads, head_dim, p.ctypes.data,
                                            p.size))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("not a prefill plan for these heads")
    return n


def pkv_prefill_attn(q, k_cache, v_cache, block_tables, plan, plan_dev, *, num_kv_heads, scale,
                     max_context_len, workspace=None, out=None, passes=0):
    """out [T, Hq, hd] = causal attention of the T new prompt tokens over their sequences'
    paged caches (see include/pkv.h). plan: the host plan from pkv_prefill_plan (NumPy int32),
    plan_dev: the same ints on the device. Allocates the workspace if none is given.
    passes: 0 both kernels, 1 the attention pass, 2 the merge of split rows."""
    _need(q, "q")
    dev = q.device
    for t, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, name, dtype=q.dtype, device=dev)
    _need(block_tables, "block_tables", dtype=torch.int32, device=dev)
    _need(plan_dev, "plan_dev", dtype=torch.int32, device=dev)
    if q.dim() != 3 or block_tables.dim() != 2:
        raise ValueError("q must be [T, Hq, hd] and block_tables [S, max_blocks]")
    T, hq, hd = q.shape
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    p = _as_c(plan, np.int32)
    if plan_dev.numel() < p.size:
        raise ValueError("plan_dev is shorter than the plan")
    S, mb = block_tables.shape
    nb = _num_blocks(k_cache, num_kv_heads, hd)
    need = pkv_prefill_workspace_bytes(hq, num_kv_heads, hd, p)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib.pkv_prefill_attn(int(passes), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), S, T, hq, num_kv_heads, hd, BLOCK_SIZE, nb, mb,
                               int(max_context_len), float(scale), pkv_dtype(q), p.ctypes.data,
                               _ptr(plan_dev), p.size, _ptr(workspace), ws_bytes,
                               _stream(dev)), "pkv_prefill_attn")
    return out


def split_workspace(workspace, batch, num_q_heads, num_kv_heads, head_dim, num_workers, kernel):
    """Views (seg int32 [B+1], ml float32 [W, 2, GS, 2], o float32 [W, 2, GS, hd]) of a stream
    workspace, for the kernel the stream pass used (1 vector, 2 matrix core)."""
    gs = num_q_heads // num_kv_heads if kernel == 2 else 1
    cells = num_workers * 2 * gs
    a0 = ((batch + 1) * 4 + 255) // 256 * 256
    a1 = (cells * 2 * 4 + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    seg = f[:(batch + 1) * 4].view(torch.int32)
    ml = f[a0:a0 + cells * 2 * 4].view(torch.float32).view(num_workers, 2, gs, 2)
    o = f[a0 + a1:a0 + a1 + cells * head_dim * 4].view(torch.float32).view(num_workers, 2, gs,
                                                                           head_dim)
    return seg, ml, o


def pkv_set_attn_kernel(which):
    """0 automatic, 1 vector kernel, 2 matrix-core kernel. Returns the previous choice."""
    return int(lib.pkv_set_attn_kernel(int(which)))


# -------------------------------------------------------------------------------------------
class BlockAllocator:
    """Host block allocator (C++), see include/pkv.h. Not thread-safe."""

    def __init__(self, num_blocks, block_size=BLOCK_SIZE, free_order=None):
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            self._order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            order = self._order.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        check(lib.pkv_alloc_create(num_blocks, block_size, order, ctypes.byref(h)),
              "pkv_alloc_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._cow = np.empty((2, 1), np.int32)  # copy-on-write pairs, reused across calls
        self._ncow = ctypes.c_int32(0)

    def close(self):
        if self._h:
            lib.pkv_alloc_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, seq):
        check(lib.pkv_alloc_add_seq(self._h, int(seq)), "pkv_alloc_add_seq")

    def append(self, seqs, ntok, want_slots=True, slots_out=None, token_ids=None):
        """Returns (slots int32 [sum ntok], cow pairs int32 [n_cow, 2]). With token_ids (sum
        ntok ids, argument order) it is pkv_alloc_append_tokens (prefix-cache indexing)."""
        seqs = _as_c(seqs, np.int64)
        ntok = _as_c(ntok, np.int32)
        n = len(seqs)
        if len(ntok) != n:
            raise ValueError("seqs and ntok lengths differ")
        slots = None
        if want_slots:
            slots = slots_out if slots_out is not None else np.empty(int(ntok.sum()), np.int32)
        if self._cow.shape[1] < max(n, 1):
            self._cow = np.empty((2, max(n, 1)), np.int32)
        cow = self._cow
        sp = slots.ctypes.data if want_slots else None
        if token_ids is None:
            check(lib.pkv_alloc_append(self._h, n, seqs.ctypes.data, ntok.ctypes.data, sp,
                                       cow[0].ctypes.data, cow[1].ctypes.data,
                                       ctypes.byref(self._ncow)), "pkv_alloc_append")
        else:
            ids = _as_c(token_ids, np.int32)
            if len(ids) != int(ntok.sum()):
                raise ValueError("token_ids must hold sum(ntok) ids")
            check(lib.pkv_alloc_append_tokens(self._h, n, seqs.ctypes.data, ntok.ctypes.data,
                                              ids.ctypes.data, sp, cow[0].ctypes.data,
                                              cow[1].ctypes.data, ctypes.byref(self._ncow)),
                  "pkv_alloc_append_tokens")
        k = self._ncow.value
        pairs = cow[:, :k].T.copy() if k else np.zeros((0, 2), np.int32)
        return slots, pairs

    def append_tokens(self, seqs, ntok, token_ids, want_slots=True, slots_out=None):
        return self.append(seqs, ntok, want_slots, slots_out, token_ids=token_ids)

    def add_seq_tokens(self, seq, token_ids, slots_out=None):
        """New sequence holding a prompt (prefix caching). Returns (slots of every prompt
        token, tokens found in the cache)."""
        ids = _as_c(token_ids, np.int32)
        slots = slots_out if slots_out is not None else np.empty(len(ids), np.int32)
        cached = ctypes.c_int32(0)
        check(lib.pkv_alloc_add_seq_tokens(self._h, int(seq), len(ids), ids.ctypes.data,
                                           slots.ctypes.data, ctypes.byref(cached)),
              "pkv_alloc_add_seq_tokens")
        return slots, cached.value

    def cached_blocks(self):
        return int(lib.pkv_alloc_cached_blocks(self._h))

    def fork(self, parent, child):
        check(lib.pkv_alloc_fork(self._h, int(parent), int(child)), "pkv_alloc_fork")

    def free(self, seq):
        check(lib.pkv_alloc_free(self._h, int(seq)), "pkv_alloc_free")

    def fork_many(self, parents, children):
        """fork(parents[k], children[k]) for every k, in order, in one call (all-or-nothing)."""
        p = _as_c(parents, np.int64)
        c = _as_c(children, np.int64)
        if p.shape != c.shape or p.ndim != 1:
            raise ValueError("parents and children must be 1-D and of one length")
        check(lib.pkv_alloc_fork_many(self._h, len(p), p.ctypes.data, c.ctypes.data),
              "pkv_alloc_fork_many")

    def free_many(self, seqs):
        """free(seqs[k]) for every k, in order, in one call (all-or-nothing)."""
        s = _as_c(seqs, np.int64)
        check(lib.pkv_alloc_free_many(self._h, len(s), s.ctypes.data), "pkv_alloc_free_many")

    def replace_many(self, parents, old, children):
        """fork_many(parents, children) then free_many(old), in one call (all-or-nothing)."""
        p = _as_c(parents, np.int64)
        o = _as_c(old, np.int64)
        c = _as_c(children, np.int64)
        if not (p.shape == o.shape == c.shape) or p.ndim != 1:
            raise ValueError("parents, old and children must be 1-D and of one length")
        check(lib.pkv_alloc_replace_many(self._h, len(p), p.ctypes.data, o.ctypes.data,
                                         c.ctypes.data), "pkv_alloc_replace_many")

    def tables(self, seqs, max_blocks, tables_out=None, lens_out=None, mark_shared=False):
        """Block tables [n, max_blocks] (pad -1) and lengths; with mark_shared, entries of
        blocks shared by several sequences carry BLOCK_SHARED (pkv_alloc_tables_marked)."""
        seqs = _as_c(seqs, np.int64)
        n = len(seqs)
        tables = tables_out if tables_out is not None else np.empty((n, max_blocks), np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, np.int32)
        fn = lib.pkv_alloc_tables_marked if mark_shared else lib.pkv_alloc_tables
        check(fn(self._h, n, seqs.ctypes.data, max_blocks, tables.ctypes.data, lens.ctypes.data),
              "pkv_alloc_tables")
        return tables, lens

    def num_free(self):
        return int(lib.pkv_alloc_num_free(self._h))

    def refcount(self, block):
        return int(lib.pkv_alloc_refcount(self._h, int(block)))

    def seq_len(self, seq):
        return int(lib.pkv_alloc_seq_len(self._h, int(seq)))

    def usage(self):
        """dict(sequences, logical_tokens, blocks_in_use, slots_filled, utilisation)."""
        out = np.zeros(4, np.int64)
        check(lib.pkv_alloc_usage(self._h, out.ctypes.data), "pkv_alloc_usage")
        seqs, logical, blocks, filled = (int(x) for x in out)
        return dict(sequences=seqs, logical_tokens=logical, blocks_in_use=blocks,
                    slots_filled=filled,
                    utilisation=filled / (blocks * self.block_size) if blocks else 0.0)

    def free_list(self):
        n = int(lib.pkv_alloc_free_list(self._h, None, 0))
        out = np.empty(max(n, 1), np.int32)
        lib.pkv_alloc_free_list(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n)
        return out[:n].tolist()


ENGINE_PLAN = 1  # PKV_ENGINE_PLAN
ENGINE_SPLIT_SHARED = 2  # PKV_ENGINE_SPLIT_SHARED
ENGINE_ONE_LAUNCH = 4  # PKV_ENGINE_ONE_LAUNCH
_ENGINE_EVENTS = 8


def _event_handles(events, buf):
    """Raw hipEvent_t handles of up to 8 events (objects with an ``ev`` handle, raw ints, or
    None) into the ctypes array buf."""
    for k in range(_ENGINE_EVENTS):
        e = events[k] if k < len(events) else None
        buf[k] = (e.ev.value if hasattr(e, "ev") else e) if e is not None else None
    return buf


class Engine:
    """Serving step engine (C++, include/pkv.h): the request queue, the running set and the
    step's staging live in the library, and one call runs a whole continuous-batching or
    beam-search step (retire, admit, append, table and plan export and upload, launches).
    Borrows ``allocator`` (kept alive here) and the caches. Not thread-safe."""

    def __init__(self, allocator, k_cache, v_cache, *, num_q_heads, num_kv_heads, head_dim,
                 max_batch, max_context_len, plan=False, shared_launch="auto"):
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            _need(t, name)
        self.alloc = allocator
        self.k_cache, self.v_cache = k_cache, v_cache
        self.Hq, self.Hkv, self.hd = num_q_heads, num_kv_heads, head_dim
        self.dtype = k_cache.dtype
        self.device = k_cache.device
        self.nb = _num_blocks(k_cache, num_kv_heads, head_dim)
        self.max_batch, self.max_ctx = int(max_batch), int(max_context_len)
        self.max_blocks = -(-self.max_ctx // BLOCK_SIZE)
        h = ctypes.c_void_p()
        check(lib.pkv_engine_create(allocator._h, _ptr(k_cache), _ptr(v_cache), self.nb,
                                    num_q_heads, num_kv_heads, head_dim, pkv_dtype(k_cache),
                                    self.max_batch, self.max_ctx,
                                    (ENGINE_PLAN if plan else 0)
                                    | ({"auto": 0, "one": ENGINE_ONE_LAUNCH,
                                        "two": ENGINE_SPLIT_SHARED}[shared_launch]
                                       if plan else 0),
                                    ctypes.byref(h)), "pkv_engine_create")
        self._h = h
        self.info = np.zeros(8, np.int64)
        self._info_p = ctypes.c_void_p(self.info.ctypes.data)
        self._ev = (ctypes.c_void_p * _ENGINE_EVENTS)()
        self._ids = np.zeros(self.max_batch, np.int32)

    def close(self):
        if self._h:
            lib.pkv_engine_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, rid, prompt_len, max_new_tokens, arrival_step=0, token_ids=None):
        ids = None
        if token_ids is not None:
            ids = _as_c(token_ids, np.int32)
            if len(ids) != prompt_len:
                raise ValueError("token_ids must hold prompt_len ids")
        check(lib.pkv_engine_submit(self._h, int(rid), int(prompt_len), int(max_new_tokens),
                                    int(arrival_step), None if ids is None else ids.ctypes.data),
              "pkv_engine_submit")

    def adopt(self, seqs):
        s = _as_c(seqs, np.int64)
        check(lib.pkv_engine_adopt(self._h, len(s), s.ctypes.data), "pkv_engine_adopt")

    def running(self):
        n = int(lib.pkv_engine_running(self._h, None, 0))
        out = np.empty(n, np.int64)
        lib.pkv_engine_running(self._h, out.ctypes.data, n)
        return out

    def queued(self):
        return int(lib.pkv_engine_queued(self._h))

    def _rows(self, t, name, heads):
        _need(t, name, dtype=self.dtype, device=self.device)
        if t.dim() != 3 or t.shape[1:] != (heads, self.hd) or t.shape[0] < self.max_batch:
            raise ValueError(f"{name} must be [>= max_batch, {heads}, {self.hd}]")

    def step(self, q, k_new, v_new, out, *, scale, k_prompt=None, v_prompt=None, q_prompt=None,
             prefill_out=None, new_ids=None, events=None):
        """pkv_engine_step. q/k_new/v_new/out hold max_batch rows (the first B are used);
        k_prompt/v_prompt (and q_prompt/prefill_out, for the prefill attention) the prompt
        rows, whose count bounds each step's admitted prompt tokens. new_ids: host int32
        (max_batch entries, the first B used) or None. Returns info (int64 [8], overwritten by
        the next step): B, T, retired, admitted, plan units, copy-on-write pairs, queued, step."""
        self._rows(q, "q", self.Hq)
        self._rows(out, "out", self.Hq)
        self._rows(k_new, "k_new", self.Hkv)
        self._rows(v_new, "v_new", self.Hkv)
        rows = 0
        if (k_prompt is None) != (v_prompt is None):
            raise ValueError("give both k_prompt and v_prompt, or neither")
        if k_prompt is not None:
            for name, t in (("k_prompt", k_prompt), ("v_prompt", v_prompt)):
                _need(t, name, dtype=self.dtype, device=self.device)
                if t.dim() != 3 or t.shape[1:] != (self.Hkv, self.hd):
                    raise ValueError(f"{name} must be [rows, {self.Hkv}, {self.hd}]")
            rows = min(k_prompt.shape[0], v_prompt.shape[0])
        if (q_prompt is None) != (prefill_out is None):
            raise ValueError("give both q_prompt and prefill_out, or neither")
        if q_prompt is not None:
            for name, t in (("q_prompt", q_prompt), ("prefill_out", prefill_out)):
                _need(t, name, dtype=self.dtype, device=self.device)
                if t.dim() != 3 or t.shape[1:] != (self.Hq, self.hd) or t.shape[0] < rows:
                    raise ValueError(f"{name} must be [>= prompt rows, {self.Hq}, {self.hd}]")
        ids = None
        if new_ids is not None:
            n = len(new_ids)
            if n > self.max_batch:
                raise ValueError("more new_ids than max_batch")
            self._ids[:n] = new_ids
            ids = self._ids.ctypes.data
        ev = _event_handles(events, self._ev) if events is not None else None
        check(lib.pkv_engine_step(self._h, _ptr(q), _ptr(k_new), _ptr(v_new), ids, _ptr(out),
                                  _ptr(k_prompt), _ptr(v_prompt), rows, _ptr(q_prompt),
                                  _ptr(prefill_out), float(scale), ev, self._info_p,
                                  _stream(self.device)), "pkv_engine_step")
        return self.info

    def beam_step(self, q, k_new, v_new, out, *, scale, parents=None, children=None,
                  events=None):
        """pkv_engine_beam_step: parents (int32 [B], rows of the running set) and children
        (int64 [B], new ids), or neither. Returns info as step()."""
        self._rows(q, "q", self.Hq)
        self._rows(out, "out", self.Hq)
        self._rows(k_new, "k_new", self.Hkv)
        self._rows(v_new, "v_new", self.Hkv)
        if (parents is None) != (children is None):
            raise ValueError("give both parents and children, or neither")
        p = c = None
        if parents is not None:
            p = _as_c(parents, np.int32)
            c = _as_c(children, np.int64)
            if p.shape != c.shape:
                raise ValueError("parents and children must have one length")
        ev = _event_handles(events, self._ev) if events is not None else None
        check(lib.pkv_engine_beam_step(self._h, None if p is None else p.ctypes.data,
                                       None if c is None else c.ctypes.data, _ptr(q),
                                       _ptr(k_new), _ptr(v_new), _ptr(out), float(scale), ev,
                                       self._info_p, _stream(self.device)),
              "pkv_engine_beam_step")
        return self.info

    def last(self):
        """What the last step did: dict(retired, admitted [(id, prompt_len, cached)],
        prompt_slots, lens, tables (marked))."""
        B, T, R, A = (int(x) for x in self.info[:4])
        retired = np.empty(R, np.int64)
        admitted = np.empty(3 * A, np.int64)
        slots = np.empty(T, np.int32)
        lens = np.empty(B, np.int32)
        tables = np.empty((B, self.max_blocks), np.int32)
        check(lib.pkv_engine_last(self._h, retired.ctypes.data, admitted.ctypes.data,
                                  slots.ctypes.data, lens.ctypes.data, tables.ctypes.data),
              "pkv_engine_last")
        return dict(retired=retired, admitted=[tuple(int(x) for x in a)
                                               for a in admitted.reshape(A, 3)],
                    prompt_slots=slots, lens=lens, tables=tables)

    def last_lens(self):
        """Lengths the last step uploaded."""
        lens = np.empty(int(self.info[0]), np.int32)
        check(lib.pkv_engine_last(self._h, None, None, None, lens.ctypes.data, None),
              "pkv_engine_last")
        return lens

    def last_tables(self):
        """(lengths, marked tables) the last step uploaded."""
        B = int(self.info[0])
        lens = np.empty(B, np.int32)
        tables = np.empty((B, self.max_blocks), np.int32)
        check(lib.pkv_engine_last(self._h, None, None, None, lens.ctypes.data,
                                  tables.ctypes.data), "pkv_engine_last")
        return lens, tables

    def sync(self):
        check(lib.pkv_engine_sync(self._h), "pkv_engine_sync")
