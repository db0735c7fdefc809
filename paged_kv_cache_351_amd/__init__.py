"""MI355X paged decode attention: Python binding of libpagedkv.

The functions here carry the names of the C-ABI entry points declared in
``include/pagedkv.h`` and do only argument marshalling: they check tensor
shapes, types, devices and contiguity, derive the integer sizes from the
shapes, and pass raw device pointers and the current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If ``libpagedkv.so`` has not been built, loading fails loudly.

PyTorch provides device memory and streams only.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PA_OK = 0
PA_ERR_NO_BLOCKS = 5
_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_lib = None


class PagedKVError(RuntimeError):
    """A non-PA_OK status from libpagedkv; ``status`` holds the code."""

    def __init__(self, status, message):
        super().__init__(f"libpagedkv status {status}: {message}")
        self.status = status


def lib():
    """The loaded libpagedkv (ctypes.CDLL), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_351_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.pa_version.restype = i32
    L.pa_version.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_decode_workspace_size.restype = sz
    L.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]  # N, Hq, Hkv, D, max_len
    L.pa_decode.restype = i32
    L.pa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                            vp, vp, sz, vp]
    L.pa_decode_cached.restype = i32
    L.pa_decode_cached.argtypes = L.pa_decode.argtypes
    L.pa_decode_append.restype = i32
    L.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                   f32, i32, vp, vp, sz, vp]
    L.pa_decode_no_alloc.restype = i32
    L.pa_decode_no_alloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                     i32, vp, vp]
    L.pa_decode_no_alloc_scratch_bytes.restype = sz
    L.pa_decode_no_alloc_scratch_bytes.argtypes = []
    L.pa_write_kv.restype = i32
    L.pa_write_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.pa_copy_blocks.restype = i32
    L.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.pa_multi_query_workspace_size.restype = sz
    L.pa_multi_query_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pa_multi_query.restype = i32
    L.pa_multi_query.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                 i32, f32, i32, vp, vp, sz, vp]
    L.pa_decode_shared_prefix_workspace_size.restype = sz
    L.pa_decode_shared_prefix_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pa_decode_shared_prefix.restype = i32
    L.pa_decode_shared_prefix.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, i32, i32, i32, f32, i32, vp, vp, sz, vp]
    L.pa_swap_blocks.restype = i32
    L.pa_swap_blocks.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32, i32, i32, i32, i32, vp]
    i64 = ctypes.c_int64
    pi32, pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    for name, res, args in (
            ("pa_bm_create", i32, [i32, i32, pi32, i32, ctypes.POINTER(vp)]),
            ("pa_bm_swap_out", i32, [vp, pi64, i32, pi32, i32, ctypes.POINTER(i32)]),
            ("pa_bm_swap_in", i32, [vp, pi64, i32, pi32, i32, ctypes.POINTER(i32)]),
            ("pa_bm_num_free_cpu", i32, [vp]),
            ("pa_bm_is_swapped", i32, [vp, i64]),
            ("pa_bm_cpu_ref_count", i32, [vp, ctypes.c_int32]),
            ("pa_bm_destroy", None, [vp]),
            ("pa_bm_allocate", i32, [vp, i64, i64]),
            ("pa_bm_append_slot", i32, [vp, i64, pi64, pi32, pi32]),
            ("pa_bm_append_step", i32, [vp, pi64, i32, pi32, pi32, ctypes.POINTER(i32)]),
            ("pa_bm_fork", i32, [vp, i64, i64]),
            ("pa_bm_free", i32, [vp, i64]),
            ("pa_bm_num_free", i32, [vp]),
            ("pa_bm_seq_len", i64, [vp, i64]),
            ("pa_bm_table", i32, [vp, i64, pi32, i32]),
            ("pa_bm_ref_count", i32, [vp, ctypes.c_int32]),
            ("pa_bm_batch", i32, [vp, pi64, i32, pi32, i32, pi32])):
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def pa_last_error():
    return lib().pa_last_error().decode()


def pa_version():
    return lib().pa_version()


def _check(status):
    if status != PA_OK:
        raise PagedKVError(status, pa_last_error())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _scratch(nbytes, device, stream, zero):
    """A uint8 device tensor of nbytes allocated (and zero-filled, if asked) on the stream
    the call will run on, so that the fill is ordered before the kernels and the caching
    allocator hands the memory to no other stream's work after this function returns."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    with torch.cuda.stream(stream):
        if zero:
            return torch.zeros(nbytes, dtype=torch.uint8, device=device)
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, max_seq_len):
    return int(lib().pa_decode_workspace_size(int(num_seqs), int(num_heads), int(num_kv_heads),
                                              int(head_dim), int(max_seq_len)))


def decode_workspace(q, num_kv_heads, max_seq_len, stream=None):
    """A zero-filled workspace tensor sized for ``pa_decode`` with these arguments (None if
    the arguments are invalid; pa_decode then reports why), allocated and filled on
    ``stream`` (default: the current stream).  Reuse it across calls on that stream: each
    call leaves it ready for the next."""
    n = pa_decode_workspace_size(q.shape[0], q.shape[1], num_kv_heads, q.shape[2], max_seq_len)
    if n == 0:
        return None
    return _scratch(n, q.device, stream, zero=True)


def pa_decode(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, *,
              max_seq_len, workspace=None, stream=None):
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over the seq_lens[s] tokens of
    sequence s, K_s/V_s fetched through block_tables[s] (see include/pagedkv.h).

    q, out: [num_seqs, num_heads, head_dim]; k_cache, v_cache:
    [num_blocks, block_size, num_kv_heads, head_dim], same dtype as q;
    block_tables: int32 [num_seqs, max_blocks_per_seq]; seq_lens: int32 [num_seqs];
    max_seq_len: host int bound on seq_lens (no device sync is made);
    workspace: uint8 tensor of at least pa_decode_workspace_size(...) bytes, allocated
    (zero-filled) here on ``stream`` if omitted (pass one to keep allocation off the hot
    path); stream: a torch.cuda.Stream, default the current one.
    """
    return _decode("pa_decode", q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale,
                   out, max_seq_len, workspace, stream)


def pa_decode_cached(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, *,
                     max_seq_len, workspace=None, stream=None):
    """pa_decode for batches whose sequences share blocks: the same result bit for bit, with
    the K/V loads under the default cache policy, so that rows read by several sequences
    can hit in the caches (pa_decode streams them; see include/pagedkv.h)."""
    return _decode("pa_decode_cached", q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads,
                   scale, out, max_seq_len, workspace, stream)


def _decode(entry, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out,
            max_seq_len, workspace, stream):
    _dev("q", q, ndim=3)
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(name, t, q.dtype, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    _dev("out", out, q.dtype)
    num_seqs, num_heads, head_dim = q.shape
    num_blocks, block_size, nkv, hd = k_cache.shape
    if nkv != num_kv_heads or hd != head_dim:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, head_dim={head_dim}")
    if out.shape != q.shape or block_tables.shape[0] != num_seqs or seq_lens.shape[0] != num_seqs:
        raise ValueError("q, out, block_tables and seq_lens disagree on num_seqs or shape")
    if workspace is None:
        workspace = decode_workspace(q, num_kv_heads, max_seq_len, stream)
    if workspace is not None:
        _dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(getattr(lib(), entry)(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
        block_tables.shape[1], int(max_seq_len), float(scale), _DTYPE[q.dtype], _ptr(out),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pa_decode_append(q, new_k, new_v, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale,
                     out, *, max_seq_len, workspace=None, stream=None):
    """Store each sequence's newest token (position seq_lens[s] - 1) into the slot its block
    table gives that position, then pa_decode, in one call: bit-identical to pa_write_kv
    into those slots followed by pa_decode (see include/pagedkv.h).

    new_k, new_v: [num_seqs, num_kv_heads, head_dim], same dtype as q; the other arguments
    as for pa_decode.  Each newest slot must belong to its sequence alone.
    """
    _dev("q", q, ndim=3)
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(name, t, q.dtype, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    _dev("out", out, q.dtype)
    num_seqs, num_heads, head_dim = q.shape
    num_blocks, block_size, nkv, hd = k_cache.shape
    if nkv != num_kv_heads or hd != head_dim:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, head_dim={head_dim}")
    for name, t in (("new_k", new_k), ("new_v", new_v)):
        _dev(name, t, q.dtype, 3)
        if tuple(t.shape) != (num_seqs, num_kv_heads, head_dim):
            raise ValueError(f"{name} must be [num_seqs, num_kv_heads, head_dim] = "
                             f"{(num_seqs, num_kv_heads, head_dim)}, got {tuple(t.shape)}")
    if out.shape != q.shape or block_tables.shape[0] != num_seqs or seq_lens.shape[0] != num_seqs:
        raise ValueError("q, out, block_tables and seq_lens disagree on num_seqs or shape")
    if workspace is None:
        workspace = decode_workspace(q, num_kv_heads, max_seq_len, stream)
    if workspace is not None:
        _dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode_append(
        _ptr(q), _ptr(new_k), _ptr(new_v), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(seq_lens), num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
        block_tables.shape[1], int(max_seq_len), float(scale), _DTYPE[q.dtype], _ptr(out),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pa_decode_no_alloc(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, *,
                       max_seq_len, stream=None):
    """pa_decode without a workspace argument and without any allocation: the library
    uses its own per-GPU device array (include/pagedkv.h).  Calls that may overlap on one
    GPU race on that array; keep them on one stream."""
    _dev("q", q, ndim=3)
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(name, t, q.dtype, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    _dev("out", out, q.dtype)
    num_seqs, num_heads, head_dim = q.shape
    num_blocks, block_size, nkv, hd = k_cache.shape
    if nkv != num_kv_heads or hd != head_dim:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, head_dim={head_dim}")
    if out.shape != q.shape or block_tables.shape[0] != num_seqs or seq_lens.shape[0] != num_seqs:
        raise ValueError("q, out, block_tables and seq_lens disagree on num_seqs or shape")
    _check(lib().pa_decode_no_alloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
        block_tables.shape[1], int(max_seq_len), float(scale), _DTYPE[q.dtype], _ptr(out),
        _stream(stream)))
    return out


def pa_decode_no_alloc_scratch_bytes():
    return int(lib().pa_decode_no_alloc_scratch_bytes())


def pa_multi_query_workspace_size(num_seqs, total_q, num_heads, num_kv_heads, head_dim, max_q_len,
                                  max_seq_len):
    return int(lib().pa_multi_query_workspace_size(int(num_seqs), int(total_q), int(num_heads),
                                                   int(num_kv_heads), int(head_dim), int(max_q_len),
                                                   int(max_seq_len)))


def pa_multi_query(q, k_cache, v_cache, block_tables, seq_lens, q_start, num_kv_heads, scale, out, *,
                   max_q_len, max_seq_len, workspace=None, stream=None):
    """Several causal queries per sequence (chunked prefill, speculative verification):
    rows q_start[s] .. q_start[s+1]-1 of q are the last n_s of sequence s's seq_lens[s]
    cached tokens; query i attends to tokens 0 .. seq_lens[s] - n_s + i (include/pagedkv.h).

    q, out: [total_q, num_heads, head_dim]; q_start: int32 [num_seqs + 1] from 0 to total_q;
    max_q_len / max_seq_len: host bounds (no device sync); workspace: uint8 tensor of at least
    pa_multi_query_workspace_size(...) bytes, allocated here if needed and omitted.
    """
    _dev("q", q, ndim=3)
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(name, t, q.dtype, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    _dev("q_start", q_start, torch.int32, 1)
    _dev("out", out, q.dtype)
    total_q, num_heads, head_dim = q.shape
    num_blocks, block_size, nkv, hd = k_cache.shape
    num_seqs = seq_lens.shape[0]
    if nkv != num_kv_heads or hd != head_dim:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, head_dim={head_dim}")
    if out.shape != q.shape or block_tables.shape[0] != num_seqs or q_start.shape[0] != num_seqs + 1:
        raise ValueError("q, out, block_tables, seq_lens and q_start disagree")
    need = pa_multi_query_workspace_size(num_seqs, total_q, num_heads, num_kv_heads, head_dim,
                                         max_q_len, max_seq_len)
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream, zero=False)
    if workspace is not None:
        _dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_multi_query(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(q_start),
        num_seqs, total_q, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
        block_tables.shape[1], int(max_q_len), int(max_seq_len), float(scale), _DTYPE[q.dtype],
        _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pa_decode_shared_prefix_workspace_size(num_seqs, num_groups, num_heads, num_kv_heads, head_dim,
                                           max_group_size, max_seq_len):
    return int(lib().pa_decode_shared_prefix_workspace_size(
        int(num_seqs), int(num_groups), int(num_heads), int(num_kv_heads), int(head_dim),
        int(max_group_size), int(max_seq_len)))


def pa_decode_shared_prefix(q, k_cache, v_cache, block_tables, seq_lens, group_start, prefix_lens,
                            num_kv_heads, scale, out, *, max_group_size, max_seq_len, workspace=None,
                            stream=None):
    """pa_decode's result, reading every group's shared prefix once (include/pagedkv.h):
    sequences group_start[j] .. group_start[j+1]-1 share the blocks of their first
    prefix_lens[j] tokens.  group_start: int32 [G + 1] from 0 to num_seqs; prefix_lens:
    int32 [G]; max_group_size / max_seq_len: host bounds (no device sync)."""
    _dev("q", q, ndim=3)
    if q.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(name, t, q.dtype, 4)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    _dev("block_tables", block_tables, torch.int32, 2)
    _dev("seq_lens", seq_lens, torch.int32, 1)
    _dev("group_start", group_start, torch.int32, 1)
    _dev("prefix_lens", prefix_lens, torch.int32, 1)
    _dev("out", out, q.dtype)
    num_seqs, num_heads, head_dim = q.shape
    num_blocks, block_size, nkv, hd = k_cache.shape
    num_groups = prefix_lens.shape[0]
    if nkv != num_kv_heads or hd != head_dim:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, head_dim={head_dim}")
    if out.shape != q.shape or block_tables.shape[0] != num_seqs or seq_lens.shape[0] != num_seqs \
            or group_start.shape[0] != num_groups + 1:
        raise ValueError("q, out, block_tables, seq_lens, group_start and prefix_lens disagree")
    need = pa_decode_shared_prefix_workspace_size(num_seqs, num_groups, num_heads, num_kv_heads,
                                                  head_dim, max_group_size, max_seq_len)
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream, zero=False)
    if workspace is not None:
        _dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode_shared_prefix(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(group_start),
        _ptr(prefix_lens), num_seqs, num_groups, num_heads, num_kv_heads, head_dim, block_size,
        num_blocks, block_tables.shape[1], int(max_group_size), int(max_seq_len), float(scale),
        _DTYPE[q.dtype], _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pa_write_kv(k, v, slot_mapping, k_cache, v_cache, *, stream=None):
    """k_cache/v_cache[slot // B, slot % B] = k[i]/v[i] for every slot_mapping[i] >= 0."""
    _dev("k", k, ndim=3)
    if k.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {k.dtype}")
    _dev("v", v, k.dtype, 3)
    _dev("slot_mapping", slot_mapping, torch.int32, 1)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(name, t, k.dtype, 4)
    num_tokens, nkv, hd = k.shape
    num_blocks, block_size, cnkv, chd = k_cache.shape
    if v.shape != k.shape or slot_mapping.shape[0] != num_tokens or (cnkv, chd) != (nkv, hd) \
            or v_cache.shape != k_cache.shape:
        raise ValueError("k, v, slot_mapping and cache shapes disagree")
    _check(lib().pa_write_kv(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                             num_tokens, nkv, hd, block_size, num_blocks, _DTYPE[k.dtype],
                             _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, src_dst_pairs, *, stream=None):
    """k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src] for every (src, dst) pair."""
    _dev("k_cache", k_cache, ndim=4)
    if k_cache.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {k_cache.dtype}")
    _dev("v_cache", v_cache, k_cache.dtype, 4)
    _dev("src_dst_pairs", src_dst_pairs, torch.int32, 2)
    if v_cache.shape != k_cache.shape or src_dst_pairs.shape[1] != 2:
        raise ValueError("cache shapes differ or pairs are not [n, 2]")
    num_blocks, block_size, nkv, hd = k_cache.shape
    _check(lib().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src_dst_pairs),
                                src_dst_pairs.shape[0], block_size, nkv, hd, num_blocks,
                                _DTYPE[k_cache.dtype], _stream(stream)))


def _acc(name, t, dtype=None, ndim=None):
    """Like _dev, but pinned host tensors are accepted too (pa_swap_blocks reads and
    writes them directly)."""
    if isinstance(t, torch.Tensor) and t.device.type == "cpu":
        if not t.is_pinned():
            raise ValueError(f"{name} must be on the GPU or in pinned host memory "
                             "(pin_memory=True)")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
        return
    _dev(name, t, dtype, ndim)


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs, *, stream=None):
    """dst_k[dst] = src_k[src] and dst_v[dst] = src_v[src] for every (src, dst) pair, between
    two pools of the same block shape: a GPU pool and a pinned host pool (either way), or two
    GPU pools.  The pairs may be a GPU tensor or a pinned host tensor.  Enqueued on the
    stream; synchronise before the host reads a host pool that was written."""
    _acc("src_k", src_k, ndim=4)
    if src_k.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {src_k.dtype}")
    _acc("src_v", src_v, src_k.dtype, 4)
    _acc("dst_k", dst_k, src_k.dtype, 4)
    _acc("dst_v", dst_v, src_k.dtype, 4)
    _acc("src_dst_pairs", src_dst_pairs, torch.int32, 2)
    if src_v.shape != src_k.shape or dst_v.shape != dst_k.shape or \
            src_k.shape[1:] != dst_k.shape[1:] or src_dst_pairs.shape[1] != 2:
        raise ValueError("pool shapes disagree or pairs are not [n, 2]")
    _, block_size, nkv, hd = src_k.shape
    _check(lib().pa_swap_blocks(_ptr(src_k), _ptr(src_v), src_k.shape[0], _ptr(dst_k), _ptr(dst_v),
                                dst_k.shape[0], _ptr(src_dst_pairs), src_dst_pairs.shape[0],
                                block_size, nkv, hd, _DTYPE[src_k.dtype], _stream(stream)))


class BlockManager:
    """Host block manager of the library (the ``pa_bm_*`` entry points): a pool of
    ``num_blocks`` blocks of ``block_size`` tokens, one block table per sequence,
    reference counts and copy-on-write.  Sequences are named by Python ints.

    Pure host bookkeeping: it yields the index inputs of the kernels -- block
    tables and lengths (``batch`` -> ``pa_decode``), write slots (``append_slot``
    -> ``pa_write_kv``) and copy-on-write pairs (-> ``pa_copy_blocks``).  Failed
    calls raise ``PagedKVError`` (status 5 when the pool is out of blocks) and
    leave the manager unchanged.
    """

    def __init__(self, num_blocks, block_size, free_order=None, num_cpu_blocks=0):
        self._h = None
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.num_cpu_blocks = int(num_cpu_blocks)
        order = None
        if free_order is not None:
            order = (ctypes.c_int32 * len(free_order))(*[int(b) for b in free_order])
            if len(free_order) != self.num_blocks:
                raise ValueError("free_order must list every block once")
        h = ctypes.c_void_p()
        _check(lib().pa_bm_create(self.num_blocks, self.block_size, order, self.num_cpu_blocks,
                                  ctypes.byref(h)))
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.pa_bm_destroy(self._h)
            self._h = None

    def allocate(self, seq, num_tokens):
        """Prefill: ``seq`` gets ceil(num_tokens / block_size) fresh blocks; returns its table."""
        _check(lib().pa_bm_allocate(self._h, int(seq), int(num_tokens)))
        return self.table(seq)

    def append_slot(self, seq):
        """Slot of ``seq``'s next token and the (src, dst) copy-on-write pair, or None."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_bm_append_slot(self._h, int(seq), ctypes.byref(slot), ctypes.byref(src),
                                       ctypes.byref(dst)))
        return slot.value, ((src.value, dst.value) if src.value >= 0 else None)

    def append_step(self, seqs):
        """One decode step for the distinct ``seqs``: (slot_mapping int32 [n], copy-on-write
        pairs int32 [p, 2]) as CPU tensors, the inputs of ``pa_write_kv`` and
        ``pa_copy_blocks`` (copy first).  All or nothing when blocks run out."""
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*[int(s) for s in seqs])
        slots = torch.empty(n, dtype=torch.int32)
        pairs = torch.empty((max(n, 1), 2), dtype=torch.int32)
        np_ = ctypes.c_int()
        as_p = lambda t: ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))
        _check(lib().pa_bm_append_step(self._h, ids, n, as_p(slots), as_p(pairs), ctypes.byref(np_)))
        return slots, pairs[:np_.value].clone()

    def _move(self, fn, seqs):
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*[int(s) for s in seqs])
        cap = sum(len(self.table(s)) for s in seqs)
        pairs = torch.empty((max(cap, 1), 2), dtype=torch.int32)
        np_ = ctypes.c_int()
        _check(fn(self._h, ids, n, ctypes.cast(pairs.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                  cap, ctypes.byref(np_)))
        return pairs[:np_.value].clone()

    def swap_out(self, seqs):
        """Preempt ``seqs`` together: (gpu_block, cpu_block) pairs, int32 CPU tensor [p, 2], to
        copy with ``pa_swap_blocks`` from the GPU pool to the host pool."""
        return self._move(lib().pa_bm_swap_out, seqs)

    def swap_in(self, seqs):
        """Restore ``seqs`` together: (cpu_block, gpu_block) pairs, int32 CPU tensor [p, 2], to
        copy with ``pa_swap_blocks`` from the host pool to the GPU pool."""
        return self._move(lib().pa_bm_swap_in, seqs)

    def num_free_cpu(self):
        return lib().pa_bm_num_free_cpu(self._h)

    def is_swapped(self, seq):
        r = lib().pa_bm_is_swapped(self._h, int(seq))
        if r < 0:
            raise KeyError(seq)
        return bool(r)

    def cpu_ref_count(self, block):
        r = lib().pa_bm_cpu_ref_count(self._h, int(block))
        if r < 0:
            raise IndexError(block)
        return r

    def fork(self, parent, child):
        _check(lib().pa_bm_fork(self._h, int(parent), int(child)))

    def free_seq(self, seq):
        _check(lib().pa_bm_free(self._h, int(seq)))

    def num_free(self):
        return lib().pa_bm_num_free(self._h)

    def seq_len(self, seq):
        n = lib().pa_bm_seq_len(self._h, int(seq))
        if n < 0:
            raise KeyError(seq)
        return n

    def table(self, seq):
        n = lib().pa_bm_table(self._h, int(seq), None, 0)
        if n < 0:
            raise KeyError(seq)
        buf = (ctypes.c_int32 * max(n, 1))()
        lib().pa_bm_table(self._h, int(seq), buf, n)
        return list(buf[:n])

    def ref_count(self, block):
        r = lib().pa_bm_ref_count(self._h, int(block))
        if r < 0:
            raise IndexError(block)
        return r

    def batch(self, seqs, max_blocks_per_seq):
        """(block_tables [n, max_blocks_per_seq], seq_lens [n]) as int32 CPU tensors, tables
        padded with -1; move them to the device for ``pa_decode``."""
        n = len(seqs)
        ids = (ctypes.c_int64 * max(n, 1))(*[int(s) for s in seqs])
        tables = torch.empty((n, int(max_blocks_per_seq)), dtype=torch.int32)
        lens = torch.empty(n, dtype=torch.int32)
        _check(lib().pa_bm_batch(
            self._h, ids, n, ctypes.cast(tables.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
            int(max_blocks_per_seq), ctypes.cast(lens.data_ptr(), ctypes.POINTER(ctypes.c_int32))))
        return tables, lens


__all__ = ["pa_decode", "pa_decode_cached", "pa_decode_append", "pa_decode_no_alloc", "pa_decode_no_alloc_scratch_bytes", "pa_multi_query", "pa_multi_query_workspace_size", "pa_decode_shared_prefix",
           "pa_decode_shared_prefix_workspace_size", "pa_write_kv",
           "pa_copy_blocks", "pa_swap_blocks", "pa_decode_workspace_size",
           "decode_workspace", "pa_last_error", "pa_version",
           "PagedKVError", "BlockManager", "lib", "LIB_PATH"]
