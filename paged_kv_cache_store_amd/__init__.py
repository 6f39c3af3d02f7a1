"""Python binding of libpa, the paged KV-cache attention library for MI355X.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/pa.h``. torch provides device memory and the stream.
The first call loads ``libpa.so`` and raises if it is missing; there is no
fallback implementation.

Pools are torch tensors in the library's layout (x = 8 for bf16, 16 for fp8):
    K: (num_blocks, num_kv_heads, head_dim // x, block_size, x)
    V: (num_blocks, num_kv_heads, block_size // x, head_dim, x)
bf16 pools have dtype torch.bfloat16, fp8 (E4M3) pools torch.uint8.
"""
import ctypes
import os
import re

import torch

__all__ = ["store_kv", "decode", "decode_noalloc", "prefill_varlen", "prefill_set_slots", "add_rmsnorm",
           "decode_workspace_size",
           "decode_partition_size", "empty_pools", "capture_step", "copy_blocks", "BlockManager",
           "PaError", "LIB_PATH", "library"]

_IN_TREE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")


def _library_path():
    """The in-tree libpa.so. Another build of the same library (a tuning
    variant) is loaded only when PA_LIBRARY names it and PA_ALLOW_OTHER_LIBRARY=1
    confirms it; PA_LIBRARY alone is an error, so a stray setting can never
    swap the library under a run unnoticed."""
    other = os.environ.get("PA_LIBRARY")
    if not other:
        return _IN_TREE
    if os.environ.get("PA_ALLOW_OTHER_LIBRARY") != "1":
        raise RuntimeError(f"PA_LIBRARY={other} is set but PA_ALLOW_OTHER_LIBRARY=1 is not: "
                           f"refusing to load a library other than {_IN_TREE}")
    return other


LIB_PATH = _library_path()

PA_KV_BF16, PA_KV_FP8_E4M3 = 0, 1


class PaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        lib = library()
        msg = lib.pa_status_string(status).decode()
        if status == -5:
            msg += ": " + lib.pa_last_hip_error().decode()
        super().__init__(f"{where}: status {status}: {msg}")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_store_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(CacheDesc)
    lib.pa_store_kv.argtypes = [P, P, P, I32, P, P, D, P]
    lib.pa_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.pa_decode_workspace_size.restype = SZ
    lib.pa_decode_partition_size.argtypes = [I32, I32, I32, I32]
    lib.pa_decode_partition_size.restype = I32
    lib.pa_decode.argtypes = [P, P, P, P, I32, P, I32, I32, I32, F, P, D, I32, P, SZ, P]
    lib.pa_store_decode.argtypes = [P, P, P, P, P, P, P, I32, P, I32, I32, I32, F, P, D, I32, P, SZ, P]
    lib.pa_decode_noalloc.argtypes = [P, P, P, P, I32, P, I32, I32, I32, F, P, D, I32, P]
    lib.pa_prefill_varlen.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P, D, P]
    lib.pa_add_rmsnorm.argtypes = [P, P, P, I32, I32, F, P, P, P]
    lib.pa_prefill_set_slots.argtypes = [I32]
    for name in ("pa_store_kv", "pa_decode", "pa_store_decode", "pa_prefill_varlen", "pa_add_rmsnorm",
                 "pa_decode_noalloc", "pa_prefill_set_slots"):
        getattr(lib, name).restype = ctypes.c_int
    I64, PI32, PI64 = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.pa_copy_blocks.argtypes = [P, P, P, I32, D, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_bm_create.argtypes = [I32, I32, I32, ctypes.POINTER(P)]
    lib.pa_bm_destroy.argtypes = [P]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_num_free_blocks.argtypes = [P]
    lib.pa_bm_num_free_blocks.restype = I32
    lib.pa_bm_add_sequence.argtypes = [P, PI32, I32, PI64, PI32]
    lib.pa_bm_append_token.argtypes = [P, I64, I32, PI32, PI32, PI32]
    lib.pa_bm_fork.argtypes = [P, I64, PI64]
    lib.pa_bm_free_sequence.argtypes = [P, I64]
    lib.pa_bm_sequence_info.argtypes = [P, I64, PI32, PI32]
    lib.pa_bm_block_table.argtypes = [P, I64, PI32, I32, I32]
    lib.pa_bm_slots.argtypes = [P, I64, I32, I32, PI32]
    lib.pa_bm_block_refcount.argtypes = [P, I32]
    lib.pa_bm_block_refcount.restype = I32
    for name in ("pa_bm_create", "pa_bm_add_sequence", "pa_bm_append_token", "pa_bm_fork",
                 "pa_bm_free_sequence", "pa_bm_sequence_info", "pa_bm_block_table", "pa_bm_slots"):
        getattr(lib, name).restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_hip_error.argtypes = []
    lib.pa_last_hip_error.restype = ctypes.c_char_p
    return lib


_lib = None


def library():
    """The loaded ctypes library; loads it on first use and raises if it is not built."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _pool_desc(k_cache, v_cache, k_scale, v_scale, need_scales=True):
    if k_cache.dtype == torch.bfloat16:
        dtype, x = PA_KV_BF16, 8
    elif k_cache.dtype == torch.uint8:
        dtype, x = PA_KV_FP8_E4M3, 16
    else:
        raise ValueError(f"k_cache dtype {k_cache.dtype} is neither bfloat16 nor uint8 (fp8)")
    _check(k_cache, "k_cache", k_cache.dtype, 5)
    _check(v_cache, "v_cache", k_cache.dtype, 5, k_cache.device)
    nb, hkv, dx, bs, xx = k_cache.shape
    if xx != x or tuple(v_cache.shape) != (nb, hkv, bs // x, dx * x, x) or bs % x:
        raise ValueError(f"pool shapes {tuple(k_cache.shape)} / {tuple(v_cache.shape)} "
                         f"do not match the layout for x={x}")
    if dtype == PA_KV_FP8_E4M3 and not need_scales:
        # calls that only move bytes: the C ABI still wants non-NULL scale pointers
        k_scale = v_scale = k_cache
    elif dtype == PA_KV_FP8_E4M3:
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            if sc is None:
                raise ValueError(f"{name} is required for an fp8 pool")
            _check(sc, name, torch.float32, 1, k_cache.device)
            if sc.numel() != hkv:
                raise ValueError(f"{name} must have num_kv_heads={hkv} entries")
    desc = CacheDesc(nb, bs, hkv, dx * x, dtype,
                     k_scale.data_ptr() if dtype == PA_KV_FP8_E4M3 else None,
                     v_scale.data_ptr() if dtype == PA_KV_FP8_E4M3 else None)
    return desc, nb, hkv, dx * x, bs


def empty_pools(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype="bf16", device="cuda"):
    """Uninitialised K and V pools in the library's layout."""
    if kv_dtype == "fp8":
        x, dt = 16, torch.uint8
    elif kv_dtype == "bf16":
        x, dt = 8, torch.bfloat16
    else:
        raise ValueError(kv_dtype)
    k = torch.empty((num_blocks, num_kv_heads, head_dim // x, block_size, x), dtype=dt, device=device)
    v = torch.empty((num_blocks, num_kv_heads, block_size // x, head_dim, x), dtype=dt, device=device)
    return k, v


def store_kv(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None, stream=None):
    """Write k, v ([T, Hkv, D] bf16) into the pools at slot_mapping ([T] int32; <0 skips)."""
    desc, nb, hkv, d, bs = _pool_desc(k_cache, v_cache, k_scale, v_scale)
    dev = k_cache.device
    _check(k, "k", torch.bfloat16, 3, dev)
    _check(v, "v", torch.bfloat16, 3, dev)
    _check(slot_mapping, "slot_mapping", torch.int32, 1, dev)
    T = k.shape[0]
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d) or slot_mapping.numel() != T:
        raise ValueError("k, v must be [T, num_kv_heads, head_dim] and slot_mapping [T]")
    st = library().pa_store_kv(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache),
                          ctypes.byref(desc), _stream(stream))
    if st != 0:
        raise PaError(st, "pa_store_kv")


def decode_partition_size(num_seqs, num_q_heads, max_context_len, partition_size=0):
    return int(library().pa_decode_partition_size(num_seqs, num_q_heads, max_context_len, partition_size))


def decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, partition_size=0):
    return int(library().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                             partition_size))


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out=None,
           k_scale=None, v_scale=None, partition_size=0, workspace=None, stream=None,
           new_k=None, new_v=None, slot_mapping=None):
    """Paged decode attention; returns out ([S, Hq, D] bf16). With new_k / new_v
    ([S, Hkv, D] bf16) and slot_mapping ([S] int32) each sequence's newest token
    is stored in the same launch (pa_store_decode)."""
    desc, nb, hkv, d, bs = _pool_desc(k_cache, v_cache, k_scale, v_scale)
    dev = k_cache.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(context_lens, "context_lens", torch.int32, 1, dev)
    S, hq, dq = q.shape
    if dq != d or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("q [S, Hq, D], block_tables [S, MB] and context_lens [S] disagree")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 3, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    mb = block_tables.shape[1]
    cap = min(int(max_context_len), mb * bs)
    need = decode_workspace_size(S, hq, d, cap, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fused = new_k is not None or new_v is not None or slot_mapping is not None
    if fused:
        for name, t in (("new_k", new_k), ("new_v", new_v)):
            _check(t, name, torch.bfloat16, 3, dev)
            if tuple(t.shape) != (S, hkv, d):
                raise ValueError(f"{name} must be [S, Hkv, D] = {(S, hkv, d)}")
        _check(slot_mapping, "slot_mapping", torch.int32, 1, dev)
        if slot_mapping.numel() != S:
            raise ValueError("slot_mapping must have one slot per sequence")
        st = library().pa_store_decode(_ptr(q), _ptr(new_k), _ptr(new_v), _ptr(slot_mapping), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_tables), mb, _ptr(context_lens), S, hq,
                                       int(max_context_len), float(scale), _ptr(out), ctypes.byref(desc),
                                       int(partition_size), _ptr(workspace), wbytes, _stream(stream))
        if st != 0:
            raise PaError(st, "pa_store_decode")
        return out
    st = library().pa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), mb,
                        _ptr(context_lens), S, hq, int(max_context_len), float(scale), _ptr(out),
                        ctypes.byref(desc), int(partition_size), _ptr(workspace), wbytes,
                        _stream(stream))
    if st != 0:
        raise PaError(st, "pa_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out,
                   k_scale=None, v_scale=None, partition_size=0, stream=None):
    """pa_decode_noalloc: pa_decode with its scratch in the library's device
    array (no workspace, nothing allocated). `out` ([S, Hq, D] bf16) is
    required. Calls that overlap on one GPU race (see include/pa.h)."""
    desc, nb, hkv, d, bs = _pool_desc(k_cache, v_cache, k_scale, v_scale)
    dev = k_cache.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(block_tables, "block_tables", torch.int32, 2, dev)
    _check(context_lens, "context_lens", torch.int32, 1, dev)
    _check(out, "out", torch.bfloat16, 3, dev)
    S, hq, dq = q.shape
    if dq != d or block_tables.shape[0] != S or context_lens.numel() != S or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q [S, Hq, D], block_tables [S, MB], context_lens [S] and out disagree")
    st = library().pa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                     block_tables.shape[1], _ptr(context_lens), S, hq, int(max_context_len),
                                     float(scale), _ptr(out), ctypes.byref(desc), int(partition_size),
                                     _stream(stream))
    if st != 0:
        raise PaError(st, "pa_decode_noalloc")
    return out


def prefill_set_slots(slots: int) -> None:
    """Resident workgroups of a persistent prefill launch (bf16 pool, blocks of at
    least 64 tokens): 0 = two per compute unit (default), > 0 = that many, < 0 = one
    workgroup per work item. Process-wide; the output is the same for every value."""
    library().pa_prefill_set_slots(int(slots))


def prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables, scale,
                   max_seqlen_q, max_seqlen_k, out=None, k_scale=None, v_scale=None, stream=None):
    """Causal varlen prefill; returns out ([Tq, Hq, D] bf16).
    Paged: k_cache / v_cache are the pools and block_tables [S, MB] int32 (fp8
    pools need k_scale / v_scale, device float32 [num_kv_heads]).
    Packed: block_tables=None and k_cache / v_cache are bf16 [Tk, Hkv, D], the
    keys of sequence s in rows cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1."""
    dev = q.device
    _check(q, "q", torch.bfloat16, 3, dev)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, dev)
    S = cu_seqlens_q.numel() - 1
    if block_tables is None:
        _check(k_cache, "k", torch.bfloat16, 3, dev)
        _check(v_cache, "v", torch.bfloat16, 3, dev)
        tk, hkv, d = k_cache.shape
        if tuple(v_cache.shape) != (tk, hkv, d):
            raise ValueError("packed k and v must both be [Tk, Hkv, D]")
        desc = CacheDesc(0, 0, hkv, d, PA_KV_BF16, None, None)
        mb, table = 0, None
    else:
        desc, nb, hkv, d, bs = _pool_desc(k_cache, v_cache, k_scale, v_scale)
        _check(block_tables, "block_tables", torch.int32, 2, dev)
        if block_tables.shape[0] != S:
            raise ValueError("block_tables must be [S, MB] with S = len(cu_seqlens_q) - 1")
        mb, table = block_tables.shape[1], block_tables
    if cu_seqlens_k.numel() != S + 1 or q.shape[2] != d:
        raise ValueError("cu_seqlens_q/k [S+1] and q [Tq, Hq, D] disagree")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", torch.bfloat16, 3, dev)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    st = library().pa_prefill_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q),
                                     _ptr(cu_seqlens_k), _ptr(table), mb, S, q.shape[1], int(max_seqlen_q),
                                     int(max_seqlen_k), float(scale), _ptr(out), ctypes.byref(desc),
                                     _stream(stream))
    if st != 0:
        raise PaError(st, "pa_prefill_varlen")
    return out


def add_rmsnorm(x, weight, eps, residual=None, out=None, residual_out=None, stream=None):
    """Residual add fused with RMSNorm over the last dimension (see pa.h).
    x, residual, out, residual_out: bf16 [T, H] on one device; weight bf16 [H].
    Returns out, or (out, residual_out) when a residual is given. Passing
    out=x and residual_out=residual works in place."""
    dev = x.device
    _check(x, "x", torch.bfloat16, 2, dev)
    T, H = x.shape
    _check(weight, "weight", torch.bfloat16, 1, dev)
    if weight.shape[0] != H:
        raise ValueError(f"weight has {weight.shape[0]} entries for hidden size {H}")
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", torch.bfloat16, 2, dev)
    if tuple(out.shape) != (T, H):
        raise ValueError("out must have the shape of x")
    if residual is not None:
        _check(residual, "residual", torch.bfloat16, 2, dev)
        if residual_out is None:
            residual_out = torch.empty_like(x)
        _check(residual_out, "residual_out", torch.bfloat16, 2, dev)
        if tuple(residual.shape) != (T, H) or tuple(residual_out.shape) != (T, H):
            raise ValueError("residual and residual_out must have the shape of x")
    st = library().pa_add_rmsnorm(_ptr(x), _ptr(residual) if residual is not None else None, _ptr(weight),
                                  T, H, float(eps), _ptr(out),
                                  _ptr(residual_out) if residual is not None else None, _stream(stream))
    if st != 0:
        raise PaError(st, "pa_add_rmsnorm")
    return out if residual is None else (out, residual_out)


def capture_step(fn, warmup=1):
    """Record the library calls made by fn() once as a HIP graph and return it;
    graph.replay() then re-issues the same kernels with the same arguments and
    no per-call host work. Every buffer fn() touches (pools, tables, outputs,
    decode workspace) must be allocated before the call and kept alive while the
    graph is used; nothing is allocated during capture. The library enqueues no
    memset and no host synchronisation, so its calls are capturable. CUDA-graph
    replay of a fixed kernel sequence is the launch-overhead removal the pages
    describe ("Nano-vLLM：轻量高效的大模型推理框架…", 三.2 (3) CUDA图与Torch编译)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def copy_blocks(k_cache, v_cache, pairs, stream=None):
    """Copy whole blocks inside the pools; pairs: device int32 [n, 2] of (src, dst)."""
    desc, *_ = _pool_desc(k_cache, v_cache, None, None, need_scales=False)
    _check(pairs, "pairs", torch.int32, 2, k_cache.device)
    st = library().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0],
                                  ctypes.byref(desc), _stream(stream))
    if st != 0:
        raise PaError(st, "pa_copy_blocks")


class BlockManager:
    """Host-side block manager with prefix caching (C++ in libpa; see
    include/pa_block_manager.h). Hands out the blocks of one pool, returns the
    block tables and slot mappings the kernels consume."""

    def __init__(self, num_blocks, block_size, prefix_caching=True):
        self._lib = library()
        h = ctypes.c_void_p()
        st = self._lib.pa_bm_create(num_blocks, block_size, 1 if prefix_caching else 0, ctypes.byref(h))
        if st != 0:
            raise PaError(st, "pa_bm_create")
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def _call(self, name, *args):
        st = getattr(self._lib, name)(self._h, *args)
        if st != 0:
            raise PaError(st, name)

    @property
    def num_free_blocks(self):
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def add_sequence(self, tokens):
        """Returns (seq_id, num_cached_tokens)."""
        arr = (ctypes.c_int32 * max(1, len(tokens)))(*tokens)
        sid, cached = ctypes.c_int64(), ctypes.c_int32()
        self._call("pa_bm_add_sequence", arr, len(tokens), ctypes.byref(sid), ctypes.byref(cached))
        return sid.value, cached.value

    def append_token(self, seq_id, token):
        """Returns (slot, (cow_src, cow_dst) or None)."""
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._call("pa_bm_append_token", seq_id, token, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def fork(self, seq_id):
        new = ctypes.c_int64()
        self._call("pa_bm_fork", seq_id, ctypes.byref(new))
        return new.value

    def free(self, seq_id):
        self._call("pa_bm_free_sequence", seq_id)

    def info(self, seq_id):
        """Returns (num_tokens, num_blocks)."""
        n, b = ctypes.c_int32(), ctypes.c_int32()
        self._call("pa_bm_sequence_info", seq_id, ctypes.byref(n), ctypes.byref(b))
        return n.value, b.value

    def block_table(self, seq_id, max_blocks, pad_block=0):
        row = (ctypes.c_int32 * max(1, max_blocks))()
        self._call("pa_bm_block_table", seq_id, row, max_blocks, pad_block)
        return list(row)[:max_blocks]

    def slots(self, seq_id, first_pos, count):
        out = (ctypes.c_int32 * max(1, count))()
        self._call("pa_bm_slots", seq_id, first_pos, count, out)
        return list(out)[:count]

    def refcount(self, block):
        return int(self._lib.pa_bm_block_refcount(self._h, block))


def header_functions(header_dir=None):
    """Names of the functions the headers in include/ declare."""
    here = os.path.dirname(os.path.abspath(__file__))
    inc = header_dir or os.path.join(os.path.dirname(here), "include")
    names = set()
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, f)).read(), flags=re.S)
            names.update(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)
