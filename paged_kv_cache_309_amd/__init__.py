"""Paged decode attention for AMD MI355X (gfx950).

Python binding of libpkv.so.  The functions below take torch tensors that
live on the GPU, turn them into raw pointers, sizes and the current HIP
stream, and call the C ABI (include/pkv.h).  They do no arithmetic: every
step runs in the HIP kernels, and an error status raises PkvError.

Cache tensors (allocate them with new_kv_cache):
    k_cache  [num_blocks, num_kv_heads, block_size, head_dim]
    v_cache  [num_blocks, num_kv_heads, block_size // 4, head_dim, 4]
Caches of dtype torch.float8_e4m3fn hold 8-bit E4M3 codes with one scale per
pool (k_scale, v_scale); the calls then route to the *_fp8 entry points.
Host pools for swapped-out blocks (new_kv_cache(..., device="cpu",
pin_memory=True)) have the same layouts in pinned host memory.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import STATIC_SCRATCH_BYTES, PkvDims, PkvError, PkvPrefixInfo

__all__ = ["reshape_and_cache", "paged_attention_decode",
           "paged_attention_decode_split", "split_workspace_bytes",
           "paged_attention_decode_split_static", "STATIC_SCRATCH_BYTES",
           "PrefixPlan", "paged_attention_decode_shared_prefix",
           "shared_prefix_workspace_bytes",
           "paged_attention_prefill", "new_kv_cache", "copy_blocks",
           "swap_blocks", "BlockManager", "PkvError", "version"]

_DTYPES = {torch.float32: _lib.PKV_F32, torch.float16: _lib.PKV_F16,
           torch.bfloat16: _lib.PKV_BF16}


def version() -> int:
    return _lib.lib().pkv_version()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t: torch.Tensor) -> int:
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpkv must be contiguous")
    return t.data_ptr()


def _on_one_device(*tensors: torch.Tensor, stream=None) -> None:
    """The kernels dereference these pointers on the GPU: every tensor must
    be a CUDA tensor, all on one device, the device the launch goes to (the
    given stream's, else the current one)."""
    for t in tensors:
        if not t.is_cuda:
            raise ValueError(f"libpkv needs CUDA tensors; got one on {t.device}")
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError(f"libpkv needs all tensors on one device; got {dev} and {t.device}")
    launch = stream.device if stream is not None else \
        torch.device("cuda", torch.cuda.current_device())
    if dev != launch:
        raise ValueError(f"tensors are on {dev} but the launch goes to {launch}")


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def new_kv_cache(num_blocks: int, num_kv_heads: int, block_size: int,
                 head_dim: int, dtype: torch.dtype, device="cuda",
                 fill: float | None = None, pin_memory: bool = False):
    """Allocate (k_cache, v_cache) in the library's block layouts (on the
    host with pin_memory=True: a pool that swap_blocks can reach)."""
    k = torch.empty((num_blocks, num_kv_heads, block_size, head_dim),
                    dtype=dtype, device=device, pin_memory=pin_memory)
    v = torch.empty((num_blocks, num_kv_heads, block_size // 4, head_dim, 4),
                    dtype=dtype, device=device, pin_memory=pin_memory)
    if fill is not None:
        k.fill_(fill)
        v.fill_(fill)
    return k, v


def _is_fp8(cache: torch.Tensor) -> bool:
    return cache.dtype == torch.float8_e4m3fn


# Shape and dtype checks.  The C ABI sizes its checks and the kernels address
# memory from the dims struct alone, so every tensor is checked against
# those dims here, before any launch: a mismatch raises ValueError.
def _expect(t, name: str, shape=None, dtypes=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtypes is not None and t.dtype not in dtypes:
        want = ", ".join(str(d) for d in dtypes)
        raise ValueError(f"{name} has dtype {t.dtype}; expected {want}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")


def _rank(t, name: str, n: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _pools(k_cache, v_cache, elem_dtype, head_dim=None, num_kv_heads=None):
    """Checks a (k_cache, v_cache) pair against the block layouts and the
    element type of the values it caches (or E4M3); returns (NB, Hkv, bs,
    D)."""
    _rank(k_cache, "k_cache", 4)
    NB, Hkv, bs, D = k_cache.shape
    _expect(k_cache, "k_cache", dtypes=(elem_dtype, torch.float8_e4m3fn))
    if head_dim is not None and D != head_dim:
        raise ValueError(f"k_cache has head_dim {D}; the queries/values have {head_dim}")
    if num_kv_heads is not None and Hkv != num_kv_heads:
        raise ValueError(f"k_cache has {Hkv} KV heads; the new keys have {num_kv_heads}")
    if bs % 4:
        raise ValueError(f"block size {bs} is not a multiple of 4")
    _expect(v_cache, "v_cache", shape=(NB, Hkv, bs // 4, D, 4), dtypes=(k_cache.dtype,))
    return NB, Hkv, bs, D


def _block_size(block_size, bs: int) -> int:
    if block_size is not None and int(block_size) != bs:
        raise ValueError(f"block_size {block_size} differs from the cache's {bs}")
    return bs


def _decode_shapes(out, q, k_cache, v_cache, block_tables, context_lens,
                   block_size) -> tuple:
    """Checks the tensors of a decode call; returns (dims, block size)."""
    _rank(q, "q", 3)
    _expect(q, "q", dtypes=tuple(_DTYPES))
    S, Hq, D = q.shape
    _expect(out, "out", shape=(S, Hq, D), dtypes=(q.dtype,))
    NB, Hkv, bs, _ = _pools(k_cache, v_cache, q.dtype, head_dim=D)
    bs = _block_size(block_size, bs)
    _rank(block_tables, "block_tables", 2)
    _expect(block_tables, "block_tables", shape=(S, block_tables.shape[1]),
            dtypes=(torch.int32,))
    _expect(context_lens, "context_lens", shape=(S,), dtypes=(torch.int32,))
    return PkvDims(S, Hq, Hkv, D, NB, block_tables.shape[1], _dtype(q)), bs


def _dims(q: torch.Tensor, k_cache: torch.Tensor,
          block_tables: torch.Tensor) -> PkvDims:
    S, Hq, D = q.shape
    NB, Hkv = k_cache.shape[0], k_cache.shape[1]
    return PkvDims(S, Hq, Hkv, D, NB, block_tables.shape[1], _dtype(q))


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor,
                      slot_mapping: torch.Tensor, stream=None,
                      k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write k[i], v[i] ([T, Hkv, D]) into slot slot_mapping[i] (int64);
    8-bit caches store the E4M3 value nearest to x / scale."""
    _rank(k, "k", 3)
    _expect(k, "k", dtypes=tuple(_DTYPES))
    T, Hkv, D = k.shape
    _expect(v, "v", shape=(T, Hkv, D), dtypes=(k.dtype,))
    NB, _, bs, _ = _pools(k_cache, v_cache, k.dtype, head_dim=D, num_kv_heads=Hkv)
    _expect(slot_mapping, "slot_mapping", shape=(T,), dtypes=(torch.int64,))
    _on_one_device(k, v, k_cache, v_cache, slot_mapping, stream=stream)
    dims = PkvDims(0, Hkv, Hkv, D, NB, 0, _dtype(k))
    if _is_fp8(k_cache):
        _lib.check(_lib.lib().reshape_and_cache_fp8(
            _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
            T, bs, float(k_scale), float(v_scale), ctypes.byref(dims),
            _stream(stream)))
        return
    _lib.check(_lib.lib().reshape_and_cache(
        _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
        T, bs, ctypes.byref(dims), _stream(stream)))


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor,
                           k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float,
                           block_size: int | None = None,
                           stream=None, k_scale: float = 1.0,
                           v_scale: float = 1.0) -> torch.Tensor:
    """out[s, h] = softmax(scale * q[s, h] . K) V over context_lens[s]
    tokens reached through block_tables[s]; single launch."""
    dims, bs = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                              context_lens, block_size)
    _on_one_device(out, q, k_cache, v_cache, block_tables, context_lens, stream=stream)
    if _is_fp8(k_cache):
        _lib.check(_lib.lib().paged_attention_decode_fp8(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), _ptr(context_lens), float(scale), bs,
            float(k_scale), float(v_scale), ctypes.byref(dims),
            _stream(stream)))
        return out
    _lib.check(_lib.lib().paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), bs, ctypes.byref(dims),
        _stream(stream)))
    return out


def split_workspace_bytes(q: torch.Tensor, k_cache: torch.Tensor,
                          block_tables: torch.Tensor, partition_size: int,
                          block_size: int | None = None) -> int:
    _rank(q, "q", 3)
    _rank(k_cache, "k_cache", 4)
    _rank(block_tables, "block_tables", 2)
    bs = _block_size(block_size, k_cache.shape[2])
    dims = _dims(q, k_cache, block_tables)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.lib().paged_attention_split_workspace_bytes(
        ctypes.byref(dims), bs, partition_size, ctypes.byref(n)))
    return n.value


def paged_attention_decode_split(out: torch.Tensor, q: torch.Tensor,
                                 k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 block_tables: torch.Tensor,
                                 context_lens: torch.Tensor, scale: float,
                                 partition_size: int,
                                 workspace: torch.Tensor,
                                 block_size: int | None = None,
                                 stream=None, k_scale: float = 1.0,
                                 v_scale: float = 1.0) -> torch.Tensor:
    """Same result as paged_attention_decode, in two launches: per-partition
    partials into `workspace` (a device byte tensor of at least
    split_workspace_bytes(...)), then the partition reduce."""
    dims, bs = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                              context_lens, block_size)
    _expect(workspace, "workspace")
    _on_one_device(out, q, k_cache, v_cache, block_tables, context_lens, workspace,
                   stream=stream)
    if _is_fp8(k_cache):
        _lib.check(_lib.lib().paged_attention_decode_split_fp8(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), _ptr(context_lens), float(scale), bs,
            int(partition_size), _ptr(workspace),
            workspace.numel() * workspace.element_size(), float(k_scale),
            float(v_scale), ctypes.byref(dims), _stream(stream)))
        return out
    _lib.check(_lib.lib().paged_attention_decode_split(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), bs, int(partition_size),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(dims), _stream(stream)))
    return out


def paged_attention_decode_split_static(out: torch.Tensor, q: torch.Tensor,
                                        k_cache: torch.Tensor,
                                        v_cache: torch.Tensor,
                                        block_tables: torch.Tensor,
                                        context_lens: torch.Tensor,
                                        scale: float, partition_size: int,
                                        block_size: int | None = None,
                                        stream=None) -> torch.Tensor:
    """paged_attention_decode_split without a workspace: the partials go to
    the library's static per-device scratch (STATIC_SCRATCH_BYTES), so the
    call allocates nothing.  Calls that overlap in time on one device race
    on that scratch.  16-bit and fp32 caches."""
    dims, bs = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                              context_lens, block_size)
    if _is_fp8(k_cache):
        raise ValueError("paged_attention_decode_split_static takes 16-bit "
                         "or fp32 caches only")
    _on_one_device(out, q, k_cache, v_cache, block_tables, context_lens, stream=stream)
    _lib.check(_lib.lib().paged_attention_decode_split_static(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), bs, int(partition_size),
        ctypes.byref(dims), _stream(stream)))
    return out


class PrefixPlan:
    """The sets of sequences that share leading blocks, found on the host by
    pkv_prefix_plan from host copies of the block tables and context
    lengths, with the plan array copied to `device` (the current GPU by
    default).  `info` holds its sizes; `host` the array itself."""

    def __init__(self, block_tables, context_lens, block_size: int,
                 min_sharers: int = 2, device=None):
        import numpy as np
        bt = np.ascontiguousarray(
            block_tables.cpu().numpy() if isinstance(block_tables, torch.Tensor)
            else block_tables, dtype=np.int32)
        cl = np.ascontiguousarray(
            context_lens.cpu().numpy() if isinstance(context_lens, torch.Tensor)
            else context_lens, dtype=np.int32)
        if bt.ndim != 2 or cl.shape != (bt.shape[0],):
            raise ValueError(f"block_tables {bt.shape} and context_lens {cl.shape} "
                             "do not describe the same sequences")
        S, MB = bt.shape
        plan = np.empty(4 * S + 1, np.int32)
        self.info = PkvPrefixInfo()
        _lib.check(_lib.lib().pkv_prefix_plan(
            bt.ctypes.data, cl.ctypes.data, S, MB, int(block_size),
            int(min_sharers), plan.ctypes.data, plan.size, ctypes.byref(self.info)))
        i = self.info
        self.host = plan[:S + 2 * i.num_groups + 1 + i.num_members].copy()
        self.block_size = int(block_size)
        dev = device if device is not None else \
            torch.device("cuda", torch.cuda.current_device())
        self.device = torch.from_numpy(self.host).to(dev)

    @property
    def seq_prefix(self):
        return self.host[:self.info.num_seqs]


def shared_prefix_workspace_bytes(q: torch.Tensor, k_cache: torch.Tensor,
                                  block_tables: torch.Tensor, plan: PrefixPlan,
                                  block_size: int | None = None) -> int:
    _rank(q, "q", 3)
    _rank(k_cache, "k_cache", 4)
    _rank(block_tables, "block_tables", 2)
    bs = _block_size(block_size, k_cache.shape[2])
    dims = _dims(q, k_cache, block_tables)
    n = ctypes.c_size_t(0)
    _lib.check(_lib.lib().paged_attention_shared_prefix_workspace_bytes(
        ctypes.byref(dims), bs, ctypes.byref(plan.info), ctypes.byref(n)))
    return n.value


def paged_attention_decode_shared_prefix(out: torch.Tensor, q: torch.Tensor,
                                         k_cache: torch.Tensor,
                                         v_cache: torch.Tensor,
                                         block_tables: torch.Tensor,
                                         context_lens: torch.Tensor,
                                         scale: float, plan: PrefixPlan,
                                         workspace: torch.Tensor,
                                         block_size: int | None = None,
                                         stream=None) -> torch.Tensor:
    """paged_attention_decode with every sharer set's common prefix computed
    once for all its members (fp16/bf16): `plan` comes from PrefixPlan over
    the same tables and lengths; `workspace` is a device byte tensor of at
    least shared_prefix_workspace_bytes(...)."""
    dims, bs = _decode_shapes(out, q, k_cache, v_cache, block_tables,
                              context_lens, block_size)
    if _is_fp8(k_cache):
        raise ValueError("paged_attention_decode_shared_prefix takes 16-bit caches")
    if not isinstance(plan, PrefixPlan):
        raise ValueError("plan must be a PrefixPlan")
    if plan.block_size != bs or plan.info.num_seqs != q.shape[0]:
        raise ValueError("the plan was built for another batch or block size")
    _expect(workspace, "workspace")
    _on_one_device(out, q, k_cache, v_cache, block_tables, context_lens,
                   plan.device, workspace, stream=stream)
    _lib.check(_lib.lib().paged_attention_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), bs, _ptr(plan.device),
        ctypes.byref(plan.info), _ptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(dims),
        _stream(stream)))
    return out


def paged_attention_prefill(out: torch.Tensor, q: torch.Tensor,
                            k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor,
                            context_lens: torch.Tensor,
                            query_start_loc: torch.Tensor, scale: float,
                            max_query_len: int | None = None,
                            block_size: int | None = None,
                            stream=None, k_scale: float = 1.0,
                            v_scale: float = 1.0) -> torch.Tensor:
    """Chunked prefill: q / out [T, Hq, D] hold the chunk tokens of every
    sequence (rows query_start_loc[s] .. query_start_loc[s+1]-1, the last
    tokens of its context, whose K/V are already in the cache); each
    attends causally.  max_query_len bounds every chunk (default T)."""
    _rank(q, "q", 3)
    _expect(q, "q", dtypes=tuple(_DTYPES))
    T, Hq, D = q.shape
    _expect(out, "out", shape=(T, Hq, D), dtypes=(q.dtype,))
    NB, Hkv, bs, _ = _pools(k_cache, v_cache, q.dtype, head_dim=D)
    bs = _block_size(block_size, bs)
    _rank(context_lens, "context_lens", 1)
    _expect(context_lens, "context_lens", dtypes=(torch.int32,))
    S = context_lens.shape[0]
    _rank(block_tables, "block_tables", 2)
    _expect(block_tables, "block_tables", shape=(S, block_tables.shape[1]),
            dtypes=(torch.int32,))
    _expect(query_start_loc, "query_start_loc", shape=(S + 1,), dtypes=(torch.int32,))
    _on_one_device(out, q, k_cache, v_cache, block_tables, context_lens,
                   query_start_loc, stream=stream)
    dims = PkvDims(S, Hq, Hkv, D, NB, block_tables.shape[1], _dtype(q))
    mq = T if max_query_len is None else int(max_query_len)
    if _is_fp8(k_cache):
        _lib.check(_lib.lib().paged_attention_prefill_fp8(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), _ptr(context_lens), _ptr(query_start_loc),
            float(scale), bs, T, mq, float(k_scale), float(v_scale),
            ctypes.byref(dims), _stream(stream)))
        return out
    _lib.check(_lib.lib().paged_attention_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start_loc), float(scale), bs, T, mq,
        ctypes.byref(dims), _stream(stream)))
    return out


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_mapping: torch.Tensor, stream=None) -> None:
    """Copy-on-write: block block_mapping[i, 1] of both caches becomes a
    copy of block block_mapping[i, 0] (device int64 [n, 2])."""
    _rank(k_cache, "k_cache", 4)
    if k_cache.dtype not in _DTYPES and not _is_fp8(k_cache):
        raise ValueError(f"k_cache has unsupported dtype {k_cache.dtype}")
    NB, Hkv, bs, D = _pools(k_cache, v_cache, k_cache.dtype)
    _rank(block_mapping, "block_mapping", 2)
    _expect(block_mapping, "block_mapping", shape=(block_mapping.shape[0], 2),
            dtypes=(torch.int64,))
    _on_one_device(k_cache, v_cache, *([block_mapping] if block_mapping.numel() else []),
                   stream=stream)
    dt = _lib.PKV_E4M3 if _is_fp8(k_cache) else _dtype(k_cache)
    dims = PkvDims(0, Hkv, Hkv, D, NB, 0, dt)
    n = block_mapping.shape[0] if block_mapping.numel() else 0
    _lib.check(_lib.lib().copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_mapping) if n else None, n,
        bs, ctypes.byref(dims), _stream(stream)))


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor,
                dst_k: torch.Tensor, dst_v: torch.Tensor,
                block_mapping: torch.Tensor, stream=None) -> None:
    """Block block_mapping[i, 1] of (dst_k, dst_v) becomes a copy of block
    block_mapping[i, 0] of (src_k, src_v); each pool is on the GPU or in
    pinned host memory, and the mapping (int64 [n, 2]) on the GPU or pinned.
    Asynchronous: synchronise the stream before reading a host pool."""
    _rank(src_k, "src_k", 4)
    if src_k.dtype not in _DTYPES and not _is_fp8(src_k):
        raise ValueError(f"src_k has unsupported dtype {src_k.dtype}")
    NB, Hkv, bs, D = _pools(src_k, src_v, src_k.dtype)
    _rank(dst_k, "dst_k", 4)
    if src_k.dtype != dst_k.dtype or src_k.shape[1:] != dst_k.shape[1:]:
        raise ValueError("source and destination pools differ in shape")
    _pools(dst_k, dst_v, dst_k.dtype)
    _rank(block_mapping, "block_mapping", 2)
    _expect(block_mapping, "block_mapping", shape=(block_mapping.shape[0], 2),
            dtypes=(torch.int64,))
    dt = _lib.PKV_E4M3 if _is_fp8(src_k) else _dtype(src_k)
    dims = PkvDims(0, Hkv, Hkv, D, 0, 0, dt)
    n = block_mapping.shape[0] if block_mapping.numel() else 0
    _lib.check(_lib.lib().swap_blocks(
        _ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v),
        _ptr(block_mapping) if n else None, n, NB, dst_k.shape[0], bs,
        ctypes.byref(dims), _stream(stream)))


class BlockManager:
    """Host block manager of the paged cache (free list, reference counts,
    block tables, copy-on-write, swapping to a host pool), a thin wrapper of
    the pkv_bm_* calls."""

    def __init__(self, num_blocks: int, block_size: int,
                 num_host_blocks: int = 0):
        import numpy as np
        self._np = np
        self._h = ctypes.c_void_p()
        _lib.check(_lib.lib().pkv_bm_create_with_host(
            num_blocks, num_host_blocks, block_size, ctypes.byref(self._h)))
        self.num_blocks = num_blocks
        self.num_host_blocks = num_host_blocks
        self.block_size = block_size

    def close(self) -> None:
        if self._h:
            _lib.lib().pkv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq_id: int, num_tokens: int):
        """Register a prompt of num_tokens; returns every token's slot."""
        slots = self._np.empty(max(num_tokens, 1), self._np.int64)
        _lib.check(_lib.lib().pkv_bm_add_sequence(
            self._h, seq_id, num_tokens, slots.ctypes.data))
        return slots[:num_tokens]

    def fork(self, parent: int, child: int) -> None:
        _lib.check(_lib.lib().pkv_bm_fork(self._h, parent, child))

    def append_tokens(self, seq_ids):
        """One new token per listed sequence: returns (slots [n] int64,
        copy pairs [k, 2] int64 to run through copy_blocks first)."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        slots = np.empty(max(n, 1), np.int64)
        pairs = np.empty((max(n, 1), 2), np.int64)
        k = ctypes.c_int32(0)
        _lib.check(_lib.lib().pkv_bm_append_tokens(
            self._h, ids.ctypes.data, n, slots.ctypes.data, pairs.ctypes.data,
            ctypes.byref(k)))
        return slots[:n], pairs[:k.value]

    def free_sequence(self, seq_id: int) -> None:
        _lib.check(_lib.lib().pkv_bm_free_sequence(self._h, seq_id))

    def batch_tables(self, seq_ids, max_blocks: int):
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        tables = np.empty((max(n, 1), max(max_blocks, 1)), np.int32)
        lens = np.empty(max(n, 1), np.int32)
        _lib.check(_lib.lib().pkv_bm_batch_tables(
            self._h, ids.ctypes.data, n, max_blocks, tables.ctypes.data,
            lens.ctypes.data))
        return tables[:n, :max_blocks], lens[:n]

    def num_free_blocks(self) -> int:
        return _lib.lib().pkv_bm_num_free_blocks(self._h)

    def refcount(self, block: int) -> int:
        return _lib.lib().pkv_bm_refcount(self._h, block)

    def num_tokens(self, seq_id: int) -> int:
        return _lib.lib().pkv_bm_num_tokens(self._h, seq_id)

    def _move(self, fn, seq_ids):
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        cap = max(self.num_blocks, self.num_host_blocks, 1)
        pairs = np.empty((cap, 2), np.int64)
        k = ctypes.c_int32(0)
        _lib.check(fn(self._h, ids.ctypes.data, ids.shape[0],
                      pairs.ctypes.data, cap, ctypes.byref(k)))
        return pairs[:k.value]

    def swap_out(self, seq_ids):
        """Move the sequences to the host pool: returns the (device block,
        host block) pairs [k, 2] to copy with swap_blocks."""
        return self._move(_lib.lib().pkv_bm_swap_out, seq_ids)

    def swap_in(self, seq_ids):
        """Bring swapped-out sequences back: (host block, device block)
        pairs [k, 2] to copy with swap_blocks."""
        return self._move(_lib.lib().pkv_bm_swap_in, seq_ids)

    def num_free_host_blocks(self) -> int:
        return _lib.lib().pkv_bm_num_free_host_blocks(self._h)

    def host_refcount(self, block: int) -> int:
        return _lib.lib().pkv_bm_host_refcount(self._h, block)

    def is_swapped(self, seq_id: int) -> int:
        return _lib.lib().pkv_bm_is_swapped(self._h, seq_id)

    def block_table(self, seq_id: int):
        np = self._np
        cap = max(self.num_blocks, self.num_host_blocks, 1)
        t = np.empty(cap, np.int32)
        k = ctypes.c_int32(0)
        _lib.check(_lib.lib().pkv_bm_block_table(
            self._h, seq_id, t.ctypes.data, cap, ctypes.byref(k)))
        return t[:k.value]


# load (and fail loudly) at import
_lib.lib()
