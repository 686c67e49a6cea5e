"""Thin Python binding of libpkv (paged KV cache + paged decode attention for
MI355X / gfx950).

Argument marshalling only: every computation runs in the library's HIP
kernels or its host C++ block manager.  Torch tensors supply device memory
(``data_ptr``) and the stream (``torch.cuda.current_stream().cuda_stream``).
Importing this module fails if ``libpkv.so`` has not been built; there is no
fallback path.

The C declarations (include/pkv.h) document layouts, ownership and errors;
the names here are the same.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_436_amd/build.py` "
                      "(or __graft_entry__.build())")
# torch ships its own HIP runtime.  Load it first so that libpkv's dependency
# on libamdhip64.so.7 resolves to that same, already loaded runtime: two HIP
# runtimes in one process do not share devices, streams or allocations.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

PKV_OK, PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_HIP = 0, -1, -2, -3, -4
PKV_KV_BF16, PKV_KV_FP8_E5M2, PKV_KV_INT8, PKV_KV_INT8_TENSOR, PKV_KV_INT8_CHANNEL, PKV_KV_INT4 = 0, 1, 2, 3, 4, 5
PKV_KV_INT8_KCHANNEL_VTENSOR = 6
PKV_DECODE_KEEP_KV_CACHED = 1
PKV_PREFILL_P_ONE_PART = 1
ELEM_BYTES = {PKV_KV_BF16: 2, PKV_KV_FP8_E5M2: 1, PKV_KV_INT8: 1}


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pkv status {status}: {msg}")
        self.status = status


class OutOfBlocks(PkvError):
    pass


class PoolConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


class PoolDesc(ctypes.Structure):
    _fields_ = [("cfg", PoolConfig), ("base", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("tile_bytes", ctypes.c_uint64), ("layer_bytes", ctypes.c_uint64)]


class KVScales(ctypes.Structure):
    _fields_ = [("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("out", ctypes.c_void_p), ("q", ctypes.c_void_p), ("pool", ctypes.POINTER(PoolDesc)),
                ("layer", ctypes.c_int32), ("key", ctypes.c_void_p), ("value", ctypes.c_void_p),
                ("block_tables", ctypes.c_void_p), ("table_width", ctypes.c_int32),
                ("context_lens", ctypes.c_void_p), ("num_seqs", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
                ("kv_scales", ctypes.POINTER(KVScales)), ("partition_size", ctypes.c_int32),
                ("sliding_window", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_uint64), ("flags", ctypes.c_uint32)]


_P = ctypes.c_void_p
_I32, _I64, _U64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_U32 = ctypes.c_uint32
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)

# every symbol declared in include/pkv.h, with its C signature
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "kv_pool_bytes": (_U64, [ctypes.POINTER(PoolConfig)]),
    "kv_pool_num_blocks_for_budget": (_I64, [ctypes.POINTER(PoolConfig), _U64]),
    "kv_pool_create": (_I32, [ctypes.POINTER(PoolConfig), _P, _U64, ctypes.POINTER(PoolDesc)]),
    "reshape_and_cache": (_I32, [ctypes.POINTER(PoolDesc), _I32, _P, _P, _P, _I32,
                                 ctypes.POINTER(KVScales), _P]),
    "copy_blocks": (_I32, [ctypes.POINTER(PoolDesc), _P, _I32, _P]),
    "swap_blocks": (_I32, [ctypes.POINTER(PoolDesc), ctypes.POINTER(PoolDesc), _P, _I32, _P]),
    "paged_attn_workspace_bytes": (_U64, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_attn_decode": (_I32, [_P, _P, ctypes.POINTER(PoolDesc), _I32, _P, _I32, _P, _I32, _I32,
                                 _F, _I32, ctypes.POINTER(KVScales), _I32, _P, _U64, _P]),
    "paged_attn_decode_append": (_I32, [_P, _P, ctypes.POINTER(PoolDesc), _I32, _P, _P, _P, _I32, _P, _I32,
                                        _I32, _F, _I32, ctypes.POINTER(KVScales), _I32, _P, _U64, _P]),
    "paged_attn_decode_ex": (_I32, [ctypes.POINTER(DecodeArgs), _P]),
    "paged_attn_decode_noalloc": (_I32, [ctypes.POINTER(DecodeArgs), _P]),
    "paged_attn_decode_shared_prefix": (_I32, [ctypes.POINTER(DecodeArgs), _P, _I32, _P]),
    "paged_attn_shared_prefix_workspace_bytes": (_U64, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_attn_prefill": (_I32, [_P, _P, ctypes.POINTER(PoolDesc), _I32, _P, _I32, _P, _P, _I32, _I32, _I32,
                                  _I32, _F, _I32, ctypes.POINTER(KVScales), _P]),
    "paged_attn_prefill_ex": (_I32, [_P, _P, ctypes.POINTER(PoolDesc), _I32, _P, _I32, _P, _P, _I32, _I32, _I32,
                                     _I32, _F, _I32, ctypes.POINTER(KVScales), _U32, _P]),
    "pkv_check_slots": (_I32, [_I64P, _I32, _I64]),
    "pkv_check_pairs": (_I32, [_I64P, _I32, _I32]),
    "pkv_check_tables": (_I32, [_I32P, _I32P, _I32, _I32, _I32, _I32]),
    "kv_bm_create": (_I32, [_I32, _I32, _I32P, ctypes.POINTER(_P)]),
    "kv_bm_destroy": (None, [_P]),
    "kv_bm_add_seq": (_I32, [_P, _I32, _I32]),
    "kv_bm_fork": (_I32, [_P, _I32, _I32]),
    "kv_bm_append": (_I32, [_P, _I32P, _I32, _I64P, _I64P, _I32P]),
    "kv_bm_free_seq": (_I32, [_P, _I32]),
    "kv_bm_block_tables": (_I32, [_P, _I32P, _I32, _I32P, _I32, _I32P]),
    "kv_bm_stats": (_I32, [_P, _I32P, _I32P, _I64P]),
    "kv_bm_ref_count": (_I32, [_P, _I32]),
    "kv_bm_add_seq_tokens": (_I32, [_P, _I32, _I32P, _I32, _I32P]),
    "kv_bm_prefix_stats": (_I32, [_P, _I64P, _I64P, _I32P]),
    "kv_bm_block_key": (_I32, [_P, _I32P, _I32, _P]),
    "kv_bm_add_seq_radix": (_I32, [_P, _I32, _I32P, _I32, _I32P, _I64P]),
    "kv_bm_radix_stats": (_I32, [_P, _I64P, _I64P, _I32P, _I32P]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def last_error() -> str:
    return _lib.pkv_last_error().decode()


def _check(st: int):
    if st != PKV_OK:
        cls = OutOfBlocks if st == PKV_ERR_OUT_OF_BLOCKS else PkvError
        raise cls(st, last_error())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _np_ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ------------------------------------------------------------------- pool
def make_config(num_layers, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype=PKV_KV_BF16):
    return PoolConfig(num_layers, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype)


def kv_pool_bytes(cfg: PoolConfig) -> int:
    n = _lib.kv_pool_bytes(ctypes.byref(cfg))
    if n == 0:
        raise PkvError(PKV_ERR_INVALID, last_error())
    return int(n)


def kv_pool_num_blocks_for_budget(cfg: PoolConfig, budget_bytes: int) -> int:
    n = _lib.kv_pool_num_blocks_for_budget(ctypes.byref(cfg), int(budget_bytes))
    if n < 0:
        raise PkvError(PKV_ERR_INVALID, last_error())
    return int(n)


class Pool:
    """A pool descriptor plus the device buffer (a torch uint8 tensor) it
    describes.  ``memory`` may be given; otherwise it is allocated with torch
    on ``device``."""

    def __init__(self, cfg: PoolConfig, memory=None, device="cuda"):
        import torch
        nbytes = kv_pool_bytes(cfg)
        if memory is None:
            memory = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.memory = memory
        self.cfg = cfg
        self.desc = PoolDesc()
        _check(_lib.kv_pool_create(ctypes.byref(cfg), _ptr(memory), memory.numel() * memory.element_size(),
                                   ctypes.byref(self.desc)))

    @property
    def nbytes(self) -> int:
        return kv_pool_bytes(self.cfg)

    def region_offsets(self):
        base = self.desc.base
        ks = self.desc.k_scale - base if self.desc.k_scale else None
        vs = self.desc.v_scale - base if self.desc.v_scale else None
        return self.desc.k - base, self.desc.v - base, ks, vs


def reshape_and_cache(pool: Pool, layer: int, key, value, slot_mapping, k_scale: float = 1.0,
                      v_scale: float = 1.0, stream=None):
    sc = KVScales(k_scale, v_scale)
    n = int(slot_mapping.numel())
    _check(_lib.reshape_and_cache(ctypes.byref(pool.desc), layer, _ptr(key), _ptr(value), _ptr(slot_mapping),
                                  n, ctypes.byref(sc), _stream(stream)))


def copy_blocks(pool: Pool, pairs, stream=None):
    n = int(pairs.numel() // 2)
    _check(_lib.copy_blocks(ctypes.byref(pool.desc), _ptr(pairs), n, _stream(stream)))


def swap_blocks(src: Pool, dst: Pool, pairs, stream=None):
    """Copy block pairs[i][0] of ``src`` to block pairs[i][1] of ``dst`` in
    every layer (pairs: device int64 [n][2]); either pool may be in pinned
    host memory."""
    n = int(pairs.numel() // 2)
    _check(_lib.swap_blocks(ctypes.byref(src.desc), ctypes.byref(dst.desc), _ptr(pairs), n, _stream(stream)))


def paged_attn_workspace_bytes(num_seqs, num_q_heads, head_dim, table_width, block_size, partition_size) -> int:
    return int(_lib.paged_attn_workspace_bytes(num_seqs, num_q_heads, head_dim, table_width, block_size,
                                               partition_size))


def paged_attn_decode(out, q, pool: Pool, layer: int, block_tables, context_lens, scale: float,
                      kv_dtype: int | None = None, k_scale: float = 1.0, v_scale: float = 1.0,
                      partition_size: int = 0, workspace=None, stream=None):
    """out: fp32 [S, Hq, D]; q: bf16 [S, Hq, D]; block_tables: int32 [S, W];
    context_lens: int32 [S]; workspace: uint8 device tensor for the split form
    (partition_size > 0); its contents are scratch."""
    S, hq, _ = q.shape
    W = block_tables.shape[1]
    kvd = pool.cfg.kv_dtype if kv_dtype is None else kv_dtype
    sc = KVScales(k_scale, v_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.paged_attn_decode(_ptr(out), _ptr(q), ctypes.byref(pool.desc), layer, _ptr(block_tables), W,
                                  _ptr(context_lens), S, hq, float(scale), kvd, ctypes.byref(sc),
                                  partition_size, _ptr(workspace), ws_bytes, _stream(stream)))


def paged_attn_decode_append(out, q, pool: Pool, layer: int, key, value, block_tables, context_lens,
                             scale: float, kv_dtype: int | None = None, k_scale: float = 1.0,
                             v_scale: float = 1.0, partition_size: int = 0, workspace=None, stream=None):
    """Decode with the cache write in the same launch: key, value are bf16
    [S, Hkv, D], stored at position context_lens[s] - 1 of each sequence."""
    S, hq, _ = q.shape
    W = block_tables.shape[1]
    kvd = pool.cfg.kv_dtype if kv_dtype is None else kv_dtype
    sc = KVScales(k_scale, v_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.paged_attn_decode_append(_ptr(out), _ptr(q), ctypes.byref(pool.desc), layer, _ptr(key),
                                         _ptr(value), _ptr(block_tables), W, _ptr(context_lens), S, hq,
                                         float(scale), kvd, ctypes.byref(sc), partition_size, _ptr(workspace),
                                         ws_bytes, _stream(stream)))


def paged_attn_decode_ex(out, q, pool: Pool, layer: int, block_tables, context_lens, scale: float,
                        kv_dtype: int | None = None, k_scale: float = 1.0, v_scale: float = 1.0,
                        partition_size: int = 0, workspace=None, key=None, value=None, sliding_window: int = 0,
                        keep_kv_cached: bool = False, stream=None):
    """Decode with every option (see pkv.h): the appending form when key and
    value are given, attention restricted to the last ``sliding_window``
    positions when it is > 0, K/V loaded with the default cache policy
    instead of streamed when ``keep_kv_cached`` (tables that share blocks)."""
    S, hq, _ = q.shape
    sc = KVScales(k_scale, v_scale)
    a = DecodeArgs()
    a.out, a.q, a.pool, a.layer = _ptr(out), _ptr(q), ctypes.pointer(pool.desc), layer
    a.key, a.value = _ptr(key), _ptr(value)
    a.block_tables, a.table_width = _ptr(block_tables), block_tables.shape[1]
    a.context_lens, a.num_seqs, a.num_q_heads = _ptr(context_lens), S, hq
    a.scale = float(scale)
    a.kv_dtype = pool.cfg.kv_dtype if kv_dtype is None else kv_dtype
    a.kv_scales = ctypes.pointer(sc)
    a.partition_size, a.sliding_window = partition_size, sliding_window
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.flags = PKV_DECODE_KEEP_KV_CACHED if keep_kv_cached else 0
    _check(_lib.paged_attn_decode_ex(ctypes.byref(a), _stream(stream)))


def paged_attn_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, table_width,
                                             block_size, kv_dtype, prefix_len) -> int:
    return int(_lib.paged_attn_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                             table_width, block_size, kv_dtype, prefix_len))


def paged_attn_decode_shared_prefix(out, q, pool: Pool, layer: int, block_tables, context_lens, scale: float,
                                    prefix_table, prefix_len: int, kv_dtype: int | None = None,
                                    k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 512,
                                    workspace=None, key=None, value=None, keep_kv_cached: bool = False,
                                    stream=None):
    """Decode of sequences sharing a prompt prefix (see pkv.h): positions
    below prefix_len are read through prefix_table (int32 device tensor of
    prefix_len / B blocks) for every sequence, once per KV head."""
    S, hq, _ = q.shape
    sc = KVScales(k_scale, v_scale)
    a = DecodeArgs()
    a.out, a.q, a.pool, a.layer = _ptr(out), _ptr(q), ctypes.pointer(pool.desc), layer
    a.key, a.value = _ptr(key), _ptr(value)
    a.block_tables, a.table_width = _ptr(block_tables), block_tables.shape[1]
    a.context_lens, a.num_seqs, a.num_q_heads = _ptr(context_lens), S, hq
    a.scale = float(scale)
    a.kv_dtype = pool.cfg.kv_dtype if kv_dtype is None else kv_dtype
    a.kv_scales = ctypes.pointer(sc)
    a.partition_size, a.sliding_window = partition_size, 0
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.flags = PKV_DECODE_KEEP_KV_CACHED if keep_kv_cached else 0
    _check(_lib.paged_attn_decode_shared_prefix(ctypes.byref(a), _ptr(prefix_table), int(prefix_len),
                                                _stream(stream)))


def paged_attn_decode_noalloc(out, q, pool: Pool, layer: int, block_tables, context_lens, scale: float,
                              kv_dtype: int | None = None, k_scale: float = 1.0, v_scale: float = 1.0,
                              partition_size: int = 0, key=None, value=None, sliding_window: int = 0,
                              keep_kv_cached: bool = False, stream=None):
    """paged_attn_decode_ex without a workspace argument: the split form's
    scratch is the library's static device array (see pkv.h)."""
    S, hq, _ = q.shape
    sc = KVScales(k_scale, v_scale)
    a = DecodeArgs()
    a.out, a.q, a.pool, a.layer = _ptr(out), _ptr(q), ctypes.pointer(pool.desc), layer
    a.key, a.value = _ptr(key), _ptr(value)
    a.block_tables, a.table_width = _ptr(block_tables), block_tables.shape[1]
    a.context_lens, a.num_seqs, a.num_q_heads = _ptr(context_lens), S, hq
    a.scale = float(scale)
    a.kv_dtype = pool.cfg.kv_dtype if kv_dtype is None else kv_dtype
    a.kv_scales = ctypes.pointer(sc)
    a.partition_size, a.sliding_window = partition_size, sliding_window
    a.workspace, a.workspace_bytes = None, 0
    a.flags = PKV_DECODE_KEEP_KV_CACHED if keep_kv_cached else 0
    _check(_lib.paged_attn_decode_noalloc(ctypes.byref(a), _stream(stream)))


def paged_attn_prefill(out, q, pool: Pool, layer: int, block_tables, context_lens, query_start, scale: float,
                       max_query_len: int, kv_dtype: int | None = None, k_scale: float = 1.0,
                       v_scale: float = 1.0, p_one_part: bool = False, stream=None):
    """Causal attention of a chunk of new tokens per sequence over its cached
    context (see pkv.h): q, out are [T][Hq][D] (bf16, fp32); query_start is
    int32 [S + 1] on the device; max_query_len bounds every chunk.
    p_one_part: paged_attn_prefill_ex with PKV_PREFILL_P_ONE_PART."""
    T, hq, _ = q.shape
    S = context_lens.shape[0]
    sc = KVScales(k_scale, v_scale)
    kvd = pool.cfg.kv_dtype if kv_dtype is None else kv_dtype
    args = (_ptr(out), _ptr(q), ctypes.byref(pool.desc), layer, _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), _ptr(query_start), S, T, int(max_query_len), hq, float(scale), kvd,
            ctypes.byref(sc))
    if p_one_part:
        _check(_lib.paged_attn_prefill_ex(*args, PKV_PREFILL_P_ONE_PART, _stream(stream)))
    else:
        _check(_lib.paged_attn_prefill(*args, _stream(stream)))


# ------------------------------------------------------------------- checks
def check_slots(slots: np.ndarray, num_slots: int):
    a = np.ascontiguousarray(slots, dtype=np.int64)
    _check(_lib.pkv_check_slots(_np_ptr(a, ctypes.c_int64), a.size, int(num_slots)))


def check_pairs(pairs: np.ndarray, num_blocks: int):
    a = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    _check(_lib.pkv_check_pairs(_np_ptr(a, ctypes.c_int64), a.shape[0], int(num_blocks)))


def check_tables(tables: np.ndarray, context_lens: np.ndarray, block_size: int, num_blocks: int):
    t = np.ascontiguousarray(tables, dtype=np.int32)
    c = np.ascontiguousarray(context_lens, dtype=np.int32)
    _check(_lib.pkv_check_tables(_np_ptr(t, ctypes.c_int32), _np_ptr(c, ctypes.c_int32), t.shape[0],
                                 t.shape[1], int(block_size), int(num_blocks)))


# ------------------------------------------------------------------- block manager
def block_key(parent: bytes | None, tokens) -> bytes:
    """The library's prefix-cache key of a block (SHA-256, see pkv.h)."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = (ctypes.c_uint8 * 32)()
    par = None if parent is None else (ctypes.c_uint8 * 32).from_buffer_copy(parent)
    _check(_lib.kv_bm_block_key(par, _np_ptr(t, ctypes.c_int32), t.size, out))
    return bytes(out)


class BlockManager:
    """Host block manager (C++).  See pkv.h for its allocation rules."""

    def __init__(self, num_blocks: int, block_size: int, initial_order=None):
        self._h = ctypes.c_void_p()
        order = None
        if initial_order is not None:
            self._order = np.ascontiguousarray(initial_order, dtype=np.int32)
            order = _np_ptr(self._order, ctypes.c_int32)
        _check(_lib.kv_bm_create(num_blocks, block_size, order, ctypes.byref(self._h)))
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            _lib.kv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_seq(self, seq: int, ctx_len: int):
        _check(_lib.kv_bm_add_seq(self._h, seq, ctx_len))

    def fork(self, parent: int, child: int):
        _check(_lib.kv_bm_fork(self._h, parent, child))

    def append(self, seqs):
        """Returns (slots int64 [n], cow pairs int64 [k, 2])."""
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        slots = np.empty(s.size, dtype=np.int64)
        pairs = np.empty((max(s.size, 1), 2), dtype=np.int64)
        npairs = ctypes.c_int32(0)
        _check(_lib.kv_bm_append(self._h, _np_ptr(s, ctypes.c_int32), s.size, _np_ptr(slots, ctypes.c_int64),
                                 _np_ptr(pairs, ctypes.c_int64), ctypes.byref(npairs)))
        return slots, pairs[:npairs.value].copy()

    def free_seq(self, seq: int):
        _check(_lib.kv_bm_free_seq(self._h, seq))

    def block_tables(self, seqs, width: int, out: np.ndarray | None = None,
                     ctx_out: np.ndarray | None = None):
        """int32 [n, width] tables and int32 [n] lengths (into ``out`` /
        ``ctx_out`` when given, e.g. pinned host buffers viewed as numpy)."""
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        tab = out if out is not None else np.empty((s.size, width), dtype=np.int32)
        ctx = ctx_out if ctx_out is not None else np.empty(s.size, dtype=np.int32)
        assert tab.dtype == np.int32 and tab.flags.c_contiguous and tab.shape == (s.size, width)
        assert ctx.dtype == np.int32 and ctx.flags.c_contiguous and ctx.size == s.size
        _check(_lib.kv_bm_block_tables(self._h, _np_ptr(s, ctypes.c_int32), s.size,
                                       _np_ptr(tab, ctypes.c_int32), width, _np_ptr(ctx, ctypes.c_int32)))
        return tab, ctx

    def add_seq_tokens(self, seq: int, tokens) -> int:
        """New sequence holding the prompt ``tokens``, reusing cached prefix
        blocks; returns the number of leading tokens whose KV is already in
        the pool."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32(0)
        _check(_lib.kv_bm_add_seq_tokens(self._h, seq, _np_ptr(t, ctypes.c_int32), t.size, ctypes.byref(cached)))
        return cached.value

    def add_seq_radix(self, seq: int, tokens):
        """New sequence holding the prompt ``tokens``, reusing its longest
        prefix found in the radix tree; returns (cached tokens, copy pair
        (src, dst) to copy before computing the rest, or None)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32(0)
        pair = np.full(2, -1, dtype=np.int64)
        _check(_lib.kv_bm_add_seq_radix(self._h, seq, _np_ptr(t, ctypes.c_int32), t.size, ctypes.byref(cached),
                                        _np_ptr(pair, ctypes.c_int64)))
        return cached.value, (None if pair[0] < 0 else (int(pair[0]), int(pair[1])))

    def radix_stats(self):
        """(lookup tokens, hit tokens, blocks in the tree, of them unreferenced)."""
        lk, hit, nodes, idle = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.kv_bm_radix_stats(self._h, ctypes.byref(lk), ctypes.byref(hit), ctypes.byref(nodes),
                                      ctypes.byref(idle)))
        return lk.value, hit.value, nodes.value, idle.value

    def prefix_stats(self):
        """(full-block lookups, hits, cached keys)."""
        lk, hit, cached = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(_lib.kv_bm_prefix_stats(self._h, ctypes.byref(lk), ctypes.byref(hit), ctypes.byref(cached)))
        return lk.value, hit.value, cached.value

    def stats(self):
        used, total, failed = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
        _check(_lib.kv_bm_stats(self._h, ctypes.byref(used), ctypes.byref(total), ctypes.byref(failed)))
        return used.value, total.value, failed.value

    def ref_count(self, block: int) -> int:
        return int(_lib.kv_bm_ref_count(self._h, block))
