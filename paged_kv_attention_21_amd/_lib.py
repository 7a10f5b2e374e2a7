"""ctypes binding of libpka.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks
dtype / device / contiguity / shape agreement, and passes raw pointers, sizes
and the current HIP stream to the C ABI declared in include/pka.h.  All work
runs in the library's HIP kernels; nothing here computes attention.  If the
library is missing, importing this module raises ImportError.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

# PKA_LIBRARY may point at another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("PKA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpka.so")
PARTITION_SIZE = 256

c_int32 = ctypes.c_int32
c_float = ctypes.c_float
c_size_t = ctypes.c_size_t
c_void_p = ctypes.c_void_p

_DTYPES = {torch.float16: 0, torch.bfloat16: 1}

STATUS = {
    0: "PKA_OK",
    1: "PKA_ERR_NULL",
    2: "PKA_ERR_SHAPE",
    3: "PKA_ERR_UNSUPPORTED",
    4: "PKA_ERR_ALIGN",
    5: "PKA_ERR_WORKSPACE",
    6: "PKA_ERR_HIP",
    7: "PKA_ERR_SCRATCH",
}


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", c_int32),
        ("block_size", c_int32),
        ("num_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("dtype", c_int32),
    ]


class PkaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


# Exported symbols: name -> (restype, argtypes)
_SIGNATURES = {
    "pka_status_str": (ctypes.c_char_p, [c_int32]),
    "pka_version": (c_int32, []),
    "pka_device_cu_count": (c_int32, []),
    "pka_kv_cache_write": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, CacheDesc, c_void_p]),
    "pka_paged_attn_decode_v1": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float, c_void_p,
         CacheDesc, c_void_p],
    ),
    "pka_paged_attn_decode_splitk": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float, c_int32, c_int32,
         c_void_p, c_void_p, c_void_p, CacheDesc, c_void_p],
    ),
    "pka_paged_attn_splitk_reduce": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32,
         c_void_p],
    ),
    "pka_splitk_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "pka_decode_choose_variant": (c_int32, [c_int32, c_int32, c_int32, c_int32]),
    "pka_paged_attn_decode": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_float, c_void_p,
         CacheDesc, c_void_p, c_size_t, c_void_p],
    ),
    "pka_paged_attn_decode_append": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
         c_float, c_void_p, CacheDesc, c_void_p, c_size_t, c_void_p],
    ),
    "pka_paged_attn_decode_noalloc": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_float, c_void_p,
         CacheDesc, c_void_p],
    ),
    "pka_paged_attn_prefill": (
        c_int32,
        [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
         c_int32, c_float, c_void_p, CacheDesc, c_void_p, c_size_t, c_void_p],
    ),
    "pka_prefill_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "pka_prefill_split_keys": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "pka_rope_table": (c_int32, [c_void_p, c_int32, c_int32, ctypes.c_double, c_void_p]),
    "pka_rope_table_bytes": (c_size_t, [c_int32, c_int32]),
    "pka_bm_create": (c_void_p, [c_int32, c_int32]),
    "pka_bm_destroy": (None, [c_void_p]),
    "pka_bm_num_free": (c_int32, [c_void_p]),
    "pka_bm_refcount": (c_int32, [c_void_p, c_int32]),
    "pka_bm_add_request": (c_int32, [c_void_p, ctypes.c_int64, c_void_p, c_int32]),
    "pka_bm_append_token": (c_int32, [c_void_p, ctypes.c_int64, c_int32]),
    "pka_bm_find_cached_prefix": (c_int32, [c_void_p, ctypes.c_int64, c_void_p, c_int32]),
    "pka_bm_admit": (c_int32, [c_void_p, ctypes.c_int64, c_int32, ctypes.POINTER(c_int32)]),
    "pka_bm_allocate": (c_int32, [c_void_p, ctypes.c_int64, c_int32]),
    "pka_bm_commit": (c_int32, [c_void_p, ctypes.c_int64, c_int32]),
    "pka_bm_free_request": (c_int32, [c_void_p, ctypes.c_int64, c_int32]),
    "pka_bm_block_table": (c_int32, [c_void_p, ctypes.c_int64, c_void_p, c_int32]),
    "pka_bm_slot_mapping": (c_int32, [c_void_p, ctypes.c_int64, c_int32, c_int32, c_void_p]),
    "pka_bm_num_computed": (c_int32, [c_void_p, ctypes.c_int64]),
    "pka_bm_decode_step": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "pka_fused_rope_kv_write": (
        c_int32,
        [c_void_p, ctypes.c_int64, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p,
         c_void_p, CacheDesc, c_void_p],
    ),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python paged_kv_attention_21_amd/build.py` "
            "(the library has no CPU fallback)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------


def _check(status: int):
    if status != 0:
        raise PkaError(status, lib.pka_status_str(status).decode())


class Prepared:
    """A library call whose arguments were checked and marshalled once.
    Calling it launches the same kernels again on the stream captured at
    preparation, with one ctypes call (what a serving loop or a timing loop
    wants).  The tensors it refers to are kept alive with it."""

    __slots__ = ("fn", "args", "keep", "result")

    def __init__(self, fn, args, keep, result=None):
        self.fn, self.args, self.keep, self.result = fn, args, keep, result

    def __call__(self):
        _check(self.fn(*self.args))
        return self.result


def _launch(fn, args, prepare, keep, result=None):
    if prepare:
        return Prepared(fn, tuple(args), keep, result)
    _check(fn(*args))
    return result


def _ptr(t: torch.Tensor | None):
    return c_void_p(t.data_ptr()) if t is not None else c_void_p(0)


def _stream(t: torch.Tensor):
    return c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _require(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    if k_cache.dtype not in _DTYPES:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    nb, bs, hkv, d = k_cache.shape
    return CacheDesc(nb, bs, hkv, d, _DTYPES[k_cache.dtype])


def _check_pool(k_cache, v_cache):
    _require(k_cache, "k_cache", ndim=4)
    _require(v_cache, "v_cache", dtype=k_cache.dtype, ndim=4, device=k_cache.device)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")


def _check_tables(block_tables, context_lens, num_seqs, device):
    _require(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=device)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=device)
    if block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs:
        raise ValueError("block_tables / context_lens do not have one row per sequence")


# ---------------------------------------------------------------------------
# operations (same names as the C ABI, without the pka_ prefix)
# ---------------------------------------------------------------------------


def version() -> int:
    return lib.pka_version()


def device_cu_count() -> int:
    n = lib.pka_device_cu_count()
    if n <= 0:
        raise PkaError(6, "could not query the CU count")
    return n


def kv_cache_write(key, value, slot_mapping, k_cache, v_cache, prepare=False):
    """Scatter key/value [T, Hkv, D] into the pool at slot_mapping (int64 [T];
    negative = skip).  Bit-exact byte copy."""
    _check_pool(k_cache, v_cache)
    dev = k_cache.device
    _require(key, "key", dtype=k_cache.dtype, ndim=3, device=dev)
    _require(value, "value", dtype=k_cache.dtype, ndim=3, device=dev)
    _require(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1, device=dev)
    T = key.shape[0]
    if value.shape != key.shape or slot_mapping.shape[0] != T or key.shape[1:] != k_cache.shape[2:]:
        raise ValueError("key/value/slot_mapping shapes disagree with each other or the pool")
    return _launch(lib.pka_kv_cache_write,
                   (_ptr(key), _ptr(value), _ptr(slot_mapping), T, _ptr(k_cache), _ptr(v_cache), cache_desc(k_cache),
                    _stream(k_cache)), prepare, (key, value, slot_mapping, k_cache, v_cache))


class BlockManager:
    """Host paged block manager (the library's C++ one): refcounted pages, an
    LRU free list and a whole-block prefix cache; produces the block tables
    and slot mappings the kernels take.  Token ids and outputs are numpy
    int32 / int64 arrays (host memory)."""

    def __init__(self, num_blocks: int, block_size: int):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self._h = lib.pka_bm_create(self.num_blocks, self.block_size)
        if not self._h:
            raise ValueError("bad block-manager sizes")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib.pka_bm_destroy(h)
            self._h = None

    @staticmethod
    def _neg(ret):
        if ret < 0:
            _check(-ret)
        return ret

    def num_free(self) -> int:
        return lib.pka_bm_num_free(self._h)

    def refcount(self, block: int) -> int:
        return lib.pka_bm_refcount(self._h, int(block))

    def add_request(self, rid: int, tokens) -> None:
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        _check(lib.pka_bm_add_request(self._h, int(rid), t.ctypes.data_as(c_void_p), int(t.size)))

    def append_token(self, rid: int, token: int) -> None:
        _check(lib.pka_bm_append_token(self._h, int(rid), int(token)))

    def find_cached_prefix(self, rid: int) -> list[int]:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = self._neg(lib.pka_bm_find_cached_prefix(self._h, int(rid), out.ctypes.data_as(c_void_p), out.size))
        return out[:n].tolist()

    def admit(self, rid: int, first_chunk: int):
        """Number of cached tokens, or None when the pool has no room."""
        cached = c_int32(0)
        ok = self._neg(lib.pka_bm_admit(self._h, int(rid), int(first_chunk), ctypes.byref(cached)))
        return cached.value if ok else None

    def allocate(self, rid: int, n: int) -> bool:
        return bool(self._neg(lib.pka_bm_allocate(self._h, int(rid), int(n))))

    def commit(self, rid: int, n: int) -> None:
        _check(lib.pka_bm_commit(self._h, int(rid), int(n)))

    def free_request(self, rid: int, drop: bool = True) -> None:
        _check(lib.pka_bm_free_request(self._h, int(rid), 0 if drop else 1))

    def block_table(self, rid: int) -> list[int]:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = self._neg(lib.pka_bm_block_table(self._h, int(rid), out.ctypes.data_as(c_void_p), out.size))
        return out[:n].tolist()

    def slot_mapping(self, rid: int, start: int, n: int) -> np.ndarray:
        out = np.empty(max(int(n), 1), dtype=np.int64)
        _check(lib.pka_bm_slot_mapping(self._h, int(rid), int(start), int(n), out.ctypes.data_as(c_void_p)))
        return out[: int(n)]

    def computed(self, rid: int) -> int:
        return self._neg(lib.pka_bm_num_computed(self._h, int(rid)))

    def decode_step(self, rids, tokens):
        """Append one token to each running request, place it and count it
        computed, in one call.  Returns (slots int64, ok bool); a request the
        pool cannot hold gets slot -1 and ok False (only its token appended)."""
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64))
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        if r.shape != t.shape:
            raise ValueError("one token per request")
        slots = np.empty(max(r.size, 1), dtype=np.int64)
        ok = np.empty(max(r.size, 1), dtype=np.int32)
        self._neg(lib.pka_bm_decode_step(self._h, int(r.size), r.ctypes.data_as(c_void_p), t.ctypes.data_as(c_void_p),
                                         slots.ctypes.data_as(c_void_p), ok.ctypes.data_as(c_void_p)))
        return slots[: r.size], ok[: r.size].astype(bool)


def rope_table(max_position, head_dim, theta, device):
    """Device table of (cos, sin) fp32 pairs [max_position, head_dim / 2, 2]
    for the fused RoPE write, computed on the GPU (double precision)."""
    n = lib.pka_rope_table_bytes(int(max_position), int(head_dim)) // 4
    table = torch.empty(max(n, 1), dtype=torch.float32, device=device)
    with torch.cuda.device(table.device):
        _check(lib.pka_rope_table(_ptr(table), int(max_position), int(head_dim), float(theta), _stream(table)))
    return table[:n].view(int(max_position), int(head_dim) // 2, 2)


def fused_rope_kv_write(qkv, positions, slot_mapping, table, num_q_heads, k_cache, v_cache, q_out=None,
                        prepare=False):
    """Rotate q and k of the fused projection rows qkv [T, (Hq + 2 Hkv) * D]
    (row stride may exceed the row) by positions (int64 [T]); returns
    q_out [T, Hq, D] and writes rotated k and raw v into the pool at
    slot_mapping (int64 [T]; negative = padding)."""
    _check_pool(k_cache, v_cache)
    dev = k_cache.device
    _require(qkv, "qkv", dtype=k_cache.dtype, ndim=2, device=dev)
    _require(positions, "positions", dtype=torch.int64, ndim=1, device=dev)
    _require(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1, device=dev)
    _require(table, "table", dtype=torch.float32, ndim=3, device=dev)
    T = qkv.shape[0]
    Hkv, D = k_cache.shape[2], k_cache.shape[3]
    if qkv.stride(1) != 1 or qkv.shape[1] != (num_q_heads + 2 * Hkv) * D:
        raise ValueError("qkv rows must be [q heads | k heads | v heads] with unit element stride")
    if positions.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("positions/slot_mapping length differs from qkv rows")
    if table.shape[1] * 2 != D or not table.is_contiguous():
        raise ValueError("rope table does not match the head size")
    if q_out is None:
        q_out = torch.empty((T, num_q_heads, D), dtype=qkv.dtype, device=dev)
    _require(q_out, "q_out", dtype=qkv.dtype, ndim=3, device=dev)
    if q_out.shape != (T, num_q_heads, D) or not q_out.is_contiguous():
        raise ValueError("q_out must be contiguous [T, Hq, D]")
    return _launch(lib.pka_fused_rope_kv_write,
                   (_ptr(qkv), qkv.stride(0), _ptr(positions), _ptr(slot_mapping), T, int(num_q_heads), _ptr(table),
                    table.shape[0], _ptr(q_out), _ptr(k_cache), _ptr(v_cache), cache_desc(k_cache), _stream(k_cache)),
                   prepare, (qkv, positions, slot_mapping, table, q_out, k_cache, v_cache), q_out)


def _decode_common(q, k_cache, v_cache, block_tables, context_lens):
    _check_pool(k_cache, v_cache)
    dev = k_cache.device
    _require(q, "q", dtype=k_cache.dtype, ndim=3, device=dev)
    if q.shape[2] != k_cache.shape[3]:
        raise ValueError("q head_dim differs from the pool's")
    _check_tables(block_tables, context_lens, q.shape[0], dev)


def _out_like(q, out):
    if out is None:
        return torch.empty_like(q)
    _require(out, "out", dtype=q.dtype, device=q.device)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return out


def paged_attn_decode_v1(q, k_cache, v_cache, block_tables, context_lens, scale, out=None, prepare=False):
    """Single-pass paged decode: q [S, Hq, D] -> out [S, Hq, D]."""
    _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    out = _out_like(q, out)
    S, Hq, _ = q.shape
    return _launch(lib.pka_paged_attn_decode_v1,
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S, Hq,
                    block_tables.shape[1], float(scale), _ptr(out), cache_desc(k_cache), _stream(q)),
                   prepare, (q, k_cache, v_cache, block_tables, context_lens, out), out)


def splitk_buffers(num_seqs, num_q_heads, head_dim, max_context_len, device):
    """Allocate (tmp_out, max_logits, exp_sums) for the split-K pass."""
    P = -(-int(max_context_len) // PARTITION_SIZE)
    tmp_out = torch.empty((num_seqs, num_q_heads, P, head_dim), dtype=torch.float32, device=device)
    max_logits = torch.empty((num_seqs, num_q_heads, P), dtype=torch.float32, device=device)
    exp_sums = torch.empty((num_seqs, num_q_heads, P), dtype=torch.float32, device=device)
    return tmp_out, max_logits, exp_sums


def paged_attn_decode_splitk(q, k_cache, v_cache, block_tables, context_lens, scale, tmp_out, max_logits, exp_sums,
                             partition_size=PARTITION_SIZE, prepare=False):
    """Split-K partition pass; fills tmp_out [S, Hq, P, D], max_logits and
    exp_sums [S, Hq, P] (fp32) for every partition inside a context."""
    _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    S, Hq, D = q.shape
    dev = q.device
    _require(tmp_out, "tmp_out", dtype=torch.float32, ndim=4, device=dev)
    _require(max_logits, "max_logits", dtype=torch.float32, ndim=3, device=dev)
    _require(exp_sums, "exp_sums", dtype=torch.float32, ndim=3, device=dev)
    P = tmp_out.shape[2]
    if tmp_out.shape != (S, Hq, P, D) or max_logits.shape != (S, Hq, P) or exp_sums.shape != (S, Hq, P):
        raise ValueError("split-K buffers have the wrong shape")
    return _launch(lib.pka_paged_attn_decode_splitk,
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S, Hq,
                    block_tables.shape[1], float(scale), partition_size, P, _ptr(tmp_out), _ptr(max_logits),
                    _ptr(exp_sums), cache_desc(k_cache), _stream(q)),
                   prepare, (q, k_cache, v_cache, block_tables, context_lens, tmp_out, max_logits, exp_sums))


def paged_attn_splitk_reduce(tmp_out, max_logits, exp_sums, context_lens, out, partition_size=PARTITION_SIZE,
                             prepare=False):
    """Merge split-K partitions into out [S, Hq, D] (fp16 or bf16)."""
    dev = out.device
    _require(out, "out", ndim=3)
    _require(tmp_out, "tmp_out", dtype=torch.float32, ndim=4, device=dev)
    _require(max_logits, "max_logits", dtype=torch.float32, ndim=3, device=dev)
    _require(exp_sums, "exp_sums", dtype=torch.float32, ndim=3, device=dev)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    S, Hq, P, D = tmp_out.shape
    if out.shape != (S, Hq, D) or context_lens.shape[0] != S:
        raise ValueError("reduce shapes disagree")
    if out.dtype not in _DTYPES:
        raise ValueError("out must be fp16 or bf16")
    return _launch(lib.pka_paged_attn_splitk_reduce,
                   (_ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums), _ptr(context_lens), S, Hq, D, partition_size, P,
                    _ptr(out), _DTYPES[out.dtype], _stream(out)),
                   prepare, (tmp_out, max_logits, exp_sums, context_lens, out), out)


def splitk_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len) -> int:
    return int(lib.pka_splitk_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len))


def splitk_workspace(num_seqs, num_q_heads, head_dim, max_context_len, device) -> torch.Tensor:
    """A workspace for the dispatched decode: uint8 device buffer of
    splitk_workspace_bytes(...) bytes, zero-filled once here (the split-K
    arrival counters at its start must be zero before the first call; every
    call leaves them zero, so the buffer is reused as is)."""
    n = max(1, splitk_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def decode_choose_variant(num_seqs, num_kv_heads, max_context_len, num_cus=None) -> int:
    if num_cus is None:
        num_cus = device_cu_count()
    return int(lib.pka_decode_choose_variant(num_seqs, num_kv_heads, max_context_len, num_cus))


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out=None,
                      workspace=None, prepare=False):
    """Paged decode with the library's dispatcher (single pass, or split-K
    with its partition merge).  max_context_len: host upper bound on
    context_lens.  workspace: optional uint8 device buffer of
    splitk_workspace_bytes(...) bytes whose first 64 KiB are zero before its
    first use (splitk_workspace() makes one); one is allocated when the split-K
    path needs it and none is given."""
    _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    out = _out_like(q, out)
    S, Hq, D = q.shape
    need = splitk_workspace_bytes(S, Hq, D, max_context_len)
    if workspace is None and decode_choose_variant(S, k_cache.shape[2], max_context_len) == 2:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _require(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
        ws_bytes = workspace.numel()
    return _launch(lib.pka_paged_attn_decode,
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S, Hq,
                    block_tables.shape[1], int(max_context_len), float(scale), _ptr(out), cache_desc(k_cache),
                    _ptr(workspace), ws_bytes, _stream(q)),
                   prepare, (q, k_cache, v_cache, block_tables, context_lens, out, workspace), out)


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out=None,
                              prepare=False):
    """paged_attn_decode without a workspace: the split-K path uses the
    library's own per-device scratch (nothing is allocated on any path when
    `out` is given).  Calls that overlap on one device race on that scratch."""
    _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    out = _out_like(q, out)
    S, Hq, _ = q.shape
    return _launch(lib.pka_paged_attn_decode_noalloc,
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S, Hq,
                    block_tables.shape[1], int(max_context_len), float(scale), _ptr(out), cache_desc(k_cache),
                    _stream(q)),
                   prepare, (q, k_cache, v_cache, block_tables, context_lens, out), out)


def paged_attn_decode_append(q, key, value, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                             out=None, workspace=None, prepare=False):
    """Decode step with the KV-cache write folded in: writes key[s] / value[s]
    ([S, Hkv, D]) at position context_lens[s] - 1 of each sequence (the slot
    its block table gives), then decodes over positions 0 .. context_lens[s] - 1
    - the same result as kv_cache_write followed by paged_attn_decode.
    Arguments otherwise as paged_attn_decode."""
    _decode_common(q, k_cache, v_cache, block_tables, context_lens)
    S, Hq, D = q.shape
    for t, name in ((key, "key"), (value, "value")):
        _require(t, name, dtype=k_cache.dtype, ndim=3, device=q.device)
        if tuple(t.shape) != (S, k_cache.shape[2], D):
            raise ValueError(f"{name} must be [{S}, {k_cache.shape[2]}, {D}], got {tuple(t.shape)}")
    out = _out_like(q, out)
    need = splitk_workspace_bytes(S, Hq, D, max_context_len)
    if workspace is None and decode_choose_variant(S, k_cache.shape[2], max_context_len) == 2:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _require(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
        ws_bytes = workspace.numel()
    return _launch(lib.pka_paged_attn_decode_append,
                   (_ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                    _ptr(context_lens), S, Hq, block_tables.shape[1], int(max_context_len), float(scale), _ptr(out),
                    cache_desc(k_cache), _ptr(workspace), ws_bytes, _stream(q)),
                   prepare, (q, key, value, k_cache, v_cache, block_tables, context_lens, out, workspace), out)


def prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len) -> int:
    return int(lib.pka_prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                                               max_context_len))


def prefill_workspace(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len,
                      device) -> torch.Tensor:
    """A workspace for paged_attn_prefill: uint8 device buffer of
    prefill_workspace_bytes(...) bytes (at least 1)."""
    n = max(1, prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def prefill_split_keys(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len) -> int:
    """Keys per split the prefill launch uses for these sizes on the current device."""
    n = int(lib.pka_prefill_split_keys(num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim, max_context_len))
    if n < 0:
        raise ValueError("invalid prefill sizes")
    return n


def paged_attn_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, max_query_len,
                       max_context_len, out=None, workspace=None, prepare=False):
    """Paged prefill over ragged chunks packed in q [Nq, Hq, D] (bottom-right
    causal; chunks attend to their cached prefix).  max_query_len /
    max_context_len: host upper bounds.  workspace: optional uint8 device
    buffer of prefill_workspace_bytes(...) bytes (allocated here when needed
    and not given).  Returns out [Nq, Hq, D]."""
    _check_pool(k_cache, v_cache)
    dev = k_cache.device
    _require(q, "q", dtype=k_cache.dtype, ndim=3, device=dev)
    S = context_lens.shape[0]
    _check_tables(block_tables, context_lens, S, dev)
    _require(query_start_loc, "query_start_loc", dtype=torch.int32, ndim=1, device=dev)
    if query_start_loc.shape[0] != S + 1:
        raise ValueError("query_start_loc must have num_seqs + 1 entries")
    out = _out_like(q, out)
    Nq, Hq, D = q.shape
    need = prefill_workspace_bytes(S, Nq, Hq, k_cache.shape[2], D, int(max_context_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _require(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
        ws_bytes = workspace.numel()
    return _launch(lib.pka_paged_attn_prefill,
                   (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
                    _ptr(query_start_loc), S, Nq, int(max_query_len), int(max_context_len), Hq, block_tables.shape[1],
                    float(scale), _ptr(out), cache_desc(k_cache), _ptr(workspace), ws_bytes, _stream(q)),
                   prepare, (q, k_cache, v_cache, block_tables, context_lens, query_start_loc, out, workspace), out)
