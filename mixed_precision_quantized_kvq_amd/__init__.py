"""Python binding of libkvq: decode attention over a mixed-precision quantized KV cache.

Argument marshalling only. Every step of the path (quantize, pack, calibrate, decode, merge)
runs in the HIP kernels of libkvq.so, reached through its C ABI (include/kvq.h); the
allocator, fit and layout planner run in the library's C++ host code. PyTorch supplies
device memory and streams. If the shared library is missing, every call raises: there is no
fallback implementation.

Names follow the C calls: cache_bytes, cache_init, calibrate_fit, allocate_bits, append,
decode_workspace_bytes, decode_attention, cache_check, region_offset, last_error.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "KvqError", "Config", "KVCache", "lib", "lib_path", "cache_bytes", "cache_init",
    "calibrate_fit", "calibrate_workspace_bytes", "allocate_bits", "append",
    "decode_workspace_bytes", "decode_attention", "decode_splitk", "decode_merge", "decode_step",
    "decode_multi_workspace_bytes", "decode_multi", "append_ragged", "decode_ragged",
    "cache_check",
    "region_offset", "last_error", "allocation_margin", "decode_attention_noalloc",
    "F16", "BF16", "QUANT_ASYM", "QUANT_HYBRID", "KEY_NORM", "AXIS_KEY", "AXIS_VALUE", "ALLOC_CAP_W",
    "EXPORTS",
]

F16, BF16 = 0, 1
QUANT_ASYM, QUANT_HYBRID = 0, 1
KEY_NORM = 0x100  # OR'ed into the quant mode: per-channel key normalization
AXIS_KEY, AXIS_VALUE = 0, 1
ALLOC_CAP_W = 1
MAX_KV_HEADS = 128
REGIONS = ("key_codes", "key_meta", "value_codes", "value_meta", "flags", "sink_keys",
           "sink_values", "ring_keys", "ring_values")

STATUS = {0: "OK", -1: "ERR_ARG", -2: "ERR_BUDGET", -3: "ERR_CAPACITY", -4: "ERR_RANGE",
          -5: "ERR_UNSUPPORTED", -6: "ERR_DEVICE", -7: "ERR_PAGE"}

EXPORTS = ("kvq_cache_bytes", "kvq_cache_init", "kvq_calibrate_workspace_bytes",
           "kvq_calibrate_fit", "kvq_allocate_bits", "kvq_append", "kvq_decode_workspace_bytes",
           "kvq_decode_attention", "kvq_decode_splitk", "kvq_decode_merge", "kvq_decode_step",
           "kvq_decode_multi_workspace_bytes", "kvq_decode_multi", "kvq_append_ragged", "kvq_decode_ragged",
           "kvq_cache_check", "kvq_cache_bytes_paged", "kvq_cache_init_paged", "kvq_cache_map_pages",
           "kvq_region_offset", "kvq_allocation_margin", "kvq_decode_attention_noalloc", "kvq_last_error")


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("quant", ctypes.c_int32),
                ("k_bits", ctypes.c_uint8 * MAX_KV_HEADS), ("v_bits", ctypes.c_uint8 * MAX_KV_HEADS)]

    @classmethod
    def make(cls, batch, n_kv_heads, n_q_heads, head_dim, capacity, n_sink, n_recent, dtype,
             quant, k_bits, v_bits, key_norm=False):
        c = cls()
        c.batch, c.n_kv_heads, c.n_q_heads, c.head_dim = batch, n_kv_heads, n_q_heads, head_dim
        c.capacity, c.group, c.n_sink, c.n_recent = capacity, 32, n_sink, n_recent
        c.dtype = dtype if isinstance(dtype, int) else {"fp16": F16, "bf16": BF16}[dtype]
        c.quant = quant if isinstance(quant, int) else {"asym": QUANT_ASYM, "hybrid": QUANT_HYBRID}[quant]
        if key_norm:
            c.quant |= KEY_NORM
        for i, b in enumerate(k_bits):
            c.k_bits[i] = int(b)
        for i, b in enumerate(v_bits):
            c.v_bits[i] = int(b)
        return c


class _Cache(ctypes.Structure):
    _fields_ = [("cfg", Config), ("dev", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
                ("len", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "libkvq.so")


def lib():
    """Load libkvq.so (built in-tree by mixed_precision_quantized_kvq_amd.build)."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: run __graft_entry__.build() first "
                              "(there is no fallback implementation)")
        L = ctypes.CDLL(path)
        P, I32, U32, U64, SZ, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32,
                                   ctypes.c_uint64, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double))
        CP = ctypes.POINTER(Config)
        KP = ctypes.POINTER(_Cache)
        sig = {
            "kvq_cache_bytes": (SZ, [CP]),
            "kvq_cache_init": (I32, [KP, CP, P, SZ, P]),
            "kvq_cache_bytes_paged": (SZ, [CP, I32]),
            "kvq_cache_init_paged": (I32, [KP, CP, I32, P, SZ, P]),
            "kvq_cache_map_pages": (I32, [KP, I32, I32, I32, P, P]),
            "kvq_calibrate_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
            "kvq_calibrate_fit": (I32, [P, I32, I32, I32, I32, I32, I32, I32, I32, P, SZ, D, D, D, P]),
            "kvq_allocate_bits": (I32, [I32, D, D, D, I32, I32, I32, U32,
                                        ctypes.POINTER(ctypes.c_uint8), D]),
            "kvq_append": (I32, [KP, P, P, I32, P]),
            "kvq_decode_workspace_bytes": (SZ, [KP, I32]),
            "kvq_decode_attention": (I32, [KP, P, P, I32, ctypes.c_float, P, SZ, P]),
            "kvq_decode_attention_noalloc": (I32, [KP, P, P, I32, ctypes.c_float, P]),
            "kvq_decode_splitk": (I32, [KP, P, I32, ctypes.c_float, P, SZ, P]),
            "kvq_decode_merge": (I32, [KP, P, I32, P, SZ, P]),
            "kvq_decode_step": (I32, [KP, P, P, I32, P, P, I32, ctypes.c_float, P, SZ, P]),
            "kvq_decode_multi_workspace_bytes": (SZ, [KP, I32, I32]),
            "kvq_decode_multi": (I32, [KP, P, I32, P, I32, ctypes.c_float, P, SZ, P]),
            "kvq_append_ragged": (I32, [KP, ctypes.POINTER(I32), ctypes.POINTER(I32), P, P, I32, P]),
            "kvq_decode_ragged": (I32, [KP, ctypes.POINTER(I32), P, P, I32, ctypes.c_float, P, SZ, P]),
            "kvq_cache_check": (I32, [KP, P]),
            "kvq_region_offset": (U64, [CP, I32, I32, I32, ctypes.POINTER(U64)]),
            "kvq_allocation_margin": (I32, [I32, D, D, D, ctypes.POINTER(ctypes.c_uint8), I32, I32, U32, D]),
            "kvq_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _LIB = L
    return _LIB


def last_error() -> str:
    return lib().kvq_last_error().decode()


def _check(st: int):
    if st != 0:
        raise KvqError(st, last_error())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _darr(x):
    vals = [float(v) for v in x]
    return (ctypes.c_double * len(vals))(*vals)


# ------------------------------------------------------------------------- host calls --

def cache_bytes(cfg: Config) -> int:
    n = lib().kvq_cache_bytes(ctypes.byref(cfg))
    if n == 0:
        raise KvqError(-1, last_error())
    return int(n)


def region_offset(cfg: Config, row: int, kv_head: int, region: int):
    size = ctypes.c_uint64(0)
    off = lib().kvq_region_offset(ctypes.byref(cfg), row, kv_head, region, ctypes.byref(size))
    if off == 0:
        raise KvqError(-1, last_error())
    return int(off), int(size.value)


def allocate_bits(alpha, beta, w, total_bits: int, b_lo: int, b_hi: int, cap: bool = False):
    """Integer bits (greedy / max-heap) and the continuous waterfilling solution."""
    n = len(alpha)
    out = (ctypes.c_uint8 * n)()
    cont = (ctypes.c_double * n)()
    _check(lib().kvq_allocate_bits(n, _darr(alpha), _darr(beta), _darr(w), int(total_bits),
                                   int(b_lo), int(b_hi), ALLOC_CAP_W if cap else 0, out, cont))
    return [int(v) for v in out], [float(v) for v in cont]


def allocation_margin(alpha, beta, w, bits, b_lo: int, b_hi: int, cap: bool = False) -> float:
    """Decision margin of an integer allocation (ln units): smallest key handed a bit minus the
    largest key left without one."""
    n = len(alpha)
    b = (ctypes.c_uint8 * n)(*[int(x) for x in bits])
    m = ctypes.c_double(0.0)
    _check(lib().kvq_allocation_margin(n, _darr(alpha), _darr(beta), _darr(w), b, int(b_lo), int(b_hi),
                                       ALLOC_CAP_W if cap else 0, ctypes.byref(m)))
    return float(m.value)


# ------------------------------------------------------------------------- device calls --

class KVCache:
    """A cache blob in a torch uint8 device tensor plus the C handle."""

    def __init__(self, cfg: Config, device="cuda", stream=None, blob=None, n_pages: int = 0):
        import torch
        self.cfg = cfg
        self.n_pages = n_pages
        nbytes = cache_bytes(cfg) if n_pages == 0 else cache_bytes_paged(cfg, n_pages)
        self.blob = blob if blob is not None else torch.empty(nbytes, dtype=torch.uint8, device=device)
        if self.blob.numel() < nbytes:
            raise ValueError("blob tensor too small")
        self.handle = _Cache()
        if n_pages == 0:
            _check(lib().kvq_cache_init(ctypes.byref(self.handle), ctypes.byref(cfg), _dptr(self.blob),
                                        nbytes, _stream(stream)))
        else:
            _check(lib().kvq_cache_init_paged(ctypes.byref(self.handle), ctypes.byref(cfg), int(n_pages),
                                              _dptr(self.blob), nbytes, _stream(stream)))

    def map_pages(self, row: int, first_tile: int, pages, stream=None):
        """Map tiles first_tile.. of `row` to the host int list/array `pages`."""
        arr = _i32_array(pages)
        _check(lib().kvq_cache_map_pages(ctypes.byref(self.handle), int(row), int(first_tile), len(pages),
                                         arr, _stream(stream)))

    def region_table(self):
        """The blob's region table as a host int64 array [batch][n_kv_heads][10]."""
        c = self.cfg
        n = c.batch * c.n_kv_heads * 10
        return self.blob[256:256 + 8 * n].cpu().numpy().view("<u8").reshape(c.batch, c.n_kv_heads, 10)

    @property
    def len(self) -> int:
        return int(self.handle.len)

    def region(self, row: int, kv_head: int, region: int):
        off, size = region_offset(self.cfg, row, kv_head, region)
        return self.blob[off:off + size]


def cache_init(cfg: Config, device="cuda", stream=None) -> KVCache:
    return KVCache(cfg, device, stream)


def cache_bytes_paged(cfg: Config, n_pages: int) -> int:
    n = lib().kvq_cache_bytes_paged(ctypes.byref(cfg), int(n_pages))
    if n == 0:
        raise KvqError(-1, last_error())
    return int(n)


def cache_init_paged(cfg: Config, n_pages: int, device="cuda", stream=None) -> KVCache:
    """A paged cache: body tiles of 64 tokens placed through a page table (all unmapped)."""
    return KVCache(cfg, device, stream, n_pages=n_pages)


def append(cache: KVCache, k, v, stream=None):
    """k, v: [batch][n_kv_heads][n_new][head_dim] 16-bit device tensors (contiguous)."""
    assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.dim() == 4
    c = cache.cfg
    assert tuple(k.shape[:2]) == (c.batch, c.n_kv_heads) and k.shape[3] == c.head_dim
    assert k.element_size() == 2 and v.element_size() == 2
    _check(lib().kvq_append(ctypes.byref(cache.handle), _dptr(k), _dptr(v), int(k.shape[2]),
                            _stream(stream)))


def decode_workspace_bytes(cache: KVCache, n_splits: int) -> int:
    n = lib().kvq_decode_workspace_bytes(ctypes.byref(cache.handle), int(n_splits))
    if n == 0:
        raise KvqError(-1, last_error())
    return int(n)


def decode_attention(cache: KVCache, q, out, n_splits: int, workspace, scale: float = 0.0,
                     stream=None):
    """q: [batch][n_q_heads][head_dim] 16-bit; out: same shape float32 (written)."""
    import torch
    c = cache.cfg
    assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
    assert tuple(q.shape) == (c.batch, c.n_q_heads, c.head_dim) and tuple(out.shape) == tuple(q.shape)
    _check(lib().kvq_decode_attention(ctypes.byref(cache.handle), _dptr(q), _dptr(out), int(n_splits),
                                      float(scale), _dptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


def decode_attention_noalloc(cache: KVCache, q, out, n_splits: int, scale: float = 0.0, stream=None):
    """decode_attention with the split partials in the library's static device scratch (no
    workspace argument; nothing is allocated)."""
    import torch
    c = cache.cfg
    assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
    assert tuple(q.shape) == (c.batch, c.n_q_heads, c.head_dim) and tuple(out.shape) == tuple(q.shape)
    _check(lib().kvq_decode_attention_noalloc(ctypes.byref(cache.handle), _dptr(q), _dptr(out), int(n_splits),
                                              float(scale), _stream(stream)))


def decode_multi_workspace_bytes(cache: KVCache, n_splits: int, n_qtok: int) -> int:
    n = lib().kvq_decode_multi_workspace_bytes(ctypes.byref(cache.handle), int(n_splits), int(n_qtok))
    if n == 0:
        raise KvqError(-1, last_error())
    return int(n)


def decode_multi(cache: KVCache, q, out, n_splits: int, workspace, scale: float = 0.0, stream=None):
    """q: [batch][n_qtok][n_q_heads][head_dim] 16-bit, the queries of the last n_qtok cached
    tokens (causal); out: same shape float32 (written)."""
    import torch
    c = cache.cfg
    assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32 and q.dim() == 4
    assert q.shape[0] == c.batch and tuple(q.shape[2:]) == (c.n_q_heads, c.head_dim)
    assert tuple(out.shape) == tuple(q.shape)
    _check(lib().kvq_decode_multi(ctypes.byref(cache.handle), _dptr(q), int(q.shape[1]), _dptr(out), int(n_splits),
                                  float(scale), _dptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))


def _i32_array(vals):
    return (ctypes.c_int32 * len(vals))(*[int(x) for x in vals])


def append_ragged(cache: KVCache, row_len, n_new, k, v, stream=None):
    """Row b (current length row_len[b]) appends the first n_new[b] of its k, v slots
    ([batch][n_kv_heads][n_max][head_dim] 16-bit). The caller updates its row_len."""
    c = cache.cfg
    assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.dim() == 4
    assert tuple(k.shape[:2]) == (c.batch, c.n_kv_heads) and k.shape[3] == c.head_dim
    assert k.element_size() == 2 and v.element_size() == 2
    assert len(row_len) == c.batch and len(n_new) == c.batch
    _check(lib().kvq_append_ragged(ctypes.byref(cache.handle), _i32_array(row_len), _i32_array(n_new), _dptr(k),
                                   _dptr(v), int(k.shape[2]), _stream(stream)))


def decode_ragged(cache: KVCache, row_len, q, out, n_splits: int, workspace, scale: float = 0.0, stream=None):
    """One query per row ([batch][n_q_heads][head_dim] 16-bit), row b over its row_len[b] tokens."""
    import torch
    c = cache.cfg
    assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
    assert tuple(q.shape) == (c.batch, c.n_q_heads, c.head_dim) and tuple(out.shape) == tuple(q.shape)
    assert len(row_len) == c.batch
    _check(lib().kvq_decode_ragged(ctypes.byref(cache.handle), _i32_array(row_len), _dptr(q), _dptr(out),
                                   int(n_splits), float(scale), _dptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_step(cache: KVCache, k, v, q, out, n_splits: int, workspace, scale: float = 0.0, stream=None):
    """Append k, v ([batch][n_kv_heads][n_new][head_dim] 16-bit) and decode q into out
    (float32 [batch][n_q_heads][head_dim]) in one call."""
    import torch
    c = cache.cfg
    assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape and k.dim() == 4
    assert tuple(k.shape[:2]) == (c.batch, c.n_kv_heads) and k.shape[3] == c.head_dim
    assert k.element_size() == 2 and v.element_size() == 2
    assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
    assert tuple(q.shape) == (c.batch, c.n_q_heads, c.head_dim) and tuple(out.shape) == tuple(q.shape)
    _check(lib().kvq_decode_step(ctypes.byref(cache.handle), _dptr(k), _dptr(v), int(k.shape[2]), _dptr(q),
                                 _dptr(out), int(n_splits), float(scale), _dptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_splitk(cache: KVCache, q, n_splits: int, workspace, scale: float = 0.0, stream=None):
    """First launch of decode_attention: the split partials, written into `workspace`."""
    c = cache.cfg
    assert q.is_contiguous() and tuple(q.shape) == (c.batch, c.n_q_heads, c.head_dim)
    _check(lib().kvq_decode_splitk(ctypes.byref(cache.handle), _dptr(q), int(n_splits), float(scale),
                                   _dptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def decode_merge(cache: KVCache, out, n_splits: int, workspace, stream=None):
    """Second launch of decode_attention: log-sum-exp merge of the partials into `out`."""
    import torch
    c = cache.cfg
    assert out.is_contiguous() and out.dtype == torch.float32
    assert tuple(out.shape) == (c.batch, c.n_q_heads, c.head_dim)
    _check(lib().kvq_decode_merge(ctypes.byref(cache.handle), _dptr(out), int(n_splits), _dptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def cache_check(cache: KVCache, stream=None):
    _check(lib().kvq_cache_check(ctypes.byref(cache.handle), _stream(stream)))


def calibrate_workspace_bytes(n_heads, n_tokens, head_dim, b_lo=2, b_hi=8) -> int:
    return int(lib().kvq_calibrate_workspace_bytes(n_heads, n_tokens, head_dim, b_lo, b_hi))


def calibrate_fit(x, dtype, axis: int, quant: int = QUANT_ASYM, b_lo: int = 2, b_hi: int = 8,
                  workspace=None, stream=None):
    """x: [n_heads][n_tokens][head_dim] 16-bit device tensor. Returns (alpha, beta, r2)."""
    import torch
    assert x.is_contiguous() and x.dim() == 3 and x.element_size() == 2
    H, T, D = x.shape
    need = calibrate_workspace_bytes(H, T, D, b_lo, b_hi)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    a = (ctypes.c_double * H)()
    b = (ctypes.c_double * H)()
    r = (ctypes.c_double * H)()
    dt = dtype if isinstance(dtype, int) else {"fp16": F16, "bf16": BF16}[dtype]
    _check(lib().kvq_calibrate_fit(_dptr(x), dt, H, T, D, axis, quant, b_lo, b_hi, _dptr(workspace),
                                   workspace.numel(), a, b, r, _stream(stream)))
    return list(a), list(b), list(r)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
