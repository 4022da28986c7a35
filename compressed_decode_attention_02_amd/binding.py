"""ctypes binding of libtq.so (include/tq.h).  Argument marshalling only: every step of
the compression and attention runs in the library's HIP kernels.  PyTorch supplies device
memory and the current stream.  Functions keep the C names (tq_*)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_RING_FULL, TQ_ERR_WORKSPACE, TQ_ERR_HIP = 0, -1, -2, -3, -4, -5
TQ_ERR_SCRATCH_LIMIT = -6
TQ_NOALLOC_SCRATCH_BYTES = 8 << 20
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2

EXPORTS = [
    "tq_build_codebook", "tq_build_rotation", "tq_tables_bytes", "tq_build_tables", "tq_tables_view",
    "tq_packed_bytes_per_token", "tq_quantize_kv", "tq_append_ring", "tq_flush",
    "tq_decode_workspace_bytes", "tq_decode_attention", "tq_decode_attention_ragged", "tq_decode_step",
    "tq_status_string", "tq_rotate", "tq_decode_scores", "tq_decode_attention_noalloc",
    "tq_prefill_workspace_bytes", "tq_prefill_attention",
    "tq_kivi_bytes_per_token", "tq_kivi_quantize", "tq_kivi_decode_workspace_bytes", "tq_kivi_decode_attention",
]


class TqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({_lib().tq_status_string(status).decode()})")
        self.status = status


class tq_config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("key_bits", ctypes.c_int32), ("value_bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("buffer_size", ctypes.c_int32)]


class tq_tables(ctypes.Structure):
    _fields_ = [("centroids", ctypes.c_void_p), ("boundaries", ctypes.c_void_p), ("sign_bits", ctypes.c_void_p),
                ("qjl_S", ctypes.c_void_p)]


class tq_packed(ctypes.Structure):
    _fields_ = [("key_words", ctypes.c_void_p), ("key_norms", ctypes.c_void_p), ("val_words", ctypes.c_void_p),
                ("val_scales", ctypes.c_void_p), ("capacity", ctypes.c_int64), ("block_table", ctypes.c_void_p),
                ("page_tokens", ctypes.c_int32), ("pages_per_slice", ctypes.c_int32), ("n_pages", ctypes.c_int64),
                ("error_flag", ctypes.c_void_p)]


class tq_kivi_store(ctypes.Structure):
    _fields_ = [("key_codes", ctypes.c_void_p), ("key_scale", ctypes.c_void_p), ("key_zero", ctypes.c_void_p),
                ("val_codes", ctypes.c_void_p), ("val_params", ctypes.c_void_p), ("capacity", ctypes.c_int64)]


class tq_ring(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


_L = None


def _lib():
    global _L
    if _L is not None:
        return _L
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m compressed_decode_attention_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    C = ctypes.POINTER(tq_config)
    T = ctypes.POINTER(tq_tables)
    K = ctypes.POINTER(tq_packed)
    R = ctypes.POINTER(tq_ring)
    sig = {
        "tq_build_codebook": (ctypes.c_int, [I32, I32, P, P]),
        "tq_build_rotation": (ctypes.c_int, [I32, ctypes.c_uint64, P, P]),
        "tq_tables_bytes": (SZ, [C]),
        "tq_build_tables": (ctypes.c_int, [C, ctypes.c_uint64, P, SZ]),
        "tq_tables_view": (ctypes.c_int, [C, P, T]),
        "tq_packed_bytes_per_token": (SZ, [C]),
        "tq_quantize_kv": (ctypes.c_int, [C, T, P, P, ctypes.c_int, I32, I64, K, I64, P]),
        "tq_append_ring": (ctypes.c_int, [C, R, P, P, ctypes.c_int, I32, I32, P]),
        "tq_flush": (ctypes.c_int, [C, T, R, I32, I32, K, I64, P]),
        "tq_decode_workspace_bytes": (SZ, [C, I32, I32, I32, I64]),
        "tq_decode_attention": (ctypes.c_int, [C, T, P, ctypes.c_int, I32, I32, I32, K, I64, R, I32, F, P, P, SZ, P]),
        "tq_decode_attention_ragged": (ctypes.c_int, [C, T, P, ctypes.c_int, I32, I32, I32, K, P, I64, R, P, I32, F,
                                                      P, P, SZ, P]),
        "tq_decode_step": (ctypes.c_int, [C, T, P, ctypes.c_int, I32, I32, I32, K, ctypes.POINTER(I64), R,
                                          ctypes.POINTER(I32), P, P, ctypes.c_int, F, P, P, SZ, P]),
        "tq_decode_attention_noalloc": (ctypes.c_int, [C, T, P, ctypes.c_int, I32, I32, I32, K, I64, R, I32, F, P,
                                                       P]),
        "tq_prefill_workspace_bytes": (SZ, [C, I32, I32, I32, I32, I64]),
        "tq_prefill_attention": (ctypes.c_int, [C, T, P, ctypes.c_int, I32, I32, I32, I32, K, I64, I64, I32, F, P,
                                                P, SZ, P]),
        "tq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "tq_kivi_bytes_per_token": (SZ, [I32]),
        "tq_kivi_quantize": (ctypes.c_int, [I32, P, P, ctypes.c_int, I32, I64, ctypes.POINTER(tq_kivi_store), I64, P]),
        "tq_kivi_decode_workspace_bytes": (SZ, [I32, I32, I32, I32, I64]),
        "tq_kivi_decode_attention": (ctypes.c_int, [I32, P, ctypes.c_int, I32, I32, I32,
                                                    ctypes.POINTER(tq_kivi_store), I64, F, P, P, SZ, P]),
        "tq_rotate": (ctypes.c_int, [C, T, P, ctypes.c_int, I64, P, P]),
        "tq_decode_scores": (ctypes.c_int, [C, T, P, ctypes.c_int, I32, I32, I32, K, I64, R, I32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _L = L
    return L


def lib():
    return _lib()


def _check(fn: str, st: int):
    if st != TQ_OK:
        raise TqError(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dtype_code(t) -> int:
    import torch
    code = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}.get(t.dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")
    return code


def _need(name: str, t, numel: int, dtype=None):
    """A device tensor argument: contiguous, of dtype `dtype` (if given) and holding at least
    `numel` elements.  Raises ValueError before anything reaches the library, which would
    otherwise read or write past the end of a buffer that is too small.  (Where the tensors
    live is checked by _on_one_gpu once every argument has passed these checks.)"""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, at least {numel} are needed")


def _on_one_gpu(*named):
    """Every given tensor is a GPU tensor, all on the same device."""
    named = [(n, t) for n, t in named if t is not None]
    for n, t in named:
        if t.device.type != "cuda":
            raise ValueError(f"{n} must be a GPU tensor, got device {t.device}")
    if len({t.device for _, t in named}) > 1:
        raise ValueError("tensors on different devices: " + ", ".join(f"{n}={t.device}" for n, t in named))


def _kv_pair(k, v, numel: int, kname="k", vname="v"):
    """k and v of one call: one dtype (the library reads both with it), contiguous, each
    holding at least numel elements."""
    if k is None or v is None:
        raise ValueError(f"{kname} and {vname} are required")
    if k.dtype != v.dtype:
        raise ValueError(f"{kname} and {vname} must share a dtype, got {k.dtype} and {v.dtype}")
    _dtype_code(k)
    _need(kname, k, numel)
    _need(vname, v, numel)


def make_config(head_dim=128, key_bits=3, value_bits=2, group_size=32, buffer_size=128) -> tq_config:
    return tq_config(head_dim, key_bits, value_bits, group_size, buffer_size)


# ------------------------------------------------------------------ host tables

def tq_build_codebook(head_dim: int, key_bits: int):
    c = np.zeros(1 << key_bits, np.float64)
    b = np.zeros((1 << key_bits) - 1, np.float64)
    _check("tq_build_codebook", _lib().tq_build_codebook(head_dim, key_bits, c.ctypes.data, b.ctypes.data))
    return c, b


def tq_build_rotation(head_dim: int, seed: int):
    s = np.zeros(head_dim, np.int8)
    S = np.zeros(head_dim * head_dim, np.uint16)
    _check("tq_build_rotation", _lib().tq_build_rotation(head_dim, seed, s.ctypes.data, S.ctypes.data))
    return s, S.reshape(head_dim, head_dim)


def tq_tables_bytes(cfg: tq_config) -> int:
    return _lib().tq_tables_bytes(ctypes.byref(cfg))


def tq_build_tables(cfg: tq_config, seed: int) -> np.ndarray:
    n = tq_tables_bytes(cfg)
    if n == 0:
        raise TqError("tq_tables_bytes", TQ_ERR_UNSUPPORTED)
    blob = np.zeros(n, np.uint8)
    _check("tq_build_tables", _lib().tq_build_tables(ctypes.byref(cfg), seed, blob.ctypes.data, n))
    return blob


class Tables:
    """The device table blob (torch uint8 tensor) and its tq_tables view."""

    def __init__(self, cfg: tq_config, seed: int, device="cuda"):
        import torch
        self.cfg = cfg
        self.host_blob = tq_build_tables(cfg, seed)
        self.blob = torch.from_numpy(self.host_blob).to(device)
        self.view = tq_tables()
        _check("tq_tables_view", _lib().tq_tables_view(ctypes.byref(cfg), _ptr(self.blob), ctypes.byref(self.view)))


def tq_packed_bytes_per_token(cfg: tq_config) -> int:
    return _lib().tq_packed_bytes_per_token(ctypes.byref(cfg))


def key_record_words(cfg: tq_config) -> int:
    """32-bit words of one key record: (key_bits + 1) head_dim / 32 (layout in tq.h)."""
    return (cfg.key_bits + 1) * cfg.head_dim // 32


class PackedStore:
    """Device arrays of the packed cache, [n_slices][capacity][...] each (layout in tq.h)."""

    def __init__(self, cfg: tq_config, n_slices: int, capacity: int, device="cuda"):
        import torch
        d, vb = cfg.head_dim, cfg.value_bits
        self.cfg, self.n_slices, self.capacity = cfg, n_slices, capacity
        self.key_words = torch.zeros((n_slices, capacity, key_record_words(cfg)), dtype=torch.int32, device=device)
        self.key_norms = torch.zeros((n_slices, capacity, 2), dtype=torch.float32, device=device)
        self.val_words = torch.zeros((n_slices, capacity, vb * d // 32), dtype=torch.int32, device=device)
        self.val_scales = torch.zeros((n_slices, capacity, d // 32), dtype=torch.int16, device=device)

    def struct(self, slice_offset: int = 0) -> tq_packed:
        """tq_packed view starting at slice `slice_offset` (e.g. one layer of a larger store)."""
        return tq_packed(self.key_words[slice_offset:].data_ptr(), self.key_norms[slice_offset:].data_ptr(),
                         self.val_words[slice_offset:].data_ptr(), self.val_scales[slice_offset:].data_ptr(),
                         self.capacity, None, 0, 0, 0, None)


class PagedStore:
    """A paged packed cache: a pool of n_pages pages of page_tokens records ([n_pages][page_tokens]
    [...] per array) and a block table [n_slices][pages_per_slice] of page indices (layout in tq.h).
    Without a table, slices take pages in a seeded random order (pages need not be contiguous)."""

    def __init__(self, cfg: tq_config, n_slices: int, page_tokens: int, pages_per_slice: int, n_pages: int,
                 table=None, seed: int = 0, device="cuda"):
        import torch
        d, vb = cfg.head_dim, cfg.value_bits
        self.cfg, self.n_slices, self.page_tokens = cfg, n_slices, page_tokens
        self.pages_per_slice, self.n_pages = pages_per_slice, n_pages
        self.capacity = pages_per_slice * page_tokens
        self.key_words = torch.zeros((n_pages, page_tokens, key_record_words(cfg)), dtype=torch.int32, device=device)
        self.key_norms = torch.zeros((n_pages, page_tokens, 2), dtype=torch.float32, device=device)
        self.val_words = torch.zeros((n_pages, page_tokens, vb * d // 32), dtype=torch.int32, device=device)
        self.val_scales = torch.zeros((n_pages, page_tokens, d // 32), dtype=torch.int16, device=device)
        if table is None:
            perm = np.random.Generator(np.random.PCG64(seed)).permutation(n_pages)[:n_slices * pages_per_slice]
            table = perm.reshape(n_slices, pages_per_slice)
        self.table_np = np.asarray(table, np.int32).reshape(n_slices, pages_per_slice)
        self.block_table = torch.from_numpy(self.table_np.copy()).to(device)
        # set to 1 by a kernel that meets a table entry outside the pool (never cleared by the library)
        self.error_flag = torch.zeros(1, dtype=torch.int32, device=device)

    def table_error(self) -> bool:
        """True when a call since the last clear_table_error() met a table entry outside the
        pool (synchronises with the device)."""
        return bool(self.error_flag.item())

    def clear_table_error(self):
        self.error_flag.zero_()

    def struct(self, slice_offset: int = 0) -> tq_packed:
        """tq_packed view of slices slice_offset.. (their block-table rows; the pool is shared)."""
        return tq_packed(self.key_words.data_ptr(), self.key_norms.data_ptr(), self.val_words.data_ptr(),
                         self.val_scales.data_ptr(), self.capacity, self.block_table[slice_offset:].data_ptr(),
                         self.page_tokens, self.pages_per_slice, self.n_pages, self.error_flag.data_ptr())

    def gather(self):
        """The store as contiguous [n_slices][capacity][...] arrays (host copies through the table)."""
        out = {}
        for name in ("key_words", "key_norms", "val_words", "val_scales"):
            pool = getattr(self, name).cpu().numpy()
            out[name] = pool[self.table_np].reshape(self.n_slices, self.capacity, *pool.shape[2:])
        return out


class Ring:
    """fp16 ring buffers [n_slices][buffer_size][d] for keys and values."""

    def __init__(self, cfg: tq_config, n_slices: int, device="cuda"):
        import torch
        shape = (n_slices, cfg.buffer_size, cfg.head_dim)
        self.k = torch.zeros(shape, dtype=torch.float16, device=device)
        self.v = torch.zeros(shape, dtype=torch.float16, device=device)

    def struct(self, slice_offset: int = 0) -> tq_ring:
        return tq_ring(self.k[slice_offset:].data_ptr(), self.v[slice_offset:].data_ptr())


# ------------------------------------------------------------------ device entry points

def tq_quantize_kv(cfg, tables: Tables, k, v, n_slices: int, n_tokens: int, dst: tq_packed, dst_offset: int,
                   stream=None):
    _kv_pair(k, v, max(n_slices, 0) * max(n_tokens, 0) * cfg.head_dim)
    _on_one_gpu(("k", k), ("v", v))
    st = _lib().tq_quantize_kv(ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(k), _ptr(v), _dtype_code(k),
                               n_slices, n_tokens, ctypes.byref(dst), dst_offset, _stream(stream))
    _check("tq_quantize_kv", st)


def tq_append_ring(cfg, ring: tq_ring, k_new, v_new, n_slices: int, n_ring: int, stream=None):
    _kv_pair(k_new, v_new, max(n_slices, 0) * cfg.head_dim, "k_new", "v_new")
    _on_one_gpu(("k_new", k_new), ("v_new", v_new))
    st = _lib().tq_append_ring(ctypes.byref(cfg), ctypes.byref(ring), _ptr(k_new), _ptr(v_new),
                               _dtype_code(k_new), n_slices, n_ring, _stream(stream))
    _check("tq_append_ring", st)


def tq_flush(cfg, tables: Tables, ring: tq_ring, n_slices: int, n_ring: int, dst: tq_packed, n_packed: int,
             stream=None):
    st = _lib().tq_flush(ctypes.byref(cfg), ctypes.byref(tables.view), ctypes.byref(ring), n_slices, n_ring,
                         ctypes.byref(dst), n_packed, _stream(stream))
    _check("tq_flush", st)


def tq_decode_workspace_bytes(cfg, batch: int, n_q_heads: int, n_kv_heads: int, max_context: int) -> int:
    return _lib().tq_decode_workspace_bytes(ctypes.byref(cfg), batch, n_q_heads, n_kv_heads, max_context)


def _decode_io(cfg, q, out, workspace, batch: int, n_q_heads: int):
    import torch
    n = max(batch, 0) * max(n_q_heads, 0) * cfg.head_dim
    _dtype_code(q)
    _need("q", q, n)
    _need("out", out, n, torch.float32)
    _need("workspace", workspace, 1)


def tq_decode_attention(cfg, tables: Tables, q, batch: int, n_q_heads: int, n_kv_heads: int,
                        packed: tq_packed | None, n_packed: int, ring: tq_ring | None, n_ring: int,
                        softmax_scale: float, out, workspace, stream=None):
    _decode_io(cfg, q, out, workspace, batch, n_q_heads)
    _on_one_gpu(("q", q), ("out", out), ("workspace", workspace))
    st = _lib().tq_decode_attention(
        ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, n_q_heads, n_kv_heads,
        ctypes.byref(packed) if packed is not None else None, n_packed,
        ctypes.byref(ring) if ring is not None else None, n_ring, ctypes.c_float(softmax_scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_decode_attention", st)


def tq_decode_attention_noalloc(cfg, tables: Tables, q, batch: int, n_q_heads: int, n_kv_heads: int,
                                packed: tq_packed | None, n_packed: int, ring: tq_ring | None, n_ring: int,
                                softmax_scale: float, out, stream=None):
    """tq_decode_attention with the library's static scratch instead of a workspace (no
    allocation; calls that may overlap on one GPU race on the scratch)."""
    import torch
    n = max(batch, 0) * max(n_q_heads, 0) * cfg.head_dim
    _dtype_code(q)
    _need("q", q, n)
    _need("out", out, n, torch.float32)
    _on_one_gpu(("q", q), ("out", out))
    st = _lib().tq_decode_attention_noalloc(
        ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, n_q_heads, n_kv_heads,
        ctypes.byref(packed) if packed is not None else None, n_packed,
        ctypes.byref(ring) if ring is not None else None, n_ring, ctypes.c_float(softmax_scale), _ptr(out),
        _stream(stream))
    _check("tq_decode_attention_noalloc", st)


def tq_rotate(cfg, tables: Tables, x, n_rows: int, out, stream=None):
    """Test hook: out = Pi x for n_rows rows (out: fp32 device tensor [n_rows][d])."""
    import torch
    _dtype_code(x)
    _need("x", x, max(n_rows, 0) * cfg.head_dim)
    _need("out", out, max(n_rows, 0) * cfg.head_dim, torch.float32)
    _on_one_gpu(("x", x), ("out", out))
    st = _lib().tq_rotate(ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(x), _dtype_code(x), n_rows, _ptr(out),
                          _stream(stream))
    _check("tq_rotate", st)


def tq_decode_scores(cfg, tables: Tables, q, batch: int, n_q_heads: int, n_kv_heads: int, packed: tq_packed | None,
                     n_packed: int, ring: tq_ring | None, n_ring: int, scores, stream=None):
    """Test hook: raw pre-softmax scores [batch][n_q_heads][n_packed + n_ring] (fp32 device tensor)."""
    import torch
    _dtype_code(q)
    _need("q", q, max(batch, 0) * max(n_q_heads, 0) * cfg.head_dim)
    _need("scores", scores, max(batch, 0) * max(n_q_heads, 0) * max(n_packed + n_ring, 0), torch.float32)
    _on_one_gpu(("q", q), ("scores", scores))
    st = _lib().tq_decode_scores(
        ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, n_q_heads, n_kv_heads,
        ctypes.byref(packed) if packed is not None else None, n_packed,
        ctypes.byref(ring) if ring is not None else None, n_ring, _ptr(scores), _stream(stream))
    _check("tq_decode_scores", st)


def tq_decode_attention_ragged(cfg, tables: Tables, q, batch: int, n_q_heads: int, n_kv_heads: int,
                               packed: tq_packed | None, seq_packed, n_packed_max: int, ring: tq_ring | None,
                               seq_ring, n_ring_max: int, softmax_scale: float, out, workspace, stream=None):
    """Decode with per-sequence lengths: seq_packed (int64) and seq_ring (int32) are device
    tensors of `batch` entries."""
    import torch
    _decode_io(cfg, q, out, workspace, batch, n_q_heads)
    _need("seq_packed", seq_packed, max(batch, 0), torch.int64)
    _need("seq_ring", seq_ring, max(batch, 0), torch.int32)
    _on_one_gpu(("q", q), ("out", out), ("workspace", workspace), ("seq_packed", seq_packed), ("seq_ring", seq_ring))
    st = _lib().tq_decode_attention_ragged(
        ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, n_q_heads, n_kv_heads,
        ctypes.byref(packed) if packed is not None else None, _ptr(seq_packed), n_packed_max,
        ctypes.byref(ring) if ring is not None else None, _ptr(seq_ring), n_ring_max, ctypes.c_float(softmax_scale),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_decode_attention_ragged", st)


def tq_decode_step(cfg, tables: Tables, q, batch: int, n_q_heads: int, n_kv_heads: int,
                   packed: tq_packed | None, n_packed: int, ring: tq_ring, n_ring: int, k_new, v_new,
                   softmax_scale: float, out, workspace, stream=None):
    """Append k_new / v_new to the ring (flushing a full ring first) and decode, in one call.
    Returns the new (n_packed, n_ring)."""
    _decode_io(cfg, q, out, workspace, batch, n_q_heads)
    _kv_pair(k_new, v_new, max(batch, 0) * max(n_kv_heads, 0) * cfg.head_dim, "k_new", "v_new")
    _on_one_gpu(("q", q), ("out", out), ("workspace", workspace), ("k_new", k_new), ("v_new", v_new))
    np_ = ctypes.c_int64(n_packed)
    nr_ = ctypes.c_int32(n_ring)
    st = _lib().tq_decode_step(
        ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, n_q_heads, n_kv_heads,
        ctypes.byref(packed) if packed is not None else None, ctypes.byref(np_), ctypes.byref(ring),
        ctypes.byref(nr_), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), ctypes.c_float(softmax_scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_decode_step", st)
    return np_.value, nr_.value


class PreparedDecodeStep:
    """One tq_decode_step call shape with its arguments checked and marshalled once, for loops
    that repeat it (a model's layers at every decode step): calling it with the fill counts runs
    tq_decode_step on the stream that was current when it was prepared and returns the new
    counts.  The tensors and views passed in must stay alive and in place."""

    def __init__(self, cfg, tables: Tables, q, batch: int, n_q_heads: int, n_kv_heads: int,
                 packed: tq_packed | None, ring: tq_ring, k_new, v_new, softmax_scale: float, out, workspace,
                 stream=None):
        _decode_io(cfg, q, out, workspace, batch, n_q_heads)
        _kv_pair(k_new, v_new, max(batch, 0) * max(n_kv_heads, 0) * cfg.head_dim, "k_new", "v_new")
        _on_one_gpu(("q", q), ("out", out), ("workspace", workspace), ("k_new", k_new), ("v_new", v_new))
        self._keep = (cfg, tables, q, packed, ring, k_new, v_new, out, workspace)
        self._np = ctypes.c_int64(0)
        self._nr = ctypes.c_int32(0)
        self._fn = _lib().tq_decode_step
        self._args = (ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, n_q_heads,
                      n_kv_heads, ctypes.byref(packed) if packed is not None else None, ctypes.byref(self._np),
                      ctypes.byref(ring), ctypes.byref(self._nr), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                      ctypes.c_float(softmax_scale), _ptr(out), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream(stream))

    def __call__(self, n_packed: int, n_ring: int):
        self._np.value = n_packed
        self._nr.value = n_ring
        st = self._fn(*self._args)
        if st != TQ_OK:
            raise TqError("tq_decode_step", st)
        return self._np.value, self._nr.value


def tq_prefill_workspace_bytes(cfg, batch: int, q_tokens: int, n_q_heads: int, n_kv_heads: int,
                               n_packed: int) -> int:
    return _lib().tq_prefill_workspace_bytes(ctypes.byref(cfg), batch, q_tokens, n_q_heads, n_kv_heads, n_packed)


def tq_prefill_attention(cfg, tables: Tables, q, batch: int, q_tokens: int, n_q_heads: int, n_kv_heads: int,
                         packed: tq_packed, n_packed: int, q_pos0: int, causal: bool, softmax_scale: float, out,
                         workspace, stream=None):
    """Prefill attention over the packed cache: q and out [batch][q_tokens][n_q_heads][d]."""
    import torch
    n = max(batch, 0) * max(q_tokens, 0) * max(n_q_heads, 0) * cfg.head_dim
    _dtype_code(q)
    _need("q", q, n)
    _need("out", out, n, torch.float32)
    _need("workspace", workspace, 1)
    _on_one_gpu(("q", q), ("out", out), ("workspace", workspace))
    st = _lib().tq_prefill_attention(
        ctypes.byref(cfg), ctypes.byref(tables.view), _ptr(q), _dtype_code(q), batch, q_tokens, n_q_heads,
        n_kv_heads, ctypes.byref(packed), n_packed, q_pos0, 1 if causal else 0, ctypes.c_float(softmax_scale),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_prefill_attention", st)


def new_prefill_workspace(cfg, batch: int, q_tokens: int, n_q_heads: int, n_kv_heads: int, n_packed: int,
                          device="cuda"):
    """Prefill workspace (scratch) of the size tq_prefill_workspace_bytes reports."""
    import torch
    n = tq_prefill_workspace_bytes(cfg, batch, q_tokens, n_q_heads, n_kv_heads, n_packed)
    if n == 0:
        raise TqError("tq_prefill_workspace_bytes", TQ_ERR_INVALID_ARG)
    return torch.empty(n, dtype=torch.uint8, device=device)


def new_workspace(cfg, batch: int, n_q_heads: int, n_kv_heads: int, max_context: int, device="cuda"):
    """Decode workspace (scratch) of the size tq_decode_workspace_bytes reports."""
    import torch
    n = tq_decode_workspace_bytes(cfg, batch, n_q_heads, n_kv_heads, max_context)
    if n == 0:
        raise TqError("tq_decode_workspace_bytes", TQ_ERR_INVALID_ARG)
    return torch.empty(n, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ KIVI 2-bit variant (layout in tq.h)

def tq_kivi_bytes_per_token(head_dim: int) -> int:
    return int(_lib().tq_kivi_bytes_per_token(head_dim))


class KiviStore:
    """Device arrays of a KIVI store, [n_slices][capacity][...] each (capacity a multiple of 32)."""

    def __init__(self, head_dim: int, n_slices: int, capacity: int, device="cuda"):
        import torch
        if capacity % 32:
            raise ValueError("capacity must be a multiple of 32")
        d = head_dim
        self.head_dim, self.n_slices, self.capacity = d, n_slices, capacity
        self.key_codes = torch.zeros((n_slices, capacity, d // 16), dtype=torch.int32, device=device)
        self.key_scale = torch.zeros((n_slices, capacity // 32, d), dtype=torch.int16, device=device)
        self.key_zero = torch.zeros((n_slices, capacity // 32, d), dtype=torch.int16, device=device)
        self.val_codes = torch.zeros((n_slices, capacity, d // 16), dtype=torch.int32, device=device)
        self.val_params = torch.zeros((n_slices, capacity, 2), dtype=torch.int16, device=device)

    def struct(self, slice_offset: int = 0) -> tq_kivi_store:
        return tq_kivi_store(self.key_codes[slice_offset:].data_ptr(), self.key_scale[slice_offset:].data_ptr(),
                             self.key_zero[slice_offset:].data_ptr(), self.val_codes[slice_offset:].data_ptr(),
                             self.val_params[slice_offset:].data_ptr(), self.capacity)


def tq_kivi_quantize(head_dim: int, k, v, n_slices: int, n_tokens: int, dst: tq_kivi_store, dst_token0: int,
                     stream=None):
    _kv_pair(k, v, max(n_slices, 0) * max(n_tokens, 0) * head_dim)
    _on_one_gpu(("k", k), ("v", v))
    st = _lib().tq_kivi_quantize(head_dim, _ptr(k), _ptr(v), _dtype_code(k), n_slices, n_tokens, ctypes.byref(dst),
                                 dst_token0, _stream(stream))
    _check("tq_kivi_quantize", st)


def tq_kivi_decode_workspace_bytes(head_dim: int, batch: int, n_q_heads: int, n_kv_heads: int,
                                   max_context: int) -> int:
    return int(_lib().tq_kivi_decode_workspace_bytes(head_dim, batch, n_q_heads, n_kv_heads, max_context))


def new_kivi_workspace(head_dim: int, batch: int, n_q_heads: int, n_kv_heads: int, max_context: int, device="cuda"):
    import torch
    n = tq_kivi_decode_workspace_bytes(head_dim, batch, n_q_heads, n_kv_heads, max_context)
    if n == 0:
        raise TqError("tq_kivi_decode_workspace_bytes", TQ_ERR_INVALID_ARG)
    return torch.empty(n, dtype=torch.uint8, device=device)


def tq_kivi_decode_attention(head_dim: int, q, batch: int, n_q_heads: int, n_kv_heads: int, src: tq_kivi_store,
                             n_packed: int, softmax_scale: float, out, workspace, stream=None):
    import torch
    _need("q", q, batch * n_q_heads * head_dim)
    _dtype_code(q)
    _need("out", out, batch * n_q_heads * head_dim, torch.float32)
    _need("workspace", workspace, 0)
    _on_one_gpu(("q", q), ("out", out), ("workspace", workspace))
    st = _lib().tq_kivi_decode_attention(head_dim, _ptr(q), _dtype_code(q), batch, n_q_heads, n_kv_heads,
                                         ctypes.byref(src), n_packed, softmax_scale, _ptr(out), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream))
    _check("tq_kivi_decode_attention", st)
