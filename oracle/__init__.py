"""CPU oracle for the TurboQuant KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It wraps ``tq_oracle.c`` (plain C, double precision) with
numpy in/out.  It shares no code with the GPU library and never imports it.

Method (pages): hotelren.com guide "企业官网建设流程全解析", section 二 -- rotation,
Lloyd-Max codebook for a Beta law, QJL residual sign bit, 2/4-bit values in groups of
32, bit packing; section 5.1 -- exact recent ring buffer plus compressed history.
Readings of what the pages leave open are stated in ``tq_oracle.c``'s header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtq_oracle.so")
_lib = None

_dp = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_fp = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_u8 = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i8 = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_u16 = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u32 = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build() -> str:
    """Compile tq_oracle.c with gcc into libtq_oracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    L = ctypes.CDLL(_LIB_PATH)
    L.orc_f16_to_double.restype = ctypes.c_double
    L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
    L.orc_double_to_f16.restype = ctypes.c_uint16
    L.orc_double_to_f16.argtypes = [ctypes.c_double]
    L.orc_splitmix64_at.restype = ctypes.c_uint64
    L.orc_splitmix64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.orc_tables.restype = None
    L.orc_tables.argtypes = [_int, ctypes.c_uint64, _i8, _u16]
    L.orc_codebook.restype = _int
    L.orc_codebook.argtypes = [_int, _int, _dp, _dp]
    L.orc_stored_codebook.restype = _int
    L.orc_stored_codebook.argtypes = [_int, _int, _dp, _dp]
    L.orc_coord_cdf.restype = ctypes.c_double
    L.orc_coord_cdf.argtypes = [_int, ctypes.c_double]
    L.orc_coord_moment.restype = ctypes.c_double
    L.orc_coord_moment.argtypes = [_int, ctypes.c_double, ctypes.c_double]
    L.orc_hadamard_entry.restype = ctypes.c_double
    L.orc_hadamard_entry.argtypes = [_int, _int]
    L.orc_rotate.restype = None
    L.orc_rotate.argtypes = [_int, _i8, _dp, _dp]
    L.orc_quantize_keys.restype = None
    L.orc_quantize_keys.argtypes = [_int, _int, _dp, _dp, _i8, _u16, _dp, _i64,
                                    _u8, _u8, _dp, _dp, _dp, _dp, ctypes.c_void_p]
    L.orc_quantize_values.restype = None
    L.orc_quantize_values.argtypes = [_int, _int, _int, _dp, _i64, _u8, _u16, _dp]
    L.orc_pack_keys.restype = None
    L.orc_pack_keys.argtypes = [_int, _int, _u8, _u8, _i64, _u32]
    L.orc_unpack_keys.restype = None
    L.orc_unpack_keys.argtypes = [_int, _int, _u32, _i64, _u8, _u8]
    L.orc_key_words.restype = _int
    L.orc_key_words.argtypes = [_int, _int]
    L.orc_pack_values.restype = None
    L.orc_pack_values.argtypes = [_int, _int, _u8, _i64, _u32]
    L.orc_unpack_values.restype = None
    L.orc_unpack_values.argtypes = [_int, _int, _u32, _i64, _u8]
    L.orc_decode.restype = None
    L.orc_decode.argtypes = [_int, _int, _int, _int, _dp, _i8, _u16, _int, _int, _int,
                             _u32, _fp, _u32, _u16, _i64, _i64, _u16, _u16, _int, _int,
                             _dp, ctypes.c_double, _dp, ctypes.c_void_p]
    _lib = L
    return L


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ----------------------------------------------------------------------------- scalars

def f16_to_double(bits: int) -> float:
    return lib().orc_f16_to_double(int(bits))


def double_to_f16(x: float) -> int:
    return int(lib().orc_double_to_f16(float(x)))


def f16_bits_to_array(bits: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_f16_to_double(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


def f16_bits_fast(bits: np.ndarray) -> np.ndarray:
    """fp16 bits -> double via a 65536-entry table built from the oracle's decoder."""
    global _F16_TABLE
    if _F16_TABLE is None:
        L = lib()
        _F16_TABLE = np.array([L.orc_f16_to_double(i) for i in range(65536)], dtype=np.float64)
    return _F16_TABLE[np.asarray(bits, dtype=np.uint16)]


_F16_TABLE = None


def splitmix64_at(seed: int, i: int) -> int:
    return int(lib().orc_splitmix64_at(seed, i))


# ----------------------------------------------------------------------------- tables

def codebook(d: int, kb: int):
    """fp64 Lloyd-Max centroids (2^kb) and boundaries (2^kb - 1); returns (c, b, iters)."""
    L = 1 << kb
    c = np.zeros(L, np.float64)
    b = np.zeros(L - 1, np.float64)
    it = lib().orc_codebook(d, kb, c, b)
    if it < 0:
        raise ValueError("bad codebook arguments")
    return c, b, it


def stored_codebook(d: int, kb: int):
    """The table values the library stores and uses (a storage format choice, not a reading
    of the pages): centroids rounded to fp16, boundaries the exact midpoints of adjacent
    stored centroids (both returned as doubles)."""
    c = np.zeros(1 << kb, np.float64)
    b = np.zeros((1 << kb) - 1, np.float64)
    if lib().orc_stored_codebook(d, kb, c, b) < 0:
        raise ValueError("bad codebook arguments")
    return c, b


def tables(d: int, seed: int):
    """(sigma int8[d], S fp16 bits uint16[d, d]) from the seeded splitmix64 stream."""
    sigma = np.zeros(d, np.int8)
    S = np.zeros(d * d, np.uint16)
    lib().orc_tables(d, seed, sigma, S)
    return sigma, S.reshape(d, d)


def coord_cdf(d: int, t: float) -> float:
    return lib().orc_coord_cdf(d, t)


def coord_moment(d: int, a: float, b: float) -> float:
    return lib().orc_coord_moment(d, a, b)


def hadamard(d: int) -> np.ndarray:
    L = lib()
    return np.array([[L.orc_hadamard_entry(i, j) for j in range(d)] for i in range(d)])


def rotate(sigma: np.ndarray, x: np.ndarray) -> np.ndarray:
    d = sigma.shape[0]
    x = _c(x, np.float64).reshape(-1, d)
    out = np.zeros_like(x)
    for r in range(x.shape[0]):
        row = np.zeros(d)
        lib().orc_rotate(d, _c(sigma, np.int8), _c(x[r], np.float64), row)
        out[r] = row
    return out


# ----------------------------------------------------------------------------- quantize

def quantize_keys(k: np.ndarray, c32, b32, sigma, S_bits, kb: int = 3, force_idx=None):
    """k: [rows, d] (values as stored).  Returns dict with idx, z, norm, rnorm, margins.
    force_idx: optional [rows, d] codebook indices to use instead of the nearest cell."""
    k = _c(k, np.float64)
    rows, d = k.shape
    idx = np.zeros((rows, d), np.uint8)
    z = np.zeros((rows, d), np.uint8)
    n = np.zeros(rows, np.float64)
    g = np.zeros(rows, np.float64)
    um = np.zeros((rows, d), np.float64)
    pm = np.zeros((rows, d), np.float64)
    lib().orc_quantize_keys(d, kb, _c(c32, np.float64), _c(b32, np.float64), _c(sigma, np.int8),
                            _c(S_bits, np.uint16).ravel(), k, rows, idx, z, n, g, um, pm,
                            None if force_idx is None else
                            _c(force_idx, np.uint8).ctypes.data_as(ctypes.c_void_p))
    return {"idx": idx, "z": z, "norm": n, "rnorm": g, "u_margin": um, "p_margin": pm}


def quantize_values(v: np.ndarray, vb: int, group: int = 32):
    v = _c(v, np.float64)
    rows, d = v.shape
    code = np.zeros((rows, d), np.uint8)
    sc = np.zeros((rows, d // group), np.uint16)
    m = np.zeros((rows, d), np.float64)
    lib().orc_quantize_values(d, vb, group, v, rows, code, sc, m)
    return {"code": code, "scale": sc, "margin": m}


def key_words(d: int, kb: int = 3) -> int:
    """Words of one key record: (kb + 1) d / 32 (kb codebook bits and one sign bit per coordinate)."""
    return lib().orc_key_words(d, kb)


def pack_keys(idx, z, kb: int = 3) -> np.ndarray:
    idx = _c(idx, np.uint8)
    rows, d = idx.shape
    out = np.zeros((rows, key_words(d, kb)), np.uint32)
    lib().orc_pack_keys(d, kb, idx, _c(z, np.uint8), rows, out)
    return out


def unpack_keys(words, d: int, kb: int = 3):
    words = _c(words, np.uint32).reshape(-1, key_words(d, kb))
    rows = words.shape[0]
    idx = np.zeros((rows, d), np.uint8)
    z = np.zeros((rows, d), np.uint8)
    lib().orc_unpack_keys(d, kb, words, rows, idx, z)
    return idx, z


def pack_values(code, vb: int) -> np.ndarray:
    code = _c(code, np.uint8)
    rows, d = code.shape
    out = np.zeros((rows, d * vb // 32), np.uint32)
    lib().orc_pack_values(d, vb, code, rows, out)
    return out


def unpack_values(words, d: int, vb: int) -> np.ndarray:
    words = _c(words, np.uint32).reshape(-1, d * vb // 32)
    rows = words.shape[0]
    code = np.zeros((rows, d), np.uint8)
    lib().orc_unpack_values(d, vb, words, rows, code)
    return code


def dequant_values(code, scale_bits, vb: int, group: int = 32) -> np.ndarray:
    """Bin-centre reconstruction (code - 2^(vb-1) + 1/2) * s."""
    code = np.asarray(code, np.float64)
    s = f16_bits_fast(scale_bits)
    return (code - (1 << (vb - 1)) + 0.5) * np.repeat(s, group, axis=-1)


# ----------------------------------------------------------------------------- decode

def decode(*, d, kb, vb, c32, sigma, S_bits, B, Hq, Hkv, kw, kn, vw, vs, cap, n_packed,
           rk, rv, buf, n_ring, q, scale, group=32, want_scores=False):
    """Hybrid decode attention in fp64.  Array layouts as in tq_oracle.c (orc_decode)."""
    out = np.zeros((B, Hq, d), np.float64)
    T = n_packed + n_ring
    scores = np.zeros((B, Hq, max(T, 1)), np.float64) if want_scores else None
    empty32 = np.zeros(1, np.uint32)
    empty16 = np.zeros(1, np.uint16)
    emptyf = np.zeros(2, np.float32)
    lib().orc_decode(
        d, kb, vb, group, _c(c32, np.float64), _c(sigma, np.int8), _c(S_bits, np.uint16).ravel(),
        B, Hq, Hkv,
        _c(kw, np.uint32).ravel() if kw is not None else empty32,
        _c(kn, np.float32).ravel() if kn is not None else emptyf,
        _c(vw, np.uint32).ravel() if vw is not None else empty32,
        _c(vs, np.uint16).ravel() if vs is not None else empty16,
        cap, n_packed,
        _c(rk, np.uint16).ravel() if rk is not None else empty16,
        _c(rv, np.uint16).ravel() if rv is not None else empty16,
        buf, n_ring, _c(q, np.float64).ravel(), float(scale), out.ravel(),
        scores.ctypes.data_as(ctypes.c_void_p) if want_scores else None)
    return (out, scores) if want_scores else out


def prefill(*, d, kb, vb, c32, sigma, S_bits, B, T, Hq, Hkv, kw, kn, vw, vs, cap, n_packed, q, pos0, causal,
            scale, group=32):
    """Prefill attention over the packed cache (guide section 三, full_tq): query token i of
    sequence b, q [B][T][Hq][d], is a decode query over that sequence's packed tokens
    [0, min(n_packed, pos0 + i + 1)) when causal, else [0, n_packed); a token with nothing to
    attend to gives zeros.  Store arrays as in decode ([B*Hkv][cap][...])."""
    out = np.zeros((B, T, Hq, d), np.float64)
    for b in range(B):
        sl = slice(b * Hkv, (b + 1) * Hkv)
        for i in range(T):
            n = min(n_packed, pos0 + i + 1) if causal else n_packed
            if n <= 0:
                continue
            out[b, i] = decode(d=d, kb=kb, vb=vb, c32=c32, sigma=sigma, S_bits=S_bits, B=1, Hq=Hq, Hkv=Hkv,
                               kw=kw[sl], kn=kn[sl], vw=vw[sl], vs=vs[sl], cap=cap, n_packed=n, rk=None, rv=None,
                               buf=0, n_ring=0, q=q[b, i][None], scale=scale, group=group)[0]
    return out

