"""CPU oracle of the KIVI 2-bit asymmetric KV quantiser -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this module.  It shares no code with the GPU library and never imports it.

Method (forum page zingnex.cn "TurboQuant-vLLM：大模型推理的KV缓存量化实战方案", section
"KIVI非对称量化：通道级与Token级混合策略"): keys are quantised per channel and values per
token, each with its own scale and zero point (asymmetric), at 2 bits; the memory table of
the same page lists KIVI 2-bit beside TurboQuant.

Readings (the page gives no more than the above):
  * 2 bits: 4 levels, code = clamp(round((x - zero) / scale), 0, 3), x^ = code scale + zero,
    with zero = the minimum and scale = (maximum - minimum) / 3 of the quantised set;
    round = to nearest, ties to even.
  * a key channel's scale and zero cover a group of 32 consecutive tokens (the page's "per
    channel" needs a set of tokens to take the minimum and maximum over; 32 = the value
    group of the TurboQuant records); a value token's pair covers its head_dim entries.
  * stored format (this library's choice): scale and zero as binary16; scale = binary16 of
    the binary32 quotient fp32(fp32(max - min) / 3); zero = binary16(min); the code from the
    binary32 quotient fp32(x - zero) / fp32(scale) (0 where the scale is 0).  Those binary32
    steps are part of the format's definition, so they are written out here with numpy's
    binary32 arithmetic (IEEE, correctly rounded).
  * attention (decode) is the plain definition over the dequantised keys and values,
    softmax(scale q . k^) v^, in double precision.
"""
from __future__ import annotations

import numpy as np

LEVELS = 3   # 2 bits: codes 0 .. 3
GROUP = 32   # tokens per key scale / zero


def asym_params(mn, mx):
    """(scale, zero) as binary16 arrays for minima `mn` and maxima `mx` (any shape)."""
    mn32 = np.asarray(mn, np.float32)
    mx32 = np.asarray(mx, np.float32)
    span = (mx32 - mn32).astype(np.float32)
    scale = (span / np.float32(LEVELS)).astype(np.float32).astype(np.float16)
    zero = mn32.astype(np.float16)
    return scale, zero


def asym_codes(x, scale, zero):
    """Codes 0 .. 3 of `x` under binary16 (scale, zero) broadcast against it."""
    x32 = np.asarray(x, np.float32)
    s32 = np.asarray(scale, np.float16).astype(np.float32)
    z32 = np.asarray(zero, np.float16).astype(np.float32)
    num = (x32 - z32).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qt = (num / np.where(s32 == 0, np.float32(1), s32)).astype(np.float32)
    code = np.clip(np.rint(qt.astype(np.float64)), 0, LEVELS)
    code = np.where(s32 == 0, 0, code)
    return code.astype(np.uint8)


def quantize_keys(k):
    """k [T, D] (T a multiple of 32): codes [T, D], scale and zero [T / 32, D] (binary16),
    per channel over each group of 32 tokens."""
    k = np.asarray(k, np.float64)
    T, D = k.shape
    assert T % GROUP == 0
    kg = k.reshape(T // GROUP, GROUP, D)
    scale, zero = asym_params(kg.min(axis=1), kg.max(axis=1))
    codes = asym_codes(kg, scale[:, None, :], zero[:, None, :]).reshape(T, D)
    return codes, scale, zero


def quantize_values(v):
    """v [T, D]: codes [T, D], scale and zero [T] (binary16), per token over its D entries."""
    v = np.asarray(v, np.float64)
    scale, zero = asym_params(v.min(axis=1), v.max(axis=1))
    codes = asym_codes(v, scale[:, None], zero[:, None])
    return codes, scale, zero


def dequant_keys(codes, scale, zero):
    T, D = codes.shape
    s = np.repeat(np.asarray(scale, np.float16).astype(np.float64), GROUP, axis=0)
    z = np.repeat(np.asarray(zero, np.float16).astype(np.float64), GROUP, axis=0)
    return codes.astype(np.float64) * s[:T] + z[:T]


def dequant_values(codes, scale, zero):
    s = np.asarray(scale, np.float16).astype(np.float64)[:, None]
    z = np.asarray(zero, np.float16).astype(np.float64)[:, None]
    return codes.astype(np.float64) * s + z


def pack_codes(codes):
    """[T, D] codes 0 .. 3 -> [T, D / 16] uint32, channel c at bits 2 (c % 16) of word c / 16."""
    T, D = codes.shape
    c = codes.astype(np.uint32).reshape(T, D // 16, 16)
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    return np.bitwise_or.reduce(c << shifts, axis=2).astype(np.uint32)


def unpack_codes(words, D):
    w = np.asarray(words, np.uint32)
    T = w.shape[0]
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, :]
    return ((w[:, :, None] >> shifts) & 3).reshape(T, D).astype(np.uint8)


def decode(q, keys, values, scale):
    """Attention of q [B, Hq, D] over dequantised keys / values [B * Hkv][T][D] (query head h
    reads kv head h / (Hq / Hkv)), softmax(scale q . k) v, in double precision."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv = len(keys) // B
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            K = keys[b * Hkv + h // G]
            V = values[b * Hkv + h // G]
            if K.shape[0] == 0:
                continue
            s = scale * (K @ q[b, h])
            p = np.exp(s - s.max())
            out[b, h] = (p @ V) / p.sum()
    return out
