"""Seeded synthetic workloads for the TurboQuant KV-cache hot path.

This module holds only input generation (shapes, seeded random draws, rounding of the
draws to their storage dtype).  It holds none of the method's arithmetic, and both the
GPU library's tests/benchmark and the CPU oracle take their inputs from here.

Workload laws (stand-ins for real model activations; no dataset is involved):
  * keys / values / queries ~ N(0, 1), drawn in fp32 and rounded to the stored dtype;
  * "outlier" key channels: a seeded choice of channels per (layer, kv head) scaled up;
  * heavy-tailed keys: every entry Student-t with nu = 3.
Seeds: numpy PCG64 with SeedSequence([config id, layer, tensor id]) on the host, or a
torch Philox generator seeded from the same triple on the device; tensor ids are
K=0, V=1, Q=2, new-token K=3, new-token V=4, outlier channels=5.
"""
from __future__ import annotations

import dataclasses

import numpy as np

TABLE_SEED = 0x7105EED  # seed of the rotation signs and the QJL matrix


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    d: int
    n_packed: int        # tokens in the compressed history per sequence
    n_ring: int          # exact recent tokens held in the ring buffer
    value_bits: int
    in_dtype: str        # "f32" | "bf16"
    key_law: str         # "outlier" | "student_t"
    outlier_channels: int
    outlier_scale: float
    outliers_in_values: bool
    key_bits: int = 3
    group: int = 32
    buffer_size: int = 128

    @property
    def g(self) -> int:
        return self.hq // self.hkv

    @property
    def context(self) -> int:
        return self.n_packed + self.n_ring

    @property
    def slices(self) -> int:
        return self.layers * self.batch * self.hkv


WORKLOADS = {
    1: Workload(1, "tiny_d128_t512", 1, 1, 4, 1, 128, 512, 0, 2, "f32", "outlier", 4, 20.0, True),
    2: Workload(2, "llama3_8b_b1_ctx32k", 1, 1, 32, 8, 128, 32640, 128, 2, "bf16", "outlier", 3, 15.0, False),
    3: Workload(3, "llama3_8b_b32_ctx8k_v4", 1, 32, 32, 8, 128, 8128, 64, 4, "bf16", "outlier", 3, 15.0, False),
    4: Workload(4, "d256_b8_ctx16k_v4_t3", 1, 8, 16, 8, 256, 16256, 128, 4, "bf16", "student_t", 0, 1.0, False),
    5: Workload(5, "llama3_8b_32layers_b4_ctx32k", 32, 4, 32, 8, 128, 32768, 1, 2, "bf16", "outlier", 3, 15.0, False),
}


def custom(base: int, **kw) -> Workload:
    """A workload with the law of WORKLOADS[base] but other sizes (for small test cases)."""
    return dataclasses.replace(WORKLOADS[base], **kw)


# --------------------------------------------------------------------------- host side

def rng(cid: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cid, layer, tensor_id])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(w: Workload, layer: int) -> np.ndarray:
    """[hkv, n_out] seeded channel indices per kv head (the same set for K and, if enabled, V)."""
    r = rng(w.cid, layer, 5)
    return np.stack([r.choice(w.d, size=w.outlier_channels, replace=False) for _ in range(w.hkv)]) \
        if w.outlier_channels else np.zeros((w.hkv, 0), np.int64)


def _student_t3(r: np.random.Generator, shape) -> np.ndarray:
    z = r.standard_normal(shape, dtype=np.float32)
    chi = sum(r.standard_normal(shape, dtype=np.float32) ** 2 for _ in range(3))
    return (z * np.sqrt(3.0 / chi)).astype(np.float32)


def host_kv(w: Workload, layer: int, n_tokens: int, tensor_ids=(0, 1)):
    """K and V for one layer as fp32 arrays [batch, hkv, n_tokens, d] holding stored values
    (already rounded to the workload's dtype), plus the stored bit patterns if bf16."""
    out = []
    ch = outlier_channels(w, layer)
    for tid, is_key in zip(tensor_ids, (True, False)):
        r = rng(w.cid, layer, tid)
        shape = (w.batch, w.hkv, n_tokens, w.d)
        if is_key and w.key_law == "student_t":
            x = _student_t3(r, shape)
        else:
            x = r.standard_normal(shape, dtype=np.float32)
        if is_key or w.outliers_in_values:
            for h in range(w.hkv):
                x[:, h, :, ch[h]] *= np.float32(w.outlier_scale)
        out.append(x)
    if w.in_dtype == "bf16":
        bits = [f32_to_bf16_bits(x) for x in out]
        return [bf16_bits_to_f32(b) for b in bits], bits
    return out, None


def host_queries(w: Workload, layer: int):
    """Queries [batch, hq, d] as stored values (fp32 array) and bf16 bits if bf16."""
    x = rng(w.cid, layer, 2).standard_normal((w.batch, w.hq, w.d), dtype=np.float32)
    if w.in_dtype == "bf16":
        b = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(b), b
    return x, None


# --------------------------------------------------------------------------- device side

def device_kv(w: Workload, layer: int, n_tokens: int, device, tensor_ids=(0, 1)):
    """Same laws as host_kv, drawn on the device (torch Philox; a different stream from the
    host generator) for workloads too large to draw on the host.  Returns stored-dtype
    tensors [batch, hkv, n_tokens, d]."""
    import torch

    dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    ch = outlier_channels(w, layer)
    res = []
    for tid, is_key in zip(tensor_ids, (True, False)):
        g = torch.Generator(device=device)
        g.manual_seed((w.cid * 1_000_003 + layer * 1009 + tid) & 0x7FFFFFFFFFFFFFFF)
        shape = (w.batch, w.hkv, n_tokens, w.d)
        if is_key and w.key_law == "student_t":
            z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            chi = torch.zeros_like(z)
            for _ in range(3):
                chi += torch.randn(shape, generator=g, device=device, dtype=torch.float32) ** 2
            x = z * torch.sqrt(3.0 / chi)
        else:
            x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if is_key or w.outliers_in_values:
            for h in range(w.hkv):
                idx = torch.as_tensor(ch[h], device=device)
                x[:, h, :, idx] *= w.outlier_scale
        res.append(x.to(dt))
    return res


def device_queries(w: Workload, layer: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((w.cid * 1_000_003 + layer * 1009 + 2) & 0x7FFFFFFFFFFFFFFF)
    dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    return torch.randn((w.batch, w.hq, w.d), generator=g, device=device, dtype=torch.float32).to(dt)


# --------------------------------------------------------------------------- byte accounting

def fp16_kv_bytes(layers: int, batch: int, heads: int, seq: int, d: int, elem_bytes: int = 2) -> int:
    """Bytes of an uncompressed K+V cache: 2 * B * L * H * T * d * bytes per element."""
    return 2 * batch * layers * heads * seq * d * elem_bytes


def packed_record_bytes(d: int, value_bits: int, key_bits: int = 3, group: int = 32) -> int:
    """Bytes of one packed token-head record in this library's format: key codes and
    sign bits (key_bits + 1 bits per coordinate), two fp32 norms, value codes and one fp16
    scale per group."""
    return d * (key_bits + 1) // 8 + 8 + d * value_bits // 8 + 2 * (d // group)


def nbytes_human(n: float) -> str:
    return f"{n / 2**20:.1f} MiB" if n < 2**30 else f"{n / 2**30:.2f} GiB"

