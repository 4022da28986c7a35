"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare with
the oracle under the comparison rules below.

Quantize (bit-exact except inside the rounding window):
  * key codes: a GPU code may differ from the oracle's only where the oracle's unit-key
    coordinate lies within 1e-6 of a decision boundary; such a row is then re-derived by
    the oracle from the GPU's codes (the residual, and so every sign bit, depends on them);
  * sign bits: may differ only where |S r| < 1e-6 (oracle, on the codes actually stored);
  * value codes and fp16 scales: bit-exact (the floor is exact on both sides);
  * norms: relative error <= 1e-6 against the fp64 values;
  * the count of window cases must be <= 1e-4 of the coordinates.
Decode (fp32 accumulation): per (batch, query head) max|o - o*| / max|o*| <= 2e-3 with
both sides reading the same packed bytes (the acceptance bound), and <= 1e-4 (a regression
bound near what the kernels reach, a few 1e-6: a loss of precision in the hot path, such as
an operand split dropped, fails it).
Window counts: with TQ_PARITY_LOG set to a file path, every quantize comparison appends its
counts to that file as one JSON line.
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

import oracle as O
import tq_workloads as W
import compressed_decode_attention_02_amd as tq

WINDOW = 1e-6
DECODE_TOL = 2e-3
DECODE_REGRESSION = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(x_np, dtype_str, device="cuda"):
    """Stored values (fp32 array) -> device tensor of the storage dtype."""
    torch = torch_mod()
    if dtype_str == "bf16":
        bits = W.f32_to_bf16_bits(x_np)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    if dtype_str == "f16":
        return torch.from_numpy(np.asarray(x_np, np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).to(device)


def dev_to_stored(t):
    """Device tensor (bf16/f16/f32) -> fp32 numpy holding exactly the stored values."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy()


class Env:
    """Library tables on the device plus the oracle's own tables, for one config."""

    def __init__(self, d: int, vb: int, buffer_size: int = 128, seed: int = W.TABLE_SEED, kb: int = 3):
        self.cfg = tq.make_config(d, kb, vb, 32, buffer_size)
        self.tables = tq.Tables(self.cfg, seed)
        self.d, self.vb, self.kb = d, vb, kb
        self.kw = O.key_words(d, kb)  # words of one key record
        self.c32, self.b32 = O.stored_codebook(d, kb)
        self.sigma, self.S = O.tables(d, seed)


def packed_to_np(store: tq.PackedStore):
    return dict(kw=store.key_words.cpu().numpy().view(np.uint32),
                kn=store.key_norms.cpu().numpy(),
                vw=store.val_words.cpu().numpy().view(np.uint32),
                vs=store.val_scales.cpu().numpy().view(np.uint16))


def check_quantize(env: Env, k_rows: np.ndarray, v_rows: np.ndarray, kw, kn, vw, vs, label=""):
    """Compare GPU records (rows aligned with k_rows / v_rows, all [rows, ...]) with the
    oracle.  Returns a dict of window counts.  Raises AssertionError on a violation."""
    d, vb = env.d, env.vb
    rows = k_rows.shape[0]
    ref = O.quantize_keys(k_rows, env.c32, env.b32, env.sigma, env.S, kb=env.kb)
    g_idx, g_z = O.unpack_keys(kw, d, env.kb)
    idx_diff = g_idx != ref["idx"]
    bad_idx = idx_diff & (ref["u_margin"] >= WINDOW)
    assert not bad_idx.any(), f"{label}: key code mismatch outside the window at {np.argwhere(bad_idx)[:5]}"
    n_idx_win = int(idx_diff.sum())
    rows_redo = np.where(idx_diff.any(axis=1))[0]
    if rows_redo.size:
        red = O.quantize_keys(k_rows[rows_redo], env.c32, env.b32, env.sigma, env.S, kb=env.kb,
                              force_idx=g_idx[rows_redo])
        for key in ("z", "rnorm", "p_margin"):
            ref[key][rows_redo] = red[key]
    z_diff = g_z != ref["z"]
    bad_z = z_diff & (ref["p_margin"] >= WINDOW)
    assert not bad_z.any(), f"{label}: sign mismatch outside the window at {np.argwhere(bad_z)[:5]}"
    n_z_win = int(z_diff.sum())
    rel_n = np.abs(kn[:, 0] - ref["norm"]) / np.maximum(ref["norm"], 1e-30)
    rel_g = np.abs(kn[:, 1] - ref["rnorm"]) / np.maximum(ref["rnorm"], 1e-30)
    assert rel_n.max() <= 1e-6, f"{label}: norm rel err {rel_n.max()}"
    assert rel_g.max() <= 1e-6, f"{label}: residual norm rel err {rel_g.max()}"
    vref = O.quantize_values(v_rows, vb)
    g_code = O.unpack_values(vw, d, vb)
    np.testing.assert_array_equal(vs, vref["scale"], err_msg=f"{label}: value scales")
    np.testing.assert_array_equal(g_code, vref["code"], err_msg=f"{label}: value codes")
    total = rows * d
    stats = dict(rows=rows, coords=total, key_window=n_idx_win, sign_window=n_z_win,
                 window_frac=(n_idx_win + n_z_win) / max(total, 1),
                 near_boundary_keys=int((ref["u_margin"] < WINDOW).sum()),
                 near_zero_signs=int((ref["p_margin"] < WINDOW).sum()),
                 value_codes_near_step=int((vref["margin"] < WINDOW).sum()))
    record_windows(label, stats)
    assert stats["window_frac"] <= 1e-4, f"{label}: window cases {stats}"
    return stats


def record_windows(label: str, stats: dict):
    """Append one comparison's window counts to the file named by TQ_PARITY_LOG (if set)."""
    path = os.environ.get("TQ_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": label, **stats}) + "\n")


def quantize_gpu(env: Env, k_dev, v_dev, n_slices: int, n_tokens: int, capacity=None, offset=0, store=None):
    torch = torch_mod()
    if store is None:
        store = tq.PackedStore(env.cfg, n_slices, capacity or n_tokens)
    tq.tq_quantize_kv(env.cfg, env.tables, k_dev, v_dev, n_slices, n_tokens, store.struct(), offset)
    torch.cuda.synchronize()
    return store


def rel_err_per_head(out, ref):
    """max |o - o*| / max |o*| for every (batch, head) row."""
    num = np.abs(out - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return num / den


def run_decode(env: Env, q_np, q_dtype, batch, hq, hkv, store, n_packed, ring, n_ring, slice_offset=0, qd=None):
    """GPU decode through the C ABI; returns (out fp64 numpy, stored queries fp64, workspace)."""
    torch = torch_mod()
    if qd is None:
        qd = to_dev(q_np, q_dtype)
    q_stored = dev_to_stored(qd).astype(np.float64)
    out = torch.zeros((batch, hq, env.d), dtype=torch.float32, device="cuda")
    ws = tq.new_workspace(env.cfg, batch, hq, hkv, n_packed + n_ring)
    tq.tq_decode_attention(env.cfg, env.tables, qd, batch, hq, hkv,
                           store.struct(slice_offset) if store is not None else None, n_packed,
                           ring.struct(slice_offset) if ring is not None else None, n_ring,
                           1.0 / math.sqrt(env.d), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), q_stored, ws


def oracle_decode(env: Env, q_stored, hq, hkv, store, n_packed, ring, n_ring, slice_offset=0, b_list=(0,)):
    """Oracle decode for the batch elements in b_list, reading the same packed bytes and ring
    contents as the GPU (only the slices of those batch elements are copied back)."""
    d = env.d
    outs = []
    for b in b_list:
        sl = slice(slice_offset + b * hkv, slice_offset + (b + 1) * hkv)
        if store is not None and n_packed > 0:
            kw = store.key_words[sl].cpu().numpy().view(np.uint32)
            kn = store.key_norms[sl].cpu().numpy()
            vw = store.val_words[sl].cpu().numpy().view(np.uint32)
            vs = store.val_scales[sl].cpu().numpy().view(np.uint16)
            cap = store.capacity
        else:
            kw = kn = vw = vs = None
            cap = 0
        if ring is not None and n_ring > 0:
            rk = ring.k[sl].cpu().numpy().view(np.uint16)
            rv = ring.v[sl].cpu().numpy().view(np.uint16)
            buf = ring.k.shape[1]
        else:
            rk = rv = None
            buf = 0
        o = O.decode(d=d, kb=env.kb, vb=env.vb, c32=env.c32, sigma=env.sigma, S_bits=env.S, B=1, Hq=hq, Hkv=hkv,
                     kw=kw, kn=kn, vw=vw, vs=vs, cap=cap, n_packed=n_packed, rk=rk, rv=rv, buf=buf,
                     n_ring=n_ring, q=q_stored[b:b + 1], scale=1.0 / math.sqrt(d))
        outs.append(o[0])
    return np.stack(outs)


def assert_decode_close(gpu, ref, label=""):
    err = rel_err_per_head(gpu, ref)
    log(f"{label}: decode max rel err {err.max():.3e} (mean {err.mean():.3e}) over {err.size} heads")
    assert err.max() <= DECODE_TOL, f"{label}: decode rel err {err.max()}"
    assert err.max() <= DECODE_REGRESSION, f"{label}: decode rel err {err.max()} above the regression bound"
    return float(err.max())
