"""Prefill attention over the packed cache (tq_prefill_attention) against the oracle's prefill
on the same packed bytes: causal and full windows, the tiled kernel (query tiles of 128 rows,
64 at head_dim 256: every key width, head_dim 64, 128 and 256, G = 1 to 8, ragged last
tiles, query tokens before and past the history's end) and the decode kernels for launches of
few query rows, paged stores."""
import math

import numpy as np
import pytest

import oracle as O
import tq_workloads as W
import compressed_decode_attention_02_amd as tq

pytestmark = pytest.mark.gpu

from gpu_common import Env, assert_decode_close, dev_to_stored, log, packed_to_np, quantize_gpu, to_dev  # noqa: E402


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    return t


def _prefill_case(torch, w: W.Workload, T: int, pos0: int, causal: bool, label: str, paged=None, q_dtype=None,
                  q_scale=1.0):
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size, kb=w.key_bits)
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, w.n_packed)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    if paged:
        pt, pps = paged
        store = tq.PagedStore(env.cfg, n_sl, pt, pps, n_sl * pps + 3, seed=11)
        quantize_gpu(env, to_dev(k, w.in_dtype), to_dev(v, w.in_dtype), n_sl, w.n_packed, store=store)
    else:
        store = quantize_gpu(env, to_dev(k, w.in_dtype), to_dev(v, w.in_dtype), n_sl, w.n_packed)
    r = np.random.default_rng(31)
    q = (q_scale * r.standard_normal((w.batch, T, w.hq, w.d))).astype(np.float32)
    qd = to_dev(q.reshape(-1, w.d), q_dtype or w.in_dtype)
    out = torch.zeros((w.batch, T, w.hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.new_prefill_workspace(env.cfg, w.batch, T, w.hq, w.hkv, w.n_packed)
    scale = 1.0 / math.sqrt(w.d)
    tq.tq_prefill_attention(env.cfg, env.tables, qd, w.batch, T, w.hq, w.hkv, store.struct(), w.n_packed, pos0,
                            causal, scale, out, ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    if paged:
        P = {k_: v_ for k_, v_ in store.gather().items()}
        P = dict(kw=P["key_words"].view(np.uint32), kn=P["key_norms"], vw=P["val_words"].view(np.uint32),
                 vs=P["val_scales"].view(np.uint16))
        cap = store.capacity
    else:
        P = packed_to_np(store)
        cap = store.capacity
    qs = dev_to_stored(qd).astype(np.float64).reshape(w.batch, T, w.hq, w.d)
    ref = O.prefill(d=w.d, kb=w.key_bits, vb=w.value_bits, c32=env.c32, sigma=env.sigma, S_bits=env.S, B=w.batch,
                    T=T, Hq=w.hq, Hkv=w.hkv, kw=P["kw"], kn=P["kn"], vw=P["vw"], vs=P["vs"], cap=cap,
                    n_packed=w.n_packed, q=qs, pos0=pos0, causal=causal, scale=scale)
    empty = np.abs(ref).max(axis=-1) == 0
    assert not g[empty].any(), f"{label}: query tokens with no packed token must give zeros"
    live = ~empty.all(axis=-1)
    assert_decode_close(g[live], ref[live], label)
    return g, store, env, qd, ws


def test_prefill_d128_causal_and_full(torch):
    w = W.custom(2, batch=2, hq=8, hkv=2, n_packed=700)
    _prefill_case(torch, w, 37, 700 - 37, True, "d128 causal, the prompt's last 37 tokens")
    _prefill_case(torch, w, 37, 700 - 37, False, "d128 full window")
    # query tokens before the history's end and before its start (positions 0..): the first
    # token attends to one packed token
    _prefill_case(torch, W.custom(2, batch=1, hq=4, hkv=1, n_packed=300), 40, 0, True, "d128 causal from 0")


def test_prefill_d256_and_gqa(torch):
    _prefill_case(torch, W.custom(4, batch=1, hq=4, hkv=2, n_packed=300), 20, 280, True, "d256 G=2 causal")
    _prefill_case(torch, W.custom(2, batch=1, hq=16, hkv=2, n_packed=400), 9, 391, True, "d128 G=8 causal")


def test_prefill_key_widths(torch):
    _prefill_case(torch, W.custom(2, d=64, key_bits=2, batch=2, hq=8, hkv=2, n_packed=500), 33, 467, True,
                  "d64 kb2 causal")
    _prefill_case(torch, W.custom(2, d=128, key_bits=4, batch=1, hq=8, hkv=2, n_packed=260), 12, 0, False,
                  "d128 kb4 full")


def test_prefill_paged_store_matches_contiguous(torch):
    w = W.custom(2, batch=2, hq=8, hkv=2, n_packed=640)
    g1, _, _, _, _ = _prefill_case(torch, w, 17, 623, True, "d128 contiguous")
    g2, paged, _, _, _ = _prefill_case(torch, w, 17, 623, True, "d128 paged", paged=(64, 10))
    np.testing.assert_array_equal(g1, g2)
    assert not paged.table_error()


def test_prefill_tiled_tiles_and_tails(torch):
    # 7 tiles of 128 rows per kv head, the last one ragged; causal from position 0 with more
    # query tokens than packed ones (tokens 150 .. 199 see all 150)
    _prefill_case(torch, W.custom(2, batch=2, hq=8, hkv=2, n_packed=150), 200, 0, True, "d128 G=4 from 0, T > n_packed")
    _prefill_case(torch, W.custom(2, batch=1, hq=2, hkv=2, n_packed=333), 150, 200, True, "d128 G=1 ragged")
    _prefill_case(torch, W.custom(3, batch=2, hq=16, hkv=2, n_packed=333), 11, 322, False, "d128 G=8 vb4 full")
    _prefill_case(torch, W.custom(3, batch=1, hq=8, hkv=4, n_packed=97), 64, 40, True, "d128 G=2 vb4 causal")
    _prefill_case(torch, W.custom(4, batch=1, hq=8, hkv=4, n_packed=170), 50, 120, True, "d256 G=2 vb4 causal")


def test_prefill_tiled_split_ranges(torch):
    # few tiles over a long history: each tile's packed range is split over up to 16
    # workgroups whose partials the decode's merge combines (splits that see none of a row's
    # tokens included: causal rows near the start)
    _prefill_case(torch, W.custom(2, batch=1, hq=8, hkv=2, n_packed=5000), 64, 4936, True, "d128 split, causal at the end")
    _prefill_case(torch, W.custom(2, batch=1, hq=8, hkv=2, n_packed=5000), 40, 100, True, "d128 split, causal near 0")
    _prefill_case(torch, W.custom(4, batch=1, hq=4, hkv=2, n_packed=2100), 40, 0, False, "d256 split, full window")
    _prefill_case(torch, W.custom(2, d=64, key_bits=2, batch=2, hq=4, hkv=1, n_packed=3000), 50, 2950, True,
                  "d64 kb2 split")


def test_prefill_tiled_key_widths(torch):
    for kb in (1, 2, 4):
        _prefill_case(torch, W.custom(2, d=64, key_bits=kb, batch=1, hq=8, hkv=2, n_packed=230), 40, 190, True,
                      f"d64 kb{kb} vb2")
    _prefill_case(torch, W.custom(3, d=64, key_bits=3, batch=1, hq=4, hkv=1, n_packed=75), 24, 51, True, "d64 kb3 vb4")
    _prefill_case(torch, W.custom(3, d=128, key_bits=1, batch=1, hq=8, hkv=2, n_packed=230), 40, 190, True,
                  "d128 kb1 vb4")
    _prefill_case(torch, W.custom(2, d=128, key_bits=2, batch=1, hq=4, hkv=2, n_packed=130), 70, 0, False,
                  "d128 kb2 full")
    _prefill_case(torch, W.custom(3, d=128, key_bits=4, batch=2, hq=8, hkv=2, n_packed=100), 33, 67, True,
                  "d128 kb4 vb4")


def test_prefill_decode_path_for_few_query_rows(torch):
    # fewer rows per kv head than half a tile (T G < 64 at head_dim 128): the decode kernels
    _prefill_case(torch, W.custom(2, batch=2, hq=8, hkv=2, n_packed=700), 5, 695, True, "d128 T=5 (decode kernels)")
    _prefill_case(torch, W.custom(2, d=64, key_bits=1, batch=1, hq=4, hkv=1, n_packed=300), 3, 10, True,
                  "d64 kb1 T=3 (decode kernels)")


def test_prefill_query_dtypes_and_magnitudes(torch):
    # fp32 and fp16 queries through the tiled path's preparation, and queries of very large and
    # very small magnitude (the preparation scales each row by a power of two before its fp16
    # split: no overflow, no subnormals)
    w = W.custom(2, batch=1, hq=8, hkv=2, n_packed=300)
    _prefill_case(torch, w, 40, 260, True, "d128 fp32 queries", q_dtype="f32")
    _prefill_case(torch, w, 40, 260, True, "d128 fp16 queries", q_dtype="f16")
    _prefill_case(torch, w, 40, 260, True, "d128 fp32 queries x 1e4", q_dtype="f32", q_scale=1e4)
    _prefill_case(torch, w, 40, 260, True, "d128 fp32 queries x 1e-4", q_dtype="f32", q_scale=1e-4)
    _prefill_case(torch, W.custom(4, batch=1, hq=4, hkv=2, n_packed=200), 30, 170, True, "d256 fp16 queries x 300",
                  q_dtype="f16", q_scale=300.0)
