"""GPU parity at the full workload sizes, in the launch configuration the benchmark
uses: the whole cache of every workload is compressed on the GPU, then sampled records
are checked against the oracle (quantize rule) and sampled batch elements are decoded by
the oracle over the full context (decode rule).  Rules: tests/gpu_common.py."""
import math

import numpy as np
import pytest

import oracle as O
import tq_workloads as W
import compressed_decode_attention_02_amd as tq

pytestmark = pytest.mark.gpu

from gpu_common import Env, assert_decode_close, check_quantize, dev_to_stored, log, oracle_decode  # noqa: E402

SAMPLE_ROWS = 1536


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    return t


def _build(torch, w: W.Workload):
    """Device inputs, packed store (all layers) and ring exactly as the benchmark builds them."""
    dev = torch.device("cuda:0")
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size)
    n_layer = w.batch * w.hkv
    n_sl = w.layers * n_layer
    Ks, Vs = [], []
    for layer in range(w.layers):
        k, v = W.device_kv(w, layer, w.n_packed, dev)
        Ks.append(k.reshape(n_layer, w.n_packed, w.d))
        Vs.append(v.reshape(n_layer, w.n_packed, w.d))
    K = torch.cat(Ks) if w.layers > 1 else Ks[0]
    V = torch.cat(Vs) if w.layers > 1 else Vs[0]
    del Ks, Vs
    store = tq.PackedStore(env.cfg, n_sl, w.n_packed + w.buffer_size, device=dev)
    tq.tq_quantize_kv(env.cfg, env.tables, K, V, n_sl, w.n_packed, store.struct(), 0)
    ring = tq.Ring(env.cfg, n_sl, device=dev)
    for t in range(w.n_ring):
        kn, vn = W.device_kv(w, 5000 + t, 1, dev, tensor_ids=(3, 4))
        kn = kn.reshape(n_layer, w.d).repeat(w.layers, 1).contiguous()
        vn = vn.reshape(n_layer, w.d).repeat(w.layers, 1).contiguous()
        tq.tq_append_ring(env.cfg, ring.struct(), kn, vn, n_sl, t)
    torch.cuda.synchronize()
    return env, K, V, store, ring, n_layer, n_sl


def _check_sampled_records(torch, env, w, K, V, store, n_sl, label):
    r = np.random.default_rng(w.cid)
    sl = r.integers(0, n_sl, SAMPLE_ROWS)
    tk = r.integers(0, w.n_packed, SAMPLE_ROWS)
    # always include the ragged ends of the range
    sl[:4] = [0, 0, n_sl - 1, n_sl - 1]
    tk[:4] = [0, w.n_packed - 1, 0, w.n_packed - 1]
    isl = torch.as_tensor(sl, device=K.device)
    itk = torch.as_tensor(tk, device=K.device)
    k_rows = dev_to_stored(K[isl, itk]).astype(np.float64)
    v_rows = dev_to_stored(V[isl, itk]).astype(np.float64)
    kw = store.key_words[isl, itk].cpu().numpy().view(np.uint32)
    kn = store.key_norms[isl, itk].cpu().numpy()
    vw = store.val_words[isl, itk].cpu().numpy().view(np.uint32)
    vs = store.val_scales[isl, itk].cpu().numpy().view(np.uint16)
    st = check_quantize(env, k_rows, v_rows, kw, kn, vw, vs, label=label)
    log(f"{label}: sampled records {st}")


def _decode_sampled(torch, env, w, store, ring, n_layer, layer, b_list, label):
    dev = store.key_words.device
    q = W.device_queries(w, layer, dev)
    out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device=dev)
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, w.n_packed + w.buffer_size, device=dev)
    off = layer * n_layer
    tq.tq_decode_attention(env.cfg, env.tables, q, w.batch, w.hq, w.hkv, store.struct(off), w.n_packed,
                           ring.struct(off), w.n_ring, 1.0 / math.sqrt(w.d), out, ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    q_stored = dev_to_stored(q).astype(np.float64)
    ref = oracle_decode(env, q_stored, w.hq, w.hkv, store, w.n_packed, ring, w.n_ring, slice_offset=off,
                        b_list=b_list)
    assert_decode_close(g[b_list], ref, f"{label} layer {layer} b {b_list}")


def _prefill_sampled(torch, env, w, store, T, picks, label):
    """Prefill attention over layer 0's packed history as the benchmark times it (the last T
    tokens of every sequence as causal query tokens, one call); the sampled (sequence, query
    token) pairs are decoded by the oracle over their causal prefix."""
    dev = store.key_words.device
    pos0 = w.n_packed - T
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.cid * 1000 + 29)
    dt = torch.bfloat16 if w.in_dtype == "bf16" else torch.float32
    q = torch.randn((w.batch, T, w.hq, w.d), generator=gen, device=dev, dtype=torch.float32).to(dt)
    out = torch.zeros((w.batch, T, w.hq, w.d), dtype=torch.float32, device=dev)
    ws = tq.new_prefill_workspace(env.cfg, w.batch, T, w.hq, w.hkv, w.n_packed)
    scale = 1.0 / math.sqrt(w.d)
    tq.tq_prefill_attention(env.cfg, env.tables, q, w.batch, T, w.hq, w.hkv, store.struct(0), w.n_packed, pos0, True,
                            scale, out, ws)
    torch.cuda.synchronize()
    for b, i in picks:
        sl = slice(b * w.hkv, (b + 1) * w.hkv)
        P = dict(kw=store.key_words[sl].cpu().numpy().view(np.uint32), kn=store.key_norms[sl].cpu().numpy(),
                 vw=store.val_words[sl].cpu().numpy().view(np.uint32),
                 vs=store.val_scales[sl].cpu().numpy().view(np.uint16))
        qs = dev_to_stored(q[b, i]).astype(np.float64)[None, None]
        ref = O.prefill(d=w.d, kb=w.key_bits, vb=w.value_bits, c32=env.c32, sigma=env.sigma, S_bits=env.S, B=1, T=1,
                        Hq=w.hq, Hkv=w.hkv, kw=P["kw"], kn=P["kn"], vw=P["vw"], vs=P["vs"], cap=store.capacity,
                        n_packed=w.n_packed, q=qs, pos0=pos0 + i, causal=True, scale=scale)
        g = out[b, i].cpu().numpy().astype(np.float64)[None, None]
        assert_decode_close(g, ref, f"{label} prefill T={T} sequence {b} query token {i}")


def test_full_llama_b1_32k(torch):
    w = W.WORKLOADS[2]
    env, K, V, store, ring, n_layer, n_sl = _build(torch, w)
    _check_sampled_records(torch, env, w, K, V, store, n_sl, w.name)
    _decode_sampled(torch, env, w, store, ring, n_layer, 0, [0], w.name)
    del K, V
    _prefill_sampled(torch, env, w, store, 512, [(0, 0), (0, 511)], w.name)


def test_full_batched_8k_v4(torch):
    w = W.WORKLOADS[3]
    env, K, V, store, ring, n_layer, n_sl = _build(torch, w)
    _check_sampled_records(torch, env, w, K, V, store, n_sl, w.name)
    _decode_sampled(torch, env, w, store, ring, n_layer, 0, [0, 17, 31], w.name)
    del K, V
    _prefill_sampled(torch, env, w, store, 512, [(0, 0), (13, 300), (31, 511)], w.name)


def test_full_d256_16k(torch):
    w = W.WORKLOADS[4]
    env, K, V, store, ring, n_layer, n_sl = _build(torch, w)
    _check_sampled_records(torch, env, w, K, V, store, n_sl, w.name)
    _decode_sampled(torch, env, w, store, ring, n_layer, 0, [0, 7], w.name)
    del K, V
    _prefill_sampled(torch, env, w, store, 512, [(0, 0), (7, 511)], w.name)


def test_full_32_layers_b4_32k(torch):
    w = W.WORKLOADS[5]
    env, K, V, store, ring, n_layer, n_sl = _build(torch, w)
    _check_sampled_records(torch, env, w, K, V, store, n_sl, w.name)
    del K, V
    torch.cuda.empty_cache()
    for layer, b_list in ((0, [0]), (31, [3])):
        _decode_sampled(torch, env, w, store, ring, n_layer, layer, b_list, w.name)
