"""GPU parity of the HIP path against the oracle at sizes the oracle finishes in seconds
(several tiles plus ragged tails), through the C ABI.  Rules: tests/gpu_common.py."""
import math

import numpy as np
import pytest

import oracle as O
import tq_workloads as W
import compressed_decode_attention_02_amd as tq

pytestmark = pytest.mark.gpu

from gpu_common import (Env, assert_decode_close, check_quantize, dev_to_stored, log, oracle_decode,  # noqa: E402
                        packed_to_np, quantize_gpu, rel_err_per_head, run_decode, to_dev, torch_mod)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    return t


def _quantize_case(env, w: W.Workload, n_tokens, cap_extra=0, offset=0, label=""):
    (k, v), _ = W.host_kv(w, 0, n_tokens)
    n_slices = w.batch * w.hkv
    k = k.reshape(n_slices, n_tokens, w.d)
    v = v.reshape(n_slices, n_tokens, w.d)
    kd, vd = to_dev(k, w.in_dtype), to_dev(v, w.in_dtype)
    store = quantize_gpu(env, kd, vd, n_slices, n_tokens, capacity=n_tokens + cap_extra + offset, offset=offset)
    P = packed_to_np(store)
    sl = slice(offset, offset + n_tokens)
    st = check_quantize(env, k.reshape(-1, w.d).astype(np.float64), v.reshape(-1, w.d).astype(np.float64),
                        P["kw"][:, sl].reshape(-1, env.kw), P["kn"][:, sl].reshape(-1, 2),
                        P["vw"][:, sl].reshape(-1, w.value_bits * w.d // 32),
                        P["vs"][:, sl].reshape(-1, w.d // 32), label=label)
    # records outside [offset, offset + n_tokens) are untouched (zero)
    if offset:
        assert not P["kw"][:, :offset].any() and not P["vw"][:, :offset].any()
    if cap_extra:
        assert not P["kw"][:, offset + n_tokens:].any()
    log(f"{label}: {st}")
    return store, (k, v)


def test_quantize_tiny_fp32(torch):
    w = W.WORKLOADS[1]
    env = Env(w.d, w.value_bits)
    _quantize_case(env, w, w.n_packed, label="tiny fp32")


def test_quantize_llama_law_ragged_with_offset(torch):
    w = W.custom(2, hkv=8)
    env = Env(w.d, w.value_bits)
    _quantize_case(env, w, 1000, cap_extra=5, offset=37, label="llama-law bf16 v2 ragged")


def test_quantize_d128_32_token_tiles(torch):
    # 12008 rows: enough 32-token tiles for one per CU (smaller inputs at d = 128 run
    # 16-token tiles), with a ragged last tile and slices that end inside tiles
    w = W.custom(2, hkv=8)
    env = Env(w.d, w.value_bits)
    _quantize_case(env, w, 1501, label="llama-law bf16 v2, 32-token tiles")


def test_quantize_value_bits4(torch):
    w = W.custom(3, batch=2, hkv=3)
    env = Env(w.d, w.value_bits)
    _quantize_case(env, w, 333, label="bf16 v4")


def test_quantize_d256_student_t(torch):
    w = W.custom(4, batch=1, hkv=4)
    env = Env(w.d, w.value_bits)
    _quantize_case(env, w, 301, label="d256 t3 v4")


def test_quantize_d256_v2_fp16_input(torch):
    w = W.custom(4, batch=1, hkv=2, value_bits=2, in_dtype="f32")
    env = Env(w.d, 2)
    (k, v), _ = W.host_kv(w, 0, 129)
    k = k.reshape(2, 129, w.d).astype(np.float16).astype(np.float32)
    v = v.reshape(2, 129, w.d).astype(np.float16).astype(np.float32)
    store = quantize_gpu(env, to_dev(k, "f16"), to_dev(v, "f16"), 2, 129)
    P = packed_to_np(store)
    check_quantize(env, k.reshape(-1, w.d).astype(np.float64), v.reshape(-1, w.d).astype(np.float64),
                   P["kw"].reshape(-1, w.d // 8), P["kn"].reshape(-1, 2), P["vw"].reshape(-1, 2 * w.d // 32),
                   P["vs"].reshape(-1, w.d // 32), label="d256 f16 input")


def test_quantize_edge_rows(torch):
    """Zero key, zero value groups, a single huge coordinate, tiny values, a one-token call."""
    env = Env(128, 2)
    r = np.random.default_rng(5)
    k = r.standard_normal((1, 40, 128)).astype(np.float32)
    v = r.standard_normal((1, 40, 128)).astype(np.float32)
    k[0, 0] = 0.0
    v[0, 1, :64] = 0.0
    k[0, 2] = 0.0
    k[0, 2, 77] = 1e4
    v[0, 3] = 1e-6
    v[0, 4, 5] = 300.0
    k[0, 5] = -k[0, 6]
    store = quantize_gpu(env, to_dev(k, "f32"), to_dev(v, "f32"), 1, 40)
    P = packed_to_np(store)
    check_quantize(env, k.reshape(-1, 128).astype(np.float64), v.reshape(-1, 128).astype(np.float64),
                   P["kw"].reshape(-1, 16), P["kn"].reshape(-1, 2), P["vw"].reshape(-1, 8),
                   P["vs"].reshape(-1, 4), label="edge rows")
    one = quantize_gpu(env, to_dev(k[:, :1], "f32"), to_dev(v[:, :1], "f32"), 1, 1)
    np.testing.assert_array_equal(one.key_words.cpu().numpy().view(np.uint32)[0, 0], P["kw"][0, 0])


def test_quantize_is_deterministic(torch):
    w = W.custom(2, hkv=4)
    env = Env(128, 2)
    (k, v), _ = W.host_kv(w, 0, 500)
    kd, vd = to_dev(k.reshape(4, 500, 128), "bf16"), to_dev(v.reshape(4, 500, 128), "bf16")
    a = packed_to_np(quantize_gpu(env, kd, vd, 4, 500))
    b = packed_to_np(quantize_gpu(env, kd, vd, 4, 500))
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_ring_append_is_exact_fp16(torch):
    env = Env(128, 2, buffer_size=16)
    ring = tq.Ring(env.cfg, 6)
    r = np.random.default_rng(8)
    ks, vs = [], []
    for slot in range(16):
        kn = r.standard_normal((6, 128)).astype(np.float32) * 3
        vn = r.standard_normal((6, 128)).astype(np.float32)
        kd, vd = to_dev(kn, "bf16"), to_dev(vn, "bf16")
        tq.tq_append_ring(env.cfg, ring.struct(), kd, vd, 6, slot)
        ks.append(dev_to_stored(kd))
        vs.append(dev_to_stored(vd))
    torch.cuda.synchronize()
    with pytest.raises(tq.TqError):
        tq.tq_append_ring(env.cfg, ring.struct(), kd, vd, 6, 16)
    exp_k = np.stack(ks, 1).astype(np.float16)
    exp_v = np.stack(vs, 1).astype(np.float16)
    np.testing.assert_array_equal(ring.k.cpu().numpy().view(np.uint16), exp_k.view(np.uint16))
    np.testing.assert_array_equal(ring.v.cpu().numpy().view(np.uint16), exp_v.view(np.uint16))


def test_flush_writes_records_after_the_history(torch):
    env = Env(128, 4, buffer_size=128)
    n_sl, n_pk, n_ring = 5, 300, 97
    w = W.custom(3, batch=1, hkv=n_sl)
    (k, v), _ = W.host_kv(w, 0, n_pk + n_ring)
    k = k.reshape(n_sl, -1, 128)
    v = v.reshape(n_sl, -1, 128)
    store = quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :n_pk]), "bf16"),
                         to_dev(np.ascontiguousarray(v[:, :n_pk]), "bf16"), n_sl, n_pk, capacity=n_pk + 128)
    ring = tq.Ring(env.cfg, n_sl)
    for t in range(n_ring):
        tq.tq_append_ring(env.cfg, ring.struct(), to_dev(np.ascontiguousarray(k[:, n_pk + t]), "bf16"),
                          to_dev(np.ascontiguousarray(v[:, n_pk + t]), "bf16"), n_sl, t)
    tq.tq_flush(env.cfg, env.tables, ring.struct(), n_sl, n_ring, store.struct(), n_pk)
    torch.cuda.synchronize()
    P = packed_to_np(store)
    kr = k[:, n_pk:].astype(np.float16).astype(np.float64).reshape(-1, 128)
    vr = v[:, n_pk:].astype(np.float16).astype(np.float64).reshape(-1, 128)
    sl = slice(n_pk, n_pk + n_ring)
    check_quantize(env, kr, vr, P["kw"][:, sl].reshape(-1, 16), P["kn"][:, sl].reshape(-1, 2),
                   P["vw"][:, sl].reshape(-1, 16), P["vs"][:, sl].reshape(-1, 4), label="flush")
    assert not P["kw"][:, n_pk + n_ring:].any()


# ------------------------------------------------------------------------- decode

def _decode_case(w: W.Workload, label, b_list=None, seed_layer=0):
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size, kb=w.key_bits)
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, seed_layer, w.n_packed + w.n_ring)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    store = None
    if w.n_packed:
        store = quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :w.n_packed]), w.in_dtype),
                             to_dev(np.ascontiguousarray(v[:, :w.n_packed]), w.in_dtype), n_sl, w.n_packed)
    ring = None
    if w.n_ring:
        ring = tq.Ring(env.cfg, n_sl)
        for t in range(w.n_ring):
            tq.tq_append_ring(env.cfg, ring.struct(), to_dev(np.ascontiguousarray(k[:, w.n_packed + t]), w.in_dtype),
                              to_dev(np.ascontiguousarray(v[:, w.n_packed + t]), w.in_dtype), n_sl, t)
    q, _ = W.host_queries(w, seed_layer)
    g, q_stored, ws = run_decode(env, q, w.in_dtype, w.batch, w.hq, w.hkv, store, w.n_packed, ring, w.n_ring)
    b_list = list(range(w.batch)) if b_list is None else b_list
    ref = oracle_decode(env, q_stored, w.hq, w.hkv, store, w.n_packed, ring, w.n_ring, b_list=b_list)
    err = assert_decode_close(g[b_list], ref, label)
    return env, store, ring, q, ws, g, err


def test_decode_tiny(torch):
    _decode_case(W.WORKLOADS[1], "tiny")


def test_decode_llama_law_packed_and_ring(torch):
    _decode_case(W.custom(2, n_packed=3000, n_ring=128), "llama-law b1")


def test_decode_batched_v4(torch):
    _decode_case(W.custom(3, batch=3, n_packed=700, n_ring=64), "b3 v4")


def test_decode_d256(torch):
    _decode_case(W.custom(4, batch=2, n_packed=1500, n_ring=128), "d256 v4")


def test_decode_gqa_groups(torch):
    for hq, hkv in ((8, 8), (16, 8), (64, 8)):
        _decode_case(W.custom(2, hq=hq, hkv=hkv, n_packed=600, n_ring=5), f"G={hq // hkv}")
    for hq, hkv in ((8, 8), (32, 8)):
        _decode_case(W.custom(4, batch=1, hq=hq, hkv=hkv, n_packed=600, n_ring=5), f"d256 G={hq // hkv}")


def test_decode_ring_only_and_single_token(torch):
    _decode_case(W.custom(2, n_packed=0, n_ring=77), "ring only")
    _decode_case(W.custom(2, n_packed=1, n_ring=0), "one packed token")
    _decode_case(W.custom(2, n_packed=257, n_ring=1), "257 + 1")


def test_decode_ring_longer_than_one_chunk(torch):
    # the ring is scored in chunks of 128 tokens with a running maximum: several chunks and a
    # ragged last one, with and without packed history, at both head sizes
    _decode_case(W.custom(2, n_packed=400, n_ring=300, buffer_size=512), "d128 ring 300")
    _decode_case(W.custom(2, n_packed=0, n_ring=257, buffer_size=512), "d128 ring only 257")
    _decode_case(W.custom(4, batch=1, n_packed=300, n_ring=200, buffer_size=256), "d256 ring 200")


def test_decode_slices_not_a_multiple_of_eight(torch):
    # slice counts that do not fill the eight XCDs evenly (6 and 3 slices)
    _decode_case(W.custom(2, batch=3, hq=8, hkv=2, n_packed=900, n_ring=17), "6 slices G=4")
    _decode_case(W.custom(4, batch=3, hq=2, hkv=1, n_packed=700, n_ring=128), "3 slices d256 G=2")


def _step_case(w: W.Workload, fill: int, label: str):
    """Two identical stores and rings, `fill` ring tokens; returns the fused step's and the
    two-call path's outputs, rings and stores."""
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size, kb=w.key_bits)
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, w.n_packed + fill + 1)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    cap = w.n_packed + w.buffer_size
    stores, rings = [], []
    for _ in range(2):
        st = tq.PackedStore(env.cfg, n_sl, cap)
        if w.n_packed:
            quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :w.n_packed]), w.in_dtype),
                         to_dev(np.ascontiguousarray(v[:, :w.n_packed]), w.in_dtype), n_sl, w.n_packed, store=st)
        rg = tq.Ring(env.cfg, n_sl)
        for t_ in range(fill):
            tq.tq_append_ring(env.cfg, rg.struct(), to_dev(np.ascontiguousarray(k[:, w.n_packed + t_]), w.in_dtype),
                              to_dev(np.ascontiguousarray(v[:, w.n_packed + t_]), w.in_dtype), n_sl, t_)
        stores.append(st)
        rings.append(rg)
    kn = to_dev(np.ascontiguousarray(k[:, w.n_packed + fill]), w.in_dtype)
    vn = to_dev(np.ascontiguousarray(v[:, w.n_packed + fill]), w.in_dtype)
    q, _ = W.host_queries(w, 0)
    qd = to_dev(q, w.in_dtype)
    scale = 1.0 / math.sqrt(w.d)
    outs = [torch_mod().zeros((w.batch, w.hq, w.d), dtype=torch_mod().float32, device="cuda") for _ in range(2)]
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, cap + 1)
    # two calls: (flush a full ring,) append, decode
    n_packed, n_ring = w.n_packed, fill
    if n_ring == w.buffer_size:
        tq.tq_flush(env.cfg, env.tables, rings[0].struct(), n_sl, n_ring, stores[0].struct(), n_packed)
        n_packed, n_ring = n_packed + n_ring, 0
    tq.tq_append_ring(env.cfg, rings[0].struct(), kn, vn, n_sl, n_ring)
    tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, stores[0].struct(), n_packed,
                           rings[0].struct(), n_ring + 1, scale, outs[0], ws)
    # the fused step
    got = tq.tq_decode_step(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, stores[1].struct(), w.n_packed,
                            rings[1].struct(), fill, kn, vn, scale, outs[1], ws)
    torch_mod().cuda.synchronize()
    assert got == (n_packed, n_ring + 1), (label, got)
    return env, q, qd, stores, rings, [o.cpu().numpy() for o in outs], got


def test_decode_step_matches_append_then_decode(torch):
    """The new token taken from the input inside the decode kernel gives the results of
    tq_append_ring + tq_decode_attention bit for bit, and the same ring."""
    for w, fill, label in ((W.custom(2, n_packed=1000, n_ring=40), 40, "d128 v2"),
                           (W.custom(3, batch=2, n_packed=500, n_ring=63), 63, "d128 v4 split edge"),
                           (W.custom(4, batch=1, n_packed=700, n_ring=20), 20, "d256"),
                           (W.custom(2, n_packed=0, n_ring=5), 5, "ring only"),
                           (W.custom(1, n_packed=512, n_ring=0), 0, "tiny fp32 empty ring")):
        env, q, qd, stores, rings, outs, (n_packed, n_ring) = _step_case(w, fill, label)
        np.testing.assert_array_equal(outs[1], outs[0], err_msg=label)
        for a_, b_ in ((rings[0].k, rings[1].k), (rings[0].v, rings[1].v)):
            np.testing.assert_array_equal(b_.cpu().numpy().view(np.uint16), a_.cpu().numpy().view(np.uint16),
                                          err_msg=label)
        ref = oracle_decode(env, dev_to_stored(qd).astype(np.float64), w.hq, w.hkv, stores[1], n_packed, rings[1],
                            n_ring, b_list=list(range(w.batch)))
        assert_decode_close(outs[1].astype(np.float64), ref, f"step {label}")


def test_prepared_decode_step_matches_direct_call(torch):
    """PreparedDecodeStep (arguments checked and marshalled once) runs the same tq_decode_step:
    the same output bit for bit and the same counts, called again with the same fill counts."""
    w = W.custom(3, batch=2, n_packed=700, n_ring=30)
    env, q, qd, stores, rings, outs, (n_packed, n_ring) = _step_case(w, 30, "prepared")
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, w.n_packed + 31)
    kn = to_dev(np.ascontiguousarray(k.reshape(n_sl, -1, w.d)[:, w.n_packed + 30]), w.in_dtype)
    vn = to_dev(np.ascontiguousarray(v.reshape(n_sl, -1, w.d)[:, w.n_packed + 30]), w.in_dtype)
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, w.n_packed + w.buffer_size + 1)
    scale = 1.0 / math.sqrt(w.d)
    a = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
    b = torch.zeros_like(a)
    got_a = tq.tq_decode_step(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, stores[1].struct(), w.n_packed,
                              rings[1].struct(), 30, kn, vn, scale, a, ws)
    call = tq.PreparedDecodeStep(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, stores[1].struct(), rings[1].struct(),
                                 kn, vn, scale, b, ws)
    got_b = call(w.n_packed, 30)
    torch.cuda.synchronize()
    assert got_a == got_b == (w.n_packed, 31)
    np.testing.assert_array_equal(b.cpu().numpy(), a.cpu().numpy())
    np.testing.assert_array_equal(a.cpu().numpy(), outs[1])


def test_decode_step_flushes_a_full_ring(torch):
    """A full ring is flushed into the packed store first: the same records, ring and
    output as tq_flush + tq_append_ring + tq_decode_attention."""
    w = W.custom(3, batch=2, n_packed=300, n_ring=64, buffer_size=64)
    env, q, qd, stores, rings, outs, (n_packed, n_ring) = _step_case(w, 64, "full ring")
    assert (n_packed, n_ring) == (364, 1)
    np.testing.assert_array_equal(outs[1], outs[0])
    P0, P1 = packed_to_np(stores[0]), packed_to_np(stores[1])
    for key in P0:
        np.testing.assert_array_equal(P1[key], P0[key], err_msg=key)
    np.testing.assert_array_equal(rings[1].k[:, :1].cpu().numpy().view(np.uint16),
                                  rings[0].k[:, :1].cpu().numpy().view(np.uint16))
    ref = oracle_decode(env, dev_to_stored(qd).astype(np.float64), w.hq, w.hkv, stores[1], n_packed, rings[1],
                        n_ring, b_list=[0, 1])
    assert_decode_close(outs[1].astype(np.float64), ref, "step after flush")


def test_decode_ragged_batch(torch):
    """Per-sequence lengths: every batch element against the oracle at its own lengths
    (including an empty sequence, a ring-only one and one longer than a split); lengths past
    the maxima are clamped."""
    for w, lens in ((W.custom(3, batch=6, n_packed=3000, n_ring=64),
                     [(0, 0), (1, 5), (700, 64), (3000, 17), (1500, 0), (0, 33)]),
                    (W.custom(4, batch=3, n_packed=900, n_ring=128), [(900, 128), (37, 2), (450, 90)])):
        env = Env(w.d, w.value_bits, buffer_size=w.buffer_size, kb=w.key_bits)
        n_sl = w.batch * w.hkv
        (k, v), _ = W.host_kv(w, 0, w.n_packed + w.n_ring)
        k = k.reshape(n_sl, -1, w.d)
        v = v.reshape(n_sl, -1, w.d)
        store = quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :w.n_packed]), w.in_dtype),
                             to_dev(np.ascontiguousarray(v[:, :w.n_packed]), w.in_dtype), n_sl, w.n_packed)
        ring = tq.Ring(env.cfg, n_sl)
        for t_ in range(w.n_ring):
            tq.tq_append_ring(env.cfg, ring.struct(), to_dev(np.ascontiguousarray(k[:, w.n_packed + t_]), w.in_dtype),
                              to_dev(np.ascontiguousarray(v[:, w.n_packed + t_]), w.in_dtype), n_sl, t_)
        q, _ = W.host_queries(w, 0)
        qd = to_dev(q, w.in_dtype)
        sp = torch.tensor([a for a, _ in lens], dtype=torch.int64, device="cuda")
        sr = torch.tensor([r for _, r in lens], dtype=torch.int32, device="cuda")
        out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
        ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, w.n_packed + w.n_ring)
        tq.tq_decode_attention_ragged(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), sp, w.n_packed,
                                      ring.struct(), sr, w.n_ring, 1.0 / math.sqrt(w.d), out, ws)
        torch.cuda.synchronize()
        g = out.cpu().numpy().astype(np.float64)
        q_stored = dev_to_stored(qd).astype(np.float64)
        for b, (n_p, n_r) in enumerate(lens):
            if n_p + n_r == 0:
                assert not g[b].any(), f"sequence {b} has no tokens"
                continue
            ref = oracle_decode(env, q_stored[b:b + 1], w.hq, w.hkv, store, n_p, ring, n_r, slice_offset=b * w.hkv,
                                b_list=[0])
            assert_decode_close(g[b:b + 1], ref, f"ragged d{w.d} b{b} ({n_p} + {n_r})")
        # every sequence at the maxima (and lengths beyond them, clamped) = the uniform decode
        sp.fill_(w.n_packed + 1000)
        sr.fill_(w.n_ring)
        tq.tq_decode_attention_ragged(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), sp, w.n_packed,
                                      ring.struct(), sr, w.n_ring, 1.0 / math.sqrt(w.d), out, ws)
        g2, _, _ = run_decode(env, q, w.in_dtype, w.batch, w.hq, w.hkv, store, w.n_packed, ring, w.n_ring, qd=qd)
        np.testing.assert_array_equal(out.cpu().numpy(), g2.astype(np.float32))


@pytest.mark.parametrize("case", ["d128_v4", "d256_v4", "d64_kb2"])
def test_paged_store_matches_contiguous(torch, case):
    """A paged store (pages in a seeded random order, spare pages in the pool) holds exactly the
    contiguous store's records, and every decode entry point reads it to the same results bit
    for bit: history quantise, full-ring flush inside the fused step, uniform, ragged and
    layer-offset (slice_offset) decodes; one case also against the oracle."""
    if case == "d128_v4":
        w = W.custom(3, batch=2, n_packed=600, n_ring=64, buffer_size=64)
        pt, pps = 64, 12                   # capacity 768 >= 600 + 64 + 1
    elif case == "d256_v4":
        w = W.custom(4, batch=2, n_packed=500, n_ring=32, buffer_size=32)
        pt, pps = 32, 18                   # capacity 576 >= 500 + 32 + 1
    else:
        w = W.custom(2, d=64, key_bits=2, batch=2, hq=8, hkv=2, n_packed=600, n_ring=64, buffer_size=64)
        pt, pps = 64, 12                   # capacity 768 >= 600 + 64 + 1
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size, kb=w.key_bits)
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, w.n_packed + w.n_ring + 1)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    cont = tq.PackedStore(env.cfg, n_sl, pt * pps)
    paged = tq.PagedStore(env.cfg, n_sl, pt, pps, n_sl * pps + 7, seed=5)
    for st in (cont, paged):
        quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :w.n_packed]), w.in_dtype),
                     to_dev(np.ascontiguousarray(v[:, :w.n_packed]), w.in_dtype), n_sl, w.n_packed, store=st)
    G = paged.gather()
    C = {n: getattr(cont, n).cpu().numpy() for n in G}
    for n in G:
        np.testing.assert_array_equal(G[n].view(np.uint8), C[n].view(np.uint8), err_msg=n)
    rings = []
    for _ in range(2):
        rg = tq.Ring(env.cfg, n_sl)
        for t_ in range(w.n_ring):
            tq.tq_append_ring(env.cfg, rg.struct(), to_dev(np.ascontiguousarray(k[:, w.n_packed + t_]), w.in_dtype),
                              to_dev(np.ascontiguousarray(v[:, w.n_packed + t_]), w.in_dtype), n_sl, t_)
        rings.append(rg)
    q, _ = W.host_queries(w, 0)
    qd = to_dev(q, w.in_dtype)
    scale = 1.0 / math.sqrt(w.d)
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, pt * pps)
    outs = [torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda") for _ in range(2)]
    # uniform decode over history + full ring
    for o, st, rg in zip(outs, (cont, paged), rings):
        tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, st.struct(), w.n_packed, rg.struct(),
                               w.n_ring, scale, o, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outs[1].cpu().numpy(), outs[0].cpu().numpy())
    # layer-offset views: the second batch element alone through slice_offset
    half = [torch.zeros((1, w.hq, w.d), dtype=torch.float32, device="cuda") for _ in range(2)]
    for o, st, rg in zip(half, (cont, paged), rings):
        tq.tq_decode_attention(env.cfg, env.tables, qd[1:], 1, w.hq, w.hkv, st.struct(w.hkv), w.n_packed,
                               rg.struct(w.hkv), w.n_ring, scale, o, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(half[1].cpu().numpy(), half[0].cpu().numpy())
    # ragged
    sp = torch.tensor([w.n_packed - 1, 37], dtype=torch.int64, device="cuda")
    sr = torch.tensor([3, w.n_ring], dtype=torch.int32, device="cuda")
    for o, st, rg in zip(outs, (cont, paged), rings):
        tq.tq_decode_attention_ragged(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, st.struct(), sp, w.n_packed,
                                      rg.struct(), sr, w.n_ring, scale, o, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outs[1].cpu().numpy(), outs[0].cpu().numpy())
    # fused step on the full ring: flush it after the history, then append and decode
    kn = to_dev(np.ascontiguousarray(k[:, w.n_packed + w.n_ring]), w.in_dtype)
    vn = to_dev(np.ascontiguousarray(v[:, w.n_packed + w.n_ring]), w.in_dtype)
    for o, st, rg in zip(outs, (cont, paged), rings):
        got = tq.tq_decode_step(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, st.struct(), w.n_packed, rg.struct(),
                                w.n_ring, kn, vn, scale, o, ws)
        assert got == (w.n_packed + w.n_ring, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(outs[1].cpu().numpy(), outs[0].cpu().numpy())
    G = paged.gather()
    for n in G:
        np.testing.assert_array_equal(G[n].view(np.uint8), getattr(cont, n).cpu().numpy().view(np.uint8), err_msg=n)
    ref = oracle_decode(env, dev_to_stored(qd).astype(np.float64), w.hq, w.hkv, cont, w.n_packed + w.n_ring,
                        rings[1], 1, b_list=[0, 1])
    assert_decode_close(outs[1].cpu().numpy().astype(np.float64), ref, "paged step")
    assert not paged.table_error()


def test_paged_store_reports_bad_table_entries(torch):
    """A block-table entry outside the pool is clamped on the device (no access leaves the pool)
    and reported through the store's error flag, by the quantiser and by the decode; a valid
    table leaves the flag clear."""
    w = W.custom(3, batch=1, n_packed=256, n_ring=0)
    env = Env(w.d, w.value_bits)
    n_sl, pt, pps = w.hkv, 64, 4
    (k, v), _ = W.host_kv(w, 0, w.n_packed)
    kd = to_dev(np.ascontiguousarray(k.reshape(n_sl, -1, w.d)), w.in_dtype)
    vd = to_dev(np.ascontiguousarray(v.reshape(n_sl, -1, w.d)), w.in_dtype)
    q, _ = W.host_queries(w, 0)
    qd = to_dev(q, w.in_dtype)
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, pt * pps)
    out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
    good = tq.PagedStore(env.cfg, n_sl, pt, pps, n_sl * pps, seed=1)
    quantize_gpu(env, kd, vd, n_sl, w.n_packed, store=good)
    tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, good.struct(), w.n_packed, None, 0,
                           1 / math.sqrt(w.d), out, ws)
    torch.cuda.synchronize()
    assert not good.table_error()
    table = good.table_np.copy()
    table[3, 2] = n_sl * pps + 5          # past the pool: clamped to its last page
    table[5, 0] = -1                      # negative: clamped to page 0
    bad = tq.PagedStore(env.cfg, n_sl, pt, pps, n_sl * pps, table=table)
    quantize_gpu(env, kd, vd, n_sl, w.n_packed, store=bad)
    assert bad.table_error()
    bad.clear_table_error()
    assert not bad.table_error()
    tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, bad.struct(), w.n_packed, None, 0,
                           1 / math.sqrt(w.d), out, ws)
    torch.cuda.synchronize()
    assert bad.table_error()


def test_decode_12_wave_groups_within_tolerance(torch):
    """Long contexts at d = 128 run one 12-wave workgroup per compute unit whose waves take
    token blocks in arrival order, so the summation order varies: repeated calls and the fused
    step agree with append + decode within 1e-5 relative (not bit for bit; measured 2e-6), and the result is
    within the decode bounds of the oracle."""
    w = W.custom(2, n_packed=32000, n_ring=20)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slices = w.batch * w.hkv
    assert slices * w.n_packed // (cus * 12 * 32) >= 2, "the case must select 12-wave workgroups"
    env, q, qd, stores, rings, outs, (n_packed, n_ring) = _step_case(w, 20, "12-wave")
    spread = rel_err_per_head(outs[1].astype(np.float64), outs[0].astype(np.float64)).max()
    log(f"12-wave: fused step vs append + decode max rel diff {spread:.3e}")
    assert spread <= 1e-5
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, n_packed + n_ring)
    first = None
    for rep in range(4):
        o = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
        tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, stores[0].struct(), n_packed,
                               rings[0].struct(), n_ring, 1 / math.sqrt(w.d), o, ws)
        torch.cuda.synchronize()
        o = o.cpu().numpy().astype(np.float64)
        if first is None:
            first = o
        diff = rel_err_per_head(o, first).max()
        log(f"12-wave: repeat {rep} max rel diff {diff:.3e}")
        assert diff <= 1e-5
    ref = oracle_decode(env, dev_to_stored(qd).astype(np.float64), w.hq, w.hkv, stores[1], n_packed, rings[1],
                        n_ring, b_list=[0])
    assert_decode_close(outs[1].astype(np.float64), ref, "12-wave step")


def test_decode_empty_context_gives_zeros(torch):
    env = Env(128, 2)
    q = np.ones((1, 4, 128), np.float32)
    g, _, _ = run_decode(env, q, "f32", 1, 4, 1, None, 0, None, 0)
    assert not g.any()


def test_decode_workspace_reuse_needs_no_reset(torch):
    """Repeated calls on one workspace, first filled with garbage, give identical results
    (the workspace is scratch: every value read is written by the same call first), also
    when the calls alternate between split counts (2000 packed tokens: 4 splits, 700: 2)."""
    w = W.custom(2, n_packed=2000, n_ring=3)
    env, store, ring, q, ws, g1, _ = _decode_case(w, "reuse", b_list=[0])
    qd = to_dev(q, w.in_dtype)
    q_stored = dev_to_stored(qd).astype(np.float64)
    out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
    ws.fill_(0x7F)  # large finite floats everywhere
    for _ in range(3):
        tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), w.n_packed,
                               ring.struct(), w.n_ring, 1 / math.sqrt(w.d), out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), g1.astype(np.float32))
    for n_packed in (700, w.n_packed):
        tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), n_packed,
                               ring.struct(), w.n_ring, 1 / math.sqrt(w.d), out, ws)
        torch.cuda.synchronize()
        if n_packed == w.n_packed:
            np.testing.assert_array_equal(out.cpu().numpy(), g1.astype(np.float32))
        else:
            ref = oracle_decode(env, q_stored, w.hq, w.hkv, store, n_packed, ring, w.n_ring, b_list=[0])
            assert_decode_close(out.cpu().numpy().astype(np.float64)[:1], ref, f"reuse n_packed={n_packed}")


def test_decode_many_splits_per_slice(torch):
    # the merge of a slice's splits past the partials it loads up front (96: one slice, 137
    # splits at d = 128), and one slice at d = 256 with two and with eight query heads
    _decode_case(W.custom(2, batch=1, hq=4, hkv=1, n_packed=70000, n_ring=128), "1 slice d128 70000")
    _decode_case(W.custom(4, batch=1, hq=2, hkv=1, n_packed=40000, n_ring=128), "1 slice d256 40000")
    _decode_case(W.custom(4, batch=1, hq=8, hkv=1, n_packed=9000, n_ring=10), "1 slice d256 G=8")


class _OracleRecords:
    """The oracle's own packed records of a history, with a PackedStore's tensor shapes (host
    tensors, read by oracle_decode like a store's)."""

    def __init__(self, torch, env: Env, k, v, n_slices, n_tokens):
        d, vb = env.d, env.vb
        kq = O.quantize_keys(k, env.c32, env.b32, env.sigma, env.S)
        vq = O.quantize_values(v, vb)
        self.capacity = n_tokens
        self.key_words = torch.from_numpy(O.pack_keys(kq["idx"], kq["z"]).view(np.int32).reshape(n_slices, n_tokens, d // 8))
        self.key_norms = torch.from_numpy(np.stack([kq["norm"], kq["rnorm"]], -1).astype(np.float32)
                                          .reshape(n_slices, n_tokens, 2))
        self.val_words = torch.from_numpy(O.pack_values(vq["code"], vb).view(np.int32).reshape(n_slices, n_tokens, -1))
        self.val_scales = torch.from_numpy(vq["scale"].view(np.int16).reshape(n_slices, n_tokens, d // 32))


def test_decode_end_to_end_against_oracle_compression(torch):
    """End to end, each side on its own records: the oracle compresses the history and
    attends over its own packed bytes, the GPU path compresses and attends over its own (the
    same ring of exact fp16 tokens).  Codes may differ only within 1e-6 of a decision
    boundary, so the two outputs meet the decode bar; the error is logged."""
    cases = ((W.WORKLOADS[1], "tiny"), (W.custom(2, batch=2, n_packed=1500, n_ring=40), "llama-law b2"),
             (W.custom(4, batch=1, n_packed=600, n_ring=20), "d256 v4"))
    for w, label in cases:
        env, store, ring, q, ws, g, _ = _decode_case(w, label + " (GPU records)")
        n_sl = w.batch * w.hkv
        (k, v), _ = W.host_kv(w, 0, w.n_packed + w.n_ring)
        k = k.reshape(n_sl, -1, w.d)[:, :w.n_packed].reshape(-1, w.d).astype(np.float64)
        v = v.reshape(n_sl, -1, w.d)[:, :w.n_packed].reshape(-1, w.d).astype(np.float64)
        recs = _OracleRecords(torch, env, k, v, n_sl, w.n_packed)
        q_stored = dev_to_stored(to_dev(q, w.in_dtype)).astype(np.float64)
        ref = oracle_decode(env, q_stored, w.hq, w.hkv, recs, w.n_packed, ring, w.n_ring, b_list=range(w.batch))
        assert_decode_close(g, ref, label + " end to end (oracle records)")


def test_rotate_hook(torch):
    """Pi x on the device against the oracle's rotation (dense Sylvester matrix), at both
    head sizes, for fp32 and bf16 rows: relative error <= 1e-6 per row, and |Pi x| = |x|."""
    for d in (128, 256):
        env = Env(d, 4)
        x = np.random.default_rng(11).standard_normal((37, d)).astype(np.float32)
        x[3] = 0.0
        for dt in ("f32", "bf16"):
            xd = to_dev(x, dt)
            xs = dev_to_stored(xd).astype(np.float64)
            out = torch.zeros((37, d), dtype=torch.float32, device="cuda")
            tq.tq_rotate(env.cfg, env.tables, xd, 37, out)
            torch.cuda.synchronize()
            g = out.cpu().numpy().astype(np.float64)
            ref = O.rotate(env.sigma, xs)
            err = np.abs(g - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)
            log(f"rotate d={d} {dt}: max rel err {err.max():.3e}")
            assert err.max() <= 1e-6 and not g[3].any()
            nrm = np.linalg.norm(xs, axis=1)
            assert np.allclose(np.linalg.norm(g, axis=1), nrm, rtol=1e-6, atol=0)


def test_decode_scores_hook(torch):
    """Raw pre-softmax scores on the device against the oracle's, on the same packed bytes and
    ring: packed tokens (the estimator) and ring tokens (exact products), both head sizes,
    GQA, a paged store.  Per (batch, head): max |s - s*| / max |s*| <= 1e-5."""
    cases = ((W.custom(2, batch=2, n_packed=700, n_ring=40), "d128 b2"),
             (W.custom(4, batch=1, hq=8, hkv=2, n_packed=300, n_ring=20), "d256 G=4"),
             (W.custom(2, d=64, key_bits=1, batch=1, hq=8, hkv=2, n_packed=300, n_ring=20), "d64 kb1"),
             (W.custom(2, d=128, key_bits=4, batch=1, hq=8, hkv=2, n_packed=300, n_ring=20), "d128 kb4"))
    for w, label in cases:
        env, store, ring, q, ws, g, _ = _decode_case(w, label)
        qd = to_dev(q, w.in_dtype)
        q_stored = dev_to_stored(qd).astype(np.float64)
        T = w.n_packed + w.n_ring
        sc = torch.zeros((w.batch, w.hq, T), dtype=torch.float32, device="cuda")
        tq.tq_decode_scores(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), w.n_packed,
                            ring.struct(), w.n_ring, sc)
        torch.cuda.synchronize()
        got = sc.cpu().numpy().astype(np.float64)
        P = packed_to_np(store)
        ref_all = []
        for b in range(w.batch):
            sl = slice(b * w.hkv, (b + 1) * w.hkv)
            _, ref = O.decode(d=w.d, kb=w.key_bits, vb=w.value_bits, c32=env.c32, sigma=env.sigma, S_bits=env.S, B=1, Hq=w.hq,
                              Hkv=w.hkv, kw=P["kw"][sl], kn=P["kn"][sl], vw=P["vw"][sl], vs=P["vs"][sl],
                              cap=store.capacity, n_packed=w.n_packed,
                              rk=ring.k[sl].cpu().numpy().view(np.uint16), rv=ring.v[sl].cpu().numpy().view(np.uint16),
                              buf=ring.k.shape[1], n_ring=w.n_ring, q=q_stored[b:b + 1], scale=1.0 / math.sqrt(w.d),
                              want_scores=True)
            ref_all.append(ref[0])
        ref = np.stack(ref_all)
        err = np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)
        log(f"{label}: scores max rel err {err.max():.3e} (packed {np.abs(got - ref)[..., :w.n_packed].max():.3e}, "
            f"ring {np.abs(got - ref)[..., w.n_packed:].max():.3e} abs)")
        assert err.max() <= 1e-5, f"{label}: score rel err {err.max()}"


def test_append_flush_decode_sequence(torch):
    """History + ring decode, then flush the ring and decode again over packed only."""
    w = W.custom(3, batch=2, n_packed=500, n_ring=64)
    env, store_unused, ring, q, ws, g, _ = _decode_case(w, "before flush")
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, w.n_packed + w.n_ring)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    store = quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :w.n_packed]), "bf16"),
                         to_dev(np.ascontiguousarray(v[:, :w.n_packed]), "bf16"), n_sl, w.n_packed,
                         capacity=w.n_packed + w.buffer_size)
    tq.tq_flush(env.cfg, env.tables, ring.struct(), n_sl, w.n_ring, store.struct(), w.n_packed)
    n_packed = w.n_packed + w.n_ring
    g2, q_stored, _ = run_decode(env, q, "bf16", w.batch, w.hq, w.hkv, store, n_packed, None, 0)
    ref = oracle_decode(env, q_stored, w.hq, w.hkv, store, n_packed, None, 0, b_list=list(range(w.batch)))
    assert_decode_close(g2, ref, "after flush")


# ------------------------------------------------------------------------- key widths 1, 2, 4 and head_dim 64
# (two-plane key records; decode through k_decode_any)

WIDTHS = [(64, 1), (64, 2), (64, 3), (64, 4), (128, 1), (128, 2), (128, 4)]


@pytest.mark.parametrize("d,kb", WIDTHS)
def test_quantize_key_widths(torch, d, kb):
    """Codes, signs, norms, value codes and scales of every key width against the oracle, for
    bf16 (values 2-bit) and fp32 (values 4-bit) inputs: 3 slices x 211 tokens, so 32-token
    tiles with a ragged last one, at a store offset."""
    for vb, dt in ((2, "bf16"), (4, "f32")):
        w = W.custom(2, d=d, key_bits=kb, batch=1, hkv=3, value_bits=vb, in_dtype=dt)
        env = Env(d, vb, kb=kb)
        _quantize_case(env, w, 211, cap_extra=3, offset=5, label=f"d{d} kb{kb} v{vb} {dt}")


@pytest.mark.parametrize("d,kb", WIDTHS)
def test_decode_key_widths(torch, d, kb):
    """Decode over packed records of every key width plus the ring, against the oracle on the
    same bytes: GQA groups 4 (several splits and the merge), 1 and 8, ring only, packed only."""
    _decode_case(W.custom(2, d=d, key_bits=kb, batch=2, hq=8, hkv=2, n_packed=1100, n_ring=9), f"d{d} kb{kb} G=4")
    if kb in (1, 4):
        _decode_case(W.custom(2, d=d, key_bits=kb, batch=1, hq=4, hkv=4, n_packed=333, n_ring=70,
                              value_bits=4), f"d{d} kb{kb} G=1 v4")
        _decode_case(W.custom(2, d=d, key_bits=kb, batch=1, hq=16, hkv=2, n_packed=200, n_ring=3),
                     f"d{d} kb{kb} G=8")
        _decode_case(W.custom(2, d=d, key_bits=kb, n_packed=0, n_ring=77), f"d{d} kb{kb} ring only")
        _decode_case(W.custom(2, d=d, key_bits=kb, n_packed=65, n_ring=0), f"d{d} kb{kb} packed only")


@pytest.mark.parametrize("d,kb", [(64, 2), (128, 4)])
def test_decode_step_key_widths(torch, d, kb):
    """The fused step (append, and a full ring's flush, then decode) equals the separate calls
    bit for bit and the oracle, on the k_decode_any path."""
    for w, fill, label in ((W.custom(2, d=d, key_bits=kb, batch=2, hq=8, hkv=2, n_packed=600, n_ring=20), 20,
                            f"d{d} kb{kb}"),
                           (W.custom(2, d=d, key_bits=kb, batch=1, hq=8, hkv=2, n_packed=300, n_ring=32,
                                     buffer_size=32), 32, f"d{d} kb{kb} flush")):
        env, q, qd, stores, rings, outs, (n_packed, n_ring) = _step_case(w, fill, label)
        np.testing.assert_array_equal(outs[1], outs[0], err_msg=label)
        ref = oracle_decode(env, dev_to_stored(qd).astype(np.float64), w.hq, w.hkv, stores[1], n_packed, rings[1],
                            n_ring, b_list=list(range(w.batch)))
        assert_decode_close(outs[1].astype(np.float64), ref, f"step {label}")


def test_decode_ragged_key_widths(torch):
    """Per-sequence lengths on the k_decode_any path, each against the oracle."""
    w = W.custom(2, d=64, key_bits=4, batch=4, hq=8, hkv=2, n_packed=1500, n_ring=40)
    lens = [(0, 0), (1500, 40), (37, 3), (900, 0)]
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size, kb=w.key_bits)
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, w.n_packed + w.n_ring)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    store = quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :w.n_packed]), w.in_dtype),
                         to_dev(np.ascontiguousarray(v[:, :w.n_packed]), w.in_dtype), n_sl, w.n_packed)
    ring = tq.Ring(env.cfg, n_sl)
    for t_ in range(w.n_ring):
        tq.tq_append_ring(env.cfg, ring.struct(), to_dev(np.ascontiguousarray(k[:, w.n_packed + t_]), w.in_dtype),
                          to_dev(np.ascontiguousarray(v[:, w.n_packed + t_]), w.in_dtype), n_sl, t_)
    q, _ = W.host_queries(w, 0)
    qd = to_dev(q, w.in_dtype)
    sp = torch.tensor([a for a, _ in lens], dtype=torch.int64, device="cuda")
    sr = torch.tensor([r for _, r in lens], dtype=torch.int32, device="cuda")
    out = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, w.n_packed + w.n_ring)
    tq.tq_decode_attention_ragged(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), sp, w.n_packed,
                                  ring.struct(), sr, w.n_ring, 1.0 / math.sqrt(w.d), out, ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    q_stored = dev_to_stored(qd).astype(np.float64)
    for b, (n_p, n_r) in enumerate(lens):
        if n_p + n_r == 0:
            assert not g[b].any()
            continue
        ref = oracle_decode(env, q_stored[b:b + 1], w.hq, w.hkv, store, n_p, ring, n_r, slice_offset=b * w.hkv,
                            b_list=[0])
        assert_decode_close(g[b:b + 1], ref, f"ragged d64 kb4 b{b} ({n_p} + {n_r})")


def test_rotate_hook_d64(torch):
    env = Env(64, 2, kb=2)
    x = np.random.default_rng(12).standard_normal((19, 64)).astype(np.float32)
    xd = to_dev(x, "f32")
    out = torch.zeros((19, 64), dtype=torch.float32, device="cuda")
    tq.tq_rotate(env.cfg, env.tables, xd, 19, out)
    torch.cuda.synchronize()
    ref = O.rotate(env.sigma, x.astype(np.float64))
    g = out.cpu().numpy().astype(np.float64)
    err = np.abs(g - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert err.max() <= 1e-6, err.max()
