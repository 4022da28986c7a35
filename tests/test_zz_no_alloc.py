"""The no-allocation decode entry point (static scratch, for callers that cannot allocate)
against tq_decode_attention with a caller workspace: the same kernels and split shapes, so the
outputs agree bit for bit (4-wave workgroups at these sizes); two calls in a row, the second on a
smaller input over the first call's leftover scratch, then a head_dim-256 call (prepared queries
in the scratch); each also against the oracle."""
import math

import numpy as np
import pytest

import tq_workloads as W
import compressed_decode_attention_02_amd as tq

from gpu_common import Env, assert_decode_close, dev_to_stored, log, oracle_decode, quantize_gpu, to_dev

pytestmark = pytest.mark.gpu


def _inputs(w, n_packed, n_ring):
    env = Env(w.d, w.value_bits, buffer_size=w.buffer_size)
    n_sl = w.batch * w.hkv
    (k, v), _ = W.host_kv(w, 0, n_packed + n_ring)
    k = k.reshape(n_sl, -1, w.d)
    v = v.reshape(n_sl, -1, w.d)
    store = quantize_gpu(env, to_dev(np.ascontiguousarray(k[:, :n_packed]), w.in_dtype),
                         to_dev(np.ascontiguousarray(v[:, :n_packed]), w.in_dtype), n_sl, n_packed)
    ring = tq.Ring(env.cfg, n_sl)
    for t in range(n_ring):
        tq.tq_append_ring(env.cfg, ring.struct(), to_dev(np.ascontiguousarray(k[:, n_packed + t]), w.in_dtype),
                          to_dev(np.ascontiguousarray(v[:, n_packed + t]), w.in_dtype), n_sl, t)
    q, _ = W.host_queries(w, 0)
    return env, store, ring, to_dev(q, w.in_dtype)


def test_noalloc_decode_matches_workspace_decode():
    import torch
    assert torch.cuda.is_available()
    cases = [("d128 v4, b4 x 3000 + 40", W.custom(3, batch=4, n_packed=3000, n_ring=40)),
             ("d128 v2, b1 x 300 + 3 (smaller, after the first)", W.custom(2, batch=1, hq=8, hkv=2, n_packed=300, n_ring=3)),
             ("d256 v4, b2 x 700 + 10", W.custom(4, batch=2, n_packed=700, n_ring=10))]
    for label, w in cases:
        log(f"noalloc case: {label}")
        env, store, ring, qd = _inputs(w, w.n_packed, w.n_ring)
        scale = 1.0 / math.sqrt(w.d)
        ref = torch.zeros((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
        ws = tq.new_workspace(env.cfg, w.batch, w.hq, w.hkv, w.n_packed + w.n_ring)
        tq.tq_decode_attention(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), w.n_packed,
                               ring.struct(), w.n_ring, scale, ref, ws)
        out = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        tq.tq_decode_attention_noalloc(env.cfg, env.tables, qd, w.batch, w.hq, w.hkv, store.struct(), w.n_packed,
                                       ring.struct(), w.n_ring, scale, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all(), label
        np.testing.assert_array_equal(got, ref.cpu().numpy(), err_msg=label)
        orc = oracle_decode(env, dev_to_stored(qd).astype(np.float64), w.hq, w.hkv, store, w.n_packed, ring,
                            w.n_ring, b_list=[0])
        assert_decode_close(got[:1].astype(np.float64), orc, f"noalloc {label}")
