"""Host-side checks of libtq.so (no GPU): exported symbols, host tables against the
oracle, byte accounting, and every error path (all are decided before any launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import tq_workloads as W
import compressed_decode_attention_02_amd as tq
from compressed_decode_attention_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_header_symbol():
    hdr = open(os.path.join(ROOT, "include", "tq.h")).read()
    declared = sorted(set(re.findall(r"^\s*(?:tq_status|size_t|const char \*)\s*(tq_\w+)\s*\(", hdr, re.M)))
    assert len(declared) >= 11
    L = ctypes.CDLL(B.LIB_PATH)
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(B.EXPORTS) == declared


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kb", [1, 2, 3, 4])
def test_codebook_matches_oracle(d, kb):
    """Two independent integrations of the same Lloyd-Max problem (incomplete beta in the
    oracle, Gauss-Legendre quadrature in the library) agree; stored fp32 values are equal."""
    c, b = tq.tq_build_codebook(d, kb)
    co, bo, _ = O.codebook(d, kb)
    np.testing.assert_allclose(c, co, rtol=0, atol=1e-12)
    np.testing.assert_allclose(b, bo, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(c.astype(np.float32), co.astype(np.float32))
    np.testing.assert_array_equal(b.astype(np.float32), bo.astype(np.float32))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("seed", [0, W.TABLE_SEED, 2**63 + 12345])
def test_rotation_tables_match_oracle_bit_exact(d, seed):
    s, S = tq.tq_build_rotation(d, seed)
    so, So = O.tables(d, seed)
    np.testing.assert_array_equal(s, so)
    np.testing.assert_array_equal(S, So)


@pytest.mark.parametrize("d,vb,kb", [(128, 2, 3), (128, 4, 3), (256, 4, 3), (256, 2, 3), (64, 2, 1), (64, 4, 2),
                                     (64, 2, 3), (64, 2, 4), (128, 2, 2), (128, 4, 4)])
def test_table_blob_layout(d, vb, kb):
    cfg = tq.make_config(d, kb, vb)
    blob = tq.tq_build_tables(cfg, W.TABLE_SEED)
    assert blob.size == tq.tq_tables_bytes(cfg) == 256 + 2 * d * d
    c32, b32 = O.stored_codebook(d, kb)
    L = 1 << kb
    np.testing.assert_array_equal(blob[0:4 * L].view(np.float32), c32.astype(np.float32))
    np.testing.assert_array_equal(blob[64:64 + 4 * (L - 1)].view(np.float32), b32.astype(np.float32))
    sigma, S = O.tables(d, W.TABLE_SEED)
    bits = blob[128:128 + d // 8].view(np.uint32)
    got = np.array([(bits[j // 32] >> (j % 32)) & 1 for j in range(d)])
    np.testing.assert_array_equal(got, (sigma < 0).astype(int))
    np.testing.assert_array_equal(blob[256:].view(np.uint16).reshape(d, d), S)


def test_packed_bytes_per_token():
    assert tq.tq_packed_bytes_per_token(tq.make_config(128, 3, 2)) == W.packed_record_bytes(128, 2) == 112
    assert tq.tq_packed_bytes_per_token(tq.make_config(128, 3, 4)) == 144
    assert tq.tq_packed_bytes_per_token(tq.make_config(256, 3, 4)) == 280
    # (kb + 1) d / 8 key bytes + 8 norm bytes + vb d / 8 value bytes + 2 d / 32 scale bytes
    for d, kb, vb in [(64, 1, 2), (64, 2, 4), (64, 4, 2), (128, 2, 2), (128, 4, 4)]:
        want = (kb + 1) * d // 8 + 8 + vb * d // 8 + 2 * d // 32
        assert tq.tq_packed_bytes_per_token(tq.make_config(d, kb, vb)) == want
        assert B.key_record_words(tq.make_config(d, kb, vb)) * 4 == (kb + 1) * d // 8


# ------------------------------------------------------------------ error paths (host only)

FAKE = 0x10000  # aligned, never dereferenced: every case below fails before a launch


def _fake_tables():
    return B.tq_tables(FAKE, FAKE, FAKE, FAKE)


def _fake_packed(cap=1000):
    return B.tq_packed(FAKE, FAKE, FAKE, FAKE, cap)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=32), B.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=576), B.TQ_ERR_UNSUPPORTED),
    (dict(key_bits=5), B.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=256, key_bits=2), B.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=256, key_bits=4), B.TQ_ERR_UNSUPPORTED),
    (dict(value_bits=3), B.TQ_ERR_UNSUPPORTED),
    (dict(group_size=64), B.TQ_ERR_UNSUPPORTED),
    (dict(head_dim=0), B.TQ_ERR_INVALID_ARG),
    (dict(buffer_size=0), B.TQ_ERR_INVALID_ARG),
])
def test_config_errors(kw, status):
    base = dict(head_dim=128, key_bits=3, value_bits=2, group_size=32, buffer_size=128)
    base.update(kw)
    cfg = tq.make_config(**base)
    L = tq.lib()
    st = L.tq_quantize_kv(ctypes.byref(cfg), ctypes.byref(_fake_tables()), FAKE, FAKE, B.TQ_BF16, 1, 16,
                          ctypes.byref(_fake_packed()), 0, None)
    assert st == status
    assert L.tq_tables_bytes(ctypes.byref(cfg)) == 0
    assert L.tq_decode_workspace_bytes(ctypes.byref(cfg), 1, 4, 1, 100) == 0


def test_quantize_argument_errors():
    cfg = tq.make_config()
    L = tq.lib()
    T, P = _fake_tables(), _fake_packed(cap=100)
    q = lambda *a: L.tq_quantize_kv(ctypes.byref(cfg), *a)
    assert q(ctypes.byref(T), FAKE, FAKE, B.TQ_BF16, 1, 101, ctypes.byref(P), 0, None) == B.TQ_ERR_INVALID_ARG
    assert q(ctypes.byref(T), FAKE, FAKE, B.TQ_BF16, 1, 50, ctypes.byref(P), 51, None) == B.TQ_ERR_INVALID_ARG
    assert q(ctypes.byref(T), FAKE + 4, FAKE, B.TQ_BF16, 1, 16, ctypes.byref(P), 0, None) == B.TQ_ERR_INVALID_ARG
    assert q(ctypes.byref(T), None, FAKE, B.TQ_BF16, 1, 16, ctypes.byref(P), 0, None) == B.TQ_ERR_INVALID_ARG
    assert q(ctypes.byref(T), FAKE, FAKE, 7, 1, 16, ctypes.byref(P), 0, None) == B.TQ_ERR_INVALID_ARG
    assert q(None, FAKE, FAKE, B.TQ_BF16, 1, 16, ctypes.byref(P), 0, None) == B.TQ_ERR_INVALID_ARG
    assert q(ctypes.byref(T), FAKE, FAKE, B.TQ_BF16, -1, 16, ctypes.byref(P), 0, None) == B.TQ_ERR_INVALID_ARG
    # empty work is a no-op even with null pointers
    assert q(ctypes.byref(T), None, None, B.TQ_BF16, 1, 0, None, 0, None) == B.TQ_OK
    assert q(ctypes.byref(T), None, None, B.TQ_BF16, 0, 10, None, 0, None) == B.TQ_OK


def test_ring_errors():
    cfg = tq.make_config(buffer_size=128)
    L = tq.lib()
    R = B.tq_ring(FAKE, FAKE)
    a = lambda n: L.tq_append_ring(ctypes.byref(cfg), ctypes.byref(R), FAKE, FAKE, B.TQ_BF16, 8, n, None)
    assert a(128) == B.TQ_ERR_RING_FULL
    assert a(129) == B.TQ_ERR_INVALID_ARG
    assert a(-1) == B.TQ_ERR_INVALID_ARG
    P = _fake_packed(cap=200)
    f = lambda n_ring, n_packed: L.tq_flush(ctypes.byref(cfg), ctypes.byref(_fake_tables()), ctypes.byref(R), 8,
                                            n_ring, ctypes.byref(P), n_packed, None)
    assert f(128, 73) == B.TQ_ERR_INVALID_ARG          # would overflow the store
    assert f(129, 0) == B.TQ_ERR_INVALID_ARG
    assert f(0, 0) == B.TQ_OK                          # nothing to flush


def test_decode_errors():
    cfg = tq.make_config()
    L = tq.lib()
    T, P, R = _fake_tables(), _fake_packed(cap=4096), B.tq_ring(FAKE, FAKE)
    need = L.tq_decode_workspace_bytes(ctypes.byref(cfg), 2, 8, 2, 4096)
    assert need > 0

    def dec(bsz=2, hq=8, hkv=2, n_packed=4096, n_ring=5, ws=need, q=FAKE):
        return L.tq_decode_attention(ctypes.byref(cfg), ctypes.byref(T), q, B.TQ_BF16, bsz, hq, hkv,
                                     ctypes.byref(P), n_packed, ctypes.byref(R), n_ring, ctypes.c_float(0.1),
                                     FAKE, FAKE, ws, None)
    assert dec(ws=need - 1) == B.TQ_ERR_WORKSPACE
    assert dec(hq=6, hkv=4) == B.TQ_ERR_INVALID_ARG        # not a multiple
    assert dec(hq=24, hkv=2) == B.TQ_ERR_UNSUPPORTED      # G = 12
    assert dec(n_packed=4097) == B.TQ_ERR_INVALID_ARG     # beyond capacity
    assert dec(n_ring=129) == B.TQ_ERR_INVALID_ARG
    assert dec(q=FAKE + 2) == B.TQ_ERR_INVALID_ARG
    # decode token indices are 32-bit: a context of 2^31 - 256 tokens or more is refused
    big = 1 << 31
    P2 = _fake_packed(cap=big)
    ws_big = L.tq_decode_workspace_bytes(ctypes.byref(cfg), 2, 8, 2, big)
    dec_big = lambda n_packed, n_ring: L.tq_decode_attention(
        ctypes.byref(cfg), ctypes.byref(T), FAKE, B.TQ_BF16, 2, 8, 2, ctypes.byref(P2), n_packed, ctypes.byref(R),
        n_ring, ctypes.c_float(0.1), FAKE, FAKE, ws_big, None)
    assert dec_big(big - 256, 0) == B.TQ_ERR_UNSUPPORTED
    assert dec_big(big - 300, 44) == B.TQ_ERR_UNSUPPORTED
    assert dec_big(big, 0) == B.TQ_ERR_UNSUPPORTED
    # a shorter context needs no more workspace than the maximum it was sized for
    for ctx in (0, 1, 255, 256, 1000, 4095):
        assert L.tq_decode_workspace_bytes(ctypes.byref(cfg), 2, 8, 2, ctx) <= need


def test_decode_step_errors_leave_the_counts():
    """tq_decode_step checks everything before it launches: each error returns with the
    caller's fill counts untouched (no GPU needed: every case here fails a check, so nothing
    is launched)."""
    cfg = tq.make_config(buffer_size=128)
    L = tq.lib()
    T, P, R = _fake_tables(), _fake_packed(cap=4096), B.tq_ring(FAKE, FAKE)
    need = L.tq_decode_workspace_bytes(ctypes.byref(cfg), 2, 8, 2, 4096)

    def step(n_packed, n_ring, ws=need, kv_dtype=B.TQ_BF16, k_new=FAKE, counts=True):
        np_, nr_ = ctypes.c_int64(n_packed), ctypes.c_int32(n_ring)
        st = L.tq_decode_step(ctypes.byref(cfg), ctypes.byref(T), FAKE, B.TQ_BF16, 2, 8, 2, ctypes.byref(P),
                              ctypes.byref(np_) if counts else None, ctypes.byref(R),
                              ctypes.byref(nr_) if counts else None, k_new, FAKE, kv_dtype, ctypes.c_float(0.1),
                              FAKE, FAKE, ws, None)
        return st, np_.value, nr_.value
    assert step(100, 5, counts=False)[0] == B.TQ_ERR_INVALID_ARG
    assert step(100, 5, ws=16) == (B.TQ_ERR_WORKSPACE, 100, 5)
    assert step(100, 129) == (B.TQ_ERR_INVALID_ARG, 100, 129)
    assert step(100, 5, kv_dtype=7) == (B.TQ_ERR_INVALID_ARG, 100, 5)
    assert step(100, 5, k_new=FAKE + 2) == (B.TQ_ERR_INVALID_ARG, 100, 5)
    assert step(4097, 5) == (B.TQ_ERR_INVALID_ARG, 4097, 5)     # more records than the store holds
    # a full ring would be flushed to records 4000..4127 of a 4096-record store: refused
    # before the flush is launched
    assert step(4000, 128) == (B.TQ_ERR_INVALID_ARG, 4000, 128)


def test_decode_ragged_errors():
    cfg = tq.make_config()
    L = tq.lib()
    T, P, R = _fake_tables(), _fake_packed(cap=4096), B.tq_ring(FAKE, FAKE)
    need = L.tq_decode_workspace_bytes(ctypes.byref(cfg), 2, 8, 2, 4096)

    def rag(sp=FAKE, sr=FAKE, n_packed_max=4096, n_ring_max=5, ws=need):
        return L.tq_decode_attention_ragged(ctypes.byref(cfg), ctypes.byref(T), FAKE, B.TQ_BF16, 2, 8, 2,
                                            ctypes.byref(P), sp, n_packed_max, ctypes.byref(R), sr, n_ring_max,
                                            ctypes.c_float(0.1), FAKE, FAKE, ws, None)
    assert rag(sp=None) == B.TQ_ERR_INVALID_ARG
    assert rag(sr=None) == B.TQ_ERR_INVALID_ARG
    assert rag(sp=FAKE + 4) == B.TQ_ERR_INVALID_ARG       # int64 lengths: 8-byte aligned
    assert rag(sr=FAKE + 2) == B.TQ_ERR_INVALID_ARG       # int32 lengths: 4-byte aligned
    assert rag(n_packed_max=4097) == B.TQ_ERR_INVALID_ARG
    assert rag(n_ring_max=129) == B.TQ_ERR_INVALID_ARG
    assert rag(ws=16) == B.TQ_ERR_WORKSPACE


def test_paged_store_errors():
    """A paged store must hold whole 32-token blocks per page, cover its capacity with its table
    and have an aligned table; each violation is refused before any launch."""
    cfg = tq.make_config()
    L = tq.lib()
    T = _fake_tables()

    def q(page_tokens=64, pps=4, n_pages=40, cap=256, table=FAKE, flag=None):
        P = B.tq_packed(FAKE, FAKE, FAKE, FAKE, cap, table, page_tokens, pps, n_pages, flag)
        return L.tq_quantize_kv(ctypes.byref(cfg), ctypes.byref(T), FAKE, FAKE, B.TQ_BF16, 8, 100,
                                ctypes.byref(P), 300, None)   # offset 300 > capacity in every case
    assert q() == B.TQ_ERR_INVALID_ARG                       # (the offset check: a valid paged store)
    assert q(page_tokens=48, cap=192) == B.TQ_ERR_INVALID_ARG  # not whole 32-token blocks
    assert q(cap=512) == B.TQ_ERR_INVALID_ARG                 # capacity != pages * page tokens
    assert q(n_pages=0) == B.TQ_ERR_INVALID_ARG
    assert q(table=FAKE + 2) == B.TQ_ERR_INVALID_ARG          # int32 table: 4-byte aligned
    assert q(flag=FAKE) == B.TQ_ERR_INVALID_ARG               # (an aligned error flag: the offset check)
    assert q(flag=FAKE + 2) == B.TQ_ERR_INVALID_ARG           # int32 error flag: 4-byte aligned



def test_test_hook_errors():
    # every case fails validation, so nothing is launched
    cfg = tq.make_config()
    L = tq.lib()
    T, P, R = _fake_tables(), _fake_packed(cap=4096), B.tq_ring(FAKE, FAKE)
    assert L.tq_rotate(None, ctypes.byref(T), FAKE, B.TQ_F32, 4, FAKE, None) == B.TQ_ERR_INVALID_ARG
    assert L.tq_rotate(ctypes.byref(cfg), None, FAKE, B.TQ_F32, 4, FAKE, None) == B.TQ_ERR_INVALID_ARG
    assert L.tq_rotate(ctypes.byref(cfg), ctypes.byref(T), FAKE, 7, 4, FAKE, None) == B.TQ_ERR_INVALID_ARG
    assert L.tq_rotate(ctypes.byref(cfg), ctypes.byref(T), FAKE, B.TQ_F32, -1, FAKE, None) == B.TQ_ERR_INVALID_ARG
    assert L.tq_rotate(ctypes.byref(cfg), ctypes.byref(T), FAKE + 4, B.TQ_F32, 4, FAKE, None) == B.TQ_ERR_INVALID_ARG
    assert L.tq_rotate(ctypes.byref(cfg), ctypes.byref(T), FAKE, B.TQ_F32, 4, None, None) == B.TQ_ERR_INVALID_ARG
    bad = tq.make_config(576)
    assert L.tq_rotate(ctypes.byref(bad), ctypes.byref(T), FAKE, B.TQ_F32, 4, FAKE, None) == B.TQ_ERR_UNSUPPORTED

    def scores(hq=8, hkv=2, n_packed=100, n_ring=5, out=FAKE, packed=P, q=FAKE):
        return L.tq_decode_scores(ctypes.byref(cfg), ctypes.byref(T), q, B.TQ_BF16, 2, hq, hkv,
                                  ctypes.byref(packed) if packed is not None else None, n_packed,
                                  ctypes.byref(R), n_ring, out, None)
    assert scores(hq=8, hkv=3) == B.TQ_ERR_INVALID_ARG
    assert scores(n_ring=129) == B.TQ_ERR_INVALID_ARG
    assert scores(n_packed=-1) == B.TQ_ERR_INVALID_ARG
    assert scores(n_packed=4097) == B.TQ_ERR_INVALID_ARG    # beyond the store's capacity
    assert scores(packed=None) == B.TQ_ERR_INVALID_ARG
    assert scores(out=None) == B.TQ_ERR_INVALID_ARG
    assert scores(out=FAKE + 4) == B.TQ_ERR_INVALID_ARG
    assert scores(q=None) == B.TQ_ERR_INVALID_ARG
    assert scores(hq=40000, hkv=1) == B.TQ_ERR_UNSUPPORTED  # batch * heads above the grid's y limit


def test_binding_rejects_bad_tensors_before_the_library():
    """The binding checks dtype agreement, contiguity, size and device of every tensor before
    the call: a k/v dtype mismatch would make the kernel read v with k's element size."""
    import torch
    cfg = tq.make_config()
    n = 2 * 16 * 128
    k32 = torch.zeros(n, dtype=torch.float32)
    kb = torch.zeros(n, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="share a dtype"):
        tq.tq_quantize_kv(cfg, None, k32, kb, 2, 16, None, 0)
    with pytest.raises(ValueError, match="share a dtype"):
        tq.tq_quantize_kv(cfg, None, kb, k32, 2, 16, None, 0)
    with pytest.raises(ValueError, match="contiguous"):
        tq.tq_quantize_kv(cfg, None, kb.view(4, -1)[:, ::2], kb.view(4, -1)[:, ::2], 1, 4, None, 0)
    with pytest.raises(ValueError, match="at least"):
        tq.tq_quantize_kv(cfg, None, kb, kb, 2, 17, None, 0)
    with pytest.raises(ValueError, match="GPU tensor"):
        tq.tq_quantize_kv(cfg, None, kb, kb, 2, 16, None, 0)
    with pytest.raises(ValueError, match="unsupported dtype"):
        ki = torch.zeros(n, dtype=torch.int16)
        tq.tq_quantize_kv(cfg, None, ki, ki, 2, 16, None, 0)
    # the ring append: one token per slice
    with pytest.raises(ValueError, match="share a dtype"):
        tq.tq_append_ring(cfg, None, k32[:256], kb[:256], 2, 0)
    with pytest.raises(ValueError, match="at least"):
        tq.tq_append_ring(cfg, None, kb[:255], kb[:255], 2, 0)
    # decode: q, out (fp32) and workspace; the fused step's new token pair
    q = torch.zeros(4 * 128, dtype=torch.bfloat16)
    out = torch.zeros(4 * 128, dtype=torch.float32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out must be"):
        tq.tq_decode_attention(cfg, None, q, 1, 4, 1, None, 0, None, 0, 0.1, out.half(), ws)
    with pytest.raises(ValueError, match="at least"):
        tq.tq_decode_attention(cfg, None, q[:500], 1, 4, 1, None, 0, None, 0, 0.1, out, ws)
    with pytest.raises(ValueError, match="share a dtype"):
        tq.tq_decode_step(cfg, None, q, 1, 4, 1, None, 0, None, 0, k32[:128], kb[:128], 0.1, out, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        tq.tq_decode_step(cfg, None, q, 1, 4, 1, None, 0, None, 0, kb[:128], kb[:128], 0.1, out, ws)


def test_noalloc_decode_errors():
    """The no-allocation decode checks its arguments like tq_decode_attention and refuses a call
    whose scratch exceeds the static array (TQ_ERR_SCRATCH_LIMIT), all before any device call."""
    cfg = tq.make_config()
    L = tq.lib()
    T, R = _fake_tables(), B.tq_ring(FAKE, FAKE)

    def dec(bsz=2, hq=8, hkv=2, n_packed=4096, cap=4096, n_ring=5, q=FAKE):
        P = _fake_packed(cap=cap)
        return L.tq_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(T), q, B.TQ_BF16, bsz, hq, hkv,
                                             ctypes.byref(P), n_packed, ctypes.byref(R), n_ring,
                                             ctypes.c_float(0.1), FAKE, None)
    assert dec(hq=6, hkv=4) == B.TQ_ERR_INVALID_ARG
    assert dec(n_packed=4097) == B.TQ_ERR_INVALID_ARG
    assert dec(q=FAKE + 2) == B.TQ_ERR_INVALID_ARG
    # a call that fits, and one that does not: 32000 slices of one query head each need
    # 32000 partial rows of 128 fp32 (16 MB)
    need = lambda bsz, hq, hkv, ctx: L.tq_decode_workspace_bytes(ctypes.byref(cfg), bsz, hq, hkv, ctx)
    assert need(4, 32, 8, 32768) <= B.TQ_NOALLOC_SCRATCH_BYTES
    assert need(1000, 32, 32, 100) > B.TQ_NOALLOC_SCRATCH_BYTES
    assert dec(bsz=1000, hq=32, hkv=32, n_packed=100, cap=100, n_ring=0) == B.TQ_ERR_SCRATCH_LIMIT
    assert B.TQ_ERR_SCRATCH_LIMIT == -6
    assert b"scratch" in L.tq_status_string(B.TQ_ERR_SCRATCH_LIMIT)


def test_prepared_decode_step_checks_its_arguments():
    """PreparedDecodeStep checks its tensors as tq_decode_step does, before marshalling."""
    import torch
    cfg = tq.make_config()
    q = torch.zeros(4 * 128, dtype=torch.bfloat16)
    out = torch.zeros(4 * 128, dtype=torch.float32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    k32 = torch.zeros(128, dtype=torch.float32)
    kb = torch.zeros(128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="share a dtype"):
        tq.PreparedDecodeStep(cfg, None, q, 1, 4, 1, None, None, k32, kb, 0.1, out, ws)
    with pytest.raises(ValueError, match="out must be"):
        tq.PreparedDecodeStep(cfg, None, q, 1, 4, 1, None, None, kb, kb, 0.1, out.half(), ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        tq.PreparedDecodeStep(cfg, None, q, 1, 4, 1, None, None, kb, kb, 0.1, out, ws)


def test_prefill_argument_errors():
    """Prefill: every argument checked on the host before a launch (fake device pointers)."""
    cfg = tq.make_config()
    L = tq.lib()
    T, P = _fake_tables(), _fake_packed(cap=1000)

    def pf(batch=2, q_tokens=16, hq=8, hkv=2, n_packed=500, pos0=0, causal=1, q=FAKE, out=FAKE, ws_bytes=1 << 30,
           packed=P, dtype=B.TQ_BF16):
        return L.tq_prefill_attention(ctypes.byref(cfg), ctypes.byref(T), q, dtype, batch, q_tokens, hq, hkv,
                                      ctypes.byref(packed) if packed is not None else None, n_packed, pos0, causal,
                                      ctypes.c_float(0.1), out, FAKE, ws_bytes, None)
    assert pf(batch=0) == B.TQ_ERR_INVALID_ARG
    assert pf(q_tokens=0) == B.TQ_ERR_INVALID_ARG
    assert pf(pos0=-1) == B.TQ_ERR_INVALID_ARG
    assert pf(causal=2) == B.TQ_ERR_INVALID_ARG
    assert pf(packed=None) == B.TQ_ERR_INVALID_ARG
    assert pf(n_packed=1001) == B.TQ_ERR_INVALID_ARG          # beyond the store's capacity
    assert pf(q=FAKE + 4) == B.TQ_ERR_INVALID_ARG             # 16-byte alignment
    assert pf(dtype=9) == B.TQ_ERR_INVALID_ARG
    assert pf(hq=24, hkv=2) == B.TQ_ERR_UNSUPPORTED          # G = 12
    assert pf(ws_bytes=16) == B.TQ_ERR_WORKSPACE
    need = L.tq_prefill_workspace_bytes(ctypes.byref(cfg), 2, 16, 8, 2, 500)
    assert need > 0 and L.tq_prefill_workspace_bytes(ctypes.byref(cfg), 0, 16, 8, 2, 500) == 0
    # long prompts run in several launches of at most 65536 / kv heads query tokens (the tiled
    # kernel; 65535 / kv heads on the decode kernels): the workspace is sized for one launch,
    # and every launch is checked before the first
    big = L.tq_prefill_workspace_bytes(ctypes.byref(cfg), 1, 40000, 8, 2, 500)
    assert big == L.tq_prefill_workspace_bytes(ctypes.byref(cfg), 1, 32768, 8, 2, 500)
    assert pf(batch=1, q_tokens=40000, ws_bytes=16) == B.TQ_ERR_WORKSPACE
    assert pf(batch=1, q_tokens=40000, n_packed=1001) == B.TQ_ERR_INVALID_ARG


def test_prefill_workspace_plan():
    """The prefill's host plan (no device: 256 compute units assumed).  Few query rows per kv head
    (T G below half a 128-row tile) take the decode kernels' workspace; more take the tiled
    kernel's, which prepares its queries itself: only when the tiles alone do not cover the
    compute units, (o, m, l) partials per row and split of the packed range (splits of whole
    64-token blocks, at least 256 tokens each, at most 16); else the 256-byte minimum."""
    cfg = tq.make_config()  # head_dim 128
    L = tq.lib()
    ws = lambda bsz, T, hq, hkv, n: L.tq_prefill_workspace_bytes(ctypes.byref(cfg), bsz, T, hq, hkv, n)
    al = lambda x: (x + 255) // 256 * 256
    # T G = 60 < 64: the decode kernels (one batch element per query token)
    assert ws(1, 15, 8, 2, 5000) == L.tq_decode_workspace_bytes(ctypes.byref(cfg), 15, 8, 2, 5000)
    # T G = 256: 2 tiles per kv head, 4 workgroups < 256 CUs, 79 blocks of 64 -> 16 splits
    rows = 64 * 8
    assert ws(1, 64, 8, 2, 5000) == al(rows * 16 * 128 * 4) + al(rows * 16 * 2 * 4)
    # a short history limits the splits: 600 tokens -> 2 splits of 320
    assert ws(1, 64, 8, 2, 600) == al(rows * 2 * 128 * 4) + al(rows * 2 * 2 * 4)
    # enough tiles to cover the CUs (32 sequences x 8 kv heads x 16 tiles), or under 256
    # tokens of history: no split
    assert ws(32, 512, 32, 8, 8128) == 256
    assert ws(1, 64, 8, 2, 100) == 256


def test_kivi_bytes_per_token():
    # key codes d/4 + key scale and zero d/8 (a 32-token group's share) + value codes d/4 + 4
    for d, want in ((64, 16 + 8 + 16 + 4), (128, 32 + 16 + 32 + 4), (256, 64 + 32 + 64 + 4)):
        assert tq.tq_kivi_bytes_per_token(d) == want
    for d in (0, 32, 96, 512):
        assert tq.tq_kivi_bytes_per_token(d) == 0


def test_kivi_argument_errors():
    """Every case fails before a launch (the store and data pointers are never dereferenced)."""
    L = B.lib()
    S = B.tq_kivi_store(FAKE, FAKE, FAKE, FAKE, FAKE, 256)
    q = lambda d=128, k=FAKE, dt=B.TQ_BF16, ns=2, nt=64, st=S, t0=0: L.tq_kivi_quantize(
        d, k, FAKE, dt, ns, nt, ctypes.byref(st) if st is not None else None, t0, None)
    assert q(d=96) == B.TQ_ERR_UNSUPPORTED
    assert q(nt=40) == B.TQ_ERR_INVALID_ARG      # not whole 32-token groups
    assert q(t0=16) == B.TQ_ERR_INVALID_ARG
    assert q(nt=256, t0=32) == B.TQ_ERR_INVALID_ARG  # past the capacity
    assert q(ns=0) == B.TQ_ERR_INVALID_ARG
    assert q(dt=9) == B.TQ_ERR_INVALID_ARG
    assert q(k=FAKE + 4) == B.TQ_ERR_INVALID_ARG
    assert q(k=None) == B.TQ_ERR_INVALID_ARG
    assert q(st=None) == B.TQ_ERR_INVALID_ARG
    assert q(st=B.tq_kivi_store(FAKE, FAKE, FAKE, FAKE, FAKE, 100)) == B.TQ_ERR_INVALID_ARG  # capacity % 32
    assert q(st=B.tq_kivi_store(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 256)) == B.TQ_ERR_INVALID_ARG
    assert q(nt=0) == B.TQ_OK  # nothing to do: returns before any launch
    need = tq.tq_kivi_decode_workspace_bytes(128, 2, 8, 2, 256)
    assert need > 0
    assert tq.tq_kivi_decode_workspace_bytes(128, 2, 6, 4, 256) == 0

    def dec(d=128, bsz=2, hq=8, hkv=2, n=256, ws=need, qp=FAKE, st=S):
        return L.tq_kivi_decode_attention(d, qp, B.TQ_BF16, bsz, hq, hkv, ctypes.byref(st), n, 0.1, FAKE, FAKE, ws,
                                          None)
    assert dec(d=32) == B.TQ_ERR_UNSUPPORTED
    assert dec(hq=6, hkv=4) == B.TQ_ERR_INVALID_ARG
    assert dec(hq=24, hkv=2) == B.TQ_ERR_UNSUPPORTED  # 12 query heads per kv head
    assert dec(n=257) == B.TQ_ERR_INVALID_ARG          # past the capacity
    assert dec(n=-1) == B.TQ_ERR_INVALID_ARG
    assert dec(qp=FAKE + 8) == B.TQ_ERR_INVALID_ARG
    assert dec(ws=need - 1) == B.TQ_ERR_WORKSPACE
    assert dec(bsz=40000, hkv=2, hq=2) == B.TQ_ERR_UNSUPPORTED  # more than 65535 slices
