"""Pins of the KIVI oracle (oracle/kivi.py) against values worked by hand and closed forms.

Forum page zingnex.cn "TurboQuant-vLLM：大模型推理的KV缓存量化实战方案", section "KIVI非对称量化":
keys per channel, values per token, each with a scale and a zero point, 2 bits.
"""
import json
import os

import numpy as np
import pytest

from oracle import kivi as K

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kivi_hand.json")))


def _hand_keys():
    t = np.arange(32, dtype=np.float64)
    k = np.zeros((32, 16))
    k[:, 0] = t / 8
    k[:, 1] = 1.5
    k[:, 2] = -t / 4
    return k


def test_kivi_hand_example_keys():
    g = GOLD["keys"]
    codes, scale, zero = K.quantize_keys(_hand_keys())
    for c in ("0", "1", "2"):
        assert int(scale[0, int(c)].view(np.uint16)) == int(g["scale_bits"][c], 16)
        assert float(scale[0, int(c)]) == g["scale_values"][c]
        assert float(zero[0, int(c)]) == g["zero_values"][c]
    t = np.arange(32)
    want0 = np.select([t <= 5, t <= 15, t <= 25], [0, 1, 2], 3)
    want2 = np.select([t <= 5, t <= 15, t <= 25], [3, 2, 1], 0)
    assert np.array_equal(codes[:, 0], want0)
    assert np.array_equal(codes[:, 1], np.zeros(32))
    assert np.array_equal(codes[:, 2], want2)
    assert np.array_equal(codes[:, 3:], np.zeros((32, 13)))
    words = K.pack_codes(codes)
    assert words.shape == (32, 1)
    assert int(words[0, 0]) == int(g["word_token0"], 16)
    assert int(words[31, 0]) == int(g["word_token31"], 16)


def test_kivi_hand_example_values():
    g = GOLD["values"]
    v = (np.arange(16, dtype=np.float64) / 2)[None, :]
    codes, scale, zero = K.quantize_values(v)
    assert int(scale[0].view(np.uint16)) == int(g["scale_bits"], 16)
    assert float(zero[0]) == g["zero"]
    assert codes[0].tolist() == g["codes"]
    assert int(K.pack_codes(codes)[0, 0]) == int(g["word"], 16)


def test_kivi_pack_words_by_hand():
    # codes 0, 1, 2, 3 repeating: every byte 0b11100100
    codes = np.tile(np.arange(4, dtype=np.uint8), 8)[None, :]
    w = K.pack_codes(codes)
    assert w.tolist() == [[0xE4E4E4E4, 0xE4E4E4E4]]
    assert np.array_equal(K.unpack_codes(w, 32), codes)
    rng = np.random.default_rng(3)
    c = rng.integers(0, 4, size=(64, 128), dtype=np.uint8)
    assert np.array_equal(K.unpack_codes(K.pack_codes(c), 128), c)


def test_kivi_grid_values_are_reproduced_exactly():
    """Inputs on a quantiser grid (zero + code * scale, both binary16, codes 0 and 3 present in
    every set) come back exactly: span = 3 scale is exact, so the scale is recovered."""
    rng = np.random.default_rng(7)
    T, D = 64, 32
    s = rng.uniform(0.01, 0.5, size=(T // 32, D)).astype(np.float16).astype(np.float64)
    z = rng.uniform(-4, 4, size=(T // 32, D)).astype(np.float16).astype(np.float64)
    codes = rng.integers(0, 4, size=(T, D))
    codes[0::32] = 0
    codes[1::32] = 3
    k = codes * np.repeat(s, 32, axis=0) + np.repeat(z, 32, axis=0)
    # the grid points themselves must be exact in binary32 for the reading to apply
    keep = np.all(k.astype(np.float32).astype(np.float64) == k, axis=0)
    c2, s2, z2 = K.quantize_keys(k[:, keep])
    assert np.array_equal(s2.astype(np.float64), s[:, keep])
    assert np.array_equal(z2.astype(np.float64), z[:, keep])
    assert np.array_equal(c2, codes[:, keep])
    assert np.array_equal(K.dequant_keys(c2, s2, z2), k[:, keep])


def test_kivi_error_bound():
    """|x - x^| <= scale / 2 inside the range, plus the binary16 roundings of the scale (3 half
    ulps at the top code) and of the zero."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((256, 128)).astype(np.float32).astype(np.float64) * 3
    for quant, deq, axis in ((K.quantize_keys, K.dequant_keys, "k"), (K.quantize_values, K.dequant_values, "v")):
        codes, s, z = quant(x)
        xh = deq(codes, s, z)
        if axis == "k":
            ss = np.repeat(s.astype(np.float64), 32, axis=0)
            zz = np.repeat(z.astype(np.float64), 32, axis=0)
            mn = np.repeat(x.reshape(-1, 32, 128).min(axis=1), 32, axis=0)
        else:
            ss = s.astype(np.float64)[:, None]
            zz = z.astype(np.float64)[:, None]
            mn = x.min(axis=1)[:, None]
        ulp = np.spacing(ss.astype(np.float16)).astype(np.float64)
        bound = ss / 2 + 3 * ulp + np.abs(zz - mn) + 1e-6 * np.abs(x)
        assert np.all(np.abs(x - xh) <= bound)
        assert codes.min() == 0 and codes.max() == 3


def test_kivi_key_channel_and_value_token_granularity():
    """Doubling one key channel doubles that channel's scale and zero only, codes unchanged;
    doubling one value token does the same for that token's pair."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((64, 32)).astype(np.float16).astype(np.float64)
    c0, s0, z0 = K.quantize_keys(k)
    k2 = k.copy()
    k2[:, 7] *= 2
    c1, s1, z1 = K.quantize_keys(k2)
    assert np.array_equal(c1, c0)
    assert np.array_equal(s1[:, 7].astype(np.float64), 2 * s0[:, 7].astype(np.float64))
    assert np.array_equal(z1[:, 7].astype(np.float64), 2 * z0[:, 7].astype(np.float64))
    others = np.arange(32) != 7
    assert np.array_equal(s1[:, others], s0[:, others]) and np.array_equal(z1[:, others], z0[:, others])
    v = rng.standard_normal((8, 64)).astype(np.float16).astype(np.float64)
    c0, s0, z0 = K.quantize_values(v)
    v2 = v.copy()
    v2[3] *= 2
    c1, s1, z1 = K.quantize_values(v2)
    assert np.array_equal(c1, c0)
    assert float(s1[3]) == 2 * float(s0[3]) and float(z1[3]) == 2 * float(z0[3])
    assert np.array_equal(np.delete(s1, 3), np.delete(s0, 3))


def test_kivi_constant_sets():
    k = np.full((32, 16), -0.75)
    codes, s, z = K.quantize_keys(k)
    assert np.all(s == 0) and np.all(z == -0.75) and np.all(codes == 0)
    assert np.all(K.dequant_keys(codes, s, z) == -0.75)
    v = np.full((3, 16), 2.0)
    codes, s, z = K.quantize_values(v)
    assert np.all(s == 0) and np.all(codes == 0) and np.all(K.dequant_values(codes, s, z) == 2.0)


@pytest.mark.parametrize("case", ["zero_query", "equal_keys", "single_token", "dominant_key"])
def test_kivi_decode_closed_forms(case):
    rng = np.random.default_rng(13)
    B, Hq, Hkv, D, T = 2, 4, 2, 32, 64
    keys = [rng.standard_normal((T, D)) for _ in range(B * Hkv)]
    vals = [rng.standard_normal((T, D)) for _ in range(B * Hkv)]
    q = rng.standard_normal((B, Hq, D))
    if case == "zero_query":
        q[:] = 0
        out = K.decode(q, keys, vals, 0.3)
        for b in range(B):
            for h in range(Hq):
                assert np.allclose(out[b, h], vals[b * Hkv + h // 2].mean(axis=0), atol=1e-12)
    elif case == "equal_keys":
        keys = [np.tile(k[:1], (T, 1)) for k in keys]
        out = K.decode(q, keys, vals, 0.3)
        for b in range(B):
            for h in range(Hq):
                assert np.allclose(out[b, h], vals[b * Hkv + h // 2].mean(axis=0), atol=1e-12)
    elif case == "single_token":
        out = K.decode(q, [k[:1] for k in keys], [v[:1] for v in vals], 0.3)
        for b in range(B):
            for h in range(Hq):
                assert np.allclose(out[b, h], vals[b * Hkv + h // 2][0], atol=1e-12)
    else:
        for i, k in enumerate(keys):
            k[17] = 50 * q[i // Hkv, (i % Hkv) * 2]  # token 17 dominates for head 2 (i % Hkv)
        out = K.decode(q, keys, vals, 1.0)
        for b in range(B):
            for kv in range(Hkv):
                assert np.allclose(out[b, 2 * kv], vals[b * Hkv + kv][17], atol=1e-9)
