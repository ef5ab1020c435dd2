"""Pins of the oracle's attention over the NVFP4 cache (the consumer of the
cache that the LongLive-2.0 summary page builds in inference pipeline step 7
and reads through sink ranges in step 9): a worked softmax example, closed
forms (uniform weights, a single key), invariants of softmax attention (key
order, the per-chunk mean and tensor scales), and scipy's softmax /
logsumexp on scores computed here with numpy from the pinned codecs."""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def _pack(vals):
    """E2M1 values [..., D] -> packed codes [..., D/2], even element low."""
    c = np.vectorize(lambda x: E2M1_CODE[abs(float(x))] | (8 if x < 0 else 0))(vals).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _hand_cache(kvals, vvals, L, S=1.0, gk=None, gv=None, mean=None):
    Hkv, T, D = kvals.shape
    nc = T // L
    sc = np.full((Hkv, T, D // 16), O.e4m3_encode(np.float32(S)).item(), np.uint8)
    return {"k_codes": _pack(kvals), "v_codes": _pack(vvals), "k_scales": sc, "v_scales": sc.copy(),
            "k_tensor_scale": np.asarray(gk if gk is not None else np.ones(nc), np.float32),
            "v_tensor_scale": np.asarray(gv if gv is not None else np.ones(nc), np.float32),
            "k_mean": None if mean is None else np.asarray(mean, np.float32)}


def _decode(codes, scales, g, mean, L):
    """Exact decode with numpy from the pinned codecs: [Hkv, T, D] float64."""
    Hkv, T, D2 = codes.shape
    D = 2 * D2
    lo, hi = codes & 15, codes >> 4
    q = np.stack([lo, hi], axis=-1).reshape(Hkv, T, D)
    v = O.e2m1_decode(q).astype(np.float64)
    S = np.repeat(O.e4m3_decode(scales).astype(np.float64), 16, axis=-1)
    ch = np.arange(T) // L
    x = v * S * np.asarray(g, np.float64)[ch][None, :, None]
    if mean is not None:
        x = x + np.asarray(mean, np.float64)[ch].transpose(1, 0, 2)
    return x


def _random_cache(Hkv, T, D, L, seed):
    k, v = W.gaussian_kv(W.KVShape(Hkv, T, D, L), seed)
    return O.smooth_quantize(W.bf16_bits(k), W.bf16_bits(v), L)


def _keys(ranges):
    return np.concatenate([np.arange(a, a + n) for a, n in ranges]) if ranges else np.zeros(0, int)


def _qf(q):
    return W.from_bits(q).float().numpy().astype(np.float64)


def test_worked_softmax_example():
    ex = json.load(open(os.path.join(GOLDEN, "attention_worked_example.json")))
    D = 16
    kv = np.zeros((1, 3, D))
    kv[0, :, 0] = ex["scores"]              # K_j = (j, 0, ...), scores q.K_j = j with q = e_0
    vv = np.zeros((1, 3, D))
    vv[0, [0, 1, 2], [0, 1, 2]] = 1.0        # V_j = e_j
    cache = _hand_cache(kv, vv, L=3)
    q = np.zeros((1, 1, D), np.uint16)
    q[0, 0, 0] = 0x3F80                      # bf16 1.0: q = e_0
    out, lse = O.kv_attention(q, cache, 3, [(0, 3)], scale=1.0)
    np.testing.assert_allclose(out[0, 0, :3], ex["softmax"], rtol=1e-15, atol=0)
    assert np.all(out[0, 0, 3:] == 0)
    assert abs(lse[0, 0] - ex["lse"]) < 1e-14
    # the K mean shifts every score by q.m: weights unchanged, lse moves by it
    mean = np.zeros((1, 1, D))
    mean[0, 0, 0] = 5.0
    cache_m = _hand_cache(kv, vv, L=3, mean=mean)
    out_m, lse_m = O.kv_attention(q, cache_m, 3, [(0, 3)], scale=1.0)
    np.testing.assert_allclose(out_m[0, 0, :3], ex["softmax"], rtol=1e-14)
    assert abs(lse_m[0, 0] - (ex["lse"] + 5.0)) < 1e-13
    # a K tensor scale of 2 doubles the scores: softmax of (0, 2, 4) = softmax of (0, 1, 2) at scale 2
    cache_g = _hand_cache(kv, vv, L=3, gk=[2.0])
    out_g, _ = O.kv_attention(q, cache_g, 3, [(0, 3)], scale=1.0)
    out_s, _ = O.kv_attention(q, cache, 3, [(0, 3)], scale=2.0)
    np.testing.assert_allclose(out_g, out_s, rtol=1e-15)
    assert out_g[0, 0, 2] > ex["softmax"][2]


def test_zero_query_is_the_mean_of_v_over_the_key_set():
    Hkv, T, D, L = 2, 96, 32, 32
    cache = _random_cache(Hkv, T, D, L, 11)
    Vx = _decode(cache["v_codes"], cache["v_scales"], cache["v_tensor_scale"], None, L)
    ranges = [(5, 20), (40, 1), (70, 26), (10, 3)]       # keys 10..12 listed twice
    keys = _keys(ranges)
    q = np.zeros((4, 3, D), np.uint16)                   # H = 4 over H_kv = 2
    out, lse = O.kv_attention(q, cache, L, ranges)
    for h in range(4):
        ref = Vx[h // 2, keys].mean(axis=0)
        np.testing.assert_allclose(out[h], np.broadcast_to(ref, (3, D)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(len(keys)), rtol=1e-15)


def test_single_key_returns_its_value():
    Hkv, T, D, L = 1, 64, 32, 16
    cache = _random_cache(Hkv, T, D, L, 12)
    Kx = _decode(cache["k_codes"], cache["k_scales"], cache["k_tensor_scale"], cache["k_mean"], L)
    Vx = _decode(cache["v_codes"], cache["v_scales"], cache["v_tensor_scale"], None, L)
    q = W.bf16_bits(W.queries(1, 2, D, 5))
    for j in (0, 17, 63):
        out, lse = O.kv_attention(q, cache, L, [(j, 1)], scale=0.3)
        np.testing.assert_array_equal(out[0], np.broadcast_to(Vx[0, j], (2, D)))
        np.testing.assert_allclose(lse[0], 0.3 * _qf(q)[0] @ Kx[0, j], rtol=1e-13)


def test_matches_scipy_softmax_on_numpy_scores():
    Hkv, T, D, L = 2, 128, 64, 32
    cache = _random_cache(Hkv, T, D, L, 13)
    Kx = _decode(cache["k_codes"], cache["k_scales"], cache["k_tensor_scale"], cache["k_mean"], L)
    Vx = _decode(cache["v_codes"], cache["v_scales"], cache["v_tensor_scale"], None, L)
    H, Tq = 4, 9
    q = W.bf16_bits(W.queries(H, Tq, D, 6))
    ranges = [(0, 16), (50, 45), (127, 1)]
    keys = _keys(ranges)
    scale = 1.0 / np.sqrt(D)
    out, lse = O.kv_attention(q, cache, L, ranges)
    qf = _qf(q)
    for h in range(H):
        s = scale * qf[h] @ Kx[h // 2, keys].T
        np.testing.assert_allclose(out[h], scipy.special.softmax(s, axis=1) @ Vx[h // 2, keys], rtol=1e-11,
                                   atol=1e-12)
        np.testing.assert_allclose(lse[h], scipy.special.logsumexp(s, axis=1), rtol=1e-13)


def test_key_order_and_splitting_do_not_matter():
    Hkv, T, D, L = 1, 128, 32, 64
    cache = _random_cache(Hkv, T, D, L, 14)
    q = W.bf16_bits(W.queries(1, 5, D, 7))
    a = O.kv_attention(q, cache, L, [(0, 128)])
    b = O.kv_attention(q, cache, L, [(100, 28), (0, 37), (37, 63)])
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14)


def test_chunk_mean_moves_that_chunk_only():
    """Two chunks with identical codes, scales and tensor scales whose K means
    differ by delta on one channel: every key of chunk 1 gets the extra weight
    w = exp(scale * q_d * delta), so the output equals chunk 0 alone and the
    log-sum-exp is that of chunk 0 plus ln(1 + w)."""
    D, L = 32, 48
    base = _random_cache(1, L, D, L, 15)
    cache = {k: (np.concatenate([v, v], axis=1) if k in ("k_codes", "v_codes", "k_scales", "v_scales") else v)
             for k, v in base.items()}
    cache["k_tensor_scale"] = np.repeat(base["k_tensor_scale"], 2)
    cache["v_tensor_scale"] = np.repeat(base["v_tensor_scale"], 2)
    m = np.repeat(base["k_mean"], 2, axis=0)
    delta, d = 1.25, 7
    m[1, 0, d] += delta
    cache["k_mean"] = m
    q = W.bf16_bits(W.queries(1, 6, D, 8))
    scale = 0.2
    one = O.kv_attention(q, base, L, [(0, L)], scale=scale)
    two = O.kv_attention(q, cache, L, [(0, 2 * L)], scale=scale)
    w = np.exp(scale * _qf(q)[0, :, d] * np.float64(np.float32(m[1, 0, d]) - np.float32(m[0, 0, d])))
    np.testing.assert_allclose(two[0], one[0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(two[1][0], one[1][0] + np.log1p(w), rtol=1e-12)


def test_value_tensor_scale_is_linear():
    Hkv, T, D, L = 1, 64, 32, 64
    cache = _random_cache(Hkv, T, D, L, 16)
    q = W.bf16_bits(W.queries(1, 4, D, 9))
    c2 = dict(cache)
    c2["v_tensor_scale"] = cache["v_tensor_scale"] * 2
    a = O.kv_attention(q, cache, L, [(3, 50)])
    b = O.kv_attention(q, c2, L, [(3, 50)])
    np.testing.assert_array_equal(b[0], 2 * a[0])
    np.testing.assert_array_equal(b[1], a[1])


def test_empty_key_set():
    cache = _random_cache(1, 32, 32, 32, 17)
    q = W.bf16_bits(W.queries(2, 3, 32, 10))
    for ranges in ([], [(4, 0)]):
        out, lse = O.kv_attention(q, cache, 32, ranges)
        assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_row_subset_matches_full_run():
    cache = _random_cache(2, 64, 32, 32, 18)
    q = W.bf16_bits(W.queries(4, 7, 32, 11))
    full = O.kv_attention(q, cache, 32, [(0, 64)])
    rows = np.array([0, 6, 13, 27])
    sub = O.kv_attention(q, cache, 32, [(0, 64)], rows=rows)
    np.testing.assert_array_equal(sub[0], full[0].reshape(-1, 32)[rows])
    np.testing.assert_array_equal(sub[1], full[1].reshape(-1)[rows])


@pytest.mark.parametrize("bad", [[(-1, 4)], [(30, 5)], [(0, -1)]])
def test_rejects_ranges_outside_the_cache(bad):
    cache = _random_cache(1, 32, 32, 32, 19)
    q = np.zeros((1, 1, 32), np.uint16)
    with pytest.raises(ValueError):
        O.kv_attention(q, cache, 32, bad)
