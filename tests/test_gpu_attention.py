"""GPU parity of nvfp4_kv_attention (attention over the NVFP4 cache) with the
oracle's fp64 attention over the exactly decoded cache.

The caches are built by the oracle quantizer from the seeded workloads, so
both sides read the same bytes.  Tolerance (derived from the kernel's
arithmetic, stated per row):
  - K~ = v * S is exact in bf16, so a logit differs from the exact one only by
    fp32 accumulation and scaling: at most
    delta = 2^-16 * sigma * sum_d |q_d| (g_K |v S|_jd + |m_d|)  (base-2 units),
    sigma = scale * log2(e);
  - with eps = ln 2 * max_j delta the normalized weights move by at most
    exp(2 eps) - 1 in total; P and V~ = bf16(v S g_V) are rounded to bf16
    (unit roundoff 2^-8 each, so at most 2^-8 max_j |V_jd| each on the
    output), exp2 is within 2^-20 relative, and out is rounded to bf16, so
      pre = max_j |V_jd| (exp(2 eps) - 1 + 2^-7 + 2^-16),
      |out - ref|_d <= pre + 2^-8 (|ref_d| + pre),
      |lse - ref|   <= eps + 2^-20 |ref| + 1e-5.
  The per-element bound assumes every rounding aligned, so each case also
  checks the RMS error against the bf16 rounding level, and the zero-query
  case (all weights exactly 1) checks the key set itself.
"""
import numpy as np
import pytest
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import attention_check as _check, decode_exact as _decode, key_list as _keys, say

pytestmark = pytest.mark.gpu



def _cache(kb, vb, L):
    return O.smooth_quantize(kb, vb, L)


def _to_gpu(c):
    keys = ("k_codes", "k_scales", "k_tensor_scale", "k_mean", "v_codes", "v_scales", "v_tensor_scale")
    return {k: (None if c.get(k) is None else torch.from_numpy(np.ascontiguousarray(c[k])).cuda()) for k in keys}


def _run_gpu(q_bits, cache, L, ranges, scale=None, mode="staged"):
    """mode: "staged" -- a workspace for every key split and the decoded
    image of every key tile (each tile decoded once per call); "staged-1" --
    one byte less (the decode on load); "split" -- a workspace for the splits
    only (each query block decodes its tiles); "unsplit" -- no workspace."""
    q = W.from_bits(q_bits, "cuda")
    H, Tq, D = q.shape
    out = torch.empty(H, Tq, D, dtype=torch.bfloat16, device="cuda")
    out.view(torch.uint8).fill_(0xFF)          # NaN: an unwritten output cannot pass
    ws = False
    if mode != "unsplit":
        Hkv, T = cache["k_codes"].shape[:2]
        n = (P.nvfp4_kv_attention_staged_workspace_bytes(H, Tq, D, Hkv, T, L, ranges) if mode.startswith("staged")
             else P.nvfp4_kv_attention_workspace_bytes(H, Tq, D))
        if mode == "staged-1":
            n -= 1
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)                         # garbage on entry
    o, lse = P.nvfp4_kv_attention(q, _to_gpu(cache), L, ranges, softmax_scale=scale, out=out, lse=True,
                                  workspace=ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _full(q_bits, cache, L, ranges, scale=None, mode="staged", **kw):
    H, Tq, D = q_bits.shape
    got, got_lse = _run_gpu(q_bits, cache, L, ranges, scale, mode)
    rows = np.arange(H * Tq)
    _check(q_bits, cache, L, ranges, got.reshape(-1, D), got_lse.reshape(-1), rows, scale, **kw)


def test_zero_query_weights_every_listed_key_equally():
    """q = 0: every logit is exactly 0, so out is the mean of V~ over the key
    set (duplicates counted) and lse = ln N; V~ and out are bf16 roundings
    (unit roundoff 2^-8 each), so a dropped, extra or misplaced key (weight
    1/N) shows."""
    H, Hkv, T, L, D, Tq = 4, 2, 600, 200, 128, 37
    say("zero query", H, Hkv, T, L, Tq)
    k, v = W.gaussian_kv(W.KVShape(Hkv, T, D, L), 21)
    cache = _cache(W.bf16_bits(k), W.bf16_bits(v), L)
    ranges = [(5, 130), (210, 1), (390, 210), (7, 3)]
    q = np.zeros((H, Tq, D), np.uint16)
    got, got_lse = _run_gpu(q, cache, L, ranges)
    keys = _keys(ranges)
    Vx = _decode(cache["v_codes"], cache["v_scales"], cache["v_tensor_scale"], L)[:, keys]
    for h in range(H):
        ref = Vx[h // 2].mean(axis=0)
        tol = 2.0 ** -8 * np.abs(Vx[h // 2]).mean(axis=0) + 2.0 ** -8 * np.abs(ref) + 1e-6
        assert np.all(np.abs(got[h] - ref) <= tol), np.abs(got[h] - ref).max()
    np.testing.assert_allclose(got_lse, np.log(len(keys)), rtol=1e-6)


RANDOM_CASES = [
    (2, 2, 640, 128, 300, [(0, 640)]),                         # 5 chunks, ragged query block
    (4, 2, 640, 128, 256, [(0, 70), (200, 77), (383, 257)]),   # grouped heads, segment edges inside tiles
    (3, 1, 512, 64, 17, [(448, 64), (0, 64), (100, 1)]),       # one cache head, single-key range
    (1, 1, 96, 96, 513, [(0, 96)]),                            # one chunk shorter than two tiles
    (2, 2, 192, 64, 1, [(64, 64)]),                            # one tile, one query
    (6, 3, 448, 64, 300, [(3, 61), (64, 65), (257, 190)]),     # pieces starting mid-chunk, a one-key piece (6 tiles)
]


def _random_case(H, Hkv, T, L, Tq):
    k, v = W.gaussian_kv(W.KVShape(Hkv, T, 128, L), 22 + T + Tq)
    return _cache(W.bf16_bits(k), W.bf16_bits(v), L), W.bf16_bits(W.queries(H, Tq, 128, 31 + Tq))


@pytest.mark.parametrize("mode", ["staged", "split", "unsplit"])
@pytest.mark.parametrize("H,Hkv,T,L,Tq,ranges", RANDOM_CASES)
def test_random_cache(H, Hkv, T, L, Tq, ranges, mode):
    say("random cache", H, Hkv, T, L, Tq, ranges, mode)
    cache, q = _random_case(H, Hkv, T, L, Tq)
    _full(q, cache, L, ranges, mode=mode)


@pytest.mark.parametrize("H,Hkv,T,L,Tq,ranges", RANDOM_CASES)
def test_staged_equals_decode_on_load(H, Hkv, T, L, Tq, ranges):
    """The staged form copies into LDS the bytes the per-block decode would
    write there and splits the keys the same way, so out and lse equal the
    decode-on-load form's bit for bit."""
    say("staged vs decode on load", H, Hkv, T, L, Tq, ranges)
    cache, q = _random_case(H, Hkv, T, L, Tq)
    a = _run_gpu(q, cache, L, ranges, mode="split")
    b = _run_gpu(q, cache, L, ranges, mode="staged")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # one byte short of the staged size: the decode on load, with the same splits
    c = _run_gpu(q, cache, L, ranges, mode="staged-1")
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_staged_narrow_and_wide_loads_agree():
    """The staging kernel copies a tile's code and scale rows with wide loads
    when the codes are 16-byte and the scales 8-byte aligned, else it gathers
    them as the decode on load does: a cache whose V codes sit 2 bytes and K
    scales 1 byte off such a boundary gives the same bits, and both match the
    oracle."""
    H, Hkv, T, L, Tq, ranges = 4, 2, 640, 128, 256, [(0, 70), (200, 77), (383, 257)]
    say("staged, unaligned cache", H, Hkv, T, L, Tq, ranges)
    cache, q_bits = _random_case(H, Hkv, T, L, Tq)
    gc = _to_gpu(cache)

    def shifted(t, off):
        flat = t.reshape(-1)
        buf = torch.empty(flat.numel() + off, dtype=torch.uint8, device="cuda")
        out = buf[off:]
        out.copy_(flat)
        return out.view(t.shape)

    mis = dict(gc)
    mis["v_codes"] = shifted(gc["v_codes"], 2)
    mis["k_scales"] = shifted(gc["k_scales"], 1)
    assert mis["v_codes"].data_ptr() % 16 == 2 and mis["k_scales"].data_ptr() % 8 == 1
    q = W.from_bits(q_bits, "cuda")
    ws = torch.empty(P.nvfp4_kv_attention_staged_workspace_bytes(H, Tq, 128, Hkv, T, L, ranges),
                     dtype=torch.uint8, device="cuda")
    a, la = P.nvfp4_kv_attention(q, gc, L, ranges, lse=True, workspace=ws)
    b, lb = P.nvfp4_kv_attention(q, mis, L, ranges, lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
    got = a.float().cpu().numpy().astype(np.float64).reshape(-1, 128)
    _check(q_bits, cache, L, ranges, got, la.cpu().numpy().astype(np.float64).reshape(-1), np.arange(H * Tq))


def test_heavy_tail_cache_and_sharp_softmax():
    """Student-t K and V with per-channel scales, and softmax_scale 1 (logits
    ~11x larger than 1/sqrt(D)): weights concentrate on few keys."""
    H, T, L, Tq = 2, 384, 128, 130
    say("heavy tail", H, T, L, Tq)
    k, v = W.heavy_tail_kv(W.KVShape(H, T, 128, L), 23)
    cache = _cache(W.bf16_bits(k), W.bf16_bits(v), L)
    q = W.bf16_bits(W.queries(H, Tq, 128, 32))
    _full(q, cache, L, [(0, T)])
    _full(q, cache, L, [(0, T)], scale=1.0)


def test_no_mean_single_key_and_empty():
    H, T, L, Tq = 2, 128, 64, 40
    say("no mean / single key / empty", H, T, L, Tq)
    k, v = W.gaussian_kv(W.KVShape(H, T, 128, L), 24)
    cache = _cache(W.bf16_bits(k), W.bf16_bits(v), L)
    q = W.bf16_bits(W.queries(H, Tq, 128, 33))
    nomean = dict(cache)
    nomean["k_mean"] = None
    _full(q, nomean, L, [(0, T)])
    _full(q, nomean, L, [(0, T)], mode="unsplit")
    _full(q, cache, L, [(77, 1)])
    got, got_lse = _run_gpu(q, cache, L, [])
    assert np.all(got == 0) and np.all(np.isneginf(got_lse))
    got, got_lse = _run_gpu(q, cache, L, [(5, 0)])
    assert np.all(got == 0) and np.all(np.isneginf(got_lse))


def test_deterministic():
    H, T, L, Tq = 2, 256, 128, 300
    k, v = W.gaussian_kv(W.KVShape(H, T, 128, L), 25)
    cache = _cache(W.bf16_bits(k), W.bf16_bits(v), L)
    q = W.bf16_bits(W.queries(H, Tq, 128, 34))
    a = _run_gpu(q, cache, L, [(0, T)])
    b = _run_gpu(q, cache, L, [(0, T)])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("layout", ["all", "sink"])
def test_full_cache_layer_sampled(layout):
    """The benchmark's workload: one chunk of queries (24 heads x 7040) over
    the 8-chunk cache layer (56320 keys), either every key or the sink layout
    (global sink, shot sink across a chunk edge, recent window); 64 sampled
    query rows, including the last, ragged query block, against the oracle."""
    shape = W.CACHE_LAYER
    say("full cache layer", layout, shape)
    k, v = W.gaussian_kv(shape, W.cache_layer_seed(0), device="cuda")
    cache = _cache(W.bf16_bits(k), W.bf16_bits(v), shape.chunk_len)
    del k, v
    q = W.bf16_bits(W.queries(shape.H, W.ATTN_QUERIES, shape.D, W.SEED_ATTN))
    ranges = [(0, shape.T)] if layout == "all" else W.sink_ranges(shape.n_chunks)
    got, got_lse = _run_gpu(q, cache, shape.chunk_len, ranges)       # staged, as the benchmark runs it
    ref = _run_gpu(q, cache, shape.chunk_len, ranges, mode="split")   # decode on load
    assert np.array_equal(got, ref[0]) and np.array_equal(got_lse, ref[1])
    del ref
    Tq = W.ATTN_QUERIES
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.integers(0, shape.H * Tq, 56), [0, Tq - 1, shape.H * Tq - 1],
                                     (shape.H - 1) * Tq + np.arange(Tq - 5, Tq)]))
    _check(q, cache, shape.chunk_len, ranges, got.reshape(-1, shape.D)[rows], got_lse.reshape(-1)[rows], rows)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse))
