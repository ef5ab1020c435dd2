"""Pins of the oracle's 3-bit and 2-bit KV quantizer (the direction to
extend the NVFP4 KV cache to 3 and 2 bits; the format is the reading stated in
tests/golden/lowbit_examples.json) against what the format definitions and
the mathematics fix: the grids' closed forms, an independent threshold
encoder over every fp32 in the quantizer's range, hand-derived worked
examples, exact-arithmetic brute force of the best-of-two choice, the
single-candidate modes as textbook absmax quantizers, invariants, and the
dequantize formula through numpy and torch's bf16 cast."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MAG = {3: np.array([0, .5, 1, 1.5]), 2: np.array([0.0, 1.0])}
DIV = {3: (1.5, 1.0), 2: (1.0, 1.5)}  # (c_a, c_b)


def _bits(x):
    return W.bf16_bits(torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16))


def _torch_e4m3(r):
    return torch.from_numpy(np.ascontiguousarray(r, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_val(s):
    return torch.from_numpy(np.ascontiguousarray(s, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _unpack(codes, bits):
    """codes [..., 2 * bits * nblocks] bytes -> element codes [..., 16 * nblocks], LSB first."""
    b = np.unpackbits(codes, axis=-1, bitorder="little").reshape(*codes.shape[:-1], -1, bits)
    return (b * (1 << np.arange(bits))).sum(-1).astype(np.uint8)


@pytest.mark.parametrize("bits", [3, 2])
def test_decode_is_the_grid(bits):
    n = len(MAG[bits])
    for c in range(2 * n):
        mag = MAG[bits][c % n]
        want = -mag if c >= n else mag
        got = O.lib().ora_lowbit_decode(bits, c)
        assert got == want and np.signbit(got) == (c >= n), (c, got)
    # E1M1 with bias 1 (the E2M1 definition with one exponent bit): e = 0 gives
    # m / 2, e = 1 gives 1 + m / 2
    if bits == 3:
        assert [0.5 * m for m in (0, 1)] + [1 + 0.5 * m for m in (0, 1)] == list(MAG[3])


def _threshold_encode(bits, y):
    """Independent encoder: magnitude index by comparing |y| with the
    midpoints, a midpoint going to the even index, saturating at the top."""
    a = np.abs(y.astype(np.float64))
    mids = (MAG[bits][:-1] + MAG[bits][1:]) / 2
    k = (a[:, None] > mids).sum(-1)
    at = (a[:, None] == mids)
    k = np.where(at.any(-1), np.where(at.argmax(-1) % 2 == 0, at.argmax(-1), at.argmax(-1) + 1), k)
    return (k | (np.signbit(y).astype(np.int64) << (bits - 1))).astype(np.uint8)


@pytest.mark.parametrize("bits", [3, 2])
def test_encode_every_fp32_in_range(bits):
    # every fp32 pattern with 2^-5 <= |y| < 4 (the ties and the saturation
    # at the top included), both signs, in slices; plus zeros and a sample of
    # everything else
    lo = np.float32(2.0 ** -5).view(np.uint32)
    hi = np.float32(4.0).view(np.uint32)
    step = 1 << 23
    for s in range(int(lo), int(hi), step):
        u = np.arange(s, min(s + step, int(hi)), dtype=np.uint32)
        for sign in (0, 0x80000000):
            y = (u | np.uint32(sign)).view(np.float32)
            assert np.array_equal(O.lowbit_encode(bits, y), _threshold_encode(bits, y)), (bits, s, sign)
    rng = np.random.default_rng(5)
    y = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    y = np.concatenate([y[np.isfinite(y)], np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    assert np.array_equal(O.lowbit_encode(bits, y), _threshold_encode(bits, y))


def _anchored_rows(blocks):
    """Rows of D = 32: the anchor 448 (so that A = C = 448, g_enc = 1), then the block."""
    blocks = np.asarray(blocks, np.float32).reshape(-1, 16)
    anchor = np.zeros((blocks.shape[0], 16), np.float32)
    anchor[0, 0] = 448.0
    rows = np.concatenate([anchor, blocks], axis=1)
    x = _bits(rows)
    assert np.array_equal(O.bf16_to_float(x), rows)  # bf16-exact inputs
    return x.reshape(1, -1, 32)


def test_worked_examples():
    ex = json.load(open(os.path.join(GOLDEN, "lowbit_examples.json")))
    for case in ex["cases"]:
        bits = case["bits"]
        blk = [-0.0 if v == "-0" else float(v) for v in case["block"]]
        x = _anchored_rows([blk])
        q = O.quantize_chunks_lowbit(x, 1, bits, O.MODE_4OVER6, want_errors=True)
        assert q["tensor_scale"][0] == 1.0, case["why"]
        if "erra" in case:
            assert q["erra"][0, 0, 1] == case["erra"] and q["errb"][0, 0, 1] == case["errb"], case["why"]
        assert q["scales"][0, 0, 1] == case["scale"], case["why"]
        assert q["codes"][0, 0, 2 * bits:].tolist() == case["codes"], case["why"]
        # dequantized with g_dec = 1: each value is v * S exactly
        d = O.dequantize_lowbit(q["codes"], q["scales"], q["tensor_scale"], None, 1, bits)
        v = MAG[bits][_unpack(q["codes"][0, 0, 2 * bits:], bits) & ((1 << (bits - 1)) - 1)]
        sgn = np.where(_unpack(q["codes"][0, 0, 2 * bits:], bits) >> (bits - 1), -1.0, 1.0)
        S = float(_e4m3_val(np.array([case["scale"]]))[0])
        assert np.array_equal(O.bf16_to_float(d)[0, 0, 16:], (sgn * v * S).astype(np.float32)), case["why"]


def _exact_candidate(bits, z, c):
    """Exact candidate with divisor c for blocks z [n, 16]: E4M3 index nearest
    to t_b / c (ties even), magnitudes nearest to |z| / S (ties even,
    saturating), and the squared error times 2^32 as an integer."""
    e4 = _e4m3_val(np.arange(127, dtype=np.uint8)).astype(np.float64)
    t = np.abs(z).max(-1).astype(np.float64)
    mids = (e4[:-1] + e4[1:]) / 2
    r = t / c
    sidx = (r[:, None] > mids).sum(-1)
    at = r[:, None] == mids
    sidx = np.where(at.any(-1), np.where(at.argmax(-1) % 2 == 0, at.argmax(-1), at.argmax(-1) + 1), sidx)
    S = e4[sidx]
    grid = MAG[bits]
    gm = (grid[:-1] + grid[1:]) / 2
    a = np.abs(z).astype(np.float64)
    thr = S[:, None, None] * gm
    k = (a[..., None] > thr).sum(-1)
    tie = a[..., None] == thr
    k = np.where(tie.any(-1), np.where(tie.argmax(-1) % 2 == 0, tie.argmax(-1), tie.argmax(-1) + 1), k)
    v = np.where(np.signbit(z), -grid[k], grid[k]) * S[:, None]
    zi = np.rint(z.astype(np.float64) * 2 ** 16).astype(np.int64)
    vi = np.rint(v * 2 ** 16).astype(np.int64)
    assert np.array_equal(zi.astype(np.float64), z.astype(np.float64) * 2 ** 16)
    assert np.array_equal(vi.astype(np.float64), v * 2 ** 16)
    return sidx.astype(np.uint8), k, ((zi - vi) ** 2).sum(-1)


@pytest.mark.parametrize("bits", [3, 2])
def test_best_of_two_matches_exact_arithmetic(bits):
    rng = np.random.default_rng(30 + bits)
    n = 40_000
    sign = rng.integers(0, 2, (n, 16))
    e = rng.integers(-5, 4, (n, 16))
    m = rng.integers(0, 128, (n, 16))
    z = ((1 + m / 128.0) * 2.0 ** e * np.where(sign, -1, 1)).astype(np.float32)
    z[: n // 4, 1:6] = z[: n // 4, :1] * np.float32(0.5)   # companions at half the maximum
    z[n // 4: n // 2, 8:] = 0.0
    z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
    x = _anchored_rows(z)
    q = O.quantize_chunks_lowbit(x, x.shape[1], bits, O.MODE_4OVER6, want_errors=True)
    assert q["tensor_scale"][0] == 1.0
    scales = q["scales"][0, :, 1]
    ca, cb = DIV[bits]
    sa, ka, ea = _exact_candidate(bits, z, ca)
    sb, kb, eb = _exact_candidate(bits, z, cb)
    # excused: the fp32 steps (t_b / c, z * fl(1/S)) land on another side of a
    # rounding boundary than the exact quotient, or the exact errors are closer
    # than the fp32 accumulation resolves
    t = np.abs(z).max(-1)
    sens = np.zeros(n, bool)
    for c, s_ex in ((ca, sa), (cb, sb)):
        sens |= _torch_e4m3((t / np.float32(c)).astype(np.float32)) != s_ex
        S = _e4m3_val(s_ex).astype(np.float32)
        R = np.where(S > 0, np.float32(1) / np.where(S > 0, S, 1), 0).astype(np.float32)
        y = (z * R[:, None]).astype(np.float32)
        mag_fl = O.lowbit_encode(bits, y) & ((1 << (bits - 1)) - 1)
        a = np.abs(z).astype(np.float64)
        grid = MAG[bits]
        gm = (grid[:-1] + grid[1:]) / 2
        thr = S.astype(np.float64)[:, None, None] * gm
        kk = (a[..., None] > thr).sum(-1)
        tie = a[..., None] == thr
        kk = np.where(tie.any(-1), np.where(tie.argmax(-1) % 2 == 0, tie.argmax(-1), tie.argmax(-1) + 1), kk)
        sens |= (mag_fl != kk).any(-1)
    close = np.abs(ea - eb) <= (np.maximum(ea, eb) >> 18) + 1
    want = np.where(eb < ea, sb, sa)
    bad = scales != want
    assert not (bad & ~(sens | close)).any(), np.nonzero(bad & ~(sens | close))[0][:10]
    assert bad.mean() < 1e-2
    # the chosen candidate's fp32 error is never above the other's
    erra, errb = q["erra"][0, :, 1], q["errb"][0, :, 1]
    chose_b = (scales == sb) & (sa != sb)
    assert np.all(np.where(chose_b, errb < erra, erra <= errb) | (sa == sb))
    assert 0.02 < (eb < ea).mean() < 0.98  # both candidates are real choices here


@pytest.mark.parametrize("bits", [3, 2])
def test_single_candidate_modes_are_absmax_quantizers(bits):
    """Mode 1 keeps c_a only, mode 2 c_b only: each is plain absmax block
    quantization, written out with numpy and torch's E4M3 cast."""
    rng = np.random.default_rng(40 + bits)
    H, T, D = 2, 64, 64
    x = _bits(rng.standard_normal((H, T, D)) * np.exp(rng.standard_normal((H, 1, D))))
    xf = O.bf16_to_float(x).astype(np.float32)
    for mode, c in ((O.MODE_FIXED6, DIV[bits][0]), (O.MODE_FIXED4, DIV[bits][1])):
        q = O.quantize_chunks_lowbit(x, T, bits, mode)
        C = np.float32(448.0 * c)
        A = np.abs(xf).max()
        g = C / A
        assert q["tensor_scale"][0] == A / C
        z = (xf * g).astype(np.float32).reshape(H, T, D // 16, 16)
        t = np.abs(z).max(-1)
        s = _torch_e4m3((t / np.float32(c)).astype(np.float32))
        assert np.array_equal(q["scales"], s)
        S = _e4m3_val(s)
        R = np.where(S > 0, np.float32(1) / np.where(S > 0, S, 1), 0).astype(np.float32)
        y = (z * R[..., None]).astype(np.float32)
        if bits == 3:
            k = np.minimum(np.rint(2 * np.abs(y)), 3).astype(np.uint8)  # rint: round half to even
        else:
            k = (np.abs(y) > 0.5).astype(np.uint8)
        codes = k | (np.signbit(y).astype(np.uint8) << (bits - 1))
        assert np.array_equal(_unpack(q["codes"], bits), codes.reshape(H, T, D))


@pytest.mark.parametrize("bits", [3, 2])
def test_invariants(bits):
    rng = np.random.default_rng(50 + bits)
    H, T, D, L = 2, 96, 64, 32
    k = W.bf16_bits(torch.from_numpy((rng.standard_normal((H, T, D)) + 3).astype(np.float32)).to(torch.bfloat16))
    v = W.bf16_bits(torch.from_numpy(rng.standard_normal((H, T, D)).astype(np.float32)).to(torch.bfloat16))
    r = O.smooth_quantize_lowbit(k, v, L, bits, want_errors=True)
    # the kept candidate's error is at most the other's
    for t in ("k", "v"):
        ea, eb = r[t + "_erra"], r[t + "_errb"]
        assert np.all(np.minimum(ea, eb) <= np.maximum(ea, eb))
    # x -> 4x: codes and scales unchanged, tensor scale and mean times 4
    k4 = _bits(O.bf16_to_float(k) * 4)
    v4 = _bits(O.bf16_to_float(v) * 4)
    r4 = O.smooth_quantize_lowbit(k4, v4, L, bits)
    for key in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert np.array_equal(r[key], r4[key]), key
    assert np.array_equal(r4["k_tensor_scale"], r["k_tensor_scale"] * 4)
    assert np.array_equal(r4["k_mean"], r["k_mean"] * 4)
    # x -> -x: every sign bit flips, nothing else
    vn = _bits(-O.bf16_to_float(v))
    rn = O.quantize_chunks_lowbit(vn, L, bits)
    sbit = np.uint8(1 << (bits - 1))
    assert np.array_equal(_unpack(rn["codes"], bits), _unpack(r["v_codes"], bits) ^ sbit)
    assert np.array_equal(rn["scales"], r["v_scales"])


@pytest.mark.parametrize("bits", [3, 2])
def test_dequant_formula_via_numpy_and_torch(bits):
    rng = np.random.default_rng(60 + bits)
    H, T, D, L = 2, 64, 48, 32
    k = _bits(rng.standard_normal((H, T, D)) + 1)
    v = _bits(rng.standard_normal((H, T, D)))
    r = O.smooth_quantize_lowbit(k, v, L, bits)
    for t, mean in (("k", r["k_mean"]), ("v", None)):
        got = O.dequantize_lowbit(r[t + "_codes"], r[t + "_scales"], r[t + "_tensor_scale"], mean, L, bits)
        c = _unpack(r[t + "_codes"], bits)
        val = np.where(c >> (bits - 1), -1.0, 1.0) * MAG[bits][c & ((1 << (bits - 1)) - 1)]
        S = np.repeat(_e4m3_val(r[t + "_scales"]), 16, axis=-1)
        g = np.repeat(r[t + "_tensor_scale"], L)[None, :, None]
        xh = ((val.astype(np.float32) * S).astype(np.float32) * g).astype(np.float32)
        if mean is not None:
            xh = (xh + np.repeat(mean, L, axis=0).transpose(1, 0, 2)).astype(np.float32)
        want = W.bf16_bits(torch.from_numpy(xh).to(torch.bfloat16))
        assert np.array_equal(got, want), t
