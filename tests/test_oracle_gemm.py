"""Pins of the oracle's W4A4 GEMM (the NVFP4 linear layers of the
LongLive-2.0 summary page's training pipeline, step 4, and inference
pipeline, step 6): a hand-worked 16-wide product, numpy's matmul on operands
decoded here from the pinned codecs, the 2D-tile layout against the same
weight expanded to 1D blocks, and linearity in the tensor scales."""
import numpy as np

import oracle as O
import workloads as W


def _decode(codes, scales, g, rows_per_scale=1):
    lo, hi = codes & 15, codes >> 4
    R, K2 = codes.shape
    v = O.e2m1_decode(np.stack([lo, hi], -1).reshape(R, 2 * K2)).astype(np.float64)
    S = O.e4m3_decode(scales).astype(np.float64)
    S = np.repeat(np.repeat(S, 16, axis=1), rows_per_scale, axis=0)
    return v * S * float(np.asarray(g).reshape(-1)[0])


def _pack(vals):
    table = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    c = np.vectorize(lambda x: table[abs(float(x))] | (8 if x < 0 else 0))(np.asarray(vals)).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def test_worked_example():
    # A = [1, 0.5, 0, ...] * S 1 * g 2;  W rows [2, 4, 0, ...] and [-6, 1, 0, ...] * S 0.5 * g 1
    a = np.zeros((1, 16)); a[0, :2] = [1.0, 0.5]
    w = np.zeros((2, 16)); w[0, :2] = [2.0, 4.0]; w[1, :2] = [-6.0, 1.0]
    A = (_pack(a), np.array([[0x38]], np.uint8), np.array([2.0], np.float32))   # E4M3 0x38 = 1.0
    Wt = (_pack(w), np.array([[0x30], [0x30]], np.uint8), np.array([1.0], np.float32))  # 0x30 = 0.5
    out = O.gemm_w4a4(A, Wt, w2d=False)
    # 2 * (1*2*0.5 + 0.5*4*0.5) = 4;  2 * (1*(-6)*0.5 + 0.5*1*0.5) = -5.5
    np.testing.assert_array_equal(out, [[4.0, -5.5]])


def test_matches_numpy_matmul_of_decoded_operands():
    x, sm, w = W.act_weight(act_rows=96, act_cols=256, w_rows=64, w_cols=256)
    a = O.quantize_1d(W.bf16_bits(x), hadamard=True, sign_mask=sm)
    q2 = O.quantize_2d(W.bf16_bits(w))
    q1 = O.quantize_1d(W.bf16_bits(w))
    A = (a["codes"], a["scales"], a["tensor_scale"])
    Ad = _decode(*A)
    for q, w2d in ((q2, True), (q1, False)):
        Wq = (q["codes"], q["scales"], q["tensor_scale"])
        Wd = _decode(*Wq, rows_per_scale=16 if w2d else 1)
        np.testing.assert_allclose(O.gemm_w4a4(A, Wq, w2d), Ad @ Wd.T, rtol=1e-12, atol=1e-12)


def test_2d_tiles_equal_expanded_1d_blocks():
    _, _, w = W.act_weight(act_rows=16, act_cols=64, w_rows=48, w_cols=64)
    x, _, _ = W.act_weight(act_rows=32, act_cols=64, w_rows=16, w_cols=64)
    a = O.quantize_1d(W.bf16_bits(x))
    q = O.quantize_2d(W.bf16_bits(w))
    A = (a["codes"], a["scales"], a["tensor_scale"])
    out2 = O.gemm_w4a4(A, (q["codes"], q["scales"], q["tensor_scale"]), True)
    out1 = O.gemm_w4a4(A, (q["codes"], np.repeat(q["scales"], 16, axis=0), q["tensor_scale"]), False)
    np.testing.assert_array_equal(out2, out1)


def test_tensor_scales_are_linear():
    x, _, w = W.act_weight(act_rows=16, act_cols=64, w_rows=32, w_cols=64)
    a = O.quantize_1d(W.bf16_bits(x))
    q = O.quantize_2d(W.bf16_bits(w))
    A = (a["codes"], a["scales"], a["tensor_scale"])
    Wq = (q["codes"], q["scales"], q["tensor_scale"])
    base = O.gemm_w4a4(A, Wq, True)
    A4 = (a["codes"], a["scales"], a["tensor_scale"] * 4)
    W2 = (q["codes"], q["scales"], q["tensor_scale"] * 0.5)
    np.testing.assert_allclose(O.gemm_w4a4(A4, W2, True), 2 * base, rtol=1e-15)
