"""GPU parity of nvfp4_gemm_w4a4 with the oracle's fp64 product of the
exactly decoded operands.  Operands come from the oracle's quantizers (the
activation with the random Hadamard transform, the weight as 2D tiles or 1D
blocks).  Tolerance from the kernel's arithmetic: the operands decode
exactly, products are exact in fp32, the fp32 accumulation of K terms is
within (K + 1) 2^-24 sum_k |a_k w_k| of the exact sum in any order, the
tensor-scale product rounds once (2^-24) and the output once to bf16 (unit
roundoff 2^-8); so with acc = (K + 2) 2^-24 sum_k |a_k w_k|,
|out - ref| <= acc + 2^-8 (|ref| + acc), plus an RMS check against the bf16
rounding level."""
import numpy as np
import pytest
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _decode(codes, scales, g, rows_per_scale=1):
    lo, hi = codes & 15, codes >> 4
    R, K2 = codes.shape
    v = O.e2m1_decode(np.stack([lo, hi], -1).reshape(R, 2 * K2)).astype(np.float64)
    S = np.repeat(np.repeat(O.e4m3_decode(scales).astype(np.float64), 16, axis=1), rows_per_scale, axis=0)
    return v * S * float(np.asarray(g).reshape(-1)[0])


def _gpu(x):
    return {k: torch.from_numpy(np.ascontiguousarray(x[k])).cuda() for k in ("codes", "scales", "tensor_scale")}


def _check(a, w, w2d, got, rows):
    A = (a["codes"][rows], a["scales"][rows], a["tensor_scale"])
    Wq = (w["codes"], w["scales"], w["tensor_scale"])
    ref = O.gemm_w4a4(A, Wq, w2d)
    Ad = np.abs(_decode(*A))
    Wd = np.abs(_decode(*Wq, rows_per_scale=16 if w2d else 1))
    K = Ad.shape[1]
    acc = (K + 2) * 2.0 ** -24 * (Ad @ Wd.T)
    tol = acc + 2.0 ** -8 * (np.abs(ref) + acc)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= tol), (f"{(err > tol).sum()} out of bound, worst excess {(err - tol).max():.3g}")
    rms, rms_ref = np.sqrt(np.mean(err ** 2)), np.sqrt(np.mean(ref ** 2))
    say(f"gemm rms err {rms:.3g} = {rms / rms_ref:.3g} x rms(ref), max err/bound {(err / np.maximum(tol, 1e-300)).max():.3g}")
    assert rms <= 2.0 ** -8 * rms_ref


@pytest.mark.parametrize("M,N,K", [(300, 80, 192), (256, 256, 64), (17, 512, 320)])
@pytest.mark.parametrize("w2d", [True, False], ids=["w2d", "w1d"])
def test_small_shapes(M, N, K, w2d):
    say("gemm", M, N, K, w2d)
    x, sm, wt = W.act_weight(act_rows=M, act_cols=K, w_rows=N, w_cols=K)
    a = O.quantize_1d(W.bf16_bits(x), hadamard=True, sign_mask=sm)
    w = O.quantize_2d(W.bf16_bits(wt)) if w2d else O.quantize_1d(W.bf16_bits(wt))
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    P.nvfp4_gemm_w4a4(_gpu(a), _gpu(w), w2d, out=out)
    torch.cuda.synchronize()
    _check(a, w, w2d, out.float().cpu().numpy().astype(np.float64), np.arange(M))


def test_activation_weight_workload_sampled():
    """The activation / weight pair of the benchmark: [16384, 3072] activation
    (1D blocks after the RHT) times the [3072, 3072] weight (2D tiles); 48
    sampled rows, the first and last included, against the oracle."""
    x, sm, wt = W.act_weight()
    say("gemm workload", tuple(x.shape), tuple(wt.shape))
    a = O.quantize_1d(W.bf16_bits(x), hadamard=True, sign_mask=sm)
    w = O.quantize_2d(W.bf16_bits(wt))
    del x, wt
    out = P.nvfp4_gemm_w4a4(_gpu(a), _gpu(w), True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    M = a["codes"].shape[0]
    rows = np.unique(np.concatenate([rng.integers(0, M, 46), [0, M - 1]]))
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    _check(a, w, True, got, rows)


def test_degenerate():
    x, sm, wt = W.act_weight(act_rows=32, act_cols=64, w_rows=16, w_cols=64)
    a = O.quantize_1d(W.bf16_bits(x))
    w = O.quantize_2d(W.bf16_bits(wt))
    zero = {k: (np.zeros_like(v) if k != "tensor_scale" else v) for k, v in w.items() if k != "use4"}
    out = P.nvfp4_gemm_w4a4(_gpu(a), _gpu(zero), True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0
    empty = {k: v[:0] for k, v in _gpu(a).items() if k != "tensor_scale"}
    empty["tensor_scale"] = _gpu(a)["tensor_scale"]
    assert P.nvfp4_gemm_w4a4(empty, _gpu(w), True).shape == (0, 16)
