"""GPU parity of the activation (1D + random Hadamard) and weight (2D tile)
quantizers against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import say, to_np

pytestmark = pytest.mark.gpu


def _filled(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0x5A)  # sentinel: a missing write cannot pass
    return t


def _check_1d(xb, mode, hadamard, mask):
    x = W.from_bits(xb, "cuda")
    rows, cols = xb.shape
    out = P.nvfp4_quantize_1d(x, mode, hadamard, mask, out={
        "codes": _filled((rows, cols // 2), torch.uint8), "scales": _filled((rows, cols // 16), torch.uint8),
        "tensor_scale": _filled((1,), torch.float32)})
    torch.cuda.synchronize()
    ref = O.quantize_1d(xb, mode, hadamard, mask)
    for key in ("codes", "scales"):
        a = out[key].cpu().numpy()
        assert np.array_equal(a, ref[key]), (key, int((a != ref[key]).sum()))
    assert out["tensor_scale"].cpu().numpy().view(np.uint32)[0] == ref["tensor_scale"].view(np.uint32)[0]
    d = P.nvfp4_dequantize(out["codes"].view(1, rows, cols // 2), out["scales"].view(1, rows, cols // 16),
                           out["tensor_scale"], None, rows, out=_filled((1, rows, cols), torch.bfloat16))
    torch.cuda.synchronize()
    rd = O.dequantize(ref["codes"][None], ref["scales"][None], ref["tensor_scale"], None, rows)
    assert np.array_equal(to_np(d), rd)
    return ref


def test_activation_workload_with_rht():
    say("activation [16384, 3072] RHT, seed", W.SEED_ACT)
    x, mask, _ = W.act_weight(act_rows=W.ACT_ROWS, act_cols=W.ACT_COLS, w_rows=16, w_cols=16)
    _check_1d(W.bf16_bits(x), O.MODE_4OVER6, True, mask)


@pytest.mark.parametrize("rows,cols,mode,had", [
    (64, 256, O.MODE_4OVER6, False), (33, 48, O.MODE_4OVER6, True), (1, 16, O.MODE_FIXED6, True),
    (100, 3072, O.MODE_FIXED4, True), (7, 4096 - 16, O.MODE_4OVER6, True),
])
def test_activation_shapes_and_modes(rows, cols, mode, had):
    say("activation", rows, cols, "mode", mode, "rht", had)
    x, mask = W.activation(rows, cols, 17 + rows)
    _check_1d(W.bf16_bits(x), mode, had, mask)


def _check_2d(wb, mode):
    w = W.from_bits(wb, "cuda")
    rows, cols = wb.shape
    out = P.nvfp4_quantize_2d(w, mode, out={
        "codes": _filled((rows, cols // 2), torch.uint8), "scales": _filled((rows // 16, cols // 16), torch.uint8),
        "tensor_scale": _filled((1,), torch.float32)})
    torch.cuda.synchronize()
    ref = O.quantize_2d(wb, mode)
    for key in ("codes", "scales"):
        a = out[key].cpu().numpy()
        assert np.array_equal(a, ref[key]), (key, int((a != ref[key]).sum()))
    assert out["tensor_scale"].cpu().numpy().view(np.uint32)[0] == ref["tensor_scale"].view(np.uint32)[0]
    d = P.nvfp4_dequantize_2d(out["codes"], out["scales"], out["tensor_scale"],
                              out=_filled((rows, cols), torch.bfloat16))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(d), O.dequantize_2d(ref["codes"], ref["scales"], ref["tensor_scale"]))


def test_weight_workload():
    say("weight [3072, 3072] 2D tiles")
    _, _, w = W.act_weight(act_rows=16, act_cols=16)
    _check_2d(W.bf16_bits(w), O.MODE_4OVER6)


@pytest.mark.parametrize("rows,cols,mode", [
    (16, 16, O.MODE_4OVER6), (48, 80, O.MODE_4OVER6), (32, 48, O.MODE_FIXED6), (160, 16, O.MODE_FIXED4),
    (16, 272, O.MODE_4OVER6),
])
def test_weight_shapes_and_modes(rows, cols, mode):
    say("weight", rows, cols, "mode", mode)
    w = W.weight(rows, cols, 23 + cols)
    # add structure so that both candidates win somewhere
    wb = W.bf16_bits(w)
    _check_2d(wb, mode)
