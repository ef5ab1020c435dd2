"""GPU parity of nvfp4_kv_quantize_v_tblocks (V blocked along tokens) with the
oracle: codes, scales and tensor scales bit-exact, for every mode, ragged
tiles (chunks that are not a multiple of the 128-token tile), several channel
groups, several 512-row statistics tiles per head with a ragged last one,
more chunks than the launch's statistics-to-quantize distance, heavy-tailed
values and the one-chunk workload; after every call the kernel's error word
(no wait timed out) is checked."""
import numpy as np
import pytest
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _run(vb, L, mode):
    v = W.from_bits(vb, "cuda")
    H, T, D = vb.shape
    out = {"codes": torch.full((H, D, T // 2), 0x5A, dtype=torch.uint8, device="cuda"),
           "scales": torch.full((H, D, T // 16), 0x5A, dtype=torch.uint8, device="cuda"),
           "tensor_scale": torch.full((T // L,), -1.0, dtype=torch.float32, device="cuda")}
    ws = torch.full((max(1, P.lib().nvfp4_kv_quantize_v_tblocks_workspace_bytes(H, T, D, L)),), 0xA5,
                    dtype=torch.uint8, device="cuda")
    ws[:4] = 0  # the sticky error word is the caller's to clear
    P.nvfp4_kv_quantize_v_tblocks(v, L, mode, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "a wait of the single-launch kernel timed out"
    return {k: t.cpu().numpy() for k, t in out.items()}


def _compare(got, ref):
    for k in ("codes", "scales"):
        if not np.array_equal(got[k], ref[k]):
            bad = np.argwhere(got[k] != ref[k])
            raise AssertionError(f"{k}: {len(bad)} mismatches, first {bad[:4].tolist()}")
    assert np.array_equal(got["tensor_scale"].view(np.uint32), ref["tensor_scale"].view(np.uint32))


@pytest.mark.parametrize("mode", [O.MODE_4OVER6, O.MODE_FIXED6, O.MODE_FIXED4])
@pytest.mark.parametrize("H,T,D,L", [(2, 256, 128, 128), (3, 352, 64, 176), (1, 96, 192, 48), (2, 4160, 128, 1040)])
def test_gaussian(H, T, D, L, mode):
    say("v tblocks", H, T, D, L, mode)
    _, v = W.gaussian_kv(W.KVShape(H, T, D, L), 60 + T)
    vb = W.bf16_bits(v)
    _compare(_run(vb, L, mode), O.quantize_v_tblocks(vb, L, mode))


def test_heavy_tail_and_one_chunk():
    _, v = W.heavy_tail_kv(W.KVShape(2, 512, 128, 256), 61)
    vb = W.bf16_bits(v)
    _compare(_run(vb, 256, O.MODE_4OVER6), O.quantize_v_tblocks(vb, 256))
    s = W.ONE_CHUNK
    say("v tblocks one chunk", s)
    _, v = W.gaussian_kv(s, W.SEED_ONE_CHUNK, device="cuda")
    vb = W.bf16_bits(v)
    _compare(_run(vb, s.chunk_len, O.MODE_4OVER6), O.quantize_v_tblocks(vb, s.chunk_len))


def test_zero_chunk():
    vb = np.zeros((1, 64, 64), np.uint16)
    got = _run(vb, 32, O.MODE_4OVER6)
    assert np.all(got["codes"] == 0) and np.all(got["scales"] == 0) and np.all(got["tensor_scale"] == 0)
