"""nvfp4_kv_smooth_quantize_noalloc (no workspace: the library's per-GPU
device array) through the C ABI against nvfp4_kv_smooth_quantize on the same
inputs, bit for bit: calls in a row on the one array, the first at the largest
shape it takes, then smaller ones (the array keeps the previous call's
contents, so everything a call needs cleared must be cleared by the call)."""
import pytest
import torch

import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import kv_outputs, say

pytestmark = pytest.mark.gpu


def _same_as_workspace_call(shape, seed, mode):
    say("noalloc", shape, "seed", seed, "mode", mode)
    H, T, D, L = shape.H, shape.T, shape.D, shape.chunk_len
    k, v = W.gaussian_kv(shape, seed, device="cuda")
    ref = P.nvfp4_kv_smooth_quantize(k, v, L, mode, choice_counts=True, out=kv_outputs(H, T, D, L))
    out = kv_outputs(H, T, D, L)  # every byte pre-filled with a sentinel
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    P.nvfp4_kv_smooth_quantize_noalloc(k, v, L, out, mode, error_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0, "a bounded wait timed out"
    for key in ref:
        assert torch.equal(ref[key], out[key]), key


def test_noalloc_matches_the_workspace_entry_point():
    # a full-cache layer: the largest workspace the array holds
    _same_as_workspace_call(W.CACHE_LAYER, W.cache_layer_seed(3), P.MODE_4OVER6)
    # then smaller inputs on the same array: ragged chunks, another mode, and
    # a head dimension that takes the two-pass kernels
    _same_as_workspace_call(W.KVShape(3, 77, 128, 7), 31, P.MODE_4OVER6)
    _same_as_workspace_call(W.KVShape(24, 7040, 128, 7040), W.SEED_ONE_CHUNK, P.MODE_FIXED6)
    _same_as_workspace_call(W.KVShape(2, 96, 48, 32), 32, P.MODE_4OVER6)
