"""Pins of the oracle's V quantizer with 16-token blocks per (head, channel)
(the V-blocking variant of the LongLive-2.0 summary page's NVFP4 V cache,
inference pipeline, step 7; the 4/6 block scale of the full-stack NVFP4
section).

- A hand-worked chunk: constant and zero channels, whose codes, scales and
  tensor scale follow from the format definitions alone.
- The same encoding through the KV path's V quantizer: a chunk transposed to
  [H, D, L] and quantized as one chunk with blocks along its last axis must
  give the same bytes, the tensor scale spanning all heads of the chunk.
  This catches a wrong transpose, nibble order along the tokens, or a tensor
  scale per head or per tensor instead of per chunk.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


def _bits(a):
    """float32 numpy array of bf16-exact values -> bf16 bit patterns."""
    return W.bf16_bits(torch.from_numpy(a).to(torch.bfloat16))


def test_worked_chunk():
    # H = 1, T = L = 16, D = 3 (channels): channel 0 is 2.0 at every token,
    # channel 1 is 0, channel 2 is -2.0.
    #   A = 2, g_enc = fl(1792 / 2) = 896, so every |z| = 1792 and t = 1792.
    #   +-6 candidate: t / 6 = 298.67 -> E4M3 288 (nearest of 288, 320);
    #   y = 1792 / 288 = 6.22 -> E2M1 6, error (1792 - 1728)^2 per element > 0.
    #   +-4 candidate: t / 4 = 448 -> E4M3 448 (byte 0x7E); y = 4 exactly,
    #   error 0, so +-4 is kept: code 6 (4.0) in every nibble, 0xE (-4.0) for
    #   channel 2.  Channel 1: t = 0 -> scale byte 0, codes +0.
    #   g_dec = fl(2 / 1792).
    v = np.zeros((1, 16, 3), np.float32)
    v[0, :, 0] = 2.0
    v[0, :, 2] = -2.0
    r = O.quantize_v_tblocks(_bits(v), 16)
    assert r["codes"].shape == (1, 3, 8) and r["scales"].shape == (1, 3, 1)
    np.testing.assert_array_equal(r["codes"][0, 0], np.full(8, 0x66, np.uint8))
    np.testing.assert_array_equal(r["codes"][0, 1], np.zeros(8, np.uint8))
    np.testing.assert_array_equal(r["codes"][0, 2], np.full(8, 0xEE, np.uint8))
    np.testing.assert_array_equal(r["scales"][0, :, 0], [0x7E, 0x00, 0x7E])
    assert r["tensor_scale"].view(np.uint32)[0] == np.float32(np.float32(2.0) / np.float32(1792.0)).view(np.uint32)


def test_token_order_of_nibbles():
    # One channel whose tokens ramp 0, 0.25, .., 3.75: token 2j sits in the
    # low nibble of byte j and token 2j + 1 in the high nibble, so the
    # magnitudes read in that order rise with the tokens.
    v = np.zeros((1, 16, 1), np.float32)
    v[0, :, 0] = np.arange(16) * 0.25
    r = O.quantize_v_tblocks(_bits(v), 16)
    codes = r["codes"][0, 0]
    lo, hi = codes & 15, codes >> 4
    mags = np.stack([lo, hi], 1).reshape(16) & 7
    # first token 0; last token the block maximum: code 7 (6.0) if +-6 is
    # kept, code 6 (4.0) if +-4 is
    assert mags[0] == 0 and mags[15] in (6, 7)
    # monotone along the tokens: swapped nibbles would put a larger code
    # before a smaller one wherever the ramp's codes step up
    assert np.all(np.diff(mags.astype(int)) >= 0)
    assert len(np.unique(mags)) >= 6


@pytest.mark.parametrize("mode", [O.MODE_4OVER6, O.MODE_FIXED6, O.MODE_FIXED4])
def test_equals_kv_v_path_on_transposed_chunks(mode):
    H, L, D, nc = 3, 48, 32, 3
    _, v = W.gaussian_kv(W.KVShape(H, nc * L, D, L), 77 + mode)
    vb = W.bf16_bits(v)
    r = O.quantize_v_tblocks(vb, L, mode)
    for c in range(nc):
        slab = np.ascontiguousarray(vb[:, c * L:(c + 1) * L, :].transpose(0, 2, 1))  # [H, D, L]
        q = O.smooth_quantize(np.zeros_like(slab), slab, D, mode)  # one chunk of D rows, blocks along L
        np.testing.assert_array_equal(r["codes"][:, :, c * L // 2:(c + 1) * L // 2], q["v_codes"])
        np.testing.assert_array_equal(r["scales"][:, :, c * L // 16:(c + 1) * L // 16], q["v_scales"])
        assert r["tensor_scale"][c].view(np.uint32) == q["v_tensor_scale"][0].view(np.uint32)
