"""GPU parity of the streaming NVFP4 KV cache: chunks are appended one at a
time (two layers, a prompt switch mid-stream, more chunks than slots, so
slots are reused), and after every commit
  - the chunk's slot holds exactly what the oracle's quantizer makes of that
    chunk (codes, scales, tensor scales and K means bit-exact: the fp64 sums
    of these bf16 inputs are exact in any order, so both means are the same
    float);
  - attention through the cache (slot ranges, chunk-major layout) matches the
    oracle's fp64 attention over the logical cache -- every chunk so far in
    video order, head-major -- restricted to the oracle's key-set model of
    the sinks and window (inference pipeline, step 9), to the attention
    tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import attention_check, mean_rule, say

pytestmark = pytest.mark.gpu


def _runs(tokens):
    """Sorted token list -> (start, len) runs."""
    out = []
    for t in tokens:
        if out and out[-1][0] + out[-1][1] == t:
            out[-1][1] += 1
        else:
            out.append([t, 1])
    return [(a, n) for a, n in out]


def _logical(chunks):
    """Per-chunk oracle caches [H, L, ...] -> one head-major cache."""
    cat = lambda key, axis: np.concatenate([c[key] for c in chunks], axis=axis)  # noqa: E731
    return {"k_codes": cat("k_codes", 1), "v_codes": cat("v_codes", 1), "k_scales": cat("k_scales", 1),
            "v_scales": cat("v_scales", 1), "k_tensor_scale": cat("k_tensor_scale", 0),
            "v_tensor_scale": cat("v_tensor_scale", 0), "k_mean": cat("k_mean", 0)}


@pytest.mark.parametrize("geom", [
    dict(H=2, L=128, F=32, Sg=1, Ss=2, W=2, cap=5, n=8, shots=(3,), Tq=70),
    dict(H=3, L=192, F=64, Sg=2, Ss=1, W=1, cap=4, n=6, shots=(2, 4), Tq=300),
])
def test_streamed_chunks(geom):
    H, L, F, D = geom["H"], geom["L"], geom["F"], 128
    layers = 2
    say("stream", geom)
    cache = P.KVCache(layers, H, D, L, geom["cap"], F, geom["Sg"], geom["Ss"], geom["W"])
    cache.storage.fill_(0x77)  # garbage: every slot byte that is read must have been written
    chunks = {layer: [] for layer in range(layers)}
    q_bits = W.bf16_bits(W.queries(H, geom["Tq"], D, 41))
    q = W.from_bits(q_bits, "cuda")
    for ch in range(geom["n"]):
        slot = cache.begin_chunk(new_shot=ch in geom["shots"])
        inputs = []
        for layer in range(layers):
            k, v = W.gaussian_kv(W.KVShape(H, L, D, L), 5000 + 10 * ch + layer)
            kb, vb = W.bf16_bits(k), W.bf16_bits(v)
            inputs.append((kb, vb))
            cache.append(layer, W.from_bits(kb, "cuda"), W.from_bits(vb, "cuda"))
        torch.cuda.synchronize()
        for layer, (kb, vb) in enumerate(inputs):
            got = {key: t[slot].cpu().numpy() for key, t in cache.slot_arrays(layer).items()
                   if key not in ("k_tensor_scale", "v_tensor_scale")}
            ts = cache.slot_arrays(layer)
            got["k_tensor_scale"] = ts["k_tensor_scale"][slot:slot + 1].cpu().numpy()
            got["v_tensor_scale"] = ts["v_tensor_scale"][slot:slot + 1].cpu().numpy()
            got["k_mean"] = got["k_mean"][None]
            ok, worst = mean_rule(kb, L, got["k_mean"])
            assert ok, (ch, layer, worst)
            ref = O.smooth_quantize(kb, vb, L, k_mean=got["k_mean"])  # parity given the GPU mean
            for key in ("k_codes", "v_codes", "k_scales", "v_scales"):
                assert np.array_equal(got[key], ref[key]), (ch, layer, key)
            for key in ("k_tensor_scale", "v_tensor_scale", "k_mean"):
                assert np.array_equal(got[key].view(np.uint32), ref[key].view(np.uint32)), (ch, layer, key)
            chunks[layer].append(ref)
        cache.end_chunk()
        tokens = O.kv_cache_key_tokens(cache.state.chunks, cache.state.shot_chunk, L, F, geom["Sg"], geom["Ss"],
                                       geom["W"])
        ranges = _runs(tokens)
        for layer in range(layers):
            out, lse = cache.attention(layer, q, lse=True)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64).reshape(-1, D)
            got_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
            attention_check(q_bits, _logical(chunks[layer]), L, ranges, got, got_lse, np.arange(H * geom["Tq"]))


def test_chunked_attention_matches_head_major():
    """nvfp4_kv_attention_chunked over a chunk-major copy of a cache gives the
    same bits as nvfp4_kv_attention over the head-major original: staged
    (the default workspace), split only, and unsplit."""
    H, T, L, D, Tq = 2, 512, 128, 128, 100
    k, v = W.gaussian_kv(W.KVShape(H, T, D, L), 42)
    ref = O.smooth_quantize(W.bf16_bits(k), W.bf16_bits(v), L)
    nc = T // L
    hm = {key: torch.from_numpy(np.ascontiguousarray(val)).cuda() for key, val in ref.items()
          if key in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tensor_scale", "v_tensor_scale", "k_mean")}
    cm = dict(hm)
    for key in ("k_codes", "v_codes", "k_scales", "v_scales"):
        a = ref[key]
        cm[key] = torch.from_numpy(np.ascontiguousarray(a.reshape(H, nc, L, -1).transpose(1, 0, 2, 3))).cuda()
    q = W.queries(H, Tq, D, 43, device="cuda")
    ranges = [(300, 200), (0, 37), (129, 1)]
    split_ws = torch.empty(P.nvfp4_kv_attention_workspace_bytes(H, Tq, D), dtype=torch.uint8, device="cuda")
    for ws in (None, split_ws, False):  # staged, key splits only, unsplit
        a, la = P.nvfp4_kv_attention(q, hm, L, ranges, lse=True, workspace=ws)
        b, lb = P.nvfp4_kv_attention_chunked(q, cm, L, ranges, lse=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb), type(ws)
