"""The entry points under HIP graph capture: a layer's smooth-quantize and
dequantize calls and an attention call are captured once (outputs and
workspace allocated beforehand; the calls allocate nothing and clear their
counters with a fill kernel, never a memset) and replayed several times,
with unrelated eager calls on the same workspace and synchronizations in
between.  Every replay must give the eager run's bits, and the overlapped
kernel's error word must stay zero."""
import pytest
import torch

import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _empty_like_dict(d):
    return {k: torch.empty_like(v) for k, v in d.items()}


def test_quantize_dequantize_attention_replays():
    s = W.KVShape(4, 1024, 128, 512)
    say("graph capture", s)
    k, v = W.gaussian_kv(s, 91, device="cuda")
    k2, v2 = W.gaussian_kv(s, 92, device="cuda")  # other data for the eager calls between replays
    q = W.queries(s.H, 300, s.D, 93, device="cuda")
    ranges = [(0, 700), (900, 124)]
    ws = torch.zeros(P.nvfp4_kv_workspace_bytes(s.H, s.T, s.D, s.chunk_len), dtype=torch.uint8, device="cuda")
    off = P.nvfp4_kv_error_word_offset(s.H, s.T, s.D, s.chunk_len)
    assert off >= 0

    # eager reference
    ref = P.nvfp4_kv_smooth_quantize(k, v, s.chunk_len, workspace=ws)
    ref_dk = P.nvfp4_dequantize(ref["k_codes"], ref["k_scales"], ref["k_tensor_scale"], ref["k_mean"], s.chunk_len)
    # room for the staged attention: a staging kernel, then the attention kernels
    aws = torch.empty(P.nvfp4_kv_attention_staged_workspace_bytes(s.H, 300, s.D, s.H, s.T, s.chunk_len, ranges),
                      dtype=torch.uint8, device="cuda")
    ref_att, ref_lse = P.nvfp4_kv_attention(q, ref, s.chunk_len, ranges, lse=True, workspace=aws)
    torch.cuda.synchronize()

    out = _empty_like_dict(ref)
    dk = torch.empty_like(ref_dk)
    att = torch.empty_like(ref_att)
    lse = torch.empty_like(ref_lse)
    other = _empty_like_dict(ref)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            P.nvfp4_kv_smooth_quantize(k, v, s.chunk_len, out=out, workspace=ws, stream=stream)
            P.nvfp4_dequantize(out["k_codes"], out["k_scales"], out["k_tensor_scale"], out["k_mean"], s.chunk_len,
                               out=dk, stream=stream)
            P.nvfp4_kv_attention(q, out, s.chunk_len, ranges, out=att, lse=lse, workspace=aws, stream=stream)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in list(out.values()) + [dk, att, lse]:
            t.view(torch.uint8).fill_(0x5A)
        # eager work on the same workspace between replays
        P.nvfp4_kv_smooth_quantize(k2, v2, s.chunk_len, out=other, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ref:
            assert torch.equal(out[key].view(torch.uint8), ref[key].view(torch.uint8)), (rep, key)
        assert torch.equal(dk.view(torch.int16), ref_dk.view(torch.int16)), rep
        assert torch.equal(att.view(torch.int16), ref_att.view(torch.int16)), rep
        assert torch.equal(lse, ref_lse), rep
        assert int(ws[off:off + 4].view(torch.int32).item()) == 0, rep
