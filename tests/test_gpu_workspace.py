"""One KV workspace reused across calls, shapes and entry points.

Every call must give the bytes of the same call on a fresh workspace (which
the other GPU tests compare with the oracle), whatever ran on the workspace
before: calls of another shape (another layout of the counters and ready
words), the two-pass kernels, the V-blocked quantizer, or nothing but random
bytes.  The calls are stream-ordered, some with no host synchronization in
between."""
import pytest
import torch

import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import say

pytestmark = pytest.mark.gpu

SHAPES = {
    "A": W.KVShape(4, 2048, 128, 1024),   # 4 units, 4 statistics and 4 quantize tiles per head
    "B": W.KVShape(3, 768, 128, 256),     # another layout: 6 units of one tile each per head
    "C": W.KVShape(1, 256, 128, 256),     # one statistics and one quantize tile per unit
    "D": W.KVShape(24, 7040, 128, 7040),  # one Wan-like chunk
}


def _inputs():
    return {name: W.gaussian_kv(s, 300 + i, device="cuda") for i, (name, s) in enumerate(SHAPES.items())}


def _fresh(k, v, L, counts):
    return P.nvfp4_kv_smooth_quantize(k, v, L, choice_counts=counts)  # the binding's zeroed workspace


def _same(a, b, what):
    for key in a:
        assert torch.equal(a[key], b[key]), (what, key)


def test_one_workspace_across_shapes_paths_and_entry_points():
    inp = _inputs()
    need = max(max(P.nvfp4_kv_workspace_bytes(s.H, s.T, s.D, s.chunk_len),
                   int(P.lib().nvfp4_kv_quantize_v_tblocks_workspace_bytes(s.H, s.T, s.D, s.chunk_len)))
               for s in SHAPES.values())
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ref = {}
    for name, s in SHAPES.items():
        ref[name] = _fresh(*inp[name], s.chunk_len, counts=True)
    torch.cuda.synchronize()
    # (shape, step): "ov" the overlapped kernel, "tp" the two-pass kernels,
    # "vt" the V-blocked quantizer on the same buffer
    seq = [("A", "ov"), ("A", "ov"), ("A", "ov"), ("B", "ov"), ("A", "ov"), ("A", "tp"), ("A", "ov"), ("A", "ov"),
           ("A", "vt"), ("A", "ov"), ("C", "ov"), ("C", "ov"), ("D", "ov"), ("D", "ov"), ("B", "ov"), ("B", "ov"),
           ("A", "ov")]
    for i, (name, step) in enumerate(seq):
        s = SHAPES[name]
        k, v = inp[name]
        say("workspace sequence", i, name, step)
        if step == "vt":
            P.nvfp4_kv_quantize_v_tblocks(v, s.chunk_len, workspace=ws)
            continue
        out = P.nvfp4_kv_smooth_quantize(k, v, s.chunk_len, choice_counts=True, workspace=ws,
                                         two_pass=(step == "tp"))
        torch.cuda.synchronize()
        assert P.kv_error_word(ws) == 0, (i, name, step)
        if step == "tp":
            # the two-pass kernels add the K sums in another order: V must agree
            for key in ("v_codes", "v_scales", "v_tensor_scale"):
                assert torch.equal(out[key], ref[name][key]), (i, key)
        else:
            _same(out, ref[name], (i, name))


def test_garbage_workspace_and_stream_ordered_reuse():
    """A workspace full of random bytes (apart from the caller's sticky error
    word), then many calls back to back on a side stream with no host
    synchronization between them."""
    s = SHAPES["A"]
    k, v = W.gaussian_kv(s, 311, device="cuda")
    ref = _fresh(k, v, s.chunk_len, counts=False)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    ws = torch.randint(0, 256, (P.nvfp4_kv_workspace_bytes(s.H, s.T, s.D, s.chunk_len),), dtype=torch.uint8,
                       device="cuda", generator=g)
    ws[:4] = 0
    outs = [{key: torch.empty_like(t) for key, t in ref.items()} for _ in range(6)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say("garbage workspace, 6 calls on a side stream")
    with torch.cuda.stream(side):
        for o in outs:
            P.nvfp4_kv_smooth_quantize(k, v, s.chunk_len, out=o, workspace=ws, stream=side)
    side.synchronize()
    assert P.kv_error_word(ws) == 0
    for i, o in enumerate(outs):
        _same(o, ref, i)
