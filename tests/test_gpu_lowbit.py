"""GPU parity of the 3-bit and 2-bit KV cache (nvfp4_kv_smooth_quantize_lowbit
/ nvfp4_dequantize_lowbit) against the CPU oracle, through the C ABI: codes,
scales, tensor scales, choice counts and dequantized values bit for bit (the
oracle fed the GPU's K mean, which must meet the 1e-6 rule), on the seeded
workloads, a full cache layer (sampled chunks), ragged shapes and degenerate
values, in both kernel forms (the overlapped kernel for D = 128, the
two-pass kernels for every D)."""
import numpy as np
import pytest
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W
from gpu_helpers import mean_rule, say, to_np

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A
PATHS = [{}, {"two_pass": True}]  # keyword options of the binding


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    P.lib()  # raises if the HIP library is missing


def _outputs(H, T, D, L, bits):
    out = P.lowbit_outputs(H, T, D, L, bits, "cuda", choice_counts=True)
    for t in out.values():
        t.view(torch.uint8).fill_(SENTINEL)
    return out


def _check(kb, vb, L, bits, mode, out, dk=None, dv=None):
    res = {key: t.cpu().numpy() for key, t in out.items()}
    ok, worst = mean_rule(kb, L, res["k_mean"])
    assert ok, f"K mean outside the 1e-6 rule ({worst:.3g})"
    ref = O.smooth_quantize_lowbit(kb, vb, L, bits, mode, k_mean=res["k_mean"])
    for key in ("k_codes", "v_codes", "k_scales", "v_scales"):
        a, b = res[key], ref[key]
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{key}: {len(bad)} mismatches, first at {bad[:5].tolist()}")
    for key in ("k_tensor_scale", "v_tensor_scale"):
        assert np.array_equal(res[key].view(np.uint32), ref[key].view(np.uint32)), key
    if "choice_counts" in res:
        n = kb.size // 16
        assert res["choice_counts"].tolist() == [[n - ref["k_useb"], ref["k_useb"]], [n - ref["v_useb"], ref["v_useb"]]]
    if dk is not None:
        rk = O.dequantize_lowbit(ref["k_codes"], ref["k_scales"], ref["k_tensor_scale"], res["k_mean"], L, bits)
        rv = O.dequantize_lowbit(ref["v_codes"], ref["v_scales"], ref["v_tensor_scale"], None, L, bits)
        assert np.array_equal(to_np(dk), rk), "dequantized K differs"
        assert np.array_equal(to_np(dv), rv), "dequantized V differs"
    return ref


def _run(kb, vb, L, bits, mode=O.MODE_4OVER6, path=None):
    H, T, D = kb.shape
    k, v = W.from_bits(kb, "cuda"), W.from_bits(vb, "cuda")
    ws = torch.full((P.nvfp4_kv_workspace_bytes(H, T, D, L),), 0xA5, dtype=torch.uint8, device="cuda")
    ws[:4] = 0  # the sticky error word is the caller's to clear
    out = P.nvfp4_kv_smooth_quantize_lowbit(k, v, L, bits, mode, out=_outputs(H, T, D, L, bits), workspace=ws,
                                            **(path or {}))
    dk = torch.full((H, T, D), -777.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full((H, T, D), -777.0, dtype=torch.bfloat16, device="cuda")
    P.nvfp4_dequantize_lowbit(out["k_codes"], out["k_scales"], out["k_tensor_scale"], out["k_mean"], L, bits, out=dk)
    P.nvfp4_dequantize_lowbit(out["v_codes"], out["v_scales"], out["v_tensor_scale"], None, L, bits, out=dv)
    torch.cuda.synchronize()
    assert P.kv_error_word(ws) == 0  # no bounded wait timed out
    return _check(kb, vb, L, bits, mode, out, dk, dv)


@pytest.mark.parametrize("path", PATHS, ids=["overlap", "two-pass"])
@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("mode", [O.MODE_4OVER6, O.MODE_FIXED6, O.MODE_FIXED4])
def test_tiny_workload(bits, mode, path):
    say("lowbit tiny", bits, mode, path)
    k, v = W.gaussian_kv(W.TINY, W.SEED_TINY)
    _run(W.bf16_bits(k), W.bf16_bits(v), W.TINY.chunk_len, bits, mode, path)


@pytest.mark.parametrize("path", PATHS, ids=["overlap", "two-pass"])
@pytest.mark.parametrize("bits", [3, 2])
def test_one_chunk_and_heavy_tail(bits, path):
    s = W.ONE_CHUNK
    for name, gen, seed in (("one chunk", W.gaussian_kv, W.SEED_ONE_CHUNK), ("heavy tail", W.heavy_tail_kv, W.SEED_HEAVY)):
        say("lowbit", name, s, "bits", bits, path)
        k, v = gen(s, seed)
        ref = _run(W.bf16_bits(k), W.bf16_bits(v), s.chunk_len, bits, O.MODE_4OVER6, path)
        n = k.numel() // 16
        assert 0 < ref["k_useb"] < n and 0 < ref["v_useb"] < n  # both candidates are chosen somewhere


@pytest.mark.parametrize("path", PATHS, ids=["overlap", "two-pass"])
@pytest.mark.parametrize("bits", [3, 2])
def test_full_cache_layer_sampled(bits, path):
    """One layer of the 8-chunk cache ([24, 56320, 128]): chunks 0, 3 and 7
    against the oracle bit for bit, the whole layer by its choice counts."""
    s = W.CACHE_LAYER
    L = s.chunk_len
    say("lowbit full layer", s, "bits", bits, path)
    k, v = W.gaussian_kv(s, W.cache_layer_seed(2), device="cuda")
    out = P.nvfp4_kv_smooth_quantize_lowbit(k, v, L, bits, out=_outputs(s.H, s.T, s.D, L, bits), **path)
    dk = P.nvfp4_dequantize_lowbit(out["k_codes"], out["k_scales"], out["k_tensor_scale"], out["k_mean"], L, bits)
    dv = P.nvfp4_dequantize_lowbit(out["v_codes"], out["v_scales"], out["v_tensor_scale"], None, L, bits)
    torch.cuda.synchronize()
    for c in (0, 3, 7):
        say("  chunk", c)
        sl = slice(c * L, (c + 1) * L)
        sub = {key: out[key][:, sl] for key in ("k_codes", "v_codes", "k_scales", "v_scales")}
        sub.update(k_mean=out["k_mean"][c:c + 1], k_tensor_scale=out["k_tensor_scale"][c:c + 1],
                   v_tensor_scale=out["v_tensor_scale"][c:c + 1])
        _check(W.bf16_bits(k[:, sl]), W.bf16_bits(v[:, sl]), L, bits, O.MODE_4OVER6, sub, dk[:, sl], dv[:, sl])
    cc = out["choice_counts"].cpu()
    assert cc.sum(1).tolist() == [k.numel() // 16] * 2


@pytest.mark.parametrize("path", PATHS, ids=["overlap", "two-pass"])
@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("H,T,D,L", [
    (3, 77, 128, 7),        # 11 chunks of 7 rows
    (2, 96, 48, 32),        # three blocks per row
    (1, 40, 4096, 8),       # widest rows
    (2, 7, 32, 1),          # one token per chunk: K' = 0
    (24, 1000, 128, 100),   # ragged tiles
])
def test_ragged_shapes(bits, H, T, D, L, path):
    say("lowbit shape", (H, T, D, L), "bits", bits, path)
    k, v = W.gaussian_kv(W.KVShape(H, T, D, L), 777 + H * T + D)
    _run(W.bf16_bits(k), W.bf16_bits(v), L, bits, O.MODE_4OVER6, path)


@pytest.mark.parametrize("path", PATHS, ids=["overlap", "two-pass"])
@pytest.mark.parametrize("bits", [3, 2])
def test_degenerate_values(bits, path):
    rng = np.random.default_rng(88)
    H, T, D, L = 2, 64, 128, 32
    cases = {
        "zeros": (np.zeros((H, T, D)), -np.zeros((H, T, D))),
        "constant": (np.broadcast_to(rng.standard_normal((H, 1, D)), (H, T, D)), np.full((H, T, D), -3.5)),
        "subnormal": (np.where(rng.random((H, T, D)) < 0.2, 3e-39, rng.standard_normal((H, T, D))),
                      rng.standard_normal((H, T, D)) * 1e-3),
        "huge": (rng.standard_normal((H, T, D)) * 1e30, rng.standard_normal((H, T, D)) * 3e37),
        "tiny": (rng.standard_normal((H, T, D)) * 1e-20, rng.standard_normal((H, T, D)) * 1e-30),
    }
    for name, (k, v) in cases.items():
        say("lowbit degenerate", name, "bits", bits, path)
        kb = W.bf16_bits(torch.as_tensor(np.asarray(k, np.float32)).to(torch.bfloat16))
        vb = W.bf16_bits(torch.as_tensor(np.asarray(v, np.float32)).to(torch.bfloat16))
        _run(kb, vb, L, bits, O.MODE_4OVER6, path)


@pytest.mark.parametrize("path", PATHS, ids=["overlap", "two-pass"])
@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("mode", [O.MODE_4OVER6, O.MODE_FIXED6, O.MODE_FIXED4])
def test_block_maxima_across_the_e4m3_range(bits, mode, path):
    # Block maxima log-uniform over 2^-22 .. 1 of the unit's largest value, so
    # that the candidate scales cover E4M3's normal and subnormal values and 0
    # (where a candidate's elements come closest to, or cross, the top
    # magnitude); a few elements of each block near its maximum.
    rng = np.random.default_rng(4242 + 10 * bits + mode)
    H, T, D, L = 2, 256, 128, 128
    nb = H * T * D // 16

    def tensor():
        scale = np.exp2(rng.uniform(-22.0, 0.0, nb))[:, None]
        x = rng.uniform(-1.0, 1.0, (nb, 16))
        x[:, 0] = np.sign(x[:, 0]) + (x[:, 0] == 0)  # the block maximum, +-1
        x[:, 1:4] = np.sign(x[:, 1:4]) * rng.uniform(0.6, 1.0, (nb, 3))
        x = rng.permuted(x, axis=1) * scale
        x = x.reshape(H, T, D)
        x[0, 0, 0] = 1.0  # the unit maximum of every chunk
        x[0, L, 0] = -1.0
        return W.bf16_bits(torch.as_tensor(x.astype(np.float32)).to(torch.bfloat16))

    say("lowbit block maxima over the E4M3 range, bits", bits, "mode", mode, path)
    _run(tensor(), tensor(), L, bits, mode, path)
