"""Shared GPU-test plumbing: run the HIP path through the binding, pull the
results to numpy, and compare them with the CPU oracle on the same inputs."""
import sys

import numpy as np
import torch

import oracle as O
import precision_kv_cache_amd as P
import workloads as W

MEAN_RTOL = 1e-6


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_np(t):
    if t.dtype == torch.bfloat16:
        return W.bf16_bits(t)
    return t.detach().cpu().numpy()


SENTINEL = 0x5A  # every output byte is pre-filled with it, so a missing write cannot pass


def kv_outputs(H, T, D, L, counts=True):
    """Output tensors for nvfp4_kv_smooth_quantize, filled with a sentinel."""
    nc = T // L

    def fill(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device="cuda")
        t.view(torch.uint8).fill_(SENTINEL)
        return t

    out = {"k_codes": fill((H, T, D // 2), torch.uint8), "v_codes": fill((H, T, D // 2), torch.uint8),
           "k_scales": fill((H, T, D // 16), torch.uint8), "v_scales": fill((H, T, D // 16), torch.uint8),
           "k_tensor_scale": fill((nc,), torch.float32), "v_tensor_scale": fill((nc,), torch.float32),
           "k_mean": fill((nc, H, D), torch.float32)}
    if counts:
        out["choice_counts"] = fill((2, 2), torch.int64)
    return out


def gpu_kv(kb, vb, L, mode=O.MODE_4OVER6, counts=True, path=None):
    """K, V given as numpy bf16 bits [H, T, D] -> GPU outputs as numpy.  The
    workspace starts out filled with garbage (its contents on entry are
    documented as ignored); after the call the overlapped kernel's error word
    must read zero (no wait timed out)."""
    k = W.from_bits(kb, "cuda")
    v = W.from_bits(vb, "cuda")
    H, T, D = kb.shape
    ws = torch.full((max(1, P.nvfp4_kv_workspace_bytes(H, T, D, L)),), 0xA5, dtype=torch.uint8, device="cuda")
    ws[:4] = 0  # the sticky error word is the caller's to clear
    out = P.nvfp4_kv_smooth_quantize(k, v, L, mode, choice_counts=counts, **(path or {}),
                                     out=kv_outputs(H, T, D, L, counts), workspace=ws)
    torch.cuda.synchronize()
    assert P.nvfp4_kv_error_word_offset(H, T, D, L) == 0
    assert P.kv_error_word(ws) == 0, "a wait of the overlapped kernel timed out"
    return {key: t.cpu().numpy() for key, t in out.items()}, out


def mean_rule(kb, L, gpu_mean):
    """Acceptance of the K mean: |m_gpu - m_ref| <= 1e-6 * max(|m_ref|,
    mean_t |K|) per channel, m_ref the fp64 mean.  Returns the worst ratio."""
    H, T, D = kb.shape
    nc = T // L
    x = O.bf16_to_float(kb).astype(np.float64).reshape(H, nc, L, D)
    ref = x.mean(2).transpose(1, 0, 2)
    scale = np.maximum(np.abs(ref), np.abs(x).mean(2).transpose(1, 0, 2))
    err = np.abs(gpu_mean.astype(np.float64) - ref)
    ok = err <= MEAN_RTOL * scale
    ratio = np.where(scale > 0, err / np.where(scale > 0, scale, 1), np.where(err > 0, np.inf, 0))
    return bool(ok.all()), float(ratio.max())


def check_kv(kb, vb, L, mode, res, dev_out=None, nthreads=0, check_dequant=True):
    """Full parity of one GPU KV call against the oracle fed with the GPU
    mean: codes, scales, tensor scales and choice counts bit-exact; the
    dequantized K (mean restored) and V bit-exact."""
    ok, worst = mean_rule(kb, L, res["k_mean"])
    assert ok, f"K mean outside 1e-6 rule (worst ratio {worst:.3g})"
    ref = O.smooth_quantize(kb, vb, L, mode, k_mean=res["k_mean"], nthreads=nthreads)
    for key in ("k_codes", "v_codes", "k_scales", "v_scales"):
        a, b = res[key], ref[key]
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{key}: {len(bad)} mismatches, first at {bad[:5].tolist()}")
    for key in ("k_tensor_scale", "v_tensor_scale"):
        assert np.array_equal(res[key].view(np.uint32), ref[key].view(np.uint32)), key
    if "choice_counts" in res:
        n = res["k_codes"].size // 8
        assert res["choice_counts"].tolist() == [[n - ref["k_use4"], ref["k_use4"]], [n - ref["v_use4"], ref["v_use4"]]]
    if check_dequant and dev_out is not None:
        H, T, D2 = res["k_codes"].shape
        dk = torch.full((H, T, 2 * D2), -777.0, dtype=torch.bfloat16, device="cuda")
        dv = torch.full((H, T, 2 * D2), -777.0, dtype=torch.bfloat16, device="cuda")
        P.nvfp4_dequantize(dev_out["k_codes"], dev_out["k_scales"], dev_out["k_tensor_scale"], dev_out["k_mean"], L,
                           out=dk)
        P.nvfp4_dequantize(dev_out["v_codes"], dev_out["v_scales"], dev_out["v_tensor_scale"], None, L, out=dv)
        torch.cuda.synchronize()
        rk = O.dequantize(ref["k_codes"], ref["k_scales"], ref["k_tensor_scale"], res["k_mean"], L, nthreads)
        rv = O.dequantize(ref["v_codes"], ref["v_scales"], ref["v_tensor_scale"], None, L, nthreads)
        assert np.array_equal(to_np(dk), rk), "dequantized K differs"
        assert np.array_equal(to_np(dv), rv), "dequantized V differs"
    return ref


# ---- attention over the NVFP4 cache ----------------------------------------

LOG2E = 1.4426950408889634


def decode_exact(codes, scales, g, L):
    """Exact decode (no mean) with numpy: [Hkv, T, D] float64."""
    Hkv, T, D2 = codes.shape
    lo, hi = codes & 15, codes >> 4
    q = np.stack([lo, hi], axis=-1).reshape(Hkv, T, 2 * D2)
    v = O.e2m1_decode(q).astype(np.float64)
    S = np.repeat(O.e4m3_decode(scales).astype(np.float64), 16, axis=-1)
    return v * S * np.asarray(g, np.float64)[np.arange(T) // L][None, :, None]



def key_list(ranges):
    return np.concatenate([np.arange(a, a + n) for a, n in ranges if n > 0]) if ranges else np.zeros(0, int)



def attention_check(q_bits, cache, L, ranges, got, got_lse, rows, scale=None, rms_rel=2.0 ** -8):
    """got [n, D], got_lse [n] for the flat rows `rows`; compare with the oracle."""
    H, Tq, D = q_bits.shape
    if scale is None:
        scale = D ** -0.5
    ref, ref_lse = O.kv_attention(q_bits, cache, L, ranges, scale=scale, rows=rows)
    Hkv = cache["k_codes"].shape[0]
    keys = key_list(ranges)
    Kp = np.abs(decode_exact(cache["k_codes"], cache["k_scales"], cache["k_tensor_scale"], L)[:, keys])
    if cache.get("k_mean") is not None:
        Kp = Kp + np.abs(np.asarray(cache["k_mean"], np.float64)[keys // L].transpose(1, 0, 2))
    Vx = decode_exact(cache["v_codes"], cache["v_scales"], cache["v_tensor_scale"], L)[:, keys]
    qf = np.abs(W.from_bits(q_bits).float().numpy().astype(np.float64)).reshape(H * Tq, D)[rows]
    heads = rows // Tq
    kvh = heads // (H // Hkv)
    tol = np.empty_like(ref)
    eps = np.empty(len(rows))
    for i, r in enumerate(rows):
        delta = 2.0 ** -16 * scale * LOG2E * (Kp[kvh[i]] @ qf[i]).max()
        eps[i] = np.log(2.0) * delta
        vmax = np.abs(Vx[kvh[i]]).max(axis=0)
        pre = vmax * (np.expm1(2 * eps[i]) + 2.0 ** -7 + 2.0 ** -16)   # error before the output rounding
        tol[i] = pre + 2.0 ** -8 * (np.abs(ref[i]) + pre)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite output"
    bad = err > tol
    assert not bad.any(), (f"{bad.sum()} elements out of bound; worst excess "
                           f"{(err - tol).max():.3g} at {np.unravel_index(np.argmax(err - tol), err.shape)}")
    lse_err = np.abs(got_lse - ref_lse)
    assert np.all(lse_err <= eps + 2.0 ** -20 * np.abs(ref_lse) + 1e-5), lse_err.max()
    rms = np.sqrt(np.mean(err ** 2))
    rms_ref = np.sqrt(np.mean(ref ** 2))
    ratio = np.divide(err, tol, out=np.zeros_like(err), where=tol > 0)
    say(f"rms err {rms:.3g} = {rms / rms_ref:.3g} x rms(out); max err / bound {ratio.max():.3g}; "
        f"max lse err {lse_err.max():.3g}")
    assert rms <= rms_rel * rms_ref, (rms, rms_ref)


