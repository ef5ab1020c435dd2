"""CPU oracle for the NVFP4 "Four-Over-Six" KV-cache smooth-quantize path,
its dequantize and attention over the cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It is
a thin numpy/ctypes wrapper over oracle.c (plain C, built with gcc), which
states what each function computes and the page passage it follows.  Inputs
are numpy arrays; bf16 tensors travel as uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

MODE_4OVER6, MODE_FIXED6, MODE_FIXED4 = 0, 1, 2

_lib = None


def lib():
    """Load liboracle.so, building it with gcc first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        i, l, f, u32 = ctypes.c_int, ctypes.c_long, ctypes.c_float, ctypes.c_uint32
        sig = {
            "ora_e2m1_encode": (ctypes.c_uint8, [f]),
            "ora_e2m1_decode": (f, [ctypes.c_uint8]),
            "ora_e4m3_encode": (ctypes.c_uint8, [f]),
            "ora_e4m3_decode": (f, [ctypes.c_uint8]),
            "ora_float_to_bf16": (ctypes.c_uint16, [f]),
            "ora_bf16_to_float": (f, [ctypes.c_uint16]),
            "ora_kv_mean": (i, [P, i, i, i, i, P, i]),
            "ora_rht16": (None, [P, l, u32, P]),
            "ora_quantize_chunks": (i, [P, i, i, i, i, i, P, i, u32, P, P, P, P, P, P, i]),
            "ora_quantize_2d": (i, [P, i, i, i, P, P, P, P, P, P, i]),
            "ora_dequantize": (i, [P, P, P, P, i, i, i, i, P, i]),
            "ora_dequantize_2d": (i, [P, P, P, i, i, P]),
            "ora_e2m1_encode_array": (None, [P, l, P, i]),
            "ora_e4m3_encode_array": (None, [P, l, P, i]),
            "ora_float_to_bf16_array": (None, [P, l, P, i]),
            "ora_e2m1_decode_array": (None, [P, l, P, i]),
            "ora_e4m3_decode_array": (None, [P, l, P, i]),
            "ora_candidate_codes": (None, [P, l, f, P]),
            "ora_lowbit_encode": (ctypes.c_uint8, [i, f]),
            "ora_lowbit_decode": (f, [i, ctypes.c_uint8]),
            "ora_lowbit_encode_array": (None, [i, P, l, P, i]),
            "ora_quantize_chunks_lowbit": (i, [P, i, i, i, i, i, i, P, P, P, P, P, P, P, i]),
            "ora_dequantize_lowbit": (i, [P, P, P, P, i, i, i, i, i, P, i]),
            "ora_gemm_w4a4": (i, [P, P, P, i, i, P, P, P, i, i, P, i]),
            "ora_kv_attention": (i, [P, i, i, i, P, P, P, P, P, P, P, i, i, i, P, i, ctypes.c_double, P, l, P, P,
                                     i]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def default_threads():
    """Worker threads for the oracle: OMP_NUM_THREADS when set (the GPU hosts
    set it to their CPU share), else the CPU count capped at 16."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(os.cpu_count() or 1, 16))


def _nt(n):
    return default_threads() if not n or n <= 0 else int(n)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ---- codecs --------------------------------------------------------------

def e2m1_encode(y, nthreads=0):
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().ora_e2m1_encode_array(_ptr(y), y.size, _ptr(out), _nt(nthreads))
    return out


def e2m1_decode(q, nthreads=0):
    q = _c(q, np.uint8)
    out = np.empty(q.shape, np.float32)
    lib().ora_e2m1_decode_array(_ptr(q), q.size, _ptr(out), _nt(nthreads))
    return out


def e4m3_encode(r, nthreads=0):
    r = _c(r, np.float32)
    out = np.empty(r.shape, np.uint8)
    lib().ora_e4m3_encode_array(_ptr(r), r.size, _ptr(out), _nt(nthreads))
    return out


def e4m3_decode(s, nthreads=0):
    s = _c(s, np.uint8)
    out = np.empty(s.shape, np.float32)
    lib().ora_e4m3_decode_array(_ptr(s), s.size, _ptr(out), _nt(nthreads))
    return out


def float_to_bf16(x, nthreads=0):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().ora_float_to_bf16_array(_ptr(x), x.size, _ptr(out), _nt(nthreads))
    return out


def bf16_to_float(h):
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def candidate_codes(t, c):
    """E4M3 code of t / c (IEEE fp32 division), as the quantizer forms a candidate."""
    t = _c(t, np.float32)
    out = np.empty(t.shape, np.uint8)
    lib().ora_candidate_codes(_ptr(t), t.size, float(c), _ptr(out))
    return out


def rht16(x, sign_mask):
    """16-point random-sign Hadamard transform of each row of x [n, 16] (fp32)."""
    x = _c(x, np.float32).reshape(-1, 16)
    out = np.empty_like(x)
    lib().ora_rht16(_ptr(x), x.shape[0], int(sign_mask) & 0xFFFF, _ptr(out))
    return out


# ---- the path ------------------------------------------------------------

def kv_mean(x, chunk_len, nthreads=0):
    """Per-chunk channel mean of x [H, T, D] (bf16 bits) -> float32 [T/L, H, D]."""
    x = _c(x, np.uint16)
    H, T, D = x.shape
    out = np.empty((T // chunk_len, H, D), np.float32)
    _check(lib().ora_kv_mean(_ptr(x), H, T, D, chunk_len, _ptr(out), _nt(nthreads)), "kv_mean")
    return out


def quantize_chunks(x, chunk_len, mode=MODE_4OVER6, mean=None, hadamard=False, sign_mask=0,
                    want_errors=False, nthreads=0):
    """Quantize x [H, T, D] (bf16 bits) chunk by chunk; see ora_quantize_chunks."""
    x = _c(x, np.uint16)
    H, T, D = x.shape
    nc = T // chunk_len
    codes = np.empty((H, T, D // 2), np.uint8)
    scales = np.empty((H, T, D // 16), np.uint8)
    ts = np.empty((nc,), np.float32)
    e6 = np.empty((H, T, D // 16), np.float32) if want_errors else None
    e4 = np.empty((H, T, D // 16), np.float32) if want_errors else None
    n4 = ctypes.c_longlong(0)
    m = None if mean is None else _c(mean, np.float32)
    rc = lib().ora_quantize_chunks(_ptr(x), H, T, D, chunk_len, mode, _ptr(m), int(bool(hadamard)),
                                   int(sign_mask) & 0xFFFF, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(e6),
                                   _ptr(e4), ctypes.byref(n4), _nt(nthreads))
    _check(rc, "quantize_chunks")
    out = {"codes": codes, "scales": scales, "tensor_scale": ts, "use4": int(n4.value)}
    if want_errors:
        out["err6"], out["err4"] = e6, e4
    return out


def smooth_quantize(k, v, chunk_len, mode=MODE_4OVER6, k_mean=None, want_errors=False, nthreads=0):
    """The KV step: per-chunk K mean (or the given one), smoothed K and raw V
    quantized per chunk.  Returns the same outputs as the GPU entry point."""
    if k_mean is None:
        k_mean = kv_mean(k, chunk_len, nthreads)
    qk = quantize_chunks(k, chunk_len, mode, mean=k_mean, want_errors=want_errors, nthreads=nthreads)
    qv = quantize_chunks(v, chunk_len, mode, mean=None, want_errors=want_errors, nthreads=nthreads)
    out = {"k_codes": qk["codes"], "v_codes": qv["codes"], "k_scales": qk["scales"], "v_scales": qv["scales"],
           "k_tensor_scale": qk["tensor_scale"], "v_tensor_scale": qv["tensor_scale"],
           "k_mean": np.asarray(k_mean, np.float32), "k_use4": qk["use4"], "v_use4": qv["use4"]}
    if want_errors:
        out.update(k_err6=qk["err6"], k_err4=qk["err4"], v_err6=qv["err6"], v_err4=qv["err4"])
    return out


def dequantize(codes, scales, tensor_scale, mean, chunk_len, nthreads=0):
    """codes [H, T, D/2], scales [H, T, D/16] -> bf16 bits [H, T, D]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    ts = _c(tensor_scale, np.float32)
    m = None if mean is None else _c(mean, np.float32)
    H, T, D2 = codes.shape
    D = 2 * D2
    out = np.empty((H, T, D), np.uint16)
    _check(lib().ora_dequantize(_ptr(codes), _ptr(scales), _ptr(ts), _ptr(m), H, T, D, chunk_len, _ptr(out),
                                _nt(nthreads)), "dequantize")
    return out


# ---- 3-bit and 2-bit KV --------------------------------------------------

def lowbit_encode(bits, y, nthreads=0):
    """Element codes of the 3-bit (E1M1) or 2-bit (E1M0) grid for fp32 y."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().ora_lowbit_encode_array(int(bits), _ptr(y), y.size, _ptr(out), _nt(nthreads))
    return out


def lowbit_decode(bits, q):
    return np.array([lib().ora_lowbit_decode(int(bits), int(c)) for c in np.asarray(q).ravel()],
                    np.float32).reshape(np.shape(q))


def quantize_chunks_lowbit(x, chunk_len, bits, mode=MODE_4OVER6, mean=None, want_errors=False, nthreads=0):
    """3-bit / 2-bit quantization of x [H, T, D] (bf16 bits) chunk by chunk;
    see ora_quantize_chunks_lowbit.  codes [H, T, D * bits / 8]."""
    x = _c(x, np.uint16)
    H, T, D = x.shape
    nc = T // chunk_len
    codes = np.empty((H, T, D * bits // 8), np.uint8)
    scales = np.empty((H, T, D // 16), np.uint8)
    ts = np.empty((nc,), np.float32)
    ea = np.empty((H, T, D // 16), np.float32) if want_errors else None
    eb = np.empty((H, T, D // 16), np.float32) if want_errors else None
    nb = ctypes.c_longlong(0)
    m = None if mean is None else _c(mean, np.float32)
    rc = lib().ora_quantize_chunks_lowbit(_ptr(x), H, T, D, chunk_len, int(bits), mode, _ptr(m), _ptr(codes),
                                          _ptr(scales), _ptr(ts), _ptr(ea), _ptr(eb), ctypes.byref(nb),
                                          _nt(nthreads))
    _check(rc, "quantize_chunks_lowbit")
    out = {"codes": codes, "scales": scales, "tensor_scale": ts, "useb": int(nb.value)}
    if want_errors:
        out["erra"], out["errb"] = ea, eb
    return out


def smooth_quantize_lowbit(k, v, chunk_len, bits, mode=MODE_4OVER6, k_mean=None, want_errors=False, nthreads=0):
    """The KV step at 3 or 2 bits: per-chunk K mean (or the given one),
    smoothed K and raw V quantized per chunk."""
    if k_mean is None:
        k_mean = kv_mean(k, chunk_len, nthreads)
    qk = quantize_chunks_lowbit(k, chunk_len, bits, mode, mean=k_mean, want_errors=want_errors, nthreads=nthreads)
    qv = quantize_chunks_lowbit(v, chunk_len, bits, mode, mean=None, want_errors=want_errors, nthreads=nthreads)
    out = {"k_codes": qk["codes"], "v_codes": qv["codes"], "k_scales": qk["scales"], "v_scales": qv["scales"],
           "k_tensor_scale": qk["tensor_scale"], "v_tensor_scale": qv["tensor_scale"],
           "k_mean": np.asarray(k_mean, np.float32), "k_useb": qk["useb"], "v_useb": qv["useb"]}
    if want_errors:
        out.update(k_erra=qk["erra"], k_errb=qk["errb"], v_erra=qv["erra"], v_errb=qv["errb"])
    return out


def dequantize_lowbit(codes, scales, tensor_scale, mean, chunk_len, bits, nthreads=0):
    """codes [H, T, D * bits / 8], scales [H, T, D/16] -> bf16 bits [H, T, D]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    ts = _c(tensor_scale, np.float32)
    m = None if mean is None else _c(mean, np.float32)
    H, T, _ = codes.shape
    D = scales.shape[2] * 16
    out = np.empty((H, T, D), np.uint16)
    _check(lib().ora_dequantize_lowbit(_ptr(codes), _ptr(scales), _ptr(ts), _ptr(m), H, T, D, chunk_len, int(bits),
                                       _ptr(out), _nt(nthreads)), "dequantize_lowbit")
    return out


def quantize_1d(x, mode=MODE_4OVER6, hadamard=False, sign_mask=0, want_errors=False, nthreads=0):
    """Activation path: x [rows, cols] (bf16 bits), 1D blocks along cols, one
    tensor scale, optional RHT first.  codes [rows, cols/2], scales [rows, cols/16]."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    r = quantize_chunks(x.reshape(1, rows, cols), rows, mode, None, hadamard, sign_mask, want_errors, nthreads)
    out = {"codes": r["codes"][0], "scales": r["scales"][0], "tensor_scale": r["tensor_scale"], "use4": r["use4"]}
    if want_errors:
        out["err6"], out["err4"] = r["err6"][0], r["err4"][0]
    return out


def quantize_2d(w, mode=MODE_4OVER6, want_errors=False, nthreads=0):
    """Weight path: w [rows, cols] (bf16 bits), 16x16 tiles.  codes [rows, cols/2],
    scales [rows/16, cols/16], tensor_scale [1]."""
    w = _c(w, np.uint16)
    rows, cols = w.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows // 16, cols // 16), np.uint8)
    ts = np.empty((1,), np.float32)
    e6 = np.empty((rows // 16, cols // 16), np.float32) if want_errors else None
    e4 = np.empty((rows // 16, cols // 16), np.float32) if want_errors else None
    n4 = ctypes.c_longlong(0)
    _check(lib().ora_quantize_2d(_ptr(w), rows, cols, mode, _ptr(codes), _ptr(scales), _ptr(ts), _ptr(e6), _ptr(e4),
                                 ctypes.byref(n4), _nt(nthreads)), "quantize_2d")
    out = {"codes": codes, "scales": scales, "tensor_scale": ts, "use4": int(n4.value)}
    if want_errors:
        out["err6"], out["err4"] = e6, e4
    return out


def dequantize_2d(codes, scales, tensor_scale):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    ts = _c(tensor_scale, np.float32)
    rows, c2 = codes.shape
    out = np.empty((rows, 2 * c2), np.uint16)
    _check(lib().ora_dequantize_2d(_ptr(codes), _ptr(scales), _ptr(ts), rows, 2 * c2, _ptr(out)), "dequantize_2d")
    return out


def kv_attention(q, cache, chunk_len, ranges, scale=None, n_kv_heads=None, rows=None, nthreads=0):
    """Softmax attention of q (bf16 bits [H, Tq, D]) over the keys listed in
    ranges ([(start, len), ...]) of an NVFP4 cache (the dict smooth_quantize
    returns; "k_mean" may be None), in double over the exactly decoded K and
    V.  scale defaults to 1/sqrt(D).  rows: None for all (h, i), else flat
    indices h * Tq + i.  Returns (out [rows, D] float64, lse [rows] float64);
    with rows None, out is [H, Tq, D] and lse [H, Tq]."""
    q = _c(q, np.uint16)
    H, Tq, D = q.shape
    kc = _c(cache["k_codes"], np.uint8)
    Hkv, T, _ = kc.shape
    if n_kv_heads is not None and n_kv_heads != Hkv:
        raise ValueError("cache head count differs from n_kv_heads")
    ks = _c(cache["k_scales"], np.uint8)
    vc = _c(cache["v_codes"], np.uint8)
    vs = _c(cache["v_scales"], np.uint8)
    kg = _c(cache["k_tensor_scale"], np.float32)
    vg = _c(cache["v_tensor_scale"], np.float32)
    km = cache.get("k_mean")
    km = None if km is None else _c(km, np.float32)
    rg = np.asarray(ranges, np.int32).reshape(-1, 2)
    rg = np.ascontiguousarray(rg)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rw = None if rows is None else _c(rows, np.int64)
    n = H * Tq if rw is None else rw.size
    out = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    _check(lib().ora_kv_attention(_ptr(q), H, Tq, D, _ptr(kc), _ptr(ks), _ptr(kg), _ptr(km), _ptr(vc), _ptr(vs),
                                  _ptr(vg), Hkv, T, chunk_len, _ptr(rg) if rg.size else None, rg.shape[0],
                                  float(scale), _ptr(rw), n, _ptr(out), _ptr(lse), _nt(nthreads)), "kv_attention")
    if rw is None:
        return out.reshape(H, Tq, D), lse.reshape(H, Tq)
    return out, lse


def kv_cache_key_tokens(chunks, shot_chunk, chunk_len, frame_tokens, sink_frames, shot_frames, window):
    """The tokens attention reads from a streaming cache after `chunks`
    committed chunks, in video token order (token i of chunk c is c * chunk_len
    + i): the union of the global sink (the first sink_frames frames of the
    video), the shot sink (the first shot_frames frames of the current shot,
    which starts at chunk shot_chunk) and the window (the last `window`
    chunks) -- inference pipeline, step 9 of the LongLive-2.0 summary page.
    Each token once, sorted."""
    keys = set()
    if chunks > 0:
        keys.update(range(0, sink_frames * frame_tokens))
        if shot_chunk < chunks:
            s0 = shot_chunk * chunk_len
            keys.update(range(s0, s0 + shot_frames * frame_tokens))
        w0 = max(0, chunks - window)
        keys.update(range(w0 * chunk_len, chunks * chunk_len))
    return sorted(keys)


def gemm_w4a4(a, w, w2d, nthreads=0):
    """out [M, N] float64 = sum over k of the exactly decoded operands:
    a = (codes [M, K/2], scales [M, K/16], tensor_scale [1]) -- the activation
    quantizer's output; w = (codes [N, K/2], scales [N, K/16] or, with w2d,
    [N/16, K/16], tensor_scale [1])."""
    ac, as_, ag = _c(a[0], np.uint8), _c(a[1], np.uint8), _c(a[2], np.float32)
    wc, ws, wg = _c(w[0], np.uint8), _c(w[1], np.uint8), _c(w[2], np.float32)
    M, K2 = ac.shape
    N = wc.shape[0]
    out = np.empty((M, N), np.float64)
    _check(lib().ora_gemm_w4a4(_ptr(ac), _ptr(as_), _ptr(ag), M, 2 * K2, _ptr(wc), _ptr(ws), _ptr(wg), N,
                               1 if w2d else 0, _ptr(out), _nt(nthreads)), "gemm_w4a4")
    return out


def quantize_v_tblocks(v, chunk_len, mode=MODE_4OVER6, nthreads=0):
    """V (bf16 bits [H, T, D]) with 16-token blocks per (head, channel): each
    chunk's [H, D, chunk_len] slab (the chunk transposed) is one 1D-blocked
    tensor with its own tensor scale -- the same encoding as the KV V path
    (inference pipeline, step 7; 4/6 block scale), blocked along tokens.
    Returns codes [H, D, T/2], scales [H, D, T/16], tensor_scale [T/L]."""
    v = _c(v, np.uint16)
    H, T, D = v.shape
    nc = T // chunk_len
    codes = np.empty((H, D, T // 2), np.uint8)
    scales = np.empty((H, D, T // 16), np.uint8)
    ts = np.empty((nc,), np.float32)
    for c in range(nc):
        x = np.ascontiguousarray(v[:, c * chunk_len:(c + 1) * chunk_len, :].transpose(0, 2, 1)).reshape(H * D,
                                                                                                        chunk_len)
        q = quantize_1d(x, mode, nthreads=nthreads)
        codes[:, :, c * chunk_len // 2:(c + 1) * chunk_len // 2] = q["codes"].reshape(H, D, chunk_len // 2)
        scales[:, :, c * chunk_len // 16:(c + 1) * chunk_len // 16] = q["scales"].reshape(H, D, chunk_len // 16)
        ts[c] = q["tensor_scale"][0]
    return {"codes": codes, "scales": scales, "tensor_scale": ts}
