"""NVFP4 "Four-Over-Six" KV-cache quantizer for MI355X (gfx950).

Thin ctypes binding over libnvfp4kv.so (HIP kernels + C ABI, declared in
include/nvfp4kv.h).  Same names as the C entry points; this module only
marshals arguments: it allocates output tensors with torch (device memory),
passes their pointers and torch's current HIP stream, and turns a non-zero
status into an exception.  Every step of the computation runs in the HIP
kernels; there is no fallback.  A missing or unloadable library raises.
"""
import ctypes
import os

import torch

__all__ = [
    "MODE_4OVER6", "MODE_FIXED6", "MODE_FIXED4", "KV_TWO_PASS", "Nvfp4Error", "lib", "nvfp4_status_string",
    "nvfp4_kv_workspace_bytes", "nvfp4_kv_error_word_offset", "nvfp4_kv_smooth_quantize", "nvfp4_kv_smooth_quantize_noalloc", "nvfp4_kv_smooth_quantize_lowbit",
    "nvfp4_dequantize_lowbit", "nvfp4_dequantize", "nvfp4_quantize_1d",
    "nvfp4_quantize_2d", "nvfp4_dequantize_2d", "nvfp4_kv_attention", "nvfp4_kv_attention_chunked",
    "nvfp4_kv_attention_workspace_bytes", "nvfp4_kv_attention_staged_workspace_bytes",
    "ATTN_MAX_RANGES", "KVCacheState", "KVCache", "nvfp4_gemm_w4a4", "nvfp4_kv_quantize_v_tblocks", "nvfp4_diag_e2m1_encode", "nvfp4_diag_candidates",
    "nvfp4_diag_reciprocal", "nvfp4_diag_bf16_round", "LIB_PATH",
]

MODE_4OVER6, MODE_FIXED6, MODE_FIXED4 = 0, 1, 2
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4kv.so")

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {nvfp4_status_string(status)} ({status})")


def lib():
    """The loaded C library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH}; build it with "
                               "`python precision_kv_cache_amd/build.py` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, i, ll, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t, ctypes.c_uint32
        sig = {
            "nvfp4_status_string": (ctypes.c_char_p, [i]),
            "nvfp4_kv_workspace_bytes": (sz, [i, i, i, i]),
            "nvfp4_kv_error_word_offset": (ll, [i, i, i, i]),
            "nvfp4_kv_smooth_quantize": (i, [P, P, i, i, i, i, i, P, P, P, P, P, P, P, P, P, sz, P]),
            "nvfp4_kv_smooth_quantize_noalloc": (i, [P, P, i, i, i, i, i, P, P, P, P, P, P, P, P, P, P]),
            "nvfp4_kv_smooth_quantize_lowbit": (i, [P, P, i, i, i, i, i, i, P, P, P, P, P, P, P, P, P, sz, P]),
            "nvfp4_dequantize_lowbit": (i, [P, P, P, P, i, i, i, i, i, P, P]),
            "nvfp4_dequantize": (i, [P, P, P, P, i, i, i, i, P, P]),
            "nvfp4_quantize_1d_workspace_bytes": (sz, [i, i]),
            "nvfp4_quantize_2d_workspace_bytes": (sz, [i, i]),
            "nvfp4_quantize_1d": (i, [P, i, i, i, i, u32, P, P, P, P, sz, P]),
            "nvfp4_quantize_2d": (i, [P, i, i, i, P, P, P, P, sz, P]),
            "nvfp4_dequantize_2d": (i, [P, P, P, i, i, P, P]),
            "nvfp4_kv_attention_workspace_bytes": (sz, [i, i, i]),
            "nvfp4_kv_attention_staged_workspace_bytes": (sz, [i, i, i, i, i, i, P, i]),
            "nvfp4_kv_attention": (i, [P, i, i, i, P, P, P, P, P, P, P, i, i, i, P, i, ctypes.c_float, P, P, P, sz,
                                       P]),
            "nvfp4_kv_attention_chunked": (i, [P, i, i, i, P, P, P, P, P, P, P, i, i, i, P, i, ctypes.c_float, P, P,
                                               P, sz, P]),
            "nvfp4_gemm_w4a4": (i, [P, P, P, i, i, P, P, P, i, i, P, P]),
            "nvfp4_kv_quantize_v_tblocks_workspace_bytes": (sz, [i, i, i, i]),
            "nvfp4_kv_quantize_v_tblocks": (i, [P, i, i, i, i, i, P, P, P, P, sz, P]),
            "nvfp4_kv_cache_layer_bytes": (sz, [i, i, i, i]),
            "nvfp4_kv_cache_offsets": (i, [P, P]),
            "nvfp4_kv_cache_init": (i, [P, i, i, i, i, i, i, i, i, i]),
            "nvfp4_kv_cache_begin_chunk": (i, [P, i]),
            "nvfp4_kv_cache_append": (i, [P, P, sz, i, P, P, i, P, sz, P]),
            "nvfp4_kv_cache_end_chunk": (i, [P]),
            "nvfp4_kv_cache_key_ranges": (i, [P, P]),
            "nvfp4_kv_cache_attention": (i, [P, P, sz, i, P, i, i, ctypes.c_float, P, P, P, sz, P]),
            "nvfp4_diag_e2m1_encode": (i, [P, ll, P, P]),
            "nvfp4_diag_candidates": (i, [P, ll, P, P, P]),
            "nvfp4_diag_reciprocal": (i, [P, ll, P, P]),
            "nvfp4_diag_bf16_round": (i, [P, ll, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def nvfp4_status_string(status):
    return lib().nvfp4_status_string(int(status)).decode()


def _check(rc, what):
    if rc != 0:
        raise Nvfp4Error(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bf16_dev(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
    return t


def nvfp4_kv_workspace_bytes(H, T, D, chunk_len):
    return int(lib().nvfp4_kv_workspace_bytes(H, T, D, chunk_len))


def kv_error_word(workspace):
    """The sticky error word of a KV or V-tblocks workspace, read after a
    synchronize (a device-to-host copy of its first 4 bytes)."""
    return int(workspace[:4].view(torch.int32).cpu()[0])


def nvfp4_kv_error_word_offset(H, T, D, chunk_len):
    """Byte offset of the workspace's sticky error word (0; -1 for an invalid
    shape).  The library never clears it; non-zero means some call on the
    workspace since it was last zeroed had a wait time out."""
    return int(lib().nvfp4_kv_error_word_offset(H, T, D, chunk_len))


KV_TWO_PASS = 0x100


def nvfp4_kv_smooth_quantize(k, v, chunk_len, mode=MODE_4OVER6, choice_counts=False, out=None, workspace=None,
                             stream=None, two_pass=False):
    """K smoothing + 4/6 NVFP4 quantization of K, V bf16 [H, T, D].

    Returns a dict with k_codes, v_codes [H, T, D/2] uint8, k_scales, v_scales
    [H, T, D/16] uint8 (E4M3FN bits), k_tensor_scale, v_tensor_scale [T/L]
    float32, k_mean [T/L, H, D] float32 and, if requested, choice_counts [2, 2]
    int64 ({K, V} x {kept +-6, kept +-4}).  ``out`` may supply these tensors
    (and ``workspace`` a uint8 device buffer) to avoid allocation.
    By default (D == 128) one overlapped launch interleaves each unit's
    statistics with the quantization of an earlier unit; ``two_pass`` forces
    the statistics-then-quantize kernels (same results).
    """
    _bf16_dev(k, "k"); _bf16_dev(v, "v")
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [H, T, D]")
    H, T, D = k.shape
    dev = k.device
    nc = T // chunk_len if chunk_len > 0 else 0
    if out is None:
        out = {
            "k_codes": torch.empty(H, T, D // 2, dtype=torch.uint8, device=dev),
            "v_codes": torch.empty(H, T, D // 2, dtype=torch.uint8, device=dev),
            "k_scales": torch.empty(H, T, D // 16, dtype=torch.uint8, device=dev),
            "v_scales": torch.empty(H, T, D // 16, dtype=torch.uint8, device=dev),
            "k_tensor_scale": torch.empty(nc, dtype=torch.float32, device=dev),
            "v_tensor_scale": torch.empty(nc, dtype=torch.float32, device=dev),
            "k_mean": torch.empty(nc, H, D, dtype=torch.float32, device=dev),
        }
        if choice_counts:
            out["choice_counts"] = torch.empty(2, 2, dtype=torch.int64, device=dev)
    ws_bytes = nvfp4_kv_workspace_bytes(H, T, D, chunk_len)
    if workspace is None and ws_bytes:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)  # sticky error word starts at 0
    rc = lib().nvfp4_kv_smooth_quantize(
        _ptr(k), _ptr(v), H, T, D, chunk_len, mode | (KV_TWO_PASS if two_pass else 0), _ptr(out["k_codes"]), _ptr(out["v_codes"]),
        _ptr(out["k_scales"]), _ptr(out["v_scales"]), _ptr(out["k_tensor_scale"]), _ptr(out["v_tensor_scale"]),
        _ptr(out["k_mean"]), _ptr(out.get("choice_counts")), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(rc, "nvfp4_kv_smooth_quantize")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # NVFP4_KV_NOALLOC_SCRATCH_BYTES


def nvfp4_kv_smooth_quantize_noalloc(k, v, chunk_len, out, mode=MODE_4OVER6, error_word=None, stream=None):
    """nvfp4_kv_smooth_quantize without a workspace (the library's per-GPU
    device array instead), for callers that cannot allocate: ``out`` must hold
    every output tensor (and "choice_counts" if wanted); ``error_word`` is an
    optional int32 device tensor the call ORs 1 into if a wait timed out.
    Allocates nothing."""
    _bf16_dev(k, "k"); _bf16_dev(v, "v")
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [H, T, D]")
    H, T, D = k.shape
    rc = lib().nvfp4_kv_smooth_quantize_noalloc(
        _ptr(k), _ptr(v), H, T, D, chunk_len, mode, _ptr(out["k_codes"]), _ptr(out["v_codes"]),
        _ptr(out["k_scales"]), _ptr(out["v_scales"]), _ptr(out["k_tensor_scale"]), _ptr(out["v_tensor_scale"]),
        _ptr(out["k_mean"]), _ptr(out.get("choice_counts")), _ptr(error_word), _stream(stream))
    _check(rc, "nvfp4_kv_smooth_quantize_noalloc")
    return out


def lowbit_outputs(H, T, D, chunk_len, bits, device, choice_counts=False):
    nc = T // chunk_len
    out = {"k_codes": torch.empty(H, T, D * bits // 8, dtype=torch.uint8, device=device),
           "v_codes": torch.empty(H, T, D * bits // 8, dtype=torch.uint8, device=device),
           "k_scales": torch.empty(H, T, D // 16, dtype=torch.uint8, device=device),
           "v_scales": torch.empty(H, T, D // 16, dtype=torch.uint8, device=device),
           "k_tensor_scale": torch.empty(nc, dtype=torch.float32, device=device),
           "v_tensor_scale": torch.empty(nc, dtype=torch.float32, device=device),
           "k_mean": torch.empty(nc, H, D, dtype=torch.float32, device=device)}
    if choice_counts:
        out["choice_counts"] = torch.empty(2, 2, dtype=torch.int64, device=device)
    return out


def nvfp4_kv_smooth_quantize_lowbit(k, v, chunk_len, bits, mode=MODE_4OVER6, choice_counts=False, out=None,
                                    workspace=None, stream=None, two_pass=False):
    """K smoothing + 3-bit or 2-bit quantization of K, V bf16 [H, T, D]: the
    outputs of nvfp4_kv_smooth_quantize with codes [H, T, D * bits / 8] and
    choice_counts {K, V} x {kept c_a, kept c_b}.  two_pass forces the two-pass
    kernels (the default is the overlapped kernel when D = 128)."""
    _bf16_dev(k, "k"); _bf16_dev(v, "v")
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [H, T, D]")
    H, T, D = k.shape
    if out is None:
        out = lowbit_outputs(H, T, D, chunk_len, bits, k.device, choice_counts)
    if workspace is None:  # zeroed: its first word is the sticky error word
        workspace = torch.zeros(max(1, nvfp4_kv_workspace_bytes(H, T, D, chunk_len)), dtype=torch.uint8,
                                device=k.device)
    rc = lib().nvfp4_kv_smooth_quantize_lowbit(
        _ptr(k), _ptr(v), H, T, D, chunk_len, bits, mode | (KV_TWO_PASS if two_pass else 0), _ptr(out["k_codes"]),
        _ptr(out["v_codes"]), _ptr(out["k_scales"]), _ptr(out["v_scales"]), _ptr(out["k_tensor_scale"]),
        _ptr(out["v_tensor_scale"]), _ptr(out["k_mean"]), _ptr(out.get("choice_counts")), _ptr(workspace),
        workspace.numel(), _stream(stream))
    _check(rc, "nvfp4_kv_smooth_quantize_lowbit")
    return out


def nvfp4_dequantize_lowbit(codes, scales, tensor_scale, mean, chunk_len, bits, out=None, stream=None):
    """codes [H, T, D * bits / 8], scales [H, T, D/16] -> bf16 [H, T, D]."""
    H, T, NB = scales.shape
    D = NB * 16
    if out is None:
        out = torch.empty(H, T, D, dtype=torch.bfloat16, device=codes.device)
    rc = lib().nvfp4_dequantize_lowbit(_ptr(codes), _ptr(scales), _ptr(tensor_scale), _ptr(mean), H, T, D, chunk_len,
                                       bits, _ptr(out), _stream(stream))
    _check(rc, "nvfp4_dequantize_lowbit")
    return out


def nvfp4_dequantize(codes, scales, tensor_scale, mean, chunk_len, out=None, stream=None):
    """codes [H, T, D/2], scales [H, T, D/16], tensor_scale [T/L], mean
    [T/L, H, D] or None -> bf16 [H, T, D]."""
    H, T, D2 = codes.shape
    D = 2 * D2
    if out is None:
        out = torch.empty(H, T, D, dtype=torch.bfloat16, device=codes.device)
    rc = lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), _ptr(mean), H, T, D, chunk_len,
                                _ptr(out), _stream(stream))
    _check(rc, "nvfp4_dequantize")
    return out


ATTN_MAX_RANGES = 8


def nvfp4_kv_attention_workspace_bytes(H, Tq, D):
    """Workspace bytes that let an attention call split every query block's
    key list as far as it helps (0 for an invalid shape)."""
    return int(lib().nvfp4_kv_attention_workspace_bytes(H, Tq, D))


def _ranges_arr(key_ranges):
    rg = [(int(a), int(n)) for a, n in key_ranges]
    return rg, (ctypes.c_int * max(1, 2 * len(rg)))(*[x for r in rg for x in r])


def nvfp4_kv_attention_staged_workspace_bytes(H, Tq, D, H_kv, T, chunk_len, key_ranges):
    """Workspace bytes for every key split plus the decoded image of every
    key tile of this key list (cache of H_kv heads, T tokens): with such a
    workspace an attention call decodes each tile once (0 for invalid
    arguments)."""
    rg, arr = _ranges_arr(key_ranges)
    return int(lib().nvfp4_kv_attention_staged_workspace_bytes(H, Tq, D, H_kv, T, chunk_len, arr, len(rg)))


def _attn_workspace(workspace, H, Tq, D, device, keys=None):
    """workspace argument -> (tensor or None, bytes): None allocates one big
    enough for every key split and, given keys = (H_kv, T, chunk_len,
    key_ranges), for the staged form too; False runs unsplit and unstaged; a
    uint8 tensor is used as it is."""
    if workspace is False:
        return None, 0
    if workspace is None:
        n = (nvfp4_kv_attention_staged_workspace_bytes(H, Tq, D, *keys) if keys is not None
             else nvfp4_kv_attention_workspace_bytes(H, Tq, D))
        if n == 0:
            return None, 0
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _lse_out(lse, H, Tq, device):
    """lse argument -> the fp32 [H, Tq] output tensor, or None."""
    if isinstance(lse, torch.Tensor):
        if lse.dtype != torch.float32 or tuple(lse.shape) != (H, Tq) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous fp32 [H, Tq] tensor")
        return lse
    return torch.empty(H, Tq, dtype=torch.float32, device=device) if lse else None


def nvfp4_kv_attention(q, cache, chunk_len, key_ranges, softmax_scale=None, out=None, lse=False, workspace=None,
                       stream=None):
    """Softmax attention of q (bf16 [H, Tq, D]) over the keys listed in
    key_ranges ([(start, len), ...], at most ATTN_MAX_RANGES) of an NVFP4
    cache: the dict nvfp4_kv_smooth_quantize returns (k_codes, k_scales,
    k_tensor_scale, k_mean (may be None), v_codes, v_scales, v_tensor_scale),
    for H_kv heads with H % H_kv == 0.  softmax_scale defaults to 1/sqrt(D).
    Returns out (bf16 [H, Tq, D]), or (out, lse fp32 [H, Tq]) when lse is
    True or a preallocated fp32 [H, Tq] tensor (written in place).
    workspace: None allocates one that allows key splits and the staged
    form (each key tile decoded once per call), False runs unsplit and
    unstaged, or a uint8 device tensor (nvfp4_kv_attention_workspace_bytes
    allows every split, nvfp4_kv_attention_staged_workspace_bytes the staged
    form as well)."""
    _bf16_dev(q, "q")
    if q.dim() != 3:
        raise ValueError("q must be [H, Tq, D]")
    H, Tq, D = q.shape
    kc = cache["k_codes"]
    H_kv, T = kc.shape[0], kc.shape[1]
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    rg, arr = _ranges_arr(key_ranges)
    if out is None:
        out = torch.empty(H, Tq, D, dtype=torch.bfloat16, device=q.device)
    lse_t = _lse_out(lse, H, Tq, q.device)
    ws, ws_bytes = _attn_workspace(workspace, H, Tq, D, q.device, (H_kv, T, chunk_len, rg))
    rc = lib().nvfp4_kv_attention(
        _ptr(q), H, Tq, D, _ptr(kc), _ptr(cache["k_scales"]), _ptr(cache["k_tensor_scale"]), _ptr(cache.get("k_mean")),
        _ptr(cache["v_codes"]), _ptr(cache["v_scales"]), _ptr(cache["v_tensor_scale"]), H_kv, T, chunk_len, arr,
        len(rg), float(softmax_scale), _ptr(out), _ptr(lse_t), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "nvfp4_kv_attention")
    return (out, lse_t) if lse_t is not None else out


def nvfp4_kv_attention_chunked(q, cache, chunk_len, key_ranges, softmax_scale=None, out=None, lse=False,
                               workspace=None, stream=None):
    """nvfp4_kv_attention over a chunk-major cache: cache arrays [n_chunks,
    H_kv, chunk_len, ...] (each chunk as one quantize call writes it), tensor
    scales [n_chunks], k_mean [n_chunks, H_kv, D]."""
    _bf16_dev(q, "q")
    H, Tq, D = q.shape
    kc = cache["k_codes"]
    nch, H_kv, L = kc.shape[0], kc.shape[1], kc.shape[2]
    if L != chunk_len:
        raise ValueError("k_codes chunk length differs from chunk_len")
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    rg, arr = _ranges_arr(key_ranges)
    if out is None:
        out = torch.empty(H, Tq, D, dtype=torch.bfloat16, device=q.device)
    lse_t = _lse_out(lse, H, Tq, q.device)
    ws, ws_bytes = _attn_workspace(workspace, H, Tq, D, q.device, (H_kv, nch * L, chunk_len, rg))
    rc = lib().nvfp4_kv_attention_chunked(
        _ptr(q), H, Tq, D, _ptr(kc), _ptr(cache["k_scales"]), _ptr(cache["k_tensor_scale"]), _ptr(cache.get("k_mean")),
        _ptr(cache["v_codes"]), _ptr(cache["v_scales"]), _ptr(cache["v_tensor_scale"]), H_kv, nch * L, chunk_len, arr,
        len(rg), float(softmax_scale), _ptr(out), _ptr(lse_t), _ptr(ws), ws_bytes, _stream(stream))
    _check(rc, "nvfp4_kv_attention_chunked")
    return (out, lse_t) if lse_t is not None else out


def nvfp4_gemm_w4a4(a, w, w_2d, out=None, stream=None):
    """out (bf16 [M, N]) = the product of two NVFP4 operands along K:
    a = (codes [M, K/2], scales [M, K/16], tensor_scale [1]) as
    nvfp4_quantize_1d returns them (a dict with those keys also works), w the
    same for the weight [N, K] with scales [N/16, K/16] (w_2d) or [N, K/16]."""
    def parts(x):
        return (x["codes"], x["scales"], x["tensor_scale"]) if isinstance(x, dict) else x
    ac, as_, ag = parts(a)
    wc, ws, wg = parts(w)
    M, K2 = ac.shape
    N = wc.shape[0]
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=ac.device)
    rc = lib().nvfp4_gemm_w4a4(_ptr(ac), _ptr(as_), _ptr(ag), M, 2 * K2, _ptr(wc), _ptr(ws), _ptr(wg), N,
                               1 if w_2d else 0, _ptr(out), _stream(stream))
    _check(rc, "nvfp4_gemm_w4a4")
    return out


def nvfp4_kv_quantize_v_tblocks(v, chunk_len, mode=MODE_4OVER6, out=None, workspace=None, stream=None):
    """V bf16 [H, T, D] -> NVFP4 with 16-token blocks per (head, channel):
    {"codes": [H, D, T/2], "scales": [H, D, T/16], "tensor_scale": [T/L]}."""
    _bf16_dev(v, "v")
    H, T, D = v.shape
    nc = T // chunk_len if chunk_len > 0 else 0
    if out is None:
        out = {"codes": torch.empty(H, D, T // 2, dtype=torch.uint8, device=v.device),
               "scales": torch.empty(H, D, T // 16, dtype=torch.uint8, device=v.device),
               "tensor_scale": torch.empty(nc, dtype=torch.float32, device=v.device)}
    if workspace is None:
        workspace = torch.zeros(max(1, int(lib().nvfp4_kv_quantize_v_tblocks_workspace_bytes(H, T, D, chunk_len))),
                                dtype=torch.uint8, device=v.device)
    rc = lib().nvfp4_kv_quantize_v_tblocks(_ptr(v), H, T, D, chunk_len, mode, _ptr(out["codes"]), _ptr(out["scales"]),
                                           _ptr(out["tensor_scale"]), _ptr(workspace), workspace.numel(),
                                           _stream(stream))
    _check(rc, "nvfp4_kv_quantize_v_tblocks")
    return out


CACHE_MAX_SLOTS = 64


class KVCacheState(ctypes.Structure):
    """Mirror of nvfp4_kv_cache_t (include/nvfp4kv.h)."""
    _fields_ = [(n, ctypes.c_int) for n in ("layers", "heads", "head_dim", "chunk_len", "capacity", "frame_tokens",
                                            "sink_frames", "shot_frames", "window")] + [
        ("chunks", ctypes.c_longlong), ("shot_chunk", ctypes.c_longlong), ("pending", ctypes.c_longlong),
        ("pending_slot", ctypes.c_int), ("pending_new_shot", ctypes.c_int),
        ("slot_chunk", ctypes.c_longlong * CACHE_MAX_SLOTS)]


class KVCache:
    """The streaming NVFP4 KV cache: a KVCacheState plus its device storage
    (one uint8 tensor, allocated here when not given).  Methods map one to
    one to the nvfp4_kv_cache_* entry points."""

    def __init__(self, layers, heads, head_dim, chunk_len, capacity, frame_tokens, sink_frames, shot_frames, window,
                 device="cuda", storage=None):
        self.state = KVCacheState()
        _check(lib().nvfp4_kv_cache_init(ctypes.byref(self.state), layers, heads, head_dim, chunk_len, capacity,
                                         frame_tokens, sink_frames, shot_frames, window), "nvfp4_kv_cache_init")
        self.layer_bytes = int(lib().nvfp4_kv_cache_layer_bytes(heads, head_dim, chunk_len, capacity))
        self.storage_bytes = self.layer_bytes * layers
        if storage is None and device is not None:
            storage = torch.empty(self.storage_bytes, dtype=torch.uint8, device=device)
        self.storage = storage
        off = (ctypes.c_size_t * 7)()
        _check(lib().nvfp4_kv_cache_offsets(ctypes.byref(self.state), off), "nvfp4_kv_cache_offsets")
        self.offsets = list(off)

    def begin_chunk(self, new_shot=False):
        rc = lib().nvfp4_kv_cache_begin_chunk(ctypes.byref(self.state), 1 if new_shot else 0)
        if rc < 0:
            raise Nvfp4Error(rc, "nvfp4_kv_cache_begin_chunk")
        return rc

    def append(self, layer, k, v, mode=MODE_4OVER6, workspace=None, stream=None):
        _bf16_dev(k, "k"); _bf16_dev(v, "v")
        st = self.state
        ws_bytes = nvfp4_kv_workspace_bytes(st.heads, st.chunk_len, st.head_dim, st.chunk_len)
        if workspace is None:
            workspace = torch.zeros(max(1, ws_bytes), dtype=torch.uint8, device=k.device)
        rc = lib().nvfp4_kv_cache_append(ctypes.byref(st), _ptr(self.storage), self.storage_bytes, layer, _ptr(k),
                                         _ptr(v), mode, _ptr(workspace), workspace.numel(), _stream(stream))
        _check(rc, "nvfp4_kv_cache_append")

    def end_chunk(self):
        _check(lib().nvfp4_kv_cache_end_chunk(ctypes.byref(self.state)), "nvfp4_kv_cache_end_chunk")

    def key_ranges(self):
        arr = (ctypes.c_int * (2 * ATTN_MAX_RANGES))()
        n = lib().nvfp4_kv_cache_key_ranges(ctypes.byref(self.state), arr)
        if n < 0:
            raise Nvfp4Error(n, "nvfp4_kv_cache_key_ranges")
        return [(arr[2 * i], arr[2 * i + 1]) for i in range(n)]

    def attention(self, layer, q, softmax_scale=None, out=None, lse=False, workspace=None, stream=None):
        _bf16_dev(q, "q")
        Hq, Tq, D = q.shape
        if softmax_scale is None:
            softmax_scale = D ** -0.5
        if out is None:
            out = torch.empty(Hq, Tq, D, dtype=torch.bfloat16, device=q.device)
        lse_t = _lse_out(lse, Hq, Tq, q.device)
        st = self.state
        keys = (st.heads, st.capacity * st.chunk_len, st.chunk_len, self.key_ranges())
        ws, ws_bytes = _attn_workspace(workspace, Hq, Tq, D, q.device, keys)
        rc = lib().nvfp4_kv_cache_attention(ctypes.byref(self.state), _ptr(self.storage), self.storage_bytes, layer,
                                            _ptr(q), Hq, Tq, float(softmax_scale), _ptr(out), _ptr(lse_t),
                                            _ptr(ws), ws_bytes, _stream(stream))
        _check(rc, "nvfp4_kv_cache_attention")
        return (out, lse_t) if lse_t is not None else out

    def slot_arrays(self, layer):
        """Views of one layer's slot arrays (k_codes, v_codes [cap, H, L,
        D/2], k_scales, v_scales [cap, H, L, D/16], k_tensor_scale,
        v_tensor_scale [cap], k_mean [cap, H, D])."""
        st = self.state
        cap, H, L, D = st.capacity, st.heads, st.chunk_len, st.head_dim
        base = layer * self.layer_bytes
        o = self.offsets
        n = cap * H * L * D
        b = lambda i, nbytes: self.storage[base + o[i]: base + o[i] + nbytes]  # noqa: E731
        return {"k_codes": b(0, n // 2).view(cap, H, L, D // 2), "v_codes": b(1, n // 2).view(cap, H, L, D // 2),
                "k_scales": b(2, n // 16).view(cap, H, L, D // 16), "v_scales": b(3, n // 16).view(cap, H, L, D // 16),
                "k_tensor_scale": b(4, cap * 4).view(torch.float32), "v_tensor_scale": b(5, cap * 4).view(torch.float32),
                "k_mean": b(6, cap * H * D * 4).view(torch.float32).view(cap, H, D)}


def nvfp4_quantize_1d(x, mode=MODE_4OVER6, hadamard=False, sign_mask=0, out=None, workspace=None, stream=None):
    """Activation x bf16 [rows, cols] -> codes [rows, cols/2], scales
    [rows, cols/16], tensor_scale [1]; optional 16-point RHT first."""
    _bf16_dev(x, "x")
    rows, cols = x.shape
    dev = x.device
    if out is None:
        out = {"codes": torch.empty(rows, cols // 2, dtype=torch.uint8, device=dev),
               "scales": torch.empty(rows, cols // 16, dtype=torch.uint8, device=dev),
               "tensor_scale": torch.empty(1, dtype=torch.float32, device=dev)}
    nws = int(lib().nvfp4_quantize_1d_workspace_bytes(rows, cols))
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    rc = lib().nvfp4_quantize_1d(_ptr(x), rows, cols, mode, int(bool(hadamard)), int(sign_mask) & 0xFFFF,
                                 _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["tensor_scale"]),
                                 _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "nvfp4_quantize_1d")
    return out


def nvfp4_quantize_2d(w, mode=MODE_4OVER6, out=None, workspace=None, stream=None):
    """Weight w bf16 [rows, cols] -> codes [rows, cols/2], scales
    [rows/16, cols/16], tensor_scale [1] (16x16 tiles)."""
    _bf16_dev(w, "w")
    rows, cols = w.shape
    dev = w.device
    if out is None:
        out = {"codes": torch.empty(rows, cols // 2, dtype=torch.uint8, device=dev),
               "scales": torch.empty(rows // 16, cols // 16, dtype=torch.uint8, device=dev),
               "tensor_scale": torch.empty(1, dtype=torch.float32, device=dev)}
    nws = int(lib().nvfp4_quantize_2d_workspace_bytes(rows, cols))
    if workspace is None:
        workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    rc = lib().nvfp4_quantize_2d(_ptr(w), rows, cols, mode, _ptr(out["codes"]), _ptr(out["scales"]),
                                 _ptr(out["tensor_scale"]), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "nvfp4_quantize_2d")
    return out


def nvfp4_dequantize_2d(codes, scales, tensor_scale, out=None, stream=None):
    rows, c2 = codes.shape
    if out is None:
        out = torch.empty(rows, 2 * c2, dtype=torch.bfloat16, device=codes.device)
    rc = lib().nvfp4_dequantize_2d(_ptr(codes), _ptr(scales), _ptr(tensor_scale), rows, 2 * c2, _ptr(out),
                                   _stream(stream))
    _check(rc, "nvfp4_dequantize_2d")
    return out


# ---- codec probes (test support) -----------------------------------------

def nvfp4_diag_e2m1_encode(y, stream=None):
    out = torch.empty(y.shape, dtype=torch.uint8, device=y.device)
    _check(lib().nvfp4_diag_e2m1_encode(_ptr(y), y.numel(), _ptr(out), _stream(stream)), "nvfp4_diag_e2m1_encode")
    return out


def nvfp4_diag_candidates(t, stream=None):
    s6 = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    s4 = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    _check(lib().nvfp4_diag_candidates(_ptr(t), t.numel(), _ptr(s6), _ptr(s4), _stream(stream)),
           "nvfp4_diag_candidates")
    return s6, s4


def nvfp4_diag_reciprocal(s, stream=None):
    out = torch.empty(s.shape, dtype=torch.float32, device=s.device)
    _check(lib().nvfp4_diag_reciprocal(_ptr(s), s.numel(), _ptr(out), _stream(stream)), "nvfp4_diag_reciprocal")
    return out


def nvfp4_diag_bf16_round(x, stream=None):
    out = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    _check(lib().nvfp4_diag_bf16_round(_ptr(x), x.numel(), _ptr(out), _stream(stream)), "nvfp4_diag_bf16_round")
    return out
