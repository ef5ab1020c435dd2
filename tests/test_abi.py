"""The C ABI without a GPU: the library loads, exports every function the
headers declare, and rejects bad arguments with the documented status before
any HIP call (so these run on a machine with no GPU, with fake pointers that
are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import precision_kv_cache_amd as P
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("nvfp4kv.h", "nvfp4kv_diag.h")]

OK, NULL, SHAPE, ALIGN, ALIAS, WORKSPACE, MODE, HIP = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    names = []
    for h in HEADERS:
        txt = open(h).read()
        names += re.findall(r"NVFP4KV_API\s+[\w\s\*]+?\b(nvfp4_\w+)\s*\(", txt)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 13
    L = P.lib()
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (nvfp4_\w+)", nm))
    assert set(names) <= exported, set(names) - exported
    # nothing else leaks out under the nvfp4_ prefix
    assert exported == set(names), exported - set(names)


def test_status_strings():
    for code in (OK, NULL, SHAPE, ALIGN, ALIAS, WORKSPACE, MODE, HIP):
        s = P.nvfp4_status_string(code)
        assert s.startswith("NVFP4")
    assert "unknown" in P.nvfp4_status_string(12345)


def test_workspace_sizes():
    assert P.nvfp4_kv_workspace_bytes(24, 7040, 128, 7040) > 0
    assert P.nvfp4_kv_workspace_bytes(24, 7040, 128, 7040) % 256 == 0
    assert P.nvfp4_kv_workspace_bytes(24, 56320, 128, 7040) > P.nvfp4_kv_workspace_bytes(24, 7040, 128, 7040)
    for bad in ((24, 7040, 100, 7040), (24, 7041, 128, 7040), (-1, 10, 16, 10), (1, 16, 8192, 16), (1, 16, 16, 0)):
        assert P.nvfp4_kv_workspace_bytes(*bad) == 0, bad
    # the sticky error word is the workspace's first word for every valid shape
    for shape in ((24, 7040, 128, 7040), (24, 56320, 128, 7040), (1, 256, 128, 256), (3, 77, 128, 7),
                  (2, 96, 48, 32)):
        assert P.nvfp4_kv_error_word_offset(*shape) == 0, shape
        assert P.nvfp4_kv_workspace_bytes(*shape) >= 256 + 4, shape
    assert P.nvfp4_kv_error_word_offset(24, 7041, 128, 7040) == -1  # invalid shape
    assert P.lib().nvfp4_quantize_1d_workspace_bytes(16, 48) > 0
    assert P.lib().nvfp4_quantize_2d_workspace_bytes(24, 48) == 0  # rows % 16


FAKE = 0x7f0000000000  # 256-byte aligned, never dereferenced


def _kvq(k=FAKE, v=FAKE + (1 << 30), H=2, T=64, D=32, L=32, mode=0, kc=FAKE + (2 << 30), vc=FAKE + (3 << 30),
         ks=FAKE + (4 << 30), vs=FAKE + (5 << 30), kt=FAKE + (6 << 30), vt=FAKE + (7 << 30), km=FAKE + (8 << 30),
         cc=None, ws=FAKE + (9 << 30), wsb=1 << 20):
    V = ctypes.c_void_p
    return P.lib().nvfp4_kv_smooth_quantize(V(k), V(v), H, T, D, L, mode, V(kc), V(vc), V(ks), V(vs), V(kt), V(vt),
                                            V(km), V(cc), V(ws), wsb, None)


def test_kv_quantize_argument_errors():
    assert _kvq(k=None) == NULL
    assert _kvq(km=None) == NULL
    assert _kvq(D=40) == SHAPE
    assert _kvq(T=65) == SHAPE
    assert _kvq(L=0) == SHAPE
    assert _kvq(H=-1) == SHAPE
    assert _kvq(D=8192) == SHAPE
    assert _kvq(mode=3) == MODE
    assert _kvq(k=FAKE + 8) == ALIGN
    assert _kvq(kc=(FAKE + (2 << 30)) + 4) == ALIGN
    assert _kvq(km=(FAKE + (8 << 30)) + 4) == ALIGN
    assert _kvq(ws=(FAKE + (9 << 30)) + 128) == ALIGN
    assert _kvq(ws=None) == WORKSPACE
    assert _kvq(wsb=16) == WORKSPACE
    assert _kvq(vc=FAKE + 64) == ALIAS            # output inside input K
    assert _kvq(vc=FAKE + (2 << 30) + 256) == ALIAS  # two outputs overlap
    assert _kvq(ws=FAKE + (1 << 30)) == ALIAS     # workspace inside V
    assert _kvq(cc=FAKE + (5 << 30)) == ALIAS     # counts inside v_scales


def test_kv_quantize_output_in_workspace_tail_is_an_alias():
    # The overlapped kernel uses more workspace than the two-pass kernels for
    # small shapes; every byte nvfp4_kv_workspace_bytes covers is the
    # library's, so an output anywhere in it is rejected.
    H, T, D, L = 1, 256, 128, 256
    need = P.nvfp4_kv_workspace_bytes(H, T, D, L)
    ws = FAKE + (9 << 30)
    assert need > 4096
    for off in (0, 4096, need - 256):
        assert _kvq(H=H, T=T, D=D, L=L, kc=ws + off, ws=ws, wsb=need) == ALIAS, off
        assert _kvq(H=H, T=T, D=D, L=L, km=ws + off, ws=ws, wsb=need) == ALIAS, off


def test_noalloc_argument_errors_before_any_hip_call():
    V = ctypes.c_void_p
    L = P.lib()

    def call(H=2, T=64, D=32, Lc=32, mode=0, ew=None, **kw):
        a = dict(k=FAKE, v=FAKE + (1 << 30), kc=FAKE + (2 << 30), vc=FAKE + (3 << 30), ks=FAKE + (4 << 30),
                 vs=FAKE + (5 << 30), kt=FAKE + (6 << 30), vt=FAKE + (7 << 30), km=FAKE + (8 << 30), cc=None)
        a.update(kw)
        return L.nvfp4_kv_smooth_quantize_noalloc(V(a["k"]), V(a["v"]), H, T, D, Lc, mode, V(a["kc"]), V(a["vc"]),
                                                  V(a["ks"]), V(a["vs"]), V(a["kt"]), V(a["vt"]), V(a["km"]),
                                                  V(a["cc"]), V(ew), None)
    # the scratch holds one full-cache layer's workspace, not two layers' worth
    assert P.nvfp4_kv_workspace_bytes(24, 56320, 128, 7040) <= P.NOALLOC_SCRATCH_BYTES
    assert P.nvfp4_kv_workspace_bytes(48, 56320, 128, 7040) > P.NOALLOC_SCRATCH_BYTES
    assert call(H=48, T=56320, D=128, Lc=7040) == WORKSPACE
    assert call(k=None) == NULL
    assert call(D=40) == SHAPE
    assert call(mode=3) == MODE
    assert call(kc=FAKE + 4) == ALIGN
    assert call(ew=FAKE + (9 << 30) + 2) == ALIGN
    assert call(ew=FAKE + 8) == ALIAS             # error word inside K
    assert call(ew=FAKE + (2 << 30) + 8) == ALIAS  # error word inside k_codes
    assert call(vc=FAKE + 64) == ALIAS
    assert call(H=0, k=None, v=None) == OK


def test_lowbit_argument_errors():
    V = ctypes.c_void_p
    L = P.lib()

    def q(bits=3, H=2, T=64, D=32, Lc=32, mode=0, **kw):
        a = dict(k=FAKE, v=FAKE + (1 << 30), kc=FAKE + (2 << 30), vc=FAKE + (3 << 30), ks=FAKE + (4 << 30),
                 vs=FAKE + (5 << 30), kt=FAKE + (6 << 30), vt=FAKE + (7 << 30), km=FAKE + (8 << 30), cc=None,
                 ws=FAKE + (9 << 30), wsb=1 << 20)
        a.update(kw)
        return L.nvfp4_kv_smooth_quantize_lowbit(V(a["k"]), V(a["v"]), H, T, D, Lc, bits, mode, V(a["kc"]),
                                                 V(a["vc"]), V(a["ks"]), V(a["vs"]), V(a["kt"]), V(a["vt"]),
                                                 V(a["km"]), V(a["cc"]), V(a["ws"]), a["wsb"], None)
    assert q(bits=4) == SHAPE and q(bits=1) == SHAPE
    assert q(D=40) == SHAPE and q(mode=3) == MODE
    assert q(k=None) == NULL
    assert q(bits=3, kc=FAKE + (2 << 30) + 1) == ALIGN   # 3-bit codes: 2-byte aligned
    assert q(bits=2, kc=FAKE + (2 << 30) + 2) == ALIGN   # 2-bit codes: 4-byte aligned
    assert q(ws=None) == WORKSPACE and q(wsb=64) == WORKSPACE
    # 3-bit codes of [2, 64, 32] are 1536 bytes: v_codes inside them is an alias
    assert q(vc=FAKE + (2 << 30) + 1024) == ALIAS
    assert q(H=0, k=None) == OK
    d = L.nvfp4_dequantize_lowbit
    assert d(V(FAKE), V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), None, 1, 32, 32, 32, 5, V(FAKE + (3 << 30)), None) == SHAPE
    assert d(V(FAKE), V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), None, 1, 32, 32, 32, 3, V(FAKE + 16), None) == ALIAS
    assert d(None, V(FAKE), V(FAKE), None, 1, 32, 32, 32, 2, V(FAKE + (3 << 30)), None) == NULL


def test_empty_calls_are_no_ops():
    assert _kvq(H=0, k=None, v=None) == OK
    assert _kvq(T=0, k=None) == OK
    assert P.lib().nvfp4_dequantize(None, None, None, None, 0, 64, 32, 32, None, None) == OK
    assert P.lib().nvfp4_quantize_1d(None, 0, 32, 0, 1, 0, None, None, None, None, 0, None) == OK
    assert P.lib().nvfp4_quantize_2d(None, 0, 32, 0, None, None, None, None, 0, None) == OK


def test_dequant_and_1d_2d_argument_errors():
    V = ctypes.c_void_p
    L = P.lib()
    assert L.nvfp4_dequantize(None, V(FAKE), V(FAKE), None, 1, 32, 32, 32, V(FAKE), None) == NULL
    assert L.nvfp4_dequantize(V(FAKE), V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), None, 1, 32, 40, 32,
                              V(FAKE + (3 << 30)), None) == SHAPE
    assert L.nvfp4_dequantize(V(FAKE), V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), None, 1, 32, 32, 32,
                              V(FAKE + 16), None) == ALIAS
    assert L.nvfp4_dequantize(V(FAKE), V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), V(FAKE + (4 << 30) + 4), 1, 32,
                              32, 32, V(FAKE + (3 << 30)), None) == ALIGN
    ws1 = L.nvfp4_quantize_1d_workspace_bytes(16, 32)
    args1d = [V(FAKE), 16, 32, 0, 1, 0, V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), V(FAKE + (3 << 30)),
              V(FAKE + (4 << 30)), ws1, None]
    a = list(args1d); a[2] = 33
    assert L.nvfp4_quantize_1d(*a) == SHAPE
    a = list(args1d); a[3] = 7
    assert L.nvfp4_quantize_1d(*a) == MODE
    a = list(args1d); a[10] = 8
    assert L.nvfp4_quantize_1d(*a) == WORKSPACE
    a = list(args1d); a[6] = V(FAKE + 32)
    assert L.nvfp4_quantize_1d(*a) == ALIAS
    assert L.nvfp4_quantize_2d(V(FAKE), 24, 32, 0, V(FAKE + (1 << 30)), V(FAKE + (2 << 30)), V(FAKE + (3 << 30)),
                               V(FAKE + (4 << 30)), L.nvfp4_quantize_2d_workspace_bytes(32, 32), None) == SHAPE
    assert L.nvfp4_dequantize_2d(V(FAKE), V(FAKE + (1 << 30)), None, 32, 32, V(FAKE + (2 << 30)), None) == NULL
    assert L.nvfp4_diag_e2m1_encode(None, 10, None, None) == NULL
    assert L.nvfp4_diag_candidates(None, -1, None, None, None) == SHAPE


def _att(q=FAKE, H=2, Tq=16, D=128, kc=FAKE + (1 << 30), ks=FAKE + (2 << 30), kg=FAKE + (3 << 30),
         km=FAKE + (4 << 30), vc=FAKE + (5 << 30), vs=FAKE + (6 << 30), vg=FAKE + (7 << 30), Hkv=1, T=64, L=32,
         ranges=((0, 64),), n=None, scale=0.088, out=FAKE + (8 << 30), lse=FAKE + (9 << 30), ws=None, wsb=0):
    V = ctypes.c_void_p
    flat = [x for r in (ranges or ()) for x in r]
    arr = (ctypes.c_int * max(1, len(flat)))(*flat) if ranges is not None else None
    n = len(ranges or ()) if n is None else n
    return P.lib().nvfp4_kv_attention(V(q), H, Tq, D, V(kc), V(ks), V(kg), V(km), V(vc), V(vs), V(vg), Hkv, T, L,
                                      arr, n, scale, V(out), V(lse), V(ws), wsb, None)


def test_attention_argument_errors():
    assert _att(D=64) == SHAPE
    assert _att(Hkv=3) == SHAPE                    # H % H_kv
    assert _att(T=65) == SHAPE                     # T % chunk_len
    assert _att(ranges=((60, 5),)) == SHAPE        # past the cache end
    assert _att(ranges=((-1, 2),)) == SHAPE
    assert _att(ranges=((0, 1),) * 9) == SHAPE     # more than the maximum count of ranges
    assert _att(scale=float("inf")) == SHAPE
    assert _att(scale=0.0) == SHAPE
    assert _att(scale=-0.1) == SHAPE
    assert _att(ranges=None, n=1) == NULL
    assert _att(q=None) == NULL
    assert _att(kc=None) == NULL
    assert _att(q=FAKE + 8) == ALIGN
    assert _att(km=FAKE + (4 << 30) + 4) == ALIGN
    assert _att(out=FAKE + 64) == ALIAS            # output inside q
    assert _att(lse=FAKE + (8 << 30) + 32) == ALIAS  # lse inside out
    assert _att(ws=FAKE + (10 << 30) + 64, wsb=1 << 20) == ALIGN  # workspace 256-byte aligned
    assert _att(ws=FAKE + (8 << 30), wsb=1 << 20) == ALIAS           # workspace over out
    assert _att(H=0, q=None, out=None) == OK       # empty call
    assert _att(Tq=0) == OK
    # workspace for every key split: partial O (fp32 D per row) and (M, l) per row, per split
    wb = P.nvfp4_kv_attention_workspace_bytes(24, 7040, 128)
    assert wb >= 4 * 24 * 7040 * (128 + 2) * 4
    assert P.nvfp4_kv_attention_workspace_bytes(24, 7040, 64) == 0


def _tiles(ranges, L):
    """Tiles of the attention's key walk: each range cut at chunk edges, each
    piece in tiles of at most 64 keys."""
    t = 0
    for a, n in ranges:
        pos, end = a, a + n
        while pos < end:
            cend = min(end, (pos // L + 1) * L)
            t += -(-(cend - pos) // 64)
            pos = cend
    return t


def test_attention_staged_workspace_bytes():
    """Every split plus one decoded image per (cache head, tile): 64 K rows
    of 272 bytes and 128 V^T rows of 144 bytes, 35,840 bytes."""
    img = 64 * 272 + 128 * 144
    for H, Tq, Hkv, T, L, ranges in [
        (24, 7040, 24, 56320, 7040, [(0, 56320)]),
        (24, 7040, 24, 56320, 7040, W.sink_ranges(8)),
        (4, 300, 2, 640, 128, [(0, 70), (200, 77), (383, 257)]),
        (3, 17, 1, 512, 64, [(448, 64), (0, 64), (100, 1)]),
        (2, 5, 2, 256, 128, []),
        (2, 5, 2, 256, 128, [(5, 0), (7, 3)]),
    ]:
        got = P.nvfp4_kv_attention_staged_workspace_bytes(H, Tq, 128, Hkv, T, L, ranges)
        assert got == P.nvfp4_kv_attention_workspace_bytes(H, Tq, 128) + Hkv * _tiles(ranges, L) * img, ranges
    assert _tiles([(0, 56320)], 7040) == 880
    bad = [dict(D=64), dict(Hkv=3), dict(T=650), dict(ranges=[(600, 50)]), dict(ranges=[(-1, 2)]),
           dict(ranges=[(0, 1)] * 9), dict(L=0), dict(H=0)]
    for b in bad:
        a = dict(H=4, Tq=10, D=128, Hkv=2, T=640, L=128, ranges=[(0, 640)])
        a.update(b)
        assert P.nvfp4_kv_attention_staged_workspace_bytes(a["H"], a["Tq"], a["D"], a["Hkv"], a["T"], a["L"],
                                                           a["ranges"]) == 0, b
    assert P.lib().nvfp4_kv_attention_staged_workspace_bytes(4, 10, 128, 2, 640, 128, None, 1) == 0
    # the staging grid (512 work-items per tile) stays below 2^32 work-items: at most 2^23 - 1 tiles,
    # a longer key list runs unstaged and needs only the split room
    splits = P.nvfp4_kv_attention_workspace_bytes(1, 1, 128)
    T = (1 << 29) - 64
    assert P.nvfp4_kv_attention_staged_workspace_bytes(1, 1, 128, 1, T, T, [(0, T)]) == splits + ((1 << 23) - 1) * img
    T = 1 << 29
    assert P.nvfp4_kv_attention_staged_workspace_bytes(1, 1, 128, 1, T, T, [(0, T)]) == splits


def _gemm(ac=FAKE, as_=FAKE + (1 << 30), ag=FAKE + (2 << 30), M=64, K=128, wc=FAKE + (3 << 30),
          ws=FAKE + (4 << 30), wg=FAKE + (5 << 30), N=32, w2d=1, out=FAKE + (6 << 30)):
    V = ctypes.c_void_p
    return P.lib().nvfp4_gemm_w4a4(V(ac), V(as_), V(ag), M, K, V(wc), V(ws), V(wg), N, w2d, V(out), None)


def test_gemm_argument_errors():
    assert _gemm(K=96) == SHAPE          # K % 64
    assert _gemm(K=0) == SHAPE
    assert _gemm(N=40) == SHAPE          # N % 16
    assert _gemm(M=-1) == SHAPE
    assert _gemm(ac=None) == NULL
    assert _gemm(wg=None) == NULL
    assert _gemm(ac=FAKE + 8) == ALIGN   # codes 16-byte aligned
    assert _gemm(out=FAKE + 4) == ALIGN
    assert _gemm(out=FAKE + 64) == ALIAS  # output inside A's codes
    assert _gemm(M=0, ac=None, out=None) == OK
    assert _gemm(N=0) == OK


def test_v_tblocks_argument_errors():
    V = ctypes.c_void_p
    L = P.lib()
    args = lambda **k: [V(k.get("v", FAKE)), k.get("H", 2), k.get("T", 256), k.get("D", 128), k.get("L", 128),  # noqa: E731
                        k.get("mode", 0), V(k.get("codes", FAKE + (1 << 30))), V(k.get("scales", FAKE + (2 << 30))),
                        V(k.get("ts", FAKE + (3 << 30))), V(k.get("ws", FAKE + (4 << 30))), k.get("wsb", 1 << 20),
                        None]
    f = L.nvfp4_kv_quantize_v_tblocks
    assert f(*args(D=96)) == SHAPE
    assert f(*args(L=24)) == SHAPE
    assert f(*args(T=200)) == SHAPE
    assert f(*args(mode=5)) == MODE
    assert f(*args(v=None)) == NULL
    assert f(*args(ws=None)) == WORKSPACE
    assert f(*args(wsb=8)) == WORKSPACE
    assert f(*args(v=FAKE + 8)) == ALIGN
    assert f(*args(codes=FAKE + 64)) == ALIAS
    assert f(*args(H=0)) == OK
    assert L.nvfp4_kv_quantize_v_tblocks_workspace_bytes(2, 256, 128, 100) == 0
    # a million 16-token chunks: 32 ready words of 256 bytes per chunk, so the
    # size passes 2^33 bytes and must come back whole (no 32-bit wrap)
    big = L.nvfp4_kv_quantize_v_tblocks_workspace_bytes(1, 1 << 24, 64, 16)
    assert big >= (1 << 20) * 32 * 256


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(P, "_lib", None)
    monkeypatch.setattr(P, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="HIP library missing"):
        P.lib()
