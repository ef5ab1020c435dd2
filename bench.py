#!/usr/bin/env python3
"""Benchmark of the NVFP4 4/6 KV-cache path on one MI355X.

Workload (one step): the full cache of 30 layers, K and V bf16 [24, 56320,
128] per layer (8 chunks of 8 frames x 880 tokens): every layer is
smooth-quantized chunk by chunk (nvfp4_kv_smooth_quantize), then the whole
cache is dequantized back to bf16 (nvfp4_dequantize, K with its means).
Inputs are resident in HBM before the timed region; they are drawn once on
the GPU from seeded generators (workloads/).  The cache (20.8 GB of bf16) is
far larger than the 256 MB Infinity Cache, so every step is a cold pass.

value = algorithmic bytes per step / time per step: every bf16 element read
once and written once, codes (0.5 B) and E4M3 scales (1/16 B) written once
and read once, plus the per-chunk means and tensor scales.

Prints one JSON line.

With --op attention it measures the consumer of the cache instead: softmax
attention of one chunk of queries (24 heads x 7040, bf16) over one layer's
whole NVFP4 cache (56320 keys), dequantizing on load (nvfp4_kv_attention);
value = 4 * heads * queries * keys * head_dim flops / time per call.

With --op stream it measures the streaming cache: one step is one new chunk
through 30 layers -- per layer, attention of the chunk's queries over the
cache's key set (global sink, shot sink, last 3 chunks: 26400 keys) on the
main stream, and the append of the chunk's K and V (quantized into a free
slot) on a second stream, overlapping the next layers' attention; the chunk
is committed at the end.  value = chunk tokens per second.

With --op gemm it measures the W4A4 GEMM: the [16384, 3072] activation
(1D blocks after the random Hadamard transform) times the [3072, 3072]
weight (2D tiles), both quantized on the GPU first; value = 2 M N K flops /
time per call.

With --op vt it measures V of one 8-chunk layer quantized with 16-token
blocks per channel (nvfp4_kv_quantize_v_tblocks); value = algorithmic bytes
(bf16 in, codes and scales out) / time per call.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
# MI355X VALU issue rate in wave-level instructions if every instruction took
# 4 cycles per SIMD (256 CUs x 4 SIMDs x 2.4 GHz / 4); used only to express
# the measured VALU load as a fraction (fp32 FMAs issue in about half that)
VALU_ISSUE_G = 256 * 4 * 2.4 / 4
# rocprofv3 HBM-traffic summaries of the KV quantize call, per kernel path
TRAFFIC_FILES = {"overlap": os.path.join(ROOT, "profiles", "kv_overlap_full_cache_traffic.md"),
                 "two-pass": os.path.join(ROOT, "profiles", "kv_two_pass_full_cache_traffic.md")}
# rocprofv3 VALU summary of the overlapped KV quantize kernel
VALU_FILE = os.path.join(ROOT, "profiles", "kv_valu_full_cache.md")


# the sources the KV quantize call's kernels are built from
KV_KERNEL_SOURCES = ("precision_kv_cache_amd/csrc/kv_quant.hip", "precision_kv_cache_amd/csrc/kv_overlap.hip",
                     "precision_kv_cache_amd/csrc/kv_overlap.hpp", "precision_kv_cache_amd/csrc/nvfp4_device.hpp",
                     "precision_kv_cache_amd/csrc/lowbit_device.hpp", "precision_kv_cache_amd/csrc/host_common.hpp",
                     "include/nvfp4kv.h")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in KV_KERNEL_SOURCES:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path):
    """HBM bytes per cache layer of a quantize call of a kernel path, from the
    committed rocprofv3 counter summary, or None once the kernel sources
    differ from the measured ones."""
    if path not in TRAFFIC_FILES:
        return None
    try:
        fields = dict(line.split(": ", 1) for line in open(TRAFFIC_FILES[path]).read().splitlines()
                      if line.startswith(("traffic_bytes_per_layer: ", "kernel_sources_sha256: ")))
    except OSError:
        return None
    if len(fields) < 2 or fields["kernel_sources_sha256"].strip() != kernel_sources_sha256():
        return None
    return int(fields["traffic_bytes_per_layer"])


def measured_valu(path):
    """(wave-level VALU instructions per cache layer, VALU busy %) of the
    overlapped kernel from the committed rocprofv3 counter summary, or None
    once the kernel sources differ from the measured ones (or for another
    path)."""
    if path != "overlap":
        return None
    keys = ("valu_instructions_per_layer: ", "valu_busy_pct: ", "kernel_sources_sha256: ")
    try:
        fields = dict(line.split(": ", 1) for line in open(VALU_FILE).read().splitlines() if line.startswith(keys))
    except OSError:
        return None
    if len(fields) < 3 or fields["kernel_sources_sha256"].strip() != kernel_sources_sha256():
        return None
    return int(fields["valu_instructions_per_layer"]), float(fields["valu_busy_pct"])
METRIC = "NVFP4 4/6 KV quantize GB/s (bytes in+out) and % of MI355X HBM peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; 200 calls for --op act / weight, which take ~0.05 ms each)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 3; 100 calls for --op act / weight, so the clocks settle)")
    ap.add_argument("--layers", type=int, default=30, help="cache layers (the workload has 30)")
    ap.add_argument("--mode", type=int, default=0, help="0 = 4/6, 1 = fixed 6, 2 = fixed 4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-pass", action="store_true", help="use the two-pass KV kernels (statistics, then quantize)")
    ap.add_argument("--schedule", choices=("whole", "layer"), default="whole",
                    help="whole: the cache head-major, one quantize call per step (the per-layer schedule is "
                         "reported beside it); layer: one quantize call per layer")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the oracle baseline")
    ap.add_argument("--bits", type=int, default=3, choices=(3, 2), help="element bits of --op lowbit")
    ap.add_argument("--op", choices=("kv", "lowbit", "chunk", "attention", "stream", "gemm", "vt", "act", "weight"),
                    default="kv",
                    help="kv: the quantize / dequantize path (default); lowbit: the same workload with 3-bit or 2-bit "
                         "elements (--bits); attention: attention over the NVFP4 cache; "
                         "stream: the streaming cache (attention + append per layer); gemm: the W4A4 GEMM; "
                         "vt: V blocked along tokens; act: the activation quantizer (RHT + 1D blocks); "
                         "weight: the weight quantizer (2D tiles)")
    ap.add_argument("--layout", choices=("all", "sink"), default="all",
                    help="attention key set: every cache key, or the sink layout (global sink, shot sink, window)")
    ap.add_argument("--attention-form", choices=("staged", "on-load"), default=None,
                    help="attention and stream: decode each key tile once per call into the workspace (staged, "
                         "the default; with key splits), or in every query block (on-load; --op stream then runs "
                         "its attention unsplit, without a workspace)")
    return ap.parse_args()


def kv_bytes(H, T, D, L, with_mean, bits=4):
    """Algorithmic bytes of one tensor's quantize (or dequantize): bf16 in,
    codes (bits per element) and scales out (or the reverse), plus tensor
    scales and means."""
    n = H * T * D
    nc = T // L
    b = 2 * n + n * bits // 8 + n // 16 + 4 * nc
    if with_mean:
        b += 4 * nc * H * D
    return b


def main():
    a = parse()
    short = a.op in ("act", "weight")  # calls of a few tens of microseconds
    if a.steps is None:
        a.steps = 200 if short else 20
    if a.warmup is None:
        a.warmup = 100 if short else 3
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this path runs on a single MI355X "
              f"(asked for --gpus {a.gpus}, WORLD_SIZE {world}); run it with --gpus 1.", flush=True)
        sys.exit(2)
    if a.op == "attention":
        attention_bench(a)
        return
    if a.op == "stream":
        stream_bench(a)
        return
    if a.op == "gemm":
        gemm_bench(a)
        return
    if a.op == "vt":
        vt_bench(a)
        return
    if a.op in ("act", "weight"):
        act_weight_bench(a)
        return
    if a.op == "chunk":
        chunk_bench(a)
        return
    kv_bench(a, 4 if a.op == "kv" else a.bits)


LOWBIT_METRIC = "{bits}-bit KV quantize GB/s (bytes in+out) and % of MI355X HBM peak"


def kv_roofline(dominant, kv_path, bits, qname, dname, ach_gbps, q_ms, qbytes, nblocks, layers):
    """The dominant call's roofline against HBM; a call covers `layers` cache
    layers (K and V), qbytes and nblocks are per call.  Every KV call is
    memory-bound: a build of the overlapped quantize kernel whose block
    encode is replaced by a trivial one runs in the same time, and the
    dequantize streams its output at the write rate.  For the overlapped
    4-bit kernel the line also carries its measured VALU load (wave-level
    instructions and busy share, from the committed counter summary) under
    "valu", and its HBM traffic under "traffic"."""
    tr = measured_traffic(kv_path) if dominant == "quantize" and bits == 4 else None
    what = f"{layers} layers" if layers > 1 else "one layer"
    kernel = f"{qname} ({what}, K and V)" if dominant == "quantize" else f"{dname} ({what}, K and V)"
    r = {"bound": "hbm", "kernel": kernel, "achieved": round(ach_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(ach_gbps / HBM_PEAK_GBPS, 4), "traffic": tr * layers if tr else None,
         "bytes_per_launch": qbytes}
    valu = measured_valu(kv_path) if dominant == "quantize" and bits == 4 else None
    if valu:
        n = valu[0] * layers
        rate = n / (q_ms * 1e-3) / 1e9
        r["valu"] = {"instructions_per_launch": n, "instructions_per_block": round(n / nblocks * 64, 1),
                     "busy_pct": valu[1], "G_instructions_per_s": round(rate, 1),
                     "frac_of_4_cycle_issue": round(rate / VALU_ISSUE_G, 4)}
    return r


def kv_bench(a, bits):
    """The full-cache workload: every layer smooth-quantized, then the whole
    cache dequantized; NVFP4 4/6 (bits = 4, the headline) or the 3-bit / 2-bit
    cache (the same readings with fewer element bits).

    Two schedules of the same work.  "whole" (the default) holds the cache
    head-major, K and V each one [H, layers * T, D] tensor in which layer l
    is tokens l * T .. (l + 1) * T - 1, and makes one quantize call and two
    dequantize calls per step: every (layer, chunk) is still its own chunk,
    with its own mean and tensor scales, and the bytes equal those of the
    per-layer calls.  "layer" makes one quantize call and two dequantize
    calls per layer on layer-major tensors.  The default line times "whole"
    and reports "layer" beside it."""
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()  # fail loudly without the HIP library
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = W.CACHE_LAYER
    H, T, D, L = s.H, s.T, s.D, s.chunk_len
    nlayers = a.layers
    nc = T // L

    t0 = time.time()
    ks, vs = [], []
    for l in range(nlayers):
        k, v = W.gaussian_kv(s, W.cache_layer_seed(l), device=dev)
        ks.append(k)
        vs.append(v)
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    def outputs(tokens, chunks):
        return {"k_codes": torch.empty(H, tokens, D * bits // 8, dtype=torch.uint8, device=dev),
                "v_codes": torch.empty(H, tokens, D * bits // 8, dtype=torch.uint8, device=dev),
                "k_scales": torch.empty(H, tokens, D // 16, dtype=torch.uint8, device=dev),
                "v_scales": torch.empty(H, tokens, D // 16, dtype=torch.uint8, device=dev),
                "k_tensor_scale": torch.empty(chunks, dtype=torch.float32, device=dev),
                "v_tensor_scale": torch.empty(chunks, dtype=torch.float32, device=dev),
                "k_mean": torch.empty(chunks, H, D, dtype=torch.float32, device=dev)}

    # dequantized output, shared by the schedules (each overwrites all of it)
    deq_buf = [torch.empty(nlayers * H * T * D, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream()

    def quant_call(k, v, o, ws):
        if bits == 4:
            P.nvfp4_kv_smooth_quantize(k, v, L, a.mode, out=o, workspace=ws, stream=stream, two_pass=a.two_pass)
        else:
            P.nvfp4_kv_smooth_quantize_lowbit(k, v, L, bits, a.mode, out=o, workspace=ws, stream=stream,
                                              two_pass=a.two_pass)

    def dequant_call(o, dk, dv):
        if bits == 4:
            P.nvfp4_dequantize(o["k_codes"], o["k_scales"], o["k_tensor_scale"], o["k_mean"], L, out=dk,
                               stream=stream)
            P.nvfp4_dequantize(o["v_codes"], o["v_scales"], o["v_tensor_scale"], None, L, out=dv, stream=stream)
        else:
            P.nvfp4_dequantize_lowbit(o["k_codes"], o["k_scales"], o["k_tensor_scale"], o["k_mean"], L, bits,
                                      out=dk, stream=stream)
            P.nvfp4_dequantize_lowbit(o["v_codes"], o["v_scales"], o["v_tensor_scale"], None, L, bits, out=dv,
                                      stream=stream)

    def schedule(kind):
        """(quantize calls, dequantize calls, outputs for the parity sample,
        dequantized (K, V) for it, workspace) of one step."""
        if kind == "whole":
            K = torch.empty(H, nlayers * T, D, dtype=torch.bfloat16, device=dev)
            V = torch.empty_like(K)
            for l in range(nlayers):
                K[:, l * T:(l + 1) * T] = ks[l]
                V[:, l * T:(l + 1) * T] = vs[l]
            o = outputs(nlayers * T, nlayers * nc)
            dk = deq_buf[0].view(H, nlayers * T, D)
            dv = deq_buf[1].view(H, nlayers * T, D)
            ws = torch.zeros(P.nvfp4_kv_workspace_bytes(H, nlayers * T, D, L), dtype=torch.uint8, device=dev)
            return ([lambda: quant_call(K, V, o, ws)], [lambda: dequant_call(o, dk, dv)], o, (dk, dv), ws)
        os_ = [outputs(T, nc) for _ in range(nlayers)]
        dks = [deq_buf[0][l * H * T * D:(l + 1) * H * T * D].view(H, T, D) for l in range(nlayers)]
        dvs = [deq_buf[1][l * H * T * D:(l + 1) * H * T * D].view(H, T, D) for l in range(nlayers)]
        ws = torch.zeros(P.nvfp4_kv_workspace_bytes(H, T, D, L), dtype=torch.uint8, device=dev)
        return ([(lambda l=l: quant_call(ks[l], vs[l], os_[l], ws)) for l in range(nlayers)],
                [(lambda l=l: dequant_call(os_[l], dks[l], dvs[l])) for l in range(nlayers)], os_[0],
                (dks[0], dvs[0]), ws)

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run(kind, warmup, steps):
        """Times `steps` steps after `warmup` untimed ones: one event pair
        around the whole run, plus an event pair around every library call of
        the last step (same stream) for the per-call durations."""
        qc, dc, o, dq, ws = schedule(kind)

        def step(qev=None, dev_=None):
            for i, f in enumerate(qc):
                if qev is not None:
                    qev[i][0].record(stream)
                f()
                if qev is not None:
                    qev[i][1].record(stream)
            for i, f in enumerate(dc):
                if dev_ is not None:
                    dev_[i][0].record(stream)
                f()
                if dev_ is not None:
                    dev_[i][1].record(stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        qev = [(E(), E()) for _ in qc]
        dev_ = [(E(), E()) for _ in dc]
        sev = [E() for _ in range(steps + 1)]  # step boundaries, for the median and minimum step
        start, stop = E(), E()
        start.record(stream)
        sev[0].record(stream)
        for i in range(steps):
            last = i == steps - 1
            step(qev if last else None, dev_ if last else None)
            sev[i + 1].record(stream)
        stop.record(stream)
        torch.cuda.synchronize()
        # every quantize call of the run shares ws: its sticky error word is
        # non-zero if any of them had a wait time out
        err = P.kv_error_word(ws)
        if err:
            print(f"bench.py: a quantize call's bounded wait timed out (error word {err}); "
                  "its outputs are invalid, so no result is reported", flush=True)
            sys.exit(3)
        per = sorted(sev[i].elapsed_time(sev[i + 1]) for i in range(steps))
        return {"ms_step": start.elapsed_time(stop) / steps,
                "step_ms": {"median": round(per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] +
                                                                                   per[steps // 2]), 4),
                            "min": round(per[0], 4), "max": round(per[-1], 4)},
                "q_call_ms": sum(e0.elapsed_time(e1) for e0, e1 in qev) / len(qev),
                "d_call_ms": sum(e0.elapsed_time(e1) for e0, e1 in dev_) / len(dev_),
                "calls_per_step": len(qc), "out": o, "deq": dq, "err": err}

    main_kind = a.schedule
    r = run(main_kind, a.warmup, a.steps)
    ms_step, wait_errors = r["ms_step"], r["err"]
    layers_per_call = nlayers if main_kind == "whole" else 1
    q_ms = r["q_call_ms"] / layers_per_call   # one layer's share of a quantize call (K and V)
    d_ms = r["d_call_ms"] / layers_per_call   # one layer's share of the dequantize calls (K and V)

    qbytes_layer = kv_bytes(H, T, D, L, True, bits) + kv_bytes(H, T, D, L, False, bits)
    dbytes_layer = qbytes_layer
    step_bytes = nlayers * (qbytes_layer + dbytes_layer)
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    q_gbps = qbytes_layer / (q_ms * 1e-3) / 1e9
    d_gbps = dbytes_layer / (d_ms * 1e-3) / 1e9
    check_out, check_deq = r["out"], r["deq"]

    # 4/6 choice histogram on one layer (outside the timed region)
    if bits == 4:
        o = P.nvfp4_kv_smooth_quantize(ks[0], vs[0], L, a.mode, choice_counts=True)
    else:
        o = P.nvfp4_kv_smooth_quantize_lowbit(ks[0], vs[0], L, bits, a.mode, choice_counts=True)
    torch.cuda.synchronize()
    cc = o["choice_counts"].cpu().tolist()

    # device copy bandwidth of a 4 GiB buffer, for context
    src = torch.empty(1 << 31, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = E(), E()
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    kv_path = "two-pass" if a.two_pass or D != 128 else "overlap"
    dominant = "quantize" if q_ms >= d_ms else "dequantize"
    ach = q_gbps if dominant == "quantize" else d_gbps
    if bits == 4:
        choice = {"K": {"kept6": cc[0][0], "kept4": cc[0][1]}, "V": {"kept6": cc[1][0], "kept4": cc[1][1]}}
        qname, dname, what = "nvfp4_kv_smooth_quantize", "nvfp4_dequantize", "4/6 smooth-quantize"
    else:
        choice = {"K": {"kept_ca": cc[0][0], "kept_cb": cc[0][1]}, "V": {"kept_ca": cc[1][0], "kept_cb": cc[1][1]}}
        qname, dname = "nvfp4_kv_smooth_quantize_lowbit", "nvfp4_dequantize_lowbit"
        what = f"{bits}-bit smooth-quantize (two-candidate block scale)"
    result = {
        "metric": METRIC if bits == 4 else LOWBIT_METRIC.format(bits=bits),
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"full 8-chunk KV cache: {nlayers} layers x K,V bf16 [24 heads, 56320 tokens, 128], "
                        f"chunks of 7040 tokens; {what} every layer, then dequantize the cache"
                        + ("; the cache held head-major, K and V each one [24, layers x 56320, 128] tensor, "
                           "one quantize call and two dequantize calls per step" if main_kind == "whole" else
                           "; one quantize call and two dequantize calls per layer"),
            "layers": nlayers, "heads": H, "tokens": T, "head_dim": D, "chunk_len": L, "element_bits": bits,
            "mode": ["4over6", "fixed6", "fixed4"][a.mode], "bytes_per_step": step_bytes,
            "kv_path": kv_path, "schedule": main_kind,
        },
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "quantize_GBps": round(q_gbps, 1),
        "dequantize_GBps": round(d_gbps, 1),
        "quantize_ms_per_layer": round(q_ms, 4),
        "dequantize_ms_per_layer": round(d_ms, 4),
        "quantize_call_ms": round(r["q_call_ms"], 4),
        "dequantize_call_ms": round(r["d_call_ms"], 4),
        "choice_counts_layer0": choice,
        "d2d_copy_GBps": round(copy_gbps, 1),
        "roofline": kv_roofline(dominant, kv_path, bits, qname, dname, ach, r["q_call_ms"],
                                layers_per_call * qbytes_layer, layers_per_call * 2 * H * T * (D // 16),
                                layers_per_call),
        "input_generation_s": round(gen_s, 2),
        "quantize_wait_timeouts": wait_errors,
    }
    if not a.no_cpu_baseline:
        # the oracle's leg: its rate on the host, and the last timed step's
        # outputs of layer 0 chunk 0 compared with it bit for bit
        result["cpu_baseline"] = cpu_baseline(ks, vs, L, a.mode, a.cpu_seconds, check=(check_out, check_deq),
                                              bits=bits)
        if not result["cpu_baseline"]["parity_check"]["bit_exact"]:
            print("bench.py: the sampled chunk differs from the oracle: " + json.dumps(result["cpu_baseline"]),
                  flush=True)
            sys.exit(3)
    del r, check_out, check_deq
    torch.cuda.empty_cache()
    if main_kind == "whole":
        # the same work in per-layer calls, for comparison
        rl = run("layer", 1, 3)
        result["per_layer_schedule"] = {
            "value": round(step_bytes / (rl["ms_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
            "ms_per_step": round(rl["ms_step"], 4), "steps": 3, "warmup": 1,
            "quantize_call_ms": round(rl["q_call_ms"], 4), "dequantize_call_ms": round(rl["d_call_ms"], 4),
            "calls_per_step": 3 * nlayers}
        del rl
        torch.cuda.empty_cache()
    del deq_buf
    torch.cuda.empty_cache()
    if bits == 4:
        result["one_chunk_configs"] = one_chunk_timing(P, W, a.mode, stream, q_ms)
        result["act_weight"] = act_weight_timing(P, W, a.mode, stream)
        result["heavy_tail_report"] = heavy_tail_report(P, W)
    print(json.dumps(result), flush=True)


def act_weight_timing(P, W, mode, stream, reps=200, warm=100):
    """The GEMM-operand quantizers on their workload: activation [16384, 3072]
    with the 16-point RHT and 1D blocks, weight [3072, 3072] with 16x16
    tiles.  Several input copies are rotated (at least 400 MB in all) so no
    call finds its input in the 256 MB Infinity Cache."""
    import torch

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    x, sign_mask, w = W.act_weight(device="cuda")
    xs = [x] + [x.clone() for _ in range(3)]
    wsz = [w] + [w.clone() for _ in range(21)]
    rows, cols = x.shape
    n = x.numel()
    xo = P.nvfp4_quantize_1d(x, mode, hadamard=True, sign_mask=sign_mask)
    wo = P.nvfp4_quantize_2d(w, mode)
    xws = torch.empty(int(P.lib().nvfp4_quantize_1d_workspace_bytes(rows, cols)) or 1, dtype=torch.uint8,
                      device="cuda")
    wws = torch.empty(int(P.lib().nvfp4_quantize_2d_workspace_bytes(*w.shape)) or 1, dtype=torch.uint8,
                      device="cuda")
    res = {}
    for name, fn, nbytes in (
            ("act_rht_quantize_1d", lambda i: P.nvfp4_quantize_1d(xs[i % len(xs)], mode, hadamard=True,
                                                                  sign_mask=sign_mask, out=xo, workspace=xws,
                                                                  stream=stream),
             2 * n + n // 2 + n // 16 + 4),
            ("weight_quantize_2d", lambda i: P.nvfp4_quantize_2d(wsz[i % len(wsz)], mode, out=wo, workspace=wws,
                                                                 stream=stream),
             2 * w.numel() + w.numel() // 2 + w.numel() // 256 + 4)):
        for i in range(warm):  # calls of tens of microseconds: let the clocks settle first
            fn(i)
        e0, e1 = E(), E()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "pct_of_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                     "bytes": nbytes}
    res["shapes"] = {"activation": [rows, cols], "weight": list(w.shape)}
    return res


def one_chunk_timing(P, W, mode, stream, layer_q_ms, sets=8, reps=6):
    """The one-chunk calls, as the streaming cache makes them for every
    generated chunk: K, V bf16 [24, 7040, 128], one chunk.  Two inputs: the
    Gaussian chunk and the heavy-tailed chunk (Student-t(3) with per-channel
    scales).  `sets` copies of inputs and outputs (8 x 86.5 MB of input) are
    rotated, so no call finds its input in the 256 MB Infinity Cache.  Each
    call is timed alone, back to back on one stream (launch gaps included),
    as the average over reps x sets calls; quantize and dequantize apart."""
    import torch

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    s = W.ONE_CHUNK
    H, T, D, L = s.H, s.T, s.D, s.chunk_len
    qbytes = kv_bytes(H, T, D, L, True) + kv_bytes(H, T, D, L, False)
    ws = torch.zeros(P.nvfp4_kv_workspace_bytes(H, T, D, L), dtype=torch.uint8, device="cuda")
    res = {"shape": [H, T, D], "chunk_len": L, "buffer_sets": sets, "calls_timed": reps * sets,
           "bytes_per_call": qbytes}
    for name, gen, seed in (("one_chunk", W.gaussian_kv, W.SEED_ONE_CHUNK),
                            ("heavy_tail", W.heavy_tail_kv, W.SEED_HEAVY)):
        k, v = gen(s, seed, device="cuda")
        ins = [(k, v)] + [(k.clone(), v.clone()) for _ in range(sets - 1)]
        outs = [P.nvfp4_kv_smooth_quantize(kk, vv, L, mode) for kk, vv in ins]
        deq = [(torch.empty_like(k), torch.empty_like(v)) for _ in range(sets)]

        def quant(i):
            kk, vv = ins[i]
            P.nvfp4_kv_smooth_quantize(kk, vv, L, mode, out=outs[i], workspace=ws, stream=stream)

        def dequant(i):
            o = outs[i]
            P.nvfp4_dequantize(o["k_codes"], o["k_scales"], o["k_tensor_scale"], o["k_mean"], L, out=deq[i][0],
                               stream=stream)
            P.nvfp4_dequantize(o["v_codes"], o["v_scales"], o["v_tensor_scale"], None, L, out=deq[i][1],
                               stream=stream)

        entry = {}
        for what, fn in (("quantize", quant), ("dequantize", dequant)):
            for i in range(sets):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = E(), E()
            e0.record(stream)
            for _ in range(reps):
                for i in range(sets):
                    fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / (reps * sets)
            gbps = qbytes / (ms * 1e-3) / 1e9
            entry[what] = {"call_ms": round(ms, 4), "GBps": round(gbps, 1),
                           "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2)}
        both = entry["quantize"]["call_ms"] + entry["dequantize"]["call_ms"]
        entry["GBps"] = round(2 * qbytes / (both * 1e-3) / 1e9, 1)
        entry["pct_of_hbm_peak"] = round(100 * entry["GBps"] / HBM_PEAK_GBPS, 2)
        # the same chunk's share of the full-layer quantize call (8 chunks per call)
        entry["quantize_vs_layer_call_per_chunk"] = (
            round(entry["quantize"]["call_ms"] / (layer_q_ms / 8), 3) if layer_q_ms else None)
        res[name] = entry
        del ins, outs, deq
    err = P.kv_error_word(ws)
    res["quantize_wait_timeouts"] = err
    if err:
        print(f"bench.py: a one-chunk quantize call's bounded wait timed out (error word {err})", flush=True)
        sys.exit(3)
    torch.cuda.empty_cache()
    return res


def chunk_bench(a):
    """The one-chunk configurations alone: the Gaussian chunk and the
    heavy-tailed chunk, quantize and dequantize calls over rotating buffers."""
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    r = one_chunk_timing(P, W, a.mode, stream, None, reps=max(1, a.steps))
    g = r["one_chunk"]
    result = {
        "metric": METRIC, "value": g["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(g["quantize"]["call_ms"] + g["dequantize"]["call_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "one chunk: K,V bf16 [24 heads, 7040 tokens, 128], smooth-quantize then dequantize, "
                               f"{r['buffer_sets']} rotating buffer sets", "mode": ["4over6", "fixed6", "fixed4"][a.mode]},
        "pct_of_hbm_peak": g["pct_of_hbm_peak"],
        "one_chunk_configs": r,
    }
    print(json.dumps(result), flush=True)


def heavy_tail_report(P, W):
    """4/6 against fixed-6 on the heavy-tailed chunk (Student-t(3) with per-
    channel scales, [24, 7040, 128]): reconstruction MSE in fp64 of the
    dequantized bf16 against the input, and the share of blocks keeping the
    +-4 candidate by decile of the block's largest magnitude.  A block's
    choice is read off its codes: the block maximum encodes to 4 (code 6)
    under +-4 and to 6 (code 7) under +-6; blocks whose largest code is
    neither (tiny E4M3 scales) are counted apart."""
    import torch

    s = W.ONE_CHUNK
    k, v = W.heavy_tail_kv(s, W.SEED_HEAVY, device="cuda")
    L = s.chunk_len
    rep = {"shape": [s.H, s.T, s.D], "chunk_len": L}
    mags = None
    for mode, name in ((P.MODE_4OVER6, "4over6"), (P.MODE_FIXED6, "fixed6")):
        o = P.nvfp4_kv_smooth_quantize(k, v, L, mode, choice_counts=True)
        dk = P.nvfp4_dequantize(o["k_codes"], o["k_scales"], o["k_tensor_scale"], o["k_mean"], L)
        dv = P.nvfp4_dequantize(o["v_codes"], o["v_scales"], o["v_tensor_scale"], None, L)
        entry = {}
        for t, x, d in (("K", k, dk), ("V", v, dv)):
            x64, d64 = x.double(), d.double()
            mse = torch.mean((d64 - x64) ** 2).item()
            entry[t] = {"mse": mse, "rel_mse": mse / torch.mean(x64 ** 2).item()}
        cc = o["choice_counts"].cpu().tolist()
        entry["kept4_share"] = {"K": cc[0][1] / max(1, sum(cc[0])), "V": cc[1][1] / max(1, sum(cc[1]))}
        if mode == P.MODE_4OVER6:
            lut = torch.tensor([0, 1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 3, 4, 5, 6, 7], dtype=torch.uint8, device="cuda")
            deciles = {}
            for t, x, codes, mean in (("K", k, o["k_codes"], o["k_mean"]), ("V", v, o["v_codes"], None)):
                xf = x.float()
                if mean is not None:  # smoothed K: x' = K - mean of its chunk
                    xf = xf - mean.permute(1, 0, 2).repeat_interleave(L, dim=1)
                amax = xf.abs().reshape(-1, 16).amax(1)
                q = codes.reshape(-1, 8)
                top = torch.maximum(lut[(q & 15).long()], lut[(q >> 4).long()]).amax(1)
                edges = torch.quantile(amax[amax > 0].float()[::97], torch.linspace(0, 1, 11, device="cuda"))
                bins = torch.bucketize(amax, edges[1:-1])
                rows = []
                for b in range(10):
                    m = bins == b
                    nb = int(m.sum())
                    rows.append({"blocks": nb, "kept4": int(((top == 6) & m).sum()),
                                 "kept6": int(((top == 7) & m).sum()),
                                 "other": int(((top != 6) & (top != 7) & m).sum())})
                deciles[t] = rows
            entry["by_block_max_decile"] = deciles
        rep[name] = entry
    rep["mse_ratio_4over6_to_fixed6"] = {t: rep["4over6"][t]["mse"] / rep["fixed6"][t]["mse"] for t in ("K", "V")}
    return rep


BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
ATT_METRIC = "NVFP4-cache attention TFLOP/s (4 * heads * queries * keys * head_dim) and % of MI355X bf16 MFMA peak"


def attention_bench(a):
    """Attention over one layer's NVFP4 cache: the cache is built on the GPU
    by nvfp4_kv_smooth_quantize from the seeded layer-0 K and V, the queries
    are one chunk of 7040 tokens.  One step = one nvfp4_kv_attention call."""
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = W.CACHE_LAYER
    H, T, D, L = s.H, s.T, s.D, s.chunk_len
    Tq = W.ATTN_QUERIES
    t0 = time.time()
    k, v = W.gaussian_kv(s, W.cache_layer_seed(0), device=dev)
    cache = P.nvfp4_kv_smooth_quantize(k, v, L)
    q = W.queries(H, Tq, D, W.SEED_ATTN, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    ranges = [(0, T)] if a.layout == "all" else W.sink_ranges(s.n_chunks)
    nk = sum(n for _, n in ranges)
    out = torch.empty_like(q)
    # workspace that lets the call split each query block's keys over several
    # workgroups (and merge them) where that fills the CUs better and, for the
    # staged form, holds every key tile decoded once per call
    staged = a.attention_form in (None, "staged")
    nws = (P.nvfp4_kv_attention_staged_workspace_bytes(H, Tq, D, H, T, L, ranges) if staged
           else P.nvfp4_kv_attention_workspace_bytes(H, Tq, D))
    aws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        P.nvfp4_kv_attention(q, cache, L, ranges, out=out, workspace=aws, stream=stream)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E()) for _ in range(a.steps)]
    start, stop = E(), E()
    start.record(stream)
    for i in range(a.steps):
        ev[i][0].record(stream)
        P.nvfp4_kv_attention(q, cache, L, ranges, out=out, workspace=aws, stream=stream)
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / a.steps
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / a.steps
    flops = 4.0 * H * Tq * nk * D
    tflops = flops / (ms_step * 1e-3) / 1e12
    call_tflops = flops / (call_ms * 1e-3) / 1e12
    cache_bytes = 2 * (H * nk * D // 2 + H * nk * D // 16)  # K and V codes + scales of the listed keys
    result = {
        "metric": ATT_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"attention of one chunk of queries [24 heads, 7040, 128] over one layer's NVFP4 cache "
                        f"({'all 56320 keys' if a.layout == 'all' else 'sink layout'}, chunks of 7040), "
                        + ("each key tile decoded once per call" if staged else "dequantized on load"),
            "form": "staged" if staged else "on-load", "workspace_bytes": nws,
            "heads": H, "queries": Tq, "keys": nk, "head_dim": D, "chunk_len": L, "key_ranges": ranges,
        },
        "pct_of_mfma_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
        "cache_bytes_read": cache_bytes,
        "roofline": {
            "bound": "mfma",
            "kernel": "nvfp4_kv_attention (one call" + (": staging and attention kernels)" if staged else ")"),
            "achieved": round(call_tflops, 1),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(call_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": flops,
        },
        "input_generation_s": round(gen_s, 2),
    }
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = attention_cpu_baseline(k, v, q, L, ranges, a.cpu_seconds)
    print(json.dumps(result), flush=True)


STREAM_METRIC = ("streaming NVFP4 cache: chunk tokens per second (30 layers x [attention over global sink + shot "
                 "sink + 3-chunk window, append of the chunk's K and V])")


def stream_bench(a):
    """One step = one chunk through the layers: attention(l) on the main
    stream, append(l) on a second stream after it (the pending slot is not in
    the key set, so the append may overlap the next layers' attention), then
    the commit.  The cache (8 slots per layer) is filled with 10 chunks and a
    prompt switch first, so slots are reused and the shot sink is off chunk 0."""
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = W.CACHE_LAYER
    H, D, L, F = s.H, s.D, s.chunk_len, W.TOKENS_PER_FRAME
    nl = a.layers
    sink, shot, window, cap = 3, 3, 3, 8
    t0 = time.time()
    cache = P.KVCache(nl, H, D, L, cap, F, sink, shot, window, device=dev)
    # per-layer K and V of one chunk (reused by every appended chunk)
    kv = [W.gaussian_kv(W.KVShape(H, L, D, L), 200000 + l, device=dev) for l in range(nl)]
    q = W.queries(H, L, D, W.SEED_ATTN, device=dev)
    out = torch.empty_like(q)
    ws = [torch.zeros(P.nvfp4_kv_workspace_bytes(H, L, D, L), dtype=torch.uint8, device=dev) for _ in range(2)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for c in range(10):
        cache.begin_chunk(new_shot=(c == 5))
        for l in range(nl):
            cache.append(l, kv[l][0], kv[l][1], workspace=ws[0], stream=main)
        cache.end_chunk()
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    ranges = cache.key_ranges()
    nk = sum(n for _, n in ranges)
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    att_staged = a.attention_form in (None, "staged")
    aws = False
    if att_staged:
        aws = torch.empty(P.nvfp4_kv_attention_staged_workspace_bytes(H, L, D, H, cap * L, L, ranges),
                          dtype=torch.uint8, device=dev)

    def step(att_ev=None, app_ev=None):
        cache.begin_chunk()
        done = [E() for _ in range(nl)]
        for l in range(nl):
            if att_ev is not None:
                att_ev[l][0].record(main)
            # staged, with key splits (the workspace); the on-load form runs
            # unsplit, since there the splits took from the appends on the side
            # stream the CUs that attention's last round leaves idle
            cache.attention(l, q, out=out, workspace=aws, stream=main)
            if att_ev is not None:
                att_ev[l][1].record(main)
            done[l].record(main)  # the layer's K and V would come out of this layer's forward
            side.wait_event(done[l])
            if app_ev is not None:
                app_ev[l][0].record(side)
            cache.append(l, kv[l][0], kv[l][1], workspace=ws[1], stream=side)
            if app_ev is not None:
                app_ev[l][1].record(side)
        main.wait_stream(side)
        cache.end_chunk()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # the appends of one chunk alone (no attention beside them), for the
    # share of their time that the overlap hides
    cache.begin_chunk()
    a0, a1 = E(), E()
    a0.record(main)
    for l in range(nl):
        cache.append(l, kv[l][0], kv[l][1], workspace=ws[0], stream=main)
    a1.record(main)
    torch.cuda.synchronize()
    cache.end_chunk()
    app_alone_ms = a0.elapsed_time(a1) / nl
    att_ev = [(E(), E()) for _ in range(nl)]
    app_ev = [(E(), E()) for _ in range(nl)]
    start, stop = E(), E()
    start.record(main)
    for i in range(a.steps):
        last = i == a.steps - 1
        step(att_ev if last else None, app_ev if last else None)
    stop.record(main)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / a.steps
    att_ms = sum(e0.elapsed_time(e1) for e0, e1 in att_ev) / nl
    app_ms = sum(e0.elapsed_time(e1) for e0, e1 in app_ev) / nl  # beside attention, waits for CUs included
    # the sticky error words of both append workspaces: non-zero if any append
    # (warm-up, alone or beside attention) had a wait time out
    wait_errors = P.kv_error_word(ws[0]) | P.kv_error_word(ws[1])
    if wait_errors:
        print(f"bench.py: an append's bounded wait timed out (error word {wait_errors}); no result is reported",
              flush=True)
        sys.exit(3)
    flops = 4.0 * H * L * nk * D
    att_tflops = flops / (att_ms * 1e-3) / 1e12
    result = {
        "metric": STREAM_METRIC,
        "value": round(L / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"streaming cache, one chunk (24 heads x 7040 tokens x 128) per step through {nl} layers: "
                        f"attention over global sink {sink} frames + shot sink {shot} frames + window {window} "
                        f"chunks ({nk} keys), append of the chunk into an 8-slot cache",
            "layers": nl, "heads": H, "chunk_len": L, "frame_tokens": F, "keys": nk, "key_ranges": ranges,
            "slots": cap,
            "attention_form": "staged, key splits" if att_staged else "on-load, unsplit",
        },
        "attention_call_ms": round(att_ms, 4),
        "append_call_ms_alone": round(app_alone_ms, 4),
        "append_call_ms_beside_attention": round(app_ms, 4),
        "serial_sum_ms": round(nl * (att_ms + app_alone_ms), 3),
        "append_wait_timeouts": wait_errors,
        "append_hidden_frac": round(max(0.0, min(1.0, (nl * (att_ms + app_alone_ms) - ms_step) /
                                                 (nl * app_alone_ms))), 3),
        "roofline": {
            "bound": "mfma",
            "kernel": "nvfp4_kv_cache_attention (one layer)",
            "achieved": round(att_tflops, 1),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": flops,
        },
        "input_generation_s": round(gen_s, 2),
    }
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = stream_cpu_baseline(kv[0], q, cache, ranges, nl, a.cpu_seconds)
    print(json.dumps(result), flush=True)


GEMM_METRIC = "W4A4 NVFP4 GEMM TFLOP/s (2 M N K) and % of MI355X fp16/bf16 MFMA peak"


def gemm_bench(a):
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    x, sm, wt = W.act_weight(device=dev)
    act = P.nvfp4_quantize_1d(x, a.mode, hadamard=True, sign_mask=sm)
    wq = P.nvfp4_quantize_2d(wt, a.mode)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    M, K = x.shape
    N = wt.shape[0]
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(a.warmup):
        P.nvfp4_gemm_w4a4(act, wq, True, out=out, stream=stream)
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev = [(E(), E()) for _ in range(a.steps)]
    start, stop = E(), E()
    start.record(stream)
    for i in range(a.steps):
        ev[i][0].record(stream)
        P.nvfp4_gemm_w4a4(act, wq, True, out=out, stream=stream)
        ev[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / a.steps
    call_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / a.steps
    flops = 2.0 * M * N * K
    tflops = flops / (ms_step * 1e-3) / 1e12
    call_tflops = flops / (call_ms * 1e-3) / 1e12
    result = {
        "metric": GEMM_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "W4A4 GEMM: activation [16384, 3072] (NVFP4 1D blocks after the RHT) x weight "
                        "[3072, 3072] (NVFP4 2D 16x16 tiles), out bf16 [16384, 3072]",
            "M": M, "N": N, "K": K, "mode": ["4over6", "fixed6", "fixed4"][a.mode],
        },
        "pct_of_mfma_peak": round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2),
        "operand_bytes": M * K // 2 + M * K // 16 + N * K // 2 + (N // 16) * (K // 16) + 8,
        "roofline": {
            "bound": "mfma",
            "kernel": "nvfp4_gemm_w4a4 (one call)",
            "achieved": round(call_tflops, 1),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(call_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": flops,
        },
        "input_generation_s": round(gen_s, 2),
    }
    if not a.no_cpu_baseline:
        import oracle as O
        nt = O.default_threads()
        ac, as_, ag = (act[k].cpu().numpy() for k in ("codes", "scales", "tensor_scale"))
        wparts = tuple(wq[k].cpu().numpy() for k in ("codes", "scales", "tensor_scale"))
        rows, t_cpu, done = 0, 0.0, 0
        rng = __import__("numpy").random.default_rng(0)
        while t_cpu < a.cpu_seconds:
            r = rng.integers(0, M, nt)
            t1 = time.perf_counter()
            O.gemm_w4a4((ac[r], as_[r], ag), wparts, True, nthreads=nt)
            t_cpu += time.perf_counter() - t1
            done += nt
        result["cpu_baseline"] = {"value": round(2.0 * done * N * K / t_cpu / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": nt, **host_cores(), "kind": "oracle",
                                  "sample": f"{done} random rows of the activation x the whole weight (fp64 over "
                                            f"the exactly decoded operands)", "seconds": round(t_cpu, 2)}
    print(json.dumps(result), flush=True)


AW_METRIC = {
    "act": "activation quantize (16-point RHT + 1D NVFP4 4/6 blocks): GB/s (bytes in + out) and % of MI355X HBM peak",
    "weight": "weight quantize (2D 16x16 NVFP4 4/6 tiles): GB/s (bytes in + out) and % of MI355X HBM peak",
}


def act_weight_bench(a):
    """The GEMM-operand quantizers on their workload: the activation
    [16384, 3072] with the RHT and 1D blocks (--op act), or the weight
    [3072, 3072] with 2D tiles (--op weight).  Each step quantizes the next of
    several seeded input copies (at least 400 MB in all), so no call finds its
    input in the 256 MB Infinity Cache."""
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    x, sign_mask, w = W.act_weight(device=dev)
    act = a.op == "act"
    src = x if act else w
    del x, w
    copies = [src] + [src.clone() for _ in range((4 if act else 22) - 1)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    rows, cols = src.shape
    n = src.numel()
    ws = torch.empty(int((P.lib().nvfp4_quantize_1d_workspace_bytes if act else
                          P.lib().nvfp4_quantize_2d_workspace_bytes)(rows, cols)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    if act:
        out = P.nvfp4_quantize_1d(src, a.mode, hadamard=True, sign_mask=sign_mask)
        call = lambda i: P.nvfp4_quantize_1d(copies[i % len(copies)], a.mode, hadamard=True,  # noqa: E731
                                             sign_mask=sign_mask, out=out, workspace=ws, stream=stream)
        nbytes = 2 * n + n // 2 + n // 16 + 4
    else:
        out = P.nvfp4_quantize_2d(src, a.mode)
        call = lambda i: P.nvfp4_quantize_2d(copies[i % len(copies)], a.mode, out=out, workspace=ws,  # noqa: E731
                                             stream=stream)
        nbytes = 2 * n + n // 2 + n // 256 + 4
    for i in range(a.warmup):
        call(i)
    torch.cuda.synchronize()
    # the calls run back to back on one stream (each is GPU-bound: a HIP
    # graph replay of the same steps measured within 3 %); one event pair
    # around all of them, none between calls, so the host never paces them
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    start, stop = E(), E()
    start.record(stream)
    for i in range(a.steps):
        call(a.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / a.steps
    call_ms = ms_step
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    call_gbps = gbps
    kind = "activation [16384, 3072] with the 16-point RHT, 1D blocks" if act else "weight [3072, 3072], 2D 16x16 tiles"
    result = {
        "metric": AW_METRIC[a.op], "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"NVFP4 4/6 quantize of a bf16 {kind}, one tensor scale; "
                               f"{len(copies)} input copies rotated",
                   "rows": rows, "cols": cols, "mode": ["4over6", "fixed6", "fixed4"][a.mode],
                   "bytes_per_step": nbytes},
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm",
                     "kernel": ("nvfp4_quantize_1d, hadamard (amax, reduce, quantize kernels)" if act else
                                "nvfp4_quantize_2d (amax, reduce, quantize kernels)"),
                     "achieved": round(call_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(call_gbps / HBM_PEAK_GBPS, 4), "traffic": None, "bytes_per_launch": nbytes},
        "input_generation_s": round(gen_s, 2),
    }
    if not a.no_cpu_baseline:
        import oracle as O
        nt = O.default_threads()
        step = 1024 if act else 3072  # rows per oracle call
        done, t_cpu = 0, 0.0
        while t_cpu < a.cpu_seconds and done < rows:
            xb = W.bf16_bits(src[done:done + step])
            t1 = time.perf_counter()
            if act:
                O.quantize_1d(xb, a.mode, True, sign_mask, nthreads=nt)
            else:
                O.quantize_2d(xb, a.mode, nthreads=nt)
            t_cpu += time.perf_counter() - t1
            done += xb.shape[0]
        nb = done * cols
        sample_bytes = 2 * nb + nb // 2 + (nb // 16 if act else nb // 256)
        result["cpu_baseline"] = {"value": round(sample_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": nt,
                                  **host_cores(),
                                  "kind": "oracle",
                                  "sample": (f"{done} of {rows} rows, {step} rows per oracle call (each call "
                                             "with its own tensor scale)" if act else f"the whole {rows} x {cols} weight"),
                                  "seconds": round(t_cpu, 2)}
    print(json.dumps(result), flush=True)


VT_METRIC = "V quantize with 16-token blocks per channel: GB/s (bytes in + out) and % of MI355X HBM peak"


def vt_bench(a):
    """V quantized with 16-token blocks per channel.  Schedule "whole" (the
    default): V of every layer held head-major as one [24, layers * 56320,
    128] tensor (layer l = tokens l * 56320 ..), one call per step; each
    (layer, chunk) keeps its own tensor scale.  The one-layer call is timed
    beside it.  Schedule "layer": one layer's V per call."""
    import torch

    import precision_kv_cache_amd as P
    import workloads as W

    P.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = W.CACHE_LAYER
    H, T, D, L = s.H, s.T, s.D, s.chunk_len
    nl = a.layers if a.schedule == "whole" else 1
    t0 = time.time()
    vl = []
    for l in range(nl):
        _, v1 = W.gaussian_kv(s, W.cache_layer_seed(l), device=dev)
        vl.append(v1)
    v = vl[0] if nl == 1 else torch.cat(vl, dim=1).contiguous()
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    stream = torch.cuda.current_stream()
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(x, warmup, steps):
        tt = x.shape[1]
        out = P.nvfp4_kv_quantize_v_tblocks(x, L, a.mode)
        ws = torch.zeros(P.lib().nvfp4_kv_quantize_v_tblocks_workspace_bytes(H, tt, D, L), dtype=torch.uint8,
                         device=dev)
        for _ in range(warmup):
            P.nvfp4_kv_quantize_v_tblocks(x, L, a.mode, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        ev = [(E(), E()) for _ in range(steps)]
        start, stop = E(), E()
        start.record(stream)
        for i in range(steps):
            ev[i][0].record(stream)
            P.nvfp4_kv_quantize_v_tblocks(x, L, a.mode, out=out, workspace=ws, stream=stream)
            ev[i][1].record(stream)
        stop.record(stream)
        torch.cuda.synchronize()
        # the sticky error word after the warm-up and timed calls (0: no wait timed out)
        err = P.kv_error_word(ws)
        if err:
            print(f"bench.py: a bounded wait timed out (error word {err}); no result is reported", flush=True)
            sys.exit(3)
        return start.elapsed_time(stop) / steps, sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps, out

    ms_step, call_ms, out = timed(v, a.warmup, a.steps)
    nbytes = nl * kv_bytes(H, T, D, L, False)
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    call_gbps = nbytes / (call_ms * 1e-3) / 1e9
    what = (f"V of {nl} 8-chunk cache layers held head-major, bf16 [24, {nl} x 56320, 128], one call" if nl > 1
            else "V of one 8-chunk cache layer, bf16 [24, 56320, 128]")
    result = {
        "metric": VT_METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": what + ", chunks of 7040, quantized with 16-token blocks per (head, channel)",
                   "layers": nl, "heads": H, "tokens": T, "head_dim": D, "chunk_len": L,
                   "mode": ["4over6", "fixed6", "fixed4"][a.mode], "bytes_per_step": nbytes,
                   "schedule": a.schedule},
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm",
                     "kernel": f"nvfp4_kv_quantize_v_tblocks ({nl} layers' V)" if nl > 1
                     else "nvfp4_kv_quantize_v_tblocks (one layer's V)",
                     "achieved": round(call_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(call_gbps / HBM_PEAK_GBPS, 4), "traffic": None, "bytes_per_launch": nbytes},
        "input_generation_s": round(gen_s, 2),
        "quantize_wait_timeouts": 0,
    }
    if nl > 1:
        # layer 0 of the whole-cache call against the one-layer call, bit for bit
        ms1, call1, out1 = timed(vl[0], 2, 10)
        nb1 = kv_bytes(H, T, D, L, False)
        same = (torch.equal(out["codes"][:, :, :T // 2], out1["codes"]) and
                torch.equal(out["scales"][:, :, :T // 16], out1["scales"]) and
                torch.equal(out["tensor_scale"][:T // L], out1["tensor_scale"]))
        result["per_layer_schedule"] = {"value": round(nb1 / (ms1 * 1e-3) / 1e9, 2), "unit": "GB/s",
                                        "ms_per_call": round(ms1, 4), "steps": 10, "warmup": 2,
                                        "layer0_bytes_equal_whole_cache_call": bool(same)}
        if not same:
            print("bench.py: layer 0 of the whole-cache call differs from the one-layer call", flush=True)
            sys.exit(3)
    v = vl[0]
    if not a.no_cpu_baseline:
        import oracle as O
        nt = O.default_threads()
        done, t_cpu = 0, 0.0
        while t_cpu < a.cpu_seconds and done < T // L:
            vb = W.bf16_bits(v[:, done * L:(done + 1) * L])
            t1 = time.perf_counter()
            O.quantize_v_tblocks(vb, L, a.mode, nthreads=nt)
            t_cpu += time.perf_counter() - t1
            done += 1
        result["cpu_baseline"] = {"value": round(done * kv_bytes(H, L, D, L, False) / t_cpu / 1e9, 3), "unit": "GB/s",
                                  "cores": nt, **host_cores(), "kind": "oracle",
                                  "sample": f"{done} chunks of V [24, 7040, 128] quantized with 16-token blocks",
                                  "seconds": round(t_cpu, 2)}
    print(json.dumps(result), flush=True)


def stream_cpu_baseline(kv0, q, cache, ranges, nl, target_s):
    """The oracle on the host cores: one layer's append (smooth-quantize of
    the chunk) timed once, attention of sampled query rows over the same key
    set (as a logical head-major cache of the committed chunks) until about
    target_s seconds; scaled to one chunk through nl layers."""
    import numpy as np

    import oracle as O
    import workloads as W

    nt = O.default_threads()
    st = cache.state
    L = st.chunk_len
    kb, vb = W.bf16_bits(kv0[0]), W.bf16_bits(kv0[1])
    t0 = time.perf_counter()
    one = O.smooth_quantize(kb, vb, L, nthreads=nt)
    t_app = time.perf_counter() - t0
    # the key set's chunks all hold this chunk's data: a logical cache of as many copies as slots
    cap = st.capacity
    logical = {key: np.concatenate([one[key]] * cap, axis=1 if one[key].ndim == 3 else 0)
               for key in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tensor_scale", "v_tensor_scale",
                           "k_mean")}
    qb = W.bf16_bits(q)
    H, Tq, D = qb.shape
    rng = np.random.default_rng(0)
    done, t_att = 0, 0.0
    batch = 4 * nt
    while t_att < target_s:
        rows = rng.integers(0, H * Tq, batch)
        t0 = time.perf_counter()
        O.kv_attention(qb, logical, L, ranges, rows=rows, nthreads=nt)
        t_att += time.perf_counter() - t0
        done += batch
    step_s = nl * (t_app + t_att / done * H * Tq)
    return {"value": round(L / step_s, 4), "unit": "tokens/s", "cores": nt, **host_cores(), "kind": "oracle",
            "sample": f"one layer's append of a [24, 7040, 128] chunk ({t_app:.2f} s) and {done} query rows of "
                      f"attention over {sum(n for _, n in ranges)} keys ({t_att:.2f} s), scaled to {nl} layers x "
                      f"24 x 7040 rows", "seconds": round(t_app + t_att, 2)}


def attention_cpu_baseline(k, v, q, L, ranges, target_s):
    """The oracle's attention as it stands, on the host cores: the cache is
    quantized by the oracle from the same K and V, then query rows are
    attended in batches until about target_s seconds of attention work."""
    import numpy as np

    import oracle as O
    import workloads as W

    nt = O.default_threads()
    cache = O.smooth_quantize(W.bf16_bits(k), W.bf16_bits(v), L, nthreads=nt)
    qb = W.bf16_bits(q)
    H, Tq, D = qb.shape
    nk = sum(n for _, n in ranges)
    rng = np.random.default_rng(0)
    done, t_total = 0, 0.0
    batch = 4 * nt
    while t_total < target_s and done < H * Tq:
        rows = rng.integers(0, H * Tq, batch)
        t0 = time.perf_counter()
        O.kv_attention(qb, cache, L, ranges, rows=rows, nthreads=nt)
        t_total += time.perf_counter() - t0
        done += batch
    flops = 4.0 * done * nk * D
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": nt, **host_cores(), "kind": "oracle",
            "sample": f"{done} random query rows of [24, 7040, 128] over {nk} keys (fp64 attention over the "
                      f"exactly decoded cache)", "seconds": round(t_total, 2)}


def host_cores():
    """The host's CPU count as this process sees it: the CPUs it may run on
    (scheduler affinity) and the machine's total."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"host_cores_usable": usable, "host_cores_total": os.cpu_count() or usable}


def cpu_baseline(ks, vs, L, mode, target_s, check=None, bits=4):
    """The oracle as it stands, on the host cores: K and V smooth-quantize +
    dequantize of whole chunks, layer 0 chunk 0 onwards, until about
    target_s seconds of work on all oracle threads; then the same chunks again
    on one thread, until about target_s / 2 seconds.  With check = (the GPU
    outputs of layer 0, its dequantized (K, V)), chunk 0 of that layer is
    then compared with the oracle fed the GPU's K mean (untimed): codes,
    scales, tensor scales and dequantized values bit for bit, the mean by the
    1e-6 rule."""
    import oracle as O
    import workloads as W

    H, T, D = ks[0].shape
    chunk_bytes = 2 * (kv_bytes(H, L, D, L, True, bits) + kv_bytes(H, L, D, L, False, bits))

    def quant(kb, vb, nt, k_mean=None):
        if bits == 4:
            return O.smooth_quantize(kb, vb, L, mode, k_mean=k_mean, nthreads=nt)
        return O.smooth_quantize_lowbit(kb, vb, L, bits, mode, k_mean=k_mean, nthreads=nt)

    def deq(r, t, mean, nt):
        if bits == 4:
            return O.dequantize(r[t + "_codes"], r[t + "_scales"], r[t + "_tensor_scale"], mean, L, nthreads=nt)
        return O.dequantize_lowbit(r[t + "_codes"], r[t + "_scales"], r[t + "_tensor_scale"], mean, L, bits,
                                   nthreads=nt)

    def run(nt, budget_s):
        done, t_total, last = 0, 0.0, (0, 0)
        for l in range(len(ks)):
            for c in range(T // L):
                kb = W.bf16_bits(ks[l][:, c * L:(c + 1) * L])
                vb = W.bf16_bits(vs[l][:, c * L:(c + 1) * L])
                t0 = time.perf_counter()
                r = quant(kb, vb, nt)
                deq(r, "k", r["k_mean"], nt)
                deq(r, "v", None, nt)
                t_total += time.perf_counter() - t0
                done += 1
                last = (l, c)
                if t_total >= budget_s:
                    return done, t_total, last
        return done, t_total, last

    nt = O.default_threads()
    done, t_total, last = run(nt, target_s)
    done1, t1, last1 = run(1, target_s / 2)
    sample = lambda n, lc: (f"{n} chunks of [{H}, {L}, {D}] K and V (layer 0 chunk 0 to layer {lc[0]} chunk "  # noqa: E731
                            f"{lc[1]}): smooth-quantize + dequantize")
    out = {"value": round(done * chunk_bytes / t_total / 1e9, 3), "unit": "GB/s", "cores": nt, **host_cores(),
           "kind": "oracle", "sample": sample(done, last), "seconds": round(t_total, 2), "threads_used": nt}
    out["single_thread"] = {"value": round(done1 * chunk_bytes / t1 / 1e9, 4), "unit": "GB/s", "threads_used": 1,
                            "sample": sample(done1, last1), "seconds": round(t1, 2)}
    if check is not None:
        import numpy as np
        o, (dk, dv) = check
        rows = slice(0, L)
        kb, vb = W.bf16_bits(ks[0][:, rows]), W.bf16_bits(vs[0][:, rows])
        gm = o["k_mean"][0:1].cpu().numpy()
        x = O.bf16_to_float(kb).astype(np.float64)
        m_ref = x.mean(1)[None]
        tol = 1e-6 * np.maximum(np.abs(m_ref), np.abs(x).mean(1)[None])
        mean_ok = bool((np.abs(gm.astype(np.float64) - m_ref) <= tol).all())
        r = quant(kb, vb, nt, k_mean=gm)
        same = {key: bool(np.array_equal(o[key][:, rows].cpu().numpy(), r[key]))
                for key in ("k_codes", "v_codes", "k_scales", "v_scales")}
        for key in ("k_tensor_scale", "v_tensor_scale"):
            same[key] = bool(np.array_equal(o[key][0:1].cpu().numpy().view(np.uint32), r[key].view(np.uint32)))
        rk = deq(r, "k", gm, nt)
        rv = deq(r, "v", None, nt)
        same["dequant_k"] = bool(np.array_equal(W.bf16_bits(dk[:, rows]), rk))
        same["dequant_v"] = bool(np.array_equal(W.bf16_bits(dv[:, rows]), rv))
        out["parity_check"] = {"sample": "layer 0, chunk 0 of the last timed step", "mean_rule": mean_ok,
                               "bit_exact": mean_ok and all(same.values()), "fields": same}
    return out


if __name__ == "__main__":
    main()
