"""Seeded synthetic inputs for the NVFP4 KV-cache quantizer.

Shared by the tests, the benchmark and the smoke check; it holds none of the
quantizer's arithmetic, only random-number recipes.  Every tensor is drawn in
fp32 with a seeded ``torch.Generator`` and rounded to bf16 (torch's
round-to-nearest-even cast).  The shapes stand in for the KV cache of the
video DiT that the LongLive-2.0 summary page builds on (training pipeline,
step 2: Wan2.2-TI2V-5B): 24 heads of 128 channels, 880 tokens per latent
frame, chunks of F_c = 8 frames (inference pipeline, step 7), 30 layers.  The
page prints no model dimensions and no quantization inputs, so the value
distributions are stated here and nowhere else:

* gaussian KV: K = N(0, 1) + offset[h, d] with offset ~ N(0, sigma=2) (the
  per-channel bias that K-smoothing removes), V = N(0, 1); every element is
  independently multiplied by 20 with probability 0.01 (outliers).
* heavy tail: K and V are Student-t with 3 degrees of freedom, z / sqrt(chi2_3
  / 3), times a per-(head, channel) scale 10**U(-1, 1); no offset.
* activation: N(0, 1) with 0.1 % of elements multiplied by 50, plus a seeded
  16-bit sign mask for the random Hadamard transform; weight: N(0, sigma=0.02).
* queries (attention over the cache): Q = N(0, 1) + offset[h, d] with
  offset ~ N(0, 1); the queries of one chunk (7040 tokens) attend to the
  8-chunk cache layer.  Key sets of the sink layout (inference pipeline, step
  9): a global sink of the first S_g frames, a shot sink of S_s frames at
  the start of the current shot, and the most recent chunks; frames are 880
  tokens, so the segment edges fall inside 64-key tiles.

Draw order inside one generator: noise, offsets, outlier masks.
"""
from dataclasses import dataclass

import torch

FRAMES_PER_CHUNK = 8
TOKENS_PER_FRAME = 880
CHUNK_TOKENS = FRAMES_PER_CHUNK * TOKENS_PER_FRAME  # 7040
HEADS = 24
HEAD_DIM = 128
LAYERS = 30
CACHE_CHUNKS = 8


@dataclass(frozen=True)
class KVShape:
    H: int
    T: int
    D: int
    chunk_len: int

    @property
    def n_chunks(self):
        return self.T // self.chunk_len


TINY = KVShape(1, 256, 128, 256)                                   # one small chunk
ONE_CHUNK = KVShape(HEADS, CHUNK_TOKENS, HEAD_DIM, CHUNK_TOKENS)   # one Wan-like chunk
CACHE_LAYER = KVShape(HEADS, CACHE_CHUNKS * CHUNK_TOKENS, HEAD_DIM, CHUNK_TOKENS)  # one layer, 8 chunks

SEED_TINY, SEED_ONE_CHUNK, SEED_CACHE, SEED_HEAVY, SEED_ACT = 1000, 1001, 1002, 1003, 1004


def cache_layer_seed(layer: int) -> int:
    """Seed of layer ``layer`` of the 30-layer cache."""
    return 100200 + layer


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian_kv(shape: KVShape, seed: int, device="cpu"):
    """K, V bf16 [H, T, D]: N(0,1) (+ N(0, 2) channel offset on K), 1 % of
    elements x20.  The offset is per (head, channel), shared by all chunks."""
    g = _gen(seed, device)
    H, T, D = shape.H, shape.T, shape.D
    k = torch.randn(H, T, D, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(H, T, D, generator=g, device=device, dtype=torch.float32)
    off = torch.randn(H, 1, D, generator=g, device=device, dtype=torch.float32) * 2.0
    k += off
    mk = torch.rand(H, T, D, generator=g, device=device) < 0.01
    k[mk] *= 20.0
    del mk
    mv = torch.rand(H, T, D, generator=g, device=device) < 0.01
    v[mv] *= 20.0
    del mv
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def heavy_tail_kv(shape: KVShape, seed: int, device="cpu"):
    """K, V bf16 [H, T, D]: Student-t(3) times a per-(h, d) scale 10**U(-1,1)."""
    g = _gen(seed, device)
    H, T, D = shape.H, shape.T, shape.D
    out = []
    for _ in range(2):
        z = torch.randn(H, T, D, generator=g, device=device, dtype=torch.float32)
        chi2 = torch.zeros(H, T, D, device=device, dtype=torch.float32)
        for _ in range(3):
            n = torch.randn(H, T, D, generator=g, device=device, dtype=torch.float32)
            chi2 += n * n
        out.append(z / torch.sqrt(chi2 / 3.0))
    for i in range(2):
        scale = torch.pow(10.0, torch.rand(H, 1, D, generator=g, device=device) * 2.0 - 1.0)
        out[i] = out[i] * scale
    return out[0].to(torch.bfloat16), out[1].to(torch.bfloat16)


def activation(rows: int, cols: int, seed: int, device="cpu"):
    """Activation bf16 [rows, cols] N(0,1) with 0.1 % outliers x50, and a
    16-bit random sign mask for the Hadamard pre-rotation."""
    g = _gen(seed, device)
    x = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    m = torch.rand(rows, cols, generator=g, device=device) < 0.001
    x[m] *= 50.0
    sign_mask = int(torch.randint(0, 1 << 16, (1,), generator=g, device=device).item())
    return x.to(torch.bfloat16), sign_mask


def weight(rows: int, cols: int, seed: int, device="cpu"):
    """Weight bf16 [rows, cols] N(0, sigma=0.02)."""
    g = _gen(seed, device)
    w = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * 0.02
    return w.to(torch.bfloat16)


ACT_ROWS, ACT_COLS = 16384, 3072
W_ROWS, W_COLS = 3072, 3072


def act_weight(seed: int = SEED_ACT, device="cpu", act_rows=ACT_ROWS, act_cols=ACT_COLS, w_rows=W_ROWS,
               w_cols=W_COLS):
    """The activation / weight pair: activation with sign mask, then weight."""
    x, sign_mask = activation(act_rows, act_cols, seed, device)
    w = weight(w_rows, w_cols, seed + 7919, device)
    return x, sign_mask, w


ATTN_QUERIES = CHUNK_TOKENS   # queries of one chunk
SEED_ATTN = 1005


def queries(H: int, Tq: int, D: int, seed: int, device="cpu"):
    """Q bf16 [H, Tq, D]: N(0, 1) plus a per-(head, channel) N(0, 1) offset."""
    g = _gen(seed, device)
    q = torch.randn(H, Tq, D, generator=g, device=device, dtype=torch.float32)
    q += torch.randn(H, 1, D, generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def sink_ranges(n_chunks: int, chunk_len: int = CHUNK_TOKENS, frame=TOKENS_PER_FRAME, sink_frames=3,
                shot_start_frame=None, shot_frames=3, window_chunks=3):
    """(start, len) key ranges of the sink layout over a cache of n_chunks
    chunks: global sink frames [0, sink_frames), shot sink frames starting at
    shot_start_frame (default: the middle of the cache), and the last
    window_chunks chunks.  Segments are disjoint for the defaults."""
    T = n_chunks * chunk_len
    if shot_start_frame is None:
        shot_start_frame = (T // frame) // 2 - 1
    win = min(window_chunks, n_chunks) * chunk_len
    r = [(0, sink_frames * frame), (shot_start_frame * frame, shot_frames * frame), (T - win, win)]
    return [(int(a), int(b)) for a, b in r]


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    import numpy as np
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a, device="cpu"):
    """numpy uint16 bit patterns -> bf16 tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)
