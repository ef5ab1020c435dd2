"""Write tests/golden/tiny_kv_oracle.npz: the oracle's outputs on the tiny KV
workload (1 head, 256 tokens, 128 channels, one chunk, seed 1000).

A regression fixture for the oracle itself: it calls only oracle/ (and the
seeded generators), never the GPU library.  Re-run it only with a commit
message that names the passage or convention behind an oracle change.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


def main():
    k, v = W.gaussian_kv(W.TINY, W.SEED_TINY)
    kb, vb = W.bf16_bits(k), W.bf16_bits(v)
    r = O.smooth_quantize(kb, vb, W.TINY.chunk_len)
    deq = O.dequantize(r["k_codes"], r["k_scales"], r["k_tensor_scale"], r["k_mean"], W.TINY.chunk_len)
    out = os.path.join(HERE, "tiny_kv_oracle.npz")
    np.savez_compressed(out, k=kb, v=vb, k_dequant=deq,
                        **{key: r[key] for key in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tensor_scale",
                                                   "v_tensor_scale", "k_mean")})
    print(out, os.path.getsize(out), "bytes")


if __name__ == "__main__":
    main()
