"""The streaming KV cache's bookkeeping (host functions of the C library, no
GPU needed): the oracle's key-set model against a hand-worked sequence of
chunks and prompt switches (inference pipeline, step 9 of the LongLive-2.0
summary page), then the library's slot ranges, mapped back to video tokens,
against that model over random event sequences, with the slot-reuse rule
(a new chunk never takes a slot the committed key set reads)."""
import json
import os

import numpy as np
import pytest

import oracle as O
import precision_kv_cache_amd as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
OK, NULL, SHAPE = 0, -1, -2


def _tokens(intervals):
    """Half-open [start, end) intervals of the fixture -> tokens."""
    return sorted(t for a, b in intervals for t in range(a, b))


def _logical(cache, ranges):
    """Slot-coordinate ranges -> video tokens, keeping duplicates."""
    st = cache.state
    L = st.chunk_len
    out = []
    for a, n in ranges:
        for j in range(a, a + n):
            out.append(st.slot_chunk[j // L] * L + j % L)
    return sorted(out)


def test_model_matches_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "stream_cache_worked_example.json")))
    for step in ex["after_commit"]:
        got = O.kv_cache_key_tokens(step["chunks"], step["shot_chunk"], ex["chunk_len"], ex["frame_tokens"],
                                    ex["sink_frames"], ex["shot_frames"], ex["window"])
        assert got == _tokens(step["ranges"]), step


def test_library_follows_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "stream_cache_worked_example.json")))
    c = P.KVCache(1, 2, 128, ex["chunk_len"], ex["window"] + 3, ex["frame_tokens"], ex["sink_frames"],
                  ex["shot_frames"], ex["window"], device=None)
    for step in ex["after_commit"]:
        chunk = step["chunks"] - 1
        c.begin_chunk(new_shot=chunk in ex["new_shot_at"])
        c.end_chunk()
        assert c.state.chunks == step["chunks"] and c.state.shot_chunk == step["shot_chunk"]
        assert _logical(c, c.key_ranges()) == _tokens(step["ranges"]), step


@pytest.mark.parametrize("seed", range(12))
def test_library_matches_model_on_random_streams(seed):
    rng = np.random.default_rng(seed)
    window = int(rng.integers(1, P.ATTN_MAX_RANGES - 1))
    capacity = int(rng.integers(window + 3, window + 7))
    L = int(rng.choice([32, 48, 64]))
    F = int(rng.choice([4, 8, 16]))
    Sg = int(rng.integers(0, L // F + 1))
    Ss = int(rng.integers(0, L // F + 1))
    c = P.KVCache(2, 1, 16, L, capacity, F, Sg, Ss, window, device=None)
    for chunk in range(40):
        before = c.key_ranges()
        read_slots = {j // L for a, n in before for j in range(a, a + n)}
        slot = c.begin_chunk(new_shot=bool(rng.random() < 0.2))
        assert slot not in read_slots, "a new chunk took a slot the committed key set reads"
        assert c.key_ranges() == before, "the pending chunk changed the committed key set"
        c.end_chunk()
        want = O.kv_cache_key_tokens(c.state.chunks, c.state.shot_chunk, L, F, Sg, Ss, window)
        got = _logical(c, c.key_ranges())
        assert got == want, (seed, chunk)
        assert len(c.key_ranges()) <= P.ATTN_MAX_RANGES


def test_cache_argument_errors():
    L = P.lib()
    st = P.KVCacheState()
    import ctypes
    s = ctypes.byref(st)
    assert L.nvfp4_kv_cache_init(None, 1, 1, 128, 64, 8, 16, 1, 1, 3) == NULL
    assert L.nvfp4_kv_cache_init(s, 1, 1, 128, 64, 5, 16, 1, 1, 3) == SHAPE   # capacity < window + 3
    assert L.nvfp4_kv_cache_init(s, 1, 1, 128, 64, 8, 16, 5, 1, 3) == SHAPE   # sink longer than a chunk
    assert L.nvfp4_kv_cache_init(s, 1, 1, 128, 64, 16, 16, 1, 1, 7) == SHAPE  # window too long for the ranges
    assert L.nvfp4_kv_cache_init(s, 1, 1, 120, 64, 8, 16, 1, 1, 3) == SHAPE   # head_dim % 16
    assert L.nvfp4_kv_cache_init(s, 1, 1, 128, 64, 65, 16, 1, 1, 3) == SHAPE  # too many slots
    assert L.nvfp4_kv_cache_init(s, 2, 1, 128, 64, 8, 16, 1, 1, 3) == OK
    assert L.nvfp4_kv_cache_end_chunk(s) == SHAPE                             # nothing pending
    assert L.nvfp4_kv_cache_append(s, ctypes.c_void_p(0x7f0000000000), 1 << 30, 0, None, None, 0, None, 0,
                                   None) == SHAPE                             # nothing pending
    assert L.nvfp4_kv_cache_begin_chunk(s, 0) == 0
    assert L.nvfp4_kv_cache_begin_chunk(s, 0) == SHAPE                        # already pending
    assert L.nvfp4_kv_cache_append(s, ctypes.c_void_p(0x7f0000000000), 1 << 30, 2, None, None, 0, None, 0,
                                   None) == SHAPE                             # layer out of range
    assert L.nvfp4_kv_cache_append(s, ctypes.c_void_p(0x7f0000000000), 16, 0, None, None, 0, None, 0,
                                   None) == SHAPE                             # storage too small
    assert L.nvfp4_kv_cache_append(s, ctypes.c_void_p(0x7f0000000010), 1 << 30, 0, None, None, 0, None, 0,
                                   None) == -3                                # storage not 256-byte aligned
    good = st.pending_slot
    st.pending_slot = 8                                                       # a corrupted state: past the slots
    assert L.nvfp4_kv_cache_append(s, ctypes.c_void_p(0x7f0000000000), 1 << 30, 0, None, None, 0, None, 0,
                                   None) == SHAPE
    st.pending_slot = good
    assert L.nvfp4_kv_cache_end_chunk(s) == OK
    assert L.nvfp4_kv_cache_layer_bytes(1, 128, 64, 0) == 0
