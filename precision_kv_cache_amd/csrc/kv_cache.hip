// kv_cache.hip -- the streaming NVFP4 KV cache: slot bookkeeping for the
// sink / window key set of the LongLive-2.0 summary page (inference
// pipeline, steps 7 to 9) on top of the quantize and attention entry points.
// Host code only: the device work is nvfp4_kv_smooth_quantize writing into a
// slot and nvfp4_kv_attention_chunked reading the slots.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4kv.h"

namespace {

using nvfp4::align_up;
using nvfp4::aligned;

struct LayerLayout {
  size_t off[7];  // k_codes, v_codes, k_scales, v_scales, k_tensor_scale, v_tensor_scale, k_mean
  size_t bytes;
};

bool geometry_ok(int heads, int head_dim, int chunk_len, int capacity) {
  return heads >= 1 && head_dim >= 16 && head_dim % 16 == 0 && head_dim <= NVFP4_KV_MAX_D && chunk_len >= 1 &&
         capacity >= 1 && capacity <= NVFP4_CACHE_MAX_SLOTS && (long long)capacity * chunk_len <= (1LL << 30);
}

LayerLayout layer_layout(int heads, int head_dim, int chunk_len, int capacity) {
  LayerLayout l{};
  const size_t n = (size_t)capacity * heads * chunk_len * head_dim;  // elements per tensor
  const size_t sz[7] = {n / 2, n / 2, n / 16, n / 16, (size_t)capacity * 4, (size_t)capacity * 4,
                        (size_t)capacity * heads * head_dim * 4};
  size_t o = 0;
  for (int i = 0; i < 7; ++i) {
    l.off[i] = o;
    o = align_up(o + sz[i], 256);
  }
  l.bytes = o;
  return l;
}

LayerLayout layout_of(const nvfp4_kv_cache_t* c) {
  return layer_layout(c->heads, c->head_dim, c->chunk_len, c->capacity);
}

// The committed window: chunks [w0, chunks).
long long window_start(const nvfp4_kv_cache_t* c) {
  const long long w0 = c->chunks - c->window;
  return w0 > 0 ? w0 : 0;
}

int slot_of(const nvfp4_kv_cache_t* c, long long chunk) {
  for (int s = 0; s < c->capacity; ++s)
    if (c->slot_chunk[s] == chunk) return s;
  return -1;
}

// Tokens of chunk `chunk` that the committed key set reads as a sink (0 if
// none): chunk 0 gives the global sink, the shot's first chunk the shot sink
// (chunk 0 may be both: the longer one).  Chunks inside the window are read
// whole, so they are not sinks.
int sink_tokens(const nvfp4_kv_cache_t* c, long long chunk) {
  if (chunk >= c->chunks || chunk >= window_start(c)) return 0;
  int frames = 0;
  if (chunk == 0) frames = c->sink_frames;
  if (chunk == c->shot_chunk && c->shot_frames > frames) frames = c->shot_frames;
  return frames * c->frame_tokens;
}

// Whether the committed key set reads chunk `chunk`.
bool is_read(const nvfp4_kv_cache_t* c, long long chunk) {
  if (chunk < 0 || chunk >= c->chunks) return false;
  return chunk >= window_start(c) || sink_tokens(c, chunk) > 0;
}

}  // namespace

extern "C" NVFP4KV_API size_t nvfp4_kv_cache_layer_bytes(int heads, int head_dim, int chunk_len,
                                                         int capacity) noexcept {
  if (!geometry_ok(heads, head_dim, chunk_len, capacity)) return 0;
  return layer_layout(heads, head_dim, chunk_len, capacity).bytes;
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_offsets(const nvfp4_kv_cache_t* c, size_t* off) noexcept {
  if (!c || !off) return NVFP4_ERR_NULL;
  if (!geometry_ok(c->heads, c->head_dim, c->chunk_len, c->capacity)) return NVFP4_ERR_SHAPE;
  const LayerLayout l = layout_of(c);
  for (int i = 0; i < 7; ++i) off[i] = l.off[i];
  return NVFP4_OK;
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_init(nvfp4_kv_cache_t* c, int layers, int heads, int head_dim,
                                               int chunk_len, int capacity, int frame_tokens, int sink_frames,
                                               int shot_frames, int window) noexcept {
  if (!c) return NVFP4_ERR_NULL;
  if (layers < 1 || !geometry_ok(heads, head_dim, chunk_len, capacity) || frame_tokens < 1 || sink_frames < 0 ||
      shot_frames < 0 || (long long)sink_frames * frame_tokens > chunk_len ||
      (long long)shot_frames * frame_tokens > chunk_len || window < 1 || window > NVFP4_ATTN_MAX_RANGES - 2 ||
      capacity < window + 3)
    return NVFP4_ERR_SHAPE;
  c->layers = layers;
  c->heads = heads;
  c->head_dim = head_dim;
  c->chunk_len = chunk_len;
  c->capacity = capacity;
  c->frame_tokens = frame_tokens;
  c->sink_frames = sink_frames;
  c->shot_frames = shot_frames;
  c->window = window;
  c->chunks = 0;
  c->shot_chunk = 0;
  c->pending = -1;
  c->pending_slot = -1;
  c->pending_new_shot = 0;
  for (int s = 0; s < NVFP4_CACHE_MAX_SLOTS; ++s) c->slot_chunk[s] = -1;
  return NVFP4_OK;
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_begin_chunk(nvfp4_kv_cache_t* c, int new_shot) noexcept {
  if (!c) return NVFP4_ERR_NULL;
  if (c->pending >= 0 || !geometry_ok(c->heads, c->head_dim, c->chunk_len, c->capacity)) return NVFP4_ERR_SHAPE;
  // an empty slot, else the slot of the oldest chunk the committed key set
  // does not read (there is one: that set spans at most window + 2 chunks)
  int pick = -1;
  for (int s = 0; s < c->capacity && pick < 0; ++s)
    if (c->slot_chunk[s] < 0) pick = s;
  if (pick < 0) {
    long long oldest = -1;
    for (int s = 0; s < c->capacity; ++s) {
      const long long ch = c->slot_chunk[s];
      if (!is_read(c, ch) && (oldest < 0 || ch < oldest)) {
        oldest = ch;
        pick = s;
      }
    }
  }
  if (pick < 0) return NVFP4_ERR_SHAPE;
  c->pending = c->chunks;
  c->pending_slot = pick;
  c->pending_new_shot = new_shot != 0;
  c->slot_chunk[pick] = c->pending;
  return pick;
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_append(const nvfp4_kv_cache_t* c, void* storage, size_t storage_bytes,
                                                 int layer, const uint16_t* k, const uint16_t* v, int mode,
                                                 void* workspace, size_t workspace_bytes, void* stream) noexcept {
  if (!c || !storage) return NVFP4_ERR_NULL;
  if (c->pending < 0 || layer < 0 || layer >= c->layers ||
      !geometry_ok(c->heads, c->head_dim, c->chunk_len, c->capacity))
    return NVFP4_ERR_SHAPE;
  // the state is caller memory: a slot outside the storage is refused, not written
  if (c->pending_slot < 0 || c->pending_slot >= c->capacity) return NVFP4_ERR_SHAPE;
  if (!aligned(storage, 256)) return NVFP4_ERR_ALIGN;
  const LayerLayout l = layout_of(c);
  if (storage_bytes < l.bytes * (size_t)c->layers) return NVFP4_ERR_SHAPE;
  uint8_t* base = static_cast<uint8_t*>(storage) + l.bytes * (size_t)layer;
  const size_t s = (size_t)c->pending_slot;
  const size_t slot_elems = (size_t)c->heads * c->chunk_len * c->head_dim;
  return nvfp4_kv_smooth_quantize(
      k, v, c->heads, c->chunk_len, c->head_dim, c->chunk_len, mode, base + l.off[0] + s * slot_elems / 2,
      base + l.off[1] + s * slot_elems / 2, base + l.off[2] + s * slot_elems / 16,
      base + l.off[3] + s * slot_elems / 16, reinterpret_cast<float*>(base + l.off[4]) + s,
      reinterpret_cast<float*>(base + l.off[5]) + s,
      reinterpret_cast<float*>(base + l.off[6]) + s * (size_t)c->heads * c->head_dim, nullptr, workspace,
      workspace_bytes, stream);
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_end_chunk(nvfp4_kv_cache_t* c) noexcept {
  if (!c) return NVFP4_ERR_NULL;
  if (c->pending < 0) return NVFP4_ERR_SHAPE;
  if (c->pending_new_shot) c->shot_chunk = c->pending;
  c->chunks = c->pending + 1;
  c->pending = -1;
  c->pending_slot = -1;
  c->pending_new_shot = 0;
  return NVFP4_OK;
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_key_ranges(const nvfp4_kv_cache_t* c, int* ranges) noexcept {
  if (!c || !ranges) return NVFP4_ERR_NULL;
  if (!geometry_ok(c->heads, c->head_dim, c->chunk_len, c->capacity)) return NVFP4_ERR_SHAPE;
  int n = 0;
  const long long L = c->chunk_len;
  auto add = [&](long long start, long long len) -> bool {
    if (len <= 0) return true;
    if (n > 0 && ranges[2 * (n - 1)] + (long long)ranges[2 * (n - 1) + 1] == start) {
      ranges[2 * (n - 1) + 1] += (int)len;  // adjacent: merge
      return true;
    }
    if (n >= NVFP4_ATTN_MAX_RANGES) return false;
    ranges[2 * n] = (int)start;
    ranges[2 * n + 1] = (int)len;
    ++n;
    return true;
  };
  // sinks (chunk 0, then the shot's chunk), then the window oldest first
  const long long sinks[2] = {0, c->shot_chunk};
  for (int i = 0; i < 2; ++i) {
    if (i == 1 && c->shot_chunk == 0) break;
    const int tok = sink_tokens(c, sinks[i]);
    if (tok == 0) continue;
    const int s = slot_of(c, sinks[i]);
    if (s < 0 || !add(s * L, tok)) return NVFP4_ERR_SHAPE;
  }
  for (long long ch = window_start(c); ch < c->chunks; ++ch) {
    const int s = slot_of(c, ch);
    if (s < 0 || !add(s * L, L)) return NVFP4_ERR_SHAPE;
  }
  return n;
}

extern "C" NVFP4KV_API int nvfp4_kv_cache_attention(const nvfp4_kv_cache_t* c, const void* storage,
                                                    size_t storage_bytes, int layer, const uint16_t* q, int Hq,
                                                    int Tq, float softmax_scale, uint16_t* out, float* lse,
                                                    void* workspace, size_t workspace_bytes, void* stream) noexcept {
  if (!c || !storage) return NVFP4_ERR_NULL;
  if (layer < 0 || layer >= c->layers || !geometry_ok(c->heads, c->head_dim, c->chunk_len, c->capacity))
    return NVFP4_ERR_SHAPE;
  if (!aligned(storage, 256)) return NVFP4_ERR_ALIGN;
  const LayerLayout l = layout_of(c);
  if (storage_bytes < l.bytes * (size_t)c->layers) return NVFP4_ERR_SHAPE;
  int ranges[2 * NVFP4_ATTN_MAX_RANGES];
  const int n = nvfp4_kv_cache_key_ranges(c, ranges);
  if (n < 0) return n;
  const uint8_t* base = static_cast<const uint8_t*>(storage) + l.bytes * (size_t)layer;
  return nvfp4_kv_attention_chunked(q, Hq, Tq, c->head_dim, base + l.off[0], base + l.off[2],
                                    reinterpret_cast<const float*>(base + l.off[4]),
                                    reinterpret_cast<const float*>(base + l.off[6]), base + l.off[1],
                                    base + l.off[3], reinterpret_cast<const float*>(base + l.off[5]), c->heads,
                                    c->capacity * c->chunk_len, c->chunk_len, ranges, n, softmax_scale, out, lse,
                                    workspace, workspace_bytes, stream);
}
