// kv_overlap.hpp -- parameters and host entry of the single-launch,
// overlapped KV quantize kernel (kv_overlap.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kOvThreads = 256;
constexpr int kOvStatsRows = 512;    // rows per statistics tile
constexpr int kOvQuantRows = 256;    // rows per quantize tile
constexpr int kOvDepth = 3;          // segments between a unit's statistics and its quantization
// Calls of at most this many (chunk, tensor) units quantize with each row's
// loads issued one row ahead, and (at 4 bits) their statistics tiles keep 8
// rows per lane in flight instead of 4: they have about one round of tiles,
// so no other workgroup hides a tile's load latency.  Larger calls keep
// fewer live registers instead.
constexpr int kOvAheadUnits = 4;
constexpr int kOvReplicas = 32;      // copies of each unit's ready word
constexpr unsigned kOvSpinLimit = 1u << 22;  // polls before a wait gives up

struct OverlapParams {
  const uint16_t* x[2];  // K, V bf16 [H, T, 128]
  uint8_t* codes[2];
  uint8_t* scales[2];
  float* tscale[2];
  float* kmean;              // [nc][H][128]
  double* ksum;              // [nc][H][nst][128] per-tile K channel sums
  uint32_t* kext;            // [nc][H][nst][128] per-tile K channel max (high half) and min (low half), bf16 bits
  float* vmax;               // [nc][H][nst] per-tile V largest magnitude
  float* hamax;              // [U][H] head maxima
  float* mcopy;              // [nc][H][128] the K means again, one 512-byte block per (chunk, head)
  unsigned long long* ready; // [kOvReplicas][U], 256 bytes apart: 1 << 32 | encode-scale bits once the unit is ready
  unsigned* cnt_head;        // [U][H] finished statistics tiles of a head
  unsigned* cnt_unit;        // [U] finished heads of a unit
  unsigned* err;             // [1] set when a wait of this call timed out (cleared per call)
  unsigned* err_sticky;      // [1] set then too, never cleared here (the workspace's first word, or the
                             // caller's word for the call that has no workspace)
  uint32_t* tally;           // [U * nq][4] per-quantize-tile 4/6 choice counts (when choice)
  int choice;
  int ahead;  // calls of few units (kOvAheadUnits): rows loaded one ahead, 8-row statistics batches
  int H, T, L, nc, nst, nqt, depth;
  unsigned spin_limit;
};

struct OverlapLayout {
  size_t ksum, kext, vmax, hamax, mcopy, ready, tally, counters, total;
  int n_zero_words;  // ready .. counters end, in 32-bit words, cleared before the launch
};

OverlapLayout overlap_layout(int H, int nc, int nst, int nqt);
size_t overlap_workspace_bound(int H, int T, int D, int L);
// Bytes at the start of every KV workspace that no per-call clearing touches:
// the sticky error word (offset 0) and padding to 256 bytes.
constexpr size_t kKvWorkspaceHeader = 256;
// NVFP4_OK after enqueueing (and the choice-count reduction when choice is
// set), a positive value when this form does not apply to the shape, or
// NVFP4_ERR_HIP.
// err_word: where a timed-out wait is recorded besides this call's own word
// (never cleared here).
// bits: 4 (NVFP4), or 3 / 2 for the low-bit cache (lowbit_device.hpp).
int overlap_try_launch(OverlapParams p, int mode, int bits, void* workspace, size_t ws_bytes,
                       unsigned long long* choice, unsigned* err_word, hipStream_t s);

}  // namespace nvfp4
