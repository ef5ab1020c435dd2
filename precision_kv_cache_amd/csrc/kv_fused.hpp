// kv_fused.hpp -- parameters and host entry of the single-read persistent KV
// quantize kernel (kv_fused.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kFusedThreads = 256;
constexpr int kFusedWgPerCu = 4;                       // resident workgroups per CU
constexpr int kFusedWavesPerEU = kFusedWgPerCu * kFusedThreads / 64 / 4;  // waves per SIMD
constexpr int kFusedMaxWG = 2048;                      // bound used to size the workspace
constexpr unsigned kFusedSpinLimit = 1u << 20;         // polls before a wait gives up

struct FusedParams {
  const uint16_t* x[2];
  uint8_t* codes[2];
  uint8_t* scales[2];
  float* tscale[2];
  float* kmean;
  unsigned long long* choice;
  double* psum;   // [nc][H][WPH][D] per-slice K channel sums
  float* pmax;    // [nc][H][WPH][D]
  float* pmin;    // [nc][H][WPH][D]
  float* pv;      // [nc][H][WPH] per-slice V maxima
  float* hamax;   // [2nc][H] head maxima
  float* genc;    // [2nc] encode scales
  unsigned* cnt_head;  // [2nc][H]
  unsigned* cnt_unit;  // [2nc]
  unsigned* flag;      // [2nc]
  unsigned* err;       // [1]
  uint32_t* tally;     // [grid][4] per-workgroup 4/6 choice counts
  int H, T, D, L, nc, WPH, RPW;
  unsigned spin_limit;
};

struct FusedLayout {
  size_t psum, pmax, pmin, pv, hamax, genc, tally, counters, total;
  int n_counters;
};

FusedLayout fused_layout(int H, int nc, int D, int WPH);
size_t fused_workspace_bound(int H, int T, int D, int L);
int fused_try_launch(FusedParams p, int mode, void* workspace, size_t ws_bytes, hipStream_t s);

// Adds up nslots per-workgroup tallies [nslots][4] into the caller's
// choice_counts [2][2] (K kept +-6, K kept +-4, V kept +-6, V kept +-4).
void launch_choice_reduce(const uint32_t* tally, size_t nslots, unsigned long long* choice, hipStream_t s);

}  // namespace nvfp4
