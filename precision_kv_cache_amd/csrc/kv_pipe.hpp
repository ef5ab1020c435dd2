// kv_pipe.hpp -- parameters and host entry of the persistent, overlapped KV
// quantize kernel (kv_pipe.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kPipeThreads = 256;
constexpr int kPipeWgPerCu = 6;          // resident workgroups per CU (both roles)
constexpr int kPipeMaxWG = 4096;         // bound used to size the workspace
constexpr int kPipeStatsRows = 256;      // rows per statistics task
constexpr int kPipeQuantRows = 128;      // rows per quantize task
constexpr unsigned kPipeSpinLimit = 1u << 20;  // polls before a wait gives up

struct PipeParams {
  const uint16_t* x[2];
  uint8_t* codes[2];
  uint8_t* scales[2];
  float* tscale[2];
  float* kmean;
  double* psum;        // [nc][H][nst][128] per-tile K channel sums
  float* pmax;         // [nc][H][nst][128]
  float* pmin;         // [nc][H][nst][128]
  float* pv;           // [nc][H][nst] per-tile V maxima
  float* hamax;        // [2nc][H] head maxima
  float* genc;         // [2nc] encode scales
  uint32_t* tally;     // [grid][4] per-workgroup 4/6 choice counts
  unsigned* cnt_head;  // [2nc][H] finished statistics tiles of a head
  unsigned* cnt_unit;  // [2nc] finished heads of a unit
  unsigned* flag;      // [2nc] unit ready to encode
  unsigned* err;       // [1]
  int choice;          // tallies wanted
  int mode;
  int H, T, L, nc, nst, nqt;
  unsigned spin_limit;
};

struct PipeLayout {
  size_t psum, pmax, pmin, pv, hamax, genc, tally, counters, total;
  int n_counters;
};

PipeLayout pipe_layout(int H, int nc, int nst);
size_t pipe_workspace_bound(int H, int T, int D, int L);
// NVFP4_OK after enqueueing (and the choice-count reduction when choice is
// set), a positive value when this form does not apply to the shape or
// device, or NVFP4_ERR_HIP.
int pipe_try_launch(PipeParams p, void* workspace, size_t ws_bytes, unsigned long long* choice, hipStream_t s);

}  // namespace nvfp4
