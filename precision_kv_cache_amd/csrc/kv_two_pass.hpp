// kv_two_pass.hpp -- geometry, workspace layout and parameters of the
// two-pass KV kernels (kv_quant.hip): a statistics kernel (channel sums, max
// and min of K, largest |V| per (chunk, tensor, head)), then a quantize
// kernel.  The 3-bit / 2-bit quantizer (kv_lowbit.hip) reuses the statistics.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "host_common.hpp"
#include "kv_overlap.hpp"

namespace nvfp4 {

constexpr int kMaxThreads = 256;
constexpr int kStatsPasses = 16;  // rows per stats tile = RP * kStatsPasses
constexpr int kQuantPasses = 4;   // rows per quant / dequant tile = RP * kQuantPasses
constexpr int kBatch = 2;         // rows whose loads are issued together
constexpr long long kMaxLaunchWGs = 1LL << 22;   // workgroups per launch (grid limits)

struct KVGeom {
  int H, T, D, L, nc;
  int NB, RP, threads;
  int rows_s, rows_q, nst, nqt;
};

inline KVGeom kv_geom(int H, int T, int D, int L) {
  KVGeom g;
  g.H = H; g.T = T; g.D = D; g.L = L;
  g.nc = L > 0 ? T / L : 0;
  g.NB = D / 16;
  g.RP = g.NB > 0 ? (kMaxThreads / g.NB > 0 ? kMaxThreads / g.NB : 1) : 1;
  g.threads = (g.NB * g.RP + 63) / 64 * 64;  // whole waves
  g.rows_s = g.RP * kStatsPasses;
  g.rows_q = g.RP * kQuantPasses;
  g.nst = (L + g.rows_s - 1) / g.rows_s;
  g.nqt = (L + g.rows_q - 1) / g.rows_q;
  return g;
}

struct KVWorkspace {
  size_t psum, pmax, pmin, pvabs, hamax, tally, counters, total;  // byte offsets
  int n_counters;
  size_t n_tally;
};

inline KVWorkspace kv_workspace_layout(const KVGeom& g) {
  KVWorkspace w;
  const size_t nch = (size_t)g.nc * g.H * g.nst * g.D;
  size_t off = kKvWorkspaceHeader;  // the sticky error word's block, shared with the overlapped form
  w.psum = off;  off = align_up(off + nch * sizeof(double), 256);
  w.pmax = off;  off = align_up(off + nch * sizeof(float), 256);
  w.pmin = off;  off = align_up(off + nch * sizeof(float), 256);
  w.pvabs = off; off = align_up(off + (size_t)g.nc * g.H * g.nst * sizeof(float), 256);
  w.hamax = off; off = align_up(off + (size_t)2 * g.nc * g.H * sizeof(float), 256);
  w.tally = off;  // [nc][2][H][nqt][4] per-workgroup 4/6 choice counts
  w.n_tally = (size_t)2 * g.nc * g.H * g.nqt;
  off = align_up(off + (size_t)w.n_tally * 4 * sizeof(uint32_t), 256);
  w.counters = off;  // one per (chunk, tensor, head)
  w.n_counters = 2 * g.nc * g.H;
  off = align_up(off + (size_t)w.n_counters * sizeof(unsigned), 256);
  w.total = off;
  return w;
}

struct KVParams {
  const uint16_t* x[2];  // K, V
  uint8_t* codes[2];
  uint8_t* scales[2];
  float* tscale[2];
  float* kmean;
  double* psum;   // [nc][H][nst][D]
  float* pmax;    // [nc][H][nst][D]
  float* pmin;    // [nc][H][nst][D]
  float* pvabs;   // [nc][H][nst]
  float* hamax;   // [2][nc][H]
  unsigned* cnt;  // [nc][2][H]
  uint32_t* tally;  // [nc][2][H][nqt][4]
  unsigned long long* choice;
  int H, T, D, L, nc, NB, RP, rows_s, rows_q, nst, nqt;
  int s0, s1;  // chunks whose statistics this launch computes
  int q0, q1;  // chunks this launch quantizes
};

// Shapes the KV entry points take.
inline bool kv_shape_ok(int H, int T, int D, int L) {
  if (H < 0 || T < 0 || D <= 0 || L <= 0) return false;
  if (D % 16 != 0 || D > NVFP4_KV_MAX_D) return false;
  if (T % L != 0) return false;
  if (H > 65535 || T / L > 16384) return false;  // launch grid limits
  // block indices and row counts stay in 31 bits
  if ((long long)H * T * (D / 16) >= (1LL << 31)) return false;
  return true;
}

// Host launches of the two-pass kernels (kv_quant.hip): clear the
// per-(chunk, tensor, head) counters; statistics of chunks [p.s0, p.s1).
void launch_kv_zero_counters(unsigned* cnt, int n, hipStream_t s);
void launch_kv_stats(const KVParams& p, unsigned n_workgroups, int threads, hipStream_t s);
void launch_choice_reduce(const uint32_t* tally, size_t nslots, unsigned long long* choice, hipStream_t s);

}  // namespace nvfp4
