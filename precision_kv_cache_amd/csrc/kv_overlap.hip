// kv_overlap.hip -- single-launch, overlapped form of the per-chunk K
// smoothing + NVFP4 4/6 quantization (LongLive-2.0 summary page: inference
// pipeline, step 7; full-stack NVFP4), for head dimension 128.
//
// A unit is one (chunk, tensor): u = tensor * n_chunks + chunk, every K
// chunk before the first V chunk (the resident workgroups then cover fewer
// separate regions of memory at a time).  A unit's tensor scale needs its
// largest |K - mean| (or |V|) before any of its blocks can be encoded, so
// each unit is read twice: once for its statistics and once to encode it.
// This kernel makes the second read come mostly from the Infinity Cache and
// runs the statistics of later units beside the encoding of earlier ones:
//
//   * one launch of ordinary (non-persistent) workgroups; the grid is a
//     sequence of segments, segment s holding the statistics tiles of unit s
//     followed by the quantize tiles of unit s - depth;
//   * a statistics tile reads 512 rows of one head with ordinary loads (the
//     lines stay in the Infinity Cache) and publishes per-channel partials;
//     the last tile of a head reduces the head (mean, head maximum), the last
//     head of a unit sets the unit's tensor scales and raises its ready words;
//   * a quantize tile waits for its unit's ready word (one lane polls one of
//     32 copies, with ~1 us back-off), reads the head's means, then re-reads
//     its 256 rows and encodes them.
//
// A quantize tile waits only for statistics tiles of an earlier segment,
// i.e. of lower workgroup index, and statistics tiles never wait; with
// in-order dispatch those are resident or finished whenever the quantize
// tile runs, so the waits cannot cycle.  They are nevertheless bounded: on
// time-out the error word is raised and the tile leaves (results invalid).
//
// Partials and per-unit results that other workgroups of the same launch read
// are written with agent-scope atomic exchanges (performed at the device's
// coherence point, not in one XCD's L2) and read with agent-scope atomic
// loads; see the hand-off notes in nvfp4_device.hpp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "kv_overlap.hpp"
#include "lowbit_device.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {

void launch_choice_reduce(const uint32_t* tally, size_t nslots, unsigned long long* choice, hipStream_t s);

namespace {

constexpr int kD = 128;                               // head dimension of this form
constexpr int kNB = kD / 16;                          // blocks per row
constexpr int kHalves = kD / 8;                       // 16-byte halves per row
constexpr int kSRowsPerPass = kOvThreads / kHalves;   // 16
constexpr int kQRowsPerPass = kOvThreads / kNB;       // 32
constexpr int kSBatch = 4;                            // rows in flight per statistics lane
constexpr int kSBatchSmall = 8;                       // the same in calls of at most kOvAheadUnits units
constexpr int kQBatch = 2;                            // rows in flight per quantize lane
constexpr int kReplicaStride = 32;                    // 64-bit words between ready words (256 B)
constexpr int kWaves = kOvThreads / 64;
// K channel sums: each lane adds its rows in fp32 runs of kRunRows = 8 rows
// (8 / SB batches of SB rows) and folds every run into fp64.  A
// run of n rows has at most n - 1 fp32 roundings, each at most 2^-24 of the
// run's magnitude sum, so the channel sum is within 7 * 2^-24 * sum |K| of
// the exact one and the rounded mean within 8 * 2^-24 * max(|m|, mean |K|):
// inside the 1e-6 acceptance of the mean, at a quarter of the per-element
// issue cost of fp64 adds (the fp32 -> fp64 convert is a half-rate
// instruction).
constexpr int kRunRows = 8;

__device__ __forceinline__ unsigned long long load64_agent(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_u32(uint32_t* p, uint32_t v, uint32_t& done) {
  done ^= __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Tile {
  int stats;    // 1: statistics tile, 0: quantize tile
  int u, h, t;  // unit, head, tile within the head
  unsigned q;   // quantize tile index over the whole launch (tally slot)
};

// Workgroup index -> tile.  Segment s (s = 0 .. U - 1 + depth) holds the
// statistics tiles of unit s (if s < U), then the quantize tiles of unit
// s - depth (if 0 <= s - depth < U); tiles of a unit run head by head.
// Putting a segment's statistics tiles first gets them dispatched, and the
// unit ready, as early as possible.  The host keeps the grid (and so every
// index here) below 2^24; the lookup is closed-form (segment_of), so its cost
// does not grow with the number of units.
__device__ __forceinline__ Tile decode(const OverlapParams& p, unsigned b) {
  const int U = 2 * p.nc;
  const unsigned NS = (unsigned)p.H * p.nst, NQ = (unsigned)p.H * p.nqt;
  int s;
  unsigned off;
  segment_of(b, U, p.depth, NS, NQ, s, off);
  const unsigned ns = s < U ? NS : 0u;
  Tile t;
  t.stats = off < ns;
  if (t.stats) {
    t.u = s; t.h = (int)(off / p.nst); t.t = (int)(off % p.nst); t.q = 0;
  } else {
    const unsigned j = off - ns;
    t.u = s - p.depth; t.h = (int)(j / p.nqt); t.t = (int)(j % p.nqt); t.q = (unsigned)t.u * NQ + j;
  }
  return t;
}

// Largest of the two bf16 magnitudes held in the halves of m (bits with the
// sign cleared), as fp32.
__device__ __forceinline__ float bf16x2_max_mag(uint32_t m) {
  const uint32_t lo = m & 0xffffu, hi = m >> 16;
  return __uint_as_float((lo > hi ? lo : hi) << 16);
}

// ------------------------------------------------------------ statistics ---

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Buffer resource over one (chunk, head) slab of rows (gfx9 descriptor:
// raw byte addressing, no swizzle; loads past `bytes` return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const uint16_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, (int)bytes, 0x00020000);
}

// One lane's 16 bytes of rows r, r + 16, ..., r + 112 of a slab: byte
// voff + sb + 4096 q for row r + 16 q (voff: the lane's offset, sb: the
// batch's first row, uniform).  With GUARD, only rows below r1.
template <int SB, bool GUARD>
__device__ __forceinline__ void load_batch(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t sb, int r, int r1,
                                           uint4 (&a)[SB]) {
#pragma unroll
  for (int q = 0; q < SB; ++q) {
    if (!GUARD || r + q * kSRowsPerPass < r1) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, sb + q * kSRowsPerPass * kD * 2, 0);
      a[q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads of the batch in flight before any use
}

// K statistics of one batch: fp32 channel sums of the batch's rows added to
// the running fp32 run sums r (a lane folds them into fp64 every
// kRunRows rows), channel max and min.
template <int SB, bool GUARD>
__device__ __forceinline__ void k_stats_batch(const uint4 (&a)[SB], int r, int r1, float (&rs)[8],
                                              float (&mx)[8], float (&mn)[8]) {
#pragma unroll
  for (int q = 0; q < SB; ++q) {
    if (GUARD && r + q * kSRowsPerPass >= r1) continue;
    const uint32_t w[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
      rs[2 * j] += lo;
      rs[2 * j + 1] += hi;
      mx[2 * j] = fmaxf(mx[2 * j], lo); mn[2 * j] = fminf(mn[2 * j], lo);
      mx[2 * j + 1] = fmaxf(mx[2 * j + 1], hi); mn[2 * j + 1] = fminf(mn[2 * j + 1], hi);
    }
    if (q & 1) __builtin_amdgcn_sched_barrier(0);  // two rows at a time: bounded live values
  }
}

// fp64 channel sums += the fp32 run sums, which restart from 0.
__device__ __forceinline__ void fold_runs(double (&s)[8], float (&rs)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] += (double)rs[i];
    rs[i] = 0.0f;
  }
}

// V statistics of one batch: the largest magnitude, on the bf16 bit
// patterns (with the sign cleared, the integer order of two bf16 magnitudes
// is their numeric order), two values per 16-bit lane of am.
template <int SB, bool GUARD>
__device__ __forceinline__ void v_stats_batch(const uint4 (&a)[SB], int r, int r1, u16x2& am) {
#pragma unroll
  for (int q = 0; q < SB; ++q) {
    if (GUARD && r + q * kSRowsPerPass >= r1) continue;
    const uint32_t w[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x2 m;
      __builtin_memcpy(&m, &w[j], 4);
      m &= (unsigned short)0x7fff;
      am = __builtin_elementwise_max(am, m);
    }
  }
}

// One (unit, head, tile) statistics task.  Lane t reads the 16-byte half
// t % 16 (channels 8 (t % 16) ..) of rows r0 + t / 16, + 16, + 32, ...
// K: fp64 channel sums and channel max / min; V: the largest magnitude.
// SB: rows each lane has in flight.
template <int MODE, int BITS, int SB>
__device__ void stats_tile(const OverlapParams& p, int u, int h, int ts, double* shs, uint32_t* shx, float* shw,
                           unsigned* sh_flag) {
  const int c = u % p.nc, tau = u / p.nc;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hc = tid % kHalves, roff = tid / kHalves;
  const int r0 = ts * kOvStatsRows;
  const int r1 = min(r0 + kOvStatsRows, p.L);
  const __amdgpu_buffer_rsrc_t rs = slab_rsrc(p.x[tau] + ((size_t)h * p.T + (size_t)c * p.L) * kD, (uint32_t)p.L * kD * 2);
  const uint32_t voff = (uint32_t)(roff * kD + hc * 8) * 2;
  const size_t tile = ((size_t)c * p.H + h) * p.nst + ts;
  constexpr int kBatchRows = SB * kSRowsPerPass;
  constexpr int kRunBatches = kRunRows / SB;
  static_assert(kRunBatches * SB == kRunRows, "whole batches per fp32 run");
  const int nfull = (r1 - r0) / kBatchRows;  // whole batches: no per-row guard
  const int rrest = r0 + nfull * kBatchRows;
  uint32_t done = 0;

  if (tau == 0) {
    double s[8];
    float run[8], mx[8], mn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { s[i] = 0.0; run[i] = 0.0f; mx[i] = -INFINITY; mn[i] = INFINITY; }
    // whole batches unguarded (no per-row branch, so the compiler keeps the
    // running max / min as plain v_max3 / v_min3), then one guarded batch
    uint4 ld[SB];
    for (int b = 0; b < nfull; ++b) {
      load_batch<SB, false>(rs, voff, (uint32_t)(r0 + b * kBatchRows) * kD * 2, 0, 0, ld);
      k_stats_batch<SB, false>(ld, 0, 0, run, mx, mn);
      if (b % kRunBatches == kRunBatches - 1) fold_runs(s, run);
    }
    // the open run holds at most kRunBatches - 1 batches, so the guarded
    // batch keeps it within kRunRows rows
    if (rrest + roff < r1) {
      load_batch<SB, true>(rs, voff, (uint32_t)rrest * kD * 2, rrest + roff, r1, ld);
      k_stats_batch<SB, true>(ld, rrest + roff, r1, run, mx, mn);
    }
    fold_runs(s, run);
    // the 4 rows of a wave (lanes hc, hc + 16, hc + 32, hc + 48), in a fixed order
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s[i] += __shfl_xor(s[i], 16, 64);
      s[i] += __shfl_xor(s[i], 32, 64);
      mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], 16, 64));
      mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], 32, 64));
      mn[i] = fminf(mn[i], __shfl_xor(mn[i], 16, 64));
      mn[i] = fminf(mn[i], __shfl_xor(mn[i], 32, 64));
    }
    if (lane < kHalves) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        shs[wv * kD + hc * 8 + i] = s[i];
        // max and min are bf16 values: both fit one word exactly
        shx[wv * kD + hc * 8 + i] = (__float_as_uint(mx[i]) & 0xffff0000u) | (__float_as_uint(mn[i]) >> 16);
      }
    }
    __syncthreads();
    if (tid < kD) {
      double acc = 0.0;
      float a = -INFINITY, b = INFINITY;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        acc += shs[q * kD + tid];
        const uint32_t e = shx[q * kD + tid];
        a = fmaxf(a, __uint_as_float(e & 0xffff0000u));
        b = fminf(b, __uint_as_float(e << 16));
      }
      publish(&p.ksum[tile * kD + tid], acc, done);
      publish_u32(&p.kext[tile * kD + tid], (__float_as_uint(a) & 0xffff0000u) | (__float_as_uint(b) >> 16), done);
    }
  } else {
    u16x2 am = {0, 0};
    uint4 ld[SB];
    for (int b = 0; b < nfull; ++b) {
      load_batch<SB, false>(rs, voff, (uint32_t)(r0 + b * kBatchRows) * kD * 2, 0, 0, ld);
      v_stats_batch<SB, false>(ld, 0, 0, am);
    }
    if (rrest + roff < r1) {
      load_batch<SB, true>(rs, voff, (uint32_t)rrest * kD * 2, rrest + roff, r1, ld);
      v_stats_batch<SB, true>(ld, rrest + roff, r1, am);
    }
    uint32_t amw;
    __builtin_memcpy(&amw, &am, 4);
    float a = wave_max(bf16x2_max_mag(amw));
    if (lane == 0) shw[wv] = a;
    __syncthreads();
    if (tid == 0) {
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) m = fmaxf(m, shw[q]);
      publish(&p.vmax[tile], m, done);
    }
  }

  // The last tile of the head reduces the head; the last head of the unit
  // sets the tensor scales and raises the unit's ready words.
  wait_published(done);
  __syncthreads();  // every thread's exchanges completed before thread 0 counts
  if (tid == 0) *sh_flag = add_agent(&p.cnt_head[(size_t)u * p.H + h], 1u) == (unsigned)(p.nst - 1);
  __syncthreads();
  if (!*sh_flag) return;
  float a = 0.0f;
  const size_t hb = ((size_t)c * p.H + h) * p.nst;
  if (tau == 0) {
    // thread t: channel t % 128 over tiles t / 128, t / 128 + 2, ... (loads in
    // batches of 8), then the two parts combined in a fixed order
    const int d = tid % kD, part = tid / kD;
    double sum = 0.0;
    float mxv = -INFINITY, mnv = INFINITY;
    for (int jb = part; jb < p.nst; jb += 2 * 8) {
      double ps[8];
      uint32_t pe[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int jj = jb + 2 * q;
        if (jj < p.nst) {
          const size_t i = (hb + jj) * kD + d;
          ps[q] = fetch(&p.ksum[i]);
          pe[q] = fetch_u32(&p.kext[i]);
        } else {
          ps[q] = 0.0;
          pe[q] = 0xff807f80u;  // max -inf, min +inf
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        sum += ps[q];
        mxv = fmaxf(mxv, __uint_as_float(pe[q] & 0xffff0000u));
        mnv = fminf(mnv, __uint_as_float(pe[q] << 16));
      }
    }
    __syncthreads();
    shs[tid] = sum;
    shx[tid] = (__float_as_uint(mxv) & 0xffff0000u) | (__float_as_uint(mnv) >> 16);
    __syncthreads();
    if (tid < kD) {
      const double s2 = shs[tid] + shs[kD + tid];
      const uint32_t e0 = shx[tid], e1 = shx[kD + tid];
      const float x2 = fmaxf(__uint_as_float(e0 & 0xffff0000u), __uint_as_float(e1 & 0xffff0000u));
      const float n2 = fminf(__uint_as_float(e0 << 16), __uint_as_float(e1 << 16));
      const float m = (float)(s2 / (double)p.L);
      p.kmean[((size_t)c * p.H + h) * kD + tid] = m;  // output only: visible at kernel end
      publish(&p.mcopy[((size_t)c * p.H + h) * kD + tid], m, done);
      const float up = x2 - m, dn = m - n2;  // each one fp32 rounding
      a = fmaxf(up, dn);
    }
  } else {
    for (int jj = tid; jj < p.nst; jj += kOvThreads) a = fmaxf(a, fetch(&p.vmax[hb + jj]));
  }
  a = wave_max(a);
  wait_published(done);  // this thread's mean exchanges
  __syncthreads();
  if (lane == 0) shw[wv] = a;
  __syncthreads();
  if (tid == 0) {
    float hm = 0.0f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) hm = fmaxf(hm, shw[q]);
    uint32_t d0 = 0;
    publish(&p.hamax[(size_t)u * p.H + h], hm, d0);
    wait_published(d0);
    *sh_flag = add_agent(&p.cnt_unit[u], 1u) == (unsigned)(p.H - 1);
  }
  __syncthreads();
  if (!*sh_flag) return;
  float A = 0.0f;
  for (int hh = tid; hh < p.H; hh += kOvThreads) A = fmaxf(A, fetch(&p.hamax[(size_t)u * p.H + hh]));
  A = wave_max(A);
  __syncthreads();
  if (lane == 0) shw[wv] = A;
  __syncthreads();
  if (tid < kOvReplicas) {
    float Am = 0.0f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) Am = fmaxf(Am, shw[q]);
    float C;  // the tensor constant of the element format
    if constexpr (BITS == 4)
      C = mode_constant(MODE);
    else
      C = lowbit_constant<BITS>(MODE);
    const float g = Am > 0.0f ? C / Am : 0.0f;
    if (tid == 0) p.tscale[tau][c] = Am / C;  // output only: visible at kernel end
    (void)__hip_atomic_exchange(p.ready + ((size_t)tid * (2 * p.nc) + u) * kReplicaStride,
                                (1ull << 32) | __float_as_uint(g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// -------------------------------------------------------------- quantize ---

// One (unit, head, tile) quantize task: wait for the unit, then encode rows
// r0 .. r0 + 255 of the head.  Lane (roff, col) takes rows r0 + roff,
// + 32, ... of column block col.  NVFP4 (BITS = 4) or the 3-bit / 2-bit
// cache.
template <int MODE, int BITS>
__device__ void quant_tile(const OverlapParams& p, int u, int h, int qt, unsigned qidx, float* sh_mean,
                           float* shw, unsigned* sh_flag, const float2* tab, unsigned* sh_tally) {
  const int c = u % p.nc, tau = u / p.nc;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const unsigned long long* rw =
        p.ready + ((size_t)(blockIdx.x % kOvReplicas) * (2 * p.nc) + u) * kReplicaStride;
    unsigned long long w = load64_agent(rw);
    unsigned it = 0;
    bool ok = true;
    while ((w >> 32) == 0ull) {
      ++it;
      if (it > p.spin_limit || ((it & 255u) == 0u && load_agent(p.err) != 0u)) {
        atomicOr(p.err, 1u);
        atomicOr(p.err_sticky, 1u);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(32);  // about 1 us: every poll is a device-scope access to a shared word
      w = load64_agent(rw);
    }
    *sh_flag = ok ? 1u : 0u;
    shw[0] = __uint_as_float((uint32_t)w);
  }
  __syncthreads();  // also orders the scale table's fill before its first use
  if (!*sh_flag) return;
  const float g = shw[0];
  const int col = tid % kNB, roff = tid / kNB;
  float m[16];
  if (tau == 0) {
    // an ordinary load is safe here: the block holds only this (chunk,
    // head)'s means, which were published before the ready word, and no
    // workgroup reads it earlier, so no L2 holds a stale copy of it
    if (tid < kD) sh_mean[tid] = p.mcopy[((size_t)c * p.H + h) * kD + tid];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) m[i] = sh_mean[col * 16 + i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) m[i] = 0.0f;
  }
  const int r0 = qt * kOvQuantRows;
  const int r1 = min(r0 + kOvQuantRows, p.L);
  const size_t row0 = (size_t)h * p.T + (size_t)c * p.L;
  uint2 n;
  constexpr int kRows = kOvQuantRows / kQRowsPerPass;  // rows per lane in a full tile
  if constexpr (BITS == 4) {
    if (p.ahead && r1 - r0 == kOvQuantRows)
      n = tau == 0 ? quant_rows_ahead<MODE, true, kRows, kNB>(p.x[0], p.codes[0], p.scales[0], row0, r0 + roff,
                                                              kQRowsPerPass, col, m, g, tab)
                   : quant_rows_ahead<MODE, false, kRows, kNB>(p.x[1], p.codes[1], p.scales[1], row0, r0 + roff,
                                                               kQRowsPerPass, col, m, g, tab);
    else
      n = tau == 0 ? quant_rows<MODE, true, true, kQBatch, kNB>(p.x[0], p.codes[0], p.scales[0], row0, r0 + roff,
                                                               r1, kQRowsPerPass, kNB, col, m, g, tab)
                   : quant_rows<MODE, false, true, kQBatch, kNB>(p.x[1], p.codes[1], p.scales[1], row0, r0 + roff,
                                                                r1, kQRowsPerPass, kNB, col, m, g, tab);
  } else
    n = tau == 0 ? lowbit_quant_rows<BITS, MODE, true, kNB>(p.x[0], p.codes[0], p.scales[0], row0, r0 + roff, r1,
                                                           kQRowsPerPass, kNB, col, m, g, tab)
                 : lowbit_quant_rows<BITS, MODE, false, kNB>(p.x[1], p.codes[1], p.scales[1], row0, r0 + roff, r1,
                                                            kQRowsPerPass, kNB, col, m, g, tab);
  if (p.choice) {
    const unsigned t[4] = {tau == 0 ? n.x : 0u, tau == 0 ? n.y : 0u, tau == 1 ? n.x : 0u, tau == 1 ? n.y : 0u};
    store_wg_tally(p.tally + (size_t)qidx * 4, t, sh_tally);
  }
}

}  // namespace

template <int MODE, int BITS>
__global__ __launch_bounds__(kOvThreads) void kv_overlap_kernel(OverlapParams p) {
  __shared__ double shs[kWaves * kD];
  __shared__ uint32_t shx[kWaves * kD];
  __shared__ float sh_mean[kD];
  __shared__ float shw[kWaves];
  __shared__ unsigned sh_flag;
  __shared__ float2 sh_tab[128];
  __shared__ unsigned sh_tally[4 * kWaves];
  const Tile t = decode(p, blockIdx.x);
  if (t.stats) {
    // calls of few units have little else to overlap the statistics with:
    // more rows in flight per lane (4-bit only: the low-bit encode would
    // lose a wave per SIMD to the extra registers)
    if (BITS == 4 && p.ahead)
      stats_tile<MODE, BITS, kSBatchSmall>(p, t.u, t.h, t.t, shs, shx, shw, &sh_flag);
    else
      stats_tile<MODE, BITS, kSBatch>(p, t.u, t.h, t.t, shs, shx, shw, &sh_flag);
  } else {
    fill_scale_table(sh_tab);
    quant_tile<MODE, BITS>(p, t.u, t.h, t.t, t.q, sh_mean, shw, &sh_flag, sh_tab, sh_tally);
  }
}

// ------------------------------------------------------------- host side ---

OverlapLayout overlap_layout(int H, int nc, int nst, int nqt) {
  OverlapLayout l;
  const int U = 2 * nc;
  const size_t part = (size_t)nc * H * nst * kD;
  size_t off = kKvWorkspaceHeader;  // the sticky error word's block
  l.ksum = off;   off = align_up(off + part * sizeof(double), 256);
  l.kext = off;   off = align_up(off + part * sizeof(uint32_t), 256);
  l.vmax = off;   off = align_up(off + (size_t)nc * H * nst * sizeof(float), 256);
  l.hamax = off;  off = align_up(off + (size_t)U * H * sizeof(float), 256);
  l.mcopy = off;  off = align_up(off + (size_t)nc * H * kD * sizeof(float), 256);
  l.tally = off;  off = align_up(off + (size_t)U * H * nqt * 4 * sizeof(uint32_t), 256);
  // cleared before each launch: ready words, then cnt_head [U][H], cnt_unit [U], err
  l.ready = off;  off += (size_t)U * kOvReplicas * kReplicaStride * sizeof(unsigned long long);
  l.counters = off;
  off += ((size_t)U * H + U + 1) * sizeof(unsigned);
  l.n_zero_words = (int)((off - l.ready) / sizeof(unsigned));
  l.total = align_up(off, 256);
  return l;
}

size_t overlap_workspace_bound(int H, int T, int D, int L) {
  if (D != kD || H <= 0 || L <= 0 || T % L != 0) return 0;
  const int nst = (L + kOvStatsRows - 1) / kOvStatsRows;
  const int nqt = (L + kOvQuantRows - 1) / kOvQuantRows;
  return overlap_layout(H, T / L, nst, nqt).total;
}

__global__ void overlap_zero_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <int BITS>
static void launch_overlap(const OverlapParams& p, int mode, unsigned grid, hipStream_t s) {
  switch (mode) {
    case kModeFixed6: kv_overlap_kernel<kModeFixed6, BITS><<<grid, kOvThreads, 0, s>>>(p); break;
    case kModeFixed4: kv_overlap_kernel<kModeFixed4, BITS><<<grid, kOvThreads, 0, s>>>(p); break;
    default: kv_overlap_kernel<kMode4over6, BITS><<<grid, kOvThreads, 0, s>>>(p); break;
  }
}

int overlap_try_launch(OverlapParams p, int mode, int bits, void* workspace, size_t ws_bytes,
                       unsigned long long* choice, unsigned* err_word, hipStream_t s) {
  if (p.H <= 0 || p.nc <= 0 || p.L <= 0 || (bits != 4 && bits != 3 && bits != 2)) return 1;
  p.nst = (p.L + kOvStatsRows - 1) / kOvStatsRows;
  p.nqt = (p.L + kOvQuantRows - 1) / kOvQuantRows;
  const int U = 2 * p.nc;
  const long long grid = (long long)U * p.H * ((long long)p.nst + p.nqt);
  if (grid >= (1LL << 24)) return 1;  // work-items of a launch (and tile indices) stay in 32 bits
  if ((long long)p.L * kD * 2 >= (1LL << 31)) return 1;  // statistics buffer offsets stay in 31 bits
  const OverlapLayout l = overlap_layout(p.H, p.nc, p.nst, p.nqt);
  if (l.total > ws_bytes) return 1;
  char* ws = static_cast<char*>(workspace);
  p.ksum = reinterpret_cast<double*>(ws + l.ksum);
  p.kext = reinterpret_cast<uint32_t*>(ws + l.kext);
  p.vmax = reinterpret_cast<float*>(ws + l.vmax);
  p.hamax = reinterpret_cast<float*>(ws + l.hamax);
  p.mcopy = reinterpret_cast<float*>(ws + l.mcopy);
  p.tally = reinterpret_cast<uint32_t*>(ws + l.tally);
  p.ready = reinterpret_cast<unsigned long long*>(ws + l.ready);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws + l.counters);
  p.cnt_head = cnt;
  p.cnt_unit = cnt + (size_t)U * p.H;
  p.err = p.cnt_unit + U;
  p.err_sticky = err_word;
  p.choice = choice != nullptr;
  p.depth = kOvDepth;
  p.ahead = U <= kOvAheadUnits ? 1 : 0;
  p.spin_limit = kOvSpinLimit;
  overlap_zero_kernel<<<(l.n_zero_words + 255) / 256, 256, 0, s>>>(reinterpret_cast<unsigned*>(ws + l.ready),
                                                                  l.n_zero_words);
  if (bits == 3)
    launch_overlap<3>(p, mode, (unsigned)grid, s);
  else if (bits == 2)
    launch_overlap<2>(p, mode, (unsigned)grid, s);
  else
    launch_overlap<4>(p, mode, (unsigned)grid, s);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  if (choice) {
    launch_choice_reduce(p.tally, (size_t)U * p.H * p.nqt, choice, s);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  }
  return NVFP4_OK;
}

}  // namespace nvfp4
