// kv_pipe.hip -- persistent, overlapped form of the per-chunk K smoothing +
// NVFP4 4/6 quantization (LongLive-2.0 summary page: inference pipeline,
// step 7; full-stack NVFP4).
//
// A unit is one (chunk, tensor): u = 2 * chunk + tensor, K before V.  The
// tensor scale of a unit needs the unit's largest |K - mean| (or |V|) before
// any of its blocks can be encoded, so every unit is read twice: once for
// its statistics and once to encode it.  The second read comes from the
// Infinity Cache when it follows the first closely enough, which is what
// this kernel arranges:
//
//   * one cooperative launch; every workgroup stays resident;
//   * each workgroup first takes its statistics tiles of unit u + 1, read
//     from HBM with ordinary loads (so the lines stay in the Infinity
//     Cache), and publishes per-tile channel partials; the last tile of a
//     head reduces the head (mean, head maximum), the last head of a unit
//     sets the unit's tensor scales and ready flag;
//   * then it waits for unit u's flag and takes its quantize tiles of unit
//     u, re-reading them (cache hits) and encoding them.
//
// Unit u's statistics finish one whole step before its quantization starts,
// so each device-wide hand-off has that much slack, and at most about two
// units are in flight (the cache footprint).  Every wait is bounded: on
// time-out a workgroup raises the error word and leaves, so no wave can
// hang; the results are then invalid.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "kv_fused.hpp"
#include "kv_pipe.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kD = 128;                  // head dimension of this form
constexpr int kNB = kD / 16;             // blocks per row
constexpr int kHalves = kD / 8;          // 16-byte halves per row
constexpr int kStatsRowsPerPass = kPipeThreads / kHalves;
constexpr int kQuantRowsPerPass = kPipeThreads / kNB;
constexpr int kStatsBatch = 8;           // rows in flight per statistics lane
constexpr int kQuantBatch = 2;           // rows in flight per quantize lane

// Bounded wait until *word >= target (one lane polls); false on time-out or
// when another workgroup has raised the error word.
__device__ bool wait_at_least(const PipeParams& p, const unsigned* word, unsigned target) {
  unsigned it = 0;
  while (load_agent(word) < target) {
    if (load_agent(p.err) != 0u || ++it > p.spin_limit) {
      atomicOr(p.err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  return true;
}

// ------------------------------------------------------------ statistics ---

// One (unit, head, tile) statistics task.  Lane t reads the 16-byte half t %
// 16 (channels 8 * (t % 16) ..) of row t / 16 of each of the tile's passes.
// K: fp64 channel sums and fp32 maxima / minima; V: the largest magnitude.
template <bool NT>
__device__ void stats_task(const PipeParams& p, int u, int h, int ts, double* shs, float* shx, float* shn,
                           float* shw, unsigned* sh_flag) {
  const int c = u >> 1, tau = u & 1;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int hc = tid % kHalves, roff = tid / kHalves;
  // tile ts of a head takes the 16-row passes ts, ts + nst, ts + 2 nst, ...:
  // the tiles of a head, running side by side, read adjacent 4 KB blocks
  const int step = p.nst * kStatsRowsPerPass;
  const int r0 = ts * kStatsRowsPerPass;
  const uint16_t* base = p.x[tau] + ((size_t)h * p.T + (size_t)c * p.L) * kD + hc * 8;
  const size_t tile = ((size_t)c * p.H + h) * p.nst + ts;
  uint32_t done = 0;

  if (tau == 0) {
    double s[8];
    float mx[8], mn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { s[i] = 0.0; mx[i] = -INFINITY; mn[i] = INFINITY; }
    for (int rb = r0 + roff; rb < p.L; rb += kStatsBatch * step) {
      uint4 a[kStatsBatch];
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q) {
        const int r = rb + q * step;
        if (r < p.L) a[q] = load16<NT>(base + (size_t)r * kD);
      }
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q) {
        if (rb + q * step >= p.L) continue;
        const uint32_t w[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
          s[2 * j] += (double)lo;
          s[2 * j + 1] += (double)hi;
          mx[2 * j] = fmaxf(mx[2 * j], lo); mn[2 * j] = fminf(mn[2 * j], lo);
          mx[2 * j + 1] = fmaxf(mx[2 * j + 1], hi); mn[2 * j + 1] = fminf(mn[2 * j + 1], hi);
        }
      }
    }
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
    __syncthreads();  // the LDS may still be read by the previous task
    if (lane < kHalves) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        shs[wv * kD + hc * 8 + i] = s[i];
        shx[wv * kD + hc * 8 + i] = mx[i];
        shn[wv * kD + hc * 8 + i] = mn[i];
      }
    }
    __syncthreads();
    if (tid < kD) {
      double acc = 0.0;
      float a = -INFINITY, b = INFINITY;
      for (int q = 0; q < kPipeThreads / 64; ++q) {
        acc += shs[q * kD + tid];
        a = fmaxf(a, shx[q * kD + tid]);
        b = fminf(b, shn[q * kD + tid]);
      }
      publish(&p.psum[tile * kD + tid], acc, done);
      publish(&p.pmax[tile * kD + tid], a, done);
      publish(&p.pmin[tile * kD + tid], b, done);
    }
  } else {
    float am = 0.0f;
    for (int rb = r0 + roff; rb < p.L; rb += kStatsBatch * step) {
      uint4 a[kStatsBatch];
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q) {
        const int r = rb + q * step;
        if (r < p.L) a[q] = load16<NT>(base + (size_t)r * kD);
      }
#pragma unroll
      for (int q = 0; q < kStatsBatch; ++q) {
        if (rb + q * step >= p.L) continue;
        const uint32_t w[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) am = fmaxf(am, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
      }
    }
    am = wave_max(am);
    __syncthreads();
    if (lane == 0) shw[wv] = am;
    __syncthreads();
    if (tid == 0) {
      float a = 0.0f;
      for (int q = 0; q < kPipeThreads / 64; ++q) a = fmaxf(a, shw[q]);
      publish(&p.pv[tile], a, done);
    }
  }

  // The last tile of the head reduces the head; the last head of the unit
  // sets the tensor scales and raises the unit's flag.
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
      float px[8], pn[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int jj = jb + 2 * q;
        if (jj < p.nst) {
          const size_t i = (hb + jj) * kD + d;
          ps[q] = fetch(&p.psum[i]); px[q] = fetch(&p.pmax[i]); pn[q] = fetch(&p.pmin[i]);
        } else {
          ps[q] = 0.0; px[q] = -INFINITY; pn[q] = INFINITY;
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) { sum += ps[q]; mxv = fmaxf(mxv, px[q]); mnv = fminf(mnv, pn[q]); }
    }
    __syncthreads();
    shs[tid] = sum;
    shx[tid] = mxv;
    shn[tid] = mnv;
    __syncthreads();
    if (tid < kD) {
      const double s2 = shs[tid] + shs[kD + tid];
      const float x2 = fmaxf(shx[tid], shx[kD + tid]), n2 = fminf(shn[tid], shn[kD + tid]);
      const float m = (float)(s2 / (double)p.L);
      publish(&p.kmean[((size_t)c * p.H + h) * kD + tid], m, done);
      const float up = x2 - m, dn = m - n2;  // each one fp32 rounding
      a = fmaxf(up, dn);
    }
  } else {
    for (int jj = tid; jj < p.nst; jj += kPipeThreads) a = fmaxf(a, fetch(&p.pv[hb + jj]));
  }
  a = wave_max(a);
  wait_published(done);  // this thread's k_mean exchanges
  __syncthreads();
  if (lane == 0) shw[wv] = a;
  __syncthreads();
  if (tid == 0) {
    float hm = 0.0f;
    for (int q = 0; q < kPipeThreads / 64; ++q) hm = fmaxf(hm, shw[q]);
    uint32_t d0 = 0;
    publish(&p.hamax[(size_t)u * p.H + h], hm, d0);
    wait_published(d0);
    *sh_flag = add_agent(&p.cnt_unit[u], 1u) == (unsigned)(p.H - 1);
  }
  __syncthreads();
  if (!*sh_flag) return;
  float A = 0.0f;
  for (int hh = tid; hh < p.H; hh += kPipeThreads) A = fmaxf(A, fetch(&p.hamax[(size_t)u * p.H + hh]));
  A = wave_max(A);
  __syncthreads();
  if (lane == 0) shw[wv] = A;
  __syncthreads();
  if (tid == 0) {
    float Am = 0.0f;
    for (int q = 0; q < kPipeThreads / 64; ++q) Am = fmaxf(Am, shw[q]);
    const float C = mode_constant(p.mode);
    uint32_t d0 = 0;
    publish(&p.genc[u], Am > 0.0f ? C / Am : 0.0f, d0);
    p.tscale[tau][c] = Am / C;  // output only: visible at kernel end
    wait_published(d0);
    store_agent(&p.flag[u], 1u);
  }
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(kPipeThreads) void kv_pipe_kernel(PipeParams p) {
  __shared__ double shs[(kPipeThreads / 64) * kD];
  __shared__ float shx[(kPipeThreads / 64) * kD];
  __shared__ float shn[(kPipeThreads / 64) * kD];
  __shared__ float sh_mean[kD];
  __shared__ float shw[kPipeThreads / 64];
  __shared__ unsigned sh_flag;
  __shared__ float2 sh_tab[128];
  const int tid = threadIdx.x;
  const long long b = blockIdx.x, G = gridDim.x;
  fill_scale_table(sh_tab);
  __syncthreads();
  const int U = 2 * p.nc;
  const long long ns = (long long)p.H * p.nst, nq = (long long)p.H * p.nqt;
  const int col = tid % kNB, roff = tid / kNB;
  unsigned t4[4] = {0u, 0u, 0u, 0u};
  bool ok = true;

  // Step u (u = 0 .. U) deals out, round-robin over the workgroups, one
  // index space: the statistics tiles of unit u (if u < U) first, then the
  // quantize tiles of unit u - 1 (if u > 0).  A workgroup therefore finishes
  // all its statistics tiles of a step before it waits for unit u - 1's
  // flag, and unit u - 1's flag depends only on statistics tiles of the
  // previous step, so the waits cannot cycle; every workgroup gets about the
  // same number of tiles per step.
  for (int u = 0; u <= U && ok; ++u) {
    const long long ss = u < U ? ns : 0, qq = u > 0 ? nq : 0;
    const int uq = u - 1, c = uq >> 1, tau = uq & 1;
    bool waited = false;
    float g = 0.0f;
    int cur_h = -1;
    for (long long t = b; t < ss + qq; t += G) {
      if (t < ss) {
        stats_task<false>(p, u, (int)(t / p.nst), (int)(t % p.nst), shs, shx, shn, shw, &sh_flag);
        continue;
      }
      if (!waited) {
        // one lane waits and reads the encode scale; a device-scope load of
        // one word by every lane of every workgroup would be serialized
        __syncthreads();  // every thread is past its last reads of sh_flag and shw
        if (tid == 0) {
          sh_flag = wait_at_least(p, &p.flag[uq], 1u);
          if (sh_flag) shw[0] = fetch(&p.genc[uq]);
        }
        __syncthreads();
        if (!sh_flag) {
          ok = false;
          break;
        }
        g = shw[0];
        waited = true;
      }
      const long long tq = t - ss;
      const int h = (int)(tq / p.nqt), qt = (int)(tq % p.nqt);
      float m[16];
      if (tau == 0) {
        if (h != cur_h) {  // the head's channel means, through LDS
          __syncthreads();  // the previous head's means may still be read
          if (tid < kD) sh_mean[tid] = fetch(&p.kmean[((size_t)c * p.H + h) * kD + tid]);
          __syncthreads();
          cur_h = h;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) m[i] = sh_mean[col * 16 + i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) m[i] = 0.0f;
      }
      const int r0 = qt * kPipeQuantRows;
      const int r1 = min(r0 + kPipeQuantRows, p.L);
      const size_t row0 = (size_t)h * p.T + (size_t)c * p.L;
      const uint2 n = tau == 0
          ? quant_rows<MODE, true, false, kQuantBatch, kNB>(p.x[0], p.codes[0], p.scales[0], row0, r0 + roff, r1,
                                                            kQuantRowsPerPass, kNB, col, m, g, sh_tab)
          : quant_rows<MODE, false, false, kQuantBatch, kNB>(p.x[1], p.codes[1], p.scales[1], row0, r0 + roff,
                                                             r1, kQuantRowsPerPass, kNB, col, m, g, sh_tab);
      t4[2 * tau] += n.x;
      t4[2 * tau + 1] += n.y;
    }
  }
  if (p.choice) {
    if (ok) {
      store_wg_tally(p.tally + (size_t)b * 4, t4, reinterpret_cast<unsigned*>(shs));
    } else if (tid == 0) {
      *reinterpret_cast<uint4*>(p.tally + (size_t)b * 4) = make_uint4(0, 0, 0, 0);
    }
  }
}

// ------------------------------------------------------------- host side ---

PipeLayout pipe_layout(int H, int nc, int nst) {
  PipeLayout l;
  const int U = 2 * nc;
  const size_t part = (size_t)nc * H * nst * kD;
  size_t off = 0;
  l.psum = off;   off = align_up(off + part * sizeof(double), 256);
  l.pmax = off;   off = align_up(off + part * sizeof(float), 256);
  l.pmin = off;   off = align_up(off + part * sizeof(float), 256);
  l.pv = off;     off = align_up(off + (size_t)nc * H * nst * sizeof(float), 256);
  l.hamax = off;  off = align_up(off + (size_t)U * H * sizeof(float), 256);
  l.genc = off;   off = align_up(off + (size_t)U * sizeof(float), 256);
  l.tally = off;  off = align_up(off + (size_t)kPipeMaxWG * 4 * sizeof(uint32_t), 256);
  l.counters = off;  // cnt_head [U][H], cnt_unit [U], flag [U], err [1]
  l.n_counters = U * H + 2 * U + 1;
  off = align_up(off + (size_t)l.n_counters * sizeof(unsigned), 256);
  l.total = off;
  return l;
}

size_t pipe_workspace_bound(int H, int T, int D, int L) {
  if (D != kD || H <= 0 || L <= 0 || T % L != 0) return 0;
  const int nst = (L + kPipeStatsRows - 1) / kPipeStatsRows;
  return pipe_layout(H, T / L, nst).total;
}

__global__ void pipe_zero_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

static const void* pipe_kernel_ptr(int mode) {
  switch (mode) {
    case kModeFixed6: return reinterpret_cast<const void*>(&kv_pipe_kernel<kModeFixed6>);
    case kModeFixed4: return reinterpret_cast<const void*>(&kv_pipe_kernel<kModeFixed4>);
    default: return reinterpret_cast<const void*>(&kv_pipe_kernel<kMode4over6>);
  }
}

int pipe_try_launch(PipeParams p, void* workspace, size_t ws_bytes, unsigned long long* choice, hipStream_t s) {
  if (p.H <= 0 || p.nc <= 0 || p.L <= 0) return 1;
  int dev = 0, ncu = 0, coop = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return NVFP4_ERR_HIP;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return 1;
  const void* kern = pipe_kernel_ptr(p.mode);
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kPipeThreads, 0) != hipSuccess) return NVFP4_ERR_HIP;
  const int per_cu = occ < kPipeWgPerCu ? occ : kPipeWgPerCu;
  if (per_cu < 1) return 1;
  const int nwg = ncu * per_cu;
  if (nwg > kPipeMaxWG) return 1;
  p.nst = (p.L + kPipeStatsRows - 1) / kPipeStatsRows;
  p.nqt = (p.L + kPipeQuantRows - 1) / kPipeQuantRows;
  const PipeLayout l = pipe_layout(p.H, p.nc, p.nst);
  if (l.total > ws_bytes) return 1;
  char* ws = static_cast<char*>(workspace);
  p.psum = reinterpret_cast<double*>(ws + l.psum);
  p.pmax = reinterpret_cast<float*>(ws + l.pmax);
  p.pmin = reinterpret_cast<float*>(ws + l.pmin);
  p.pv = reinterpret_cast<float*>(ws + l.pv);
  p.hamax = reinterpret_cast<float*>(ws + l.hamax);
  p.genc = reinterpret_cast<float*>(ws + l.genc);
  p.tally = reinterpret_cast<uint32_t*>(ws + l.tally);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws + l.counters);
  const int U = 2 * p.nc;
  p.cnt_head = cnt;
  p.cnt_unit = cnt + (size_t)U * p.H;
  p.flag = p.cnt_unit + U;
  p.err = p.flag + U;
  p.choice = choice != nullptr;
  p.spin_limit = kPipeSpinLimit;
  pipe_zero_kernel<<<(l.n_counters + 255) / 256, 256, 0, s>>>(cnt, l.n_counters);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  void* args[] = {&p};
  if (hipLaunchCooperativeKernel(kern, dim3(nwg), dim3(kPipeThreads), args, 0, s) != hipSuccess) {
    (void)hipGetLastError();
    return NVFP4_ERR_HIP;
  }
  if (choice) {
    launch_choice_reduce(p.tally, nwg, choice, s);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  }
  return NVFP4_OK;
}

}  // namespace nvfp4
