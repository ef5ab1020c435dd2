// kv_fused.hip -- single-read, persistent form of the per-chunk K smoothing +
// NVFP4 4/6 quantization (LongLive-2.0 summary page: inference pipeline,
// step 7; full-stack NVFP4).
//
// The tensor scale of a chunk needs the chunk's largest |K - mean| before any
// block can be encoded, and re-reading a 43 MB tensor-chunk costs as much as
// reading it (the Infinity Cache gives no extra bandwidth for it).  So each
// (chunk, tensor) "unit" is read from HBM once and kept in registers:
//
//   * one persistent workgroup per slot, all co-resident (cooperative launch);
//     workgroup w owns a fixed row slice of head w / WPH for every unit;
//   * per unit: channel statistics of the slice from registers -> workspace;
//     the last workgroup of a head (atomic counter) reduces the head (mean,
//     head maximum), the last head of the unit computes the tensor scales
//     and raises the unit's ready flag;
//   * every workgroup waits for the flag (bounded spin; on time-out it sets
//     an error word and leaves, so no wave can hang), then encodes its slice,
//     refilling each register slot with the next unit's data as soon as the
//     slot is encoded, so HBM reads of unit u+1 overlap the VALU work of u.
//
// Units run K then V of chunk 0, K then V of chunk 1, ...  The arithmetic
// per block is the multi-kernel path's; only the order in which the fp64
// channel sums are combined differs (the mean is rounded to fp32 once).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "kv_fused.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

template <int NB, int BPT, int MODE>
__global__ __launch_bounds__(kFusedThreads, kFusedWavesPerEU) void kv_fused_kernel(FusedParams p) {
  constexpr int RPP = kFusedThreads / NB;  // rows per pass of the workgroup
  __shared__ double sh[16 * (kFusedThreads + 1)];
  __shared__ float shw[kFusedThreads / 64];
  __shared__ float sh_mean[NB * 16];
  __shared__ unsigned sh_flag;
  __shared__ float sh_g;
  __shared__ float2 sh_tab[128];

  const int w = blockIdx.x;
  if (w >= p.WPH * p.H) {  // spare workgroup: owns no rows
    if (p.choice && threadIdx.x == 0) *reinterpret_cast<uint4*>(p.tally + (size_t)w * 4) = make_uint4(0, 0, 0, 0);
    return;
  }
  fill_scale_table(sh_tab);
  __syncthreads();
  const int h = w / p.WPH, j = w % p.WPH;
  const int tid = threadIdx.x, col = tid % NB, roff = tid / NB;
  const int r0 = j * p.RPW;
  const int r1 = min(r0 + p.RPW, p.L);
  const int U = 2 * p.nc;
  const int D = NB * 16;

  uint4 buf[BPT][2];
  unsigned n4[2] = {0u, 0u}, nblk[2] = {0u, 0u};

  auto valid = [&](int k) { return r0 + roff + k * RPP < r1; };
  // slot k of the lane: element offset from the workgroup's first row
  const uint32_t lane_off = (uint32_t)(roff * D + col * 16);
  auto base_of = [&](int u) {  // uniform per unit
    const int c = u >> 1, tau = u & 1;
    return p.x[tau] + ((size_t)h * p.T + (size_t)c * p.L + r0) * D;
  };
  auto src_of = [&](int u, int k) { return base_of(u) + (lane_off + (uint32_t)(k * RPP * D)); };

#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    if (valid(k)) {
      const uint16_t* s = src_of(0, k);
      buf[k][0] = load_nt(s);
      buf[k][1] = load_nt(s + 8);
    } else {
      buf[k][0] = make_uint4(0, 0, 0, 0);
      buf[k][1] = make_uint4(0, 0, 0, 0);
    }
  }

  for (int u = 0; u < U; ++u) {
    const int c = u >> 1, tau = u & 1;
    uint32_t done = 0;  // completion of this thread's published values

    // ---- statistics of this workgroup's slice --------------------------
    if (tau == 0) {
      const int stride = kFusedThreads + 1;
      const size_t pb = (((size_t)c * p.H + h) * p.WPH + j) * D;
      float* shf = reinterpret_cast<float*>(sh);
      __syncthreads();  // the LDS buffer may still be read from the last unit
      // channel sums (fp64), then maxima and minima, 8 channels at a time
      // to keep the register footprint small
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        double s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = 0.0;
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
          if (!valid(k)) continue;
          const uint4 wv = buf[k][half];
          const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            s[2 * q] += (double)bf16_lo(wd[q]);
            s[2 * q + 1] += (double)bf16_hi(wd[q]);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) sh[(8 * half + i) * stride + tid] = s[i];
      }
      __syncthreads();
      for (int d = tid; d < D; d += kFusedThreads) {
        const int cc = d >> 4, i = d & 15;
        double acc = 0.0;
        for (int q = 0; q < RPP; ++q) acc += sh[i * stride + q * NB + cc];
        publish(&p.psum[pb + d], acc, done);
      }
      __syncthreads();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float mx[8], mn[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { mx[i] = -INFINITY; mn[i] = INFINITY; }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
          if (!valid(k)) continue;
          const uint4 wv = buf[k][half];
          const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float a = bf16_lo(wd[q]), b = bf16_hi(wd[q]);
            mx[2 * q] = fmaxf(mx[2 * q], a); mn[2 * q] = fminf(mn[2 * q], a);
            mx[2 * q + 1] = fmaxf(mx[2 * q + 1], b); mn[2 * q + 1] = fminf(mn[2 * q + 1], b);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          shf[(8 * half + i) * stride + tid] = mx[i];
          shf[(16 + 8 * half + i) * stride + tid] = mn[i];
        }
      }
      __syncthreads();
      for (int d = tid; d < D; d += kFusedThreads) {
        const int cc = d >> 4, i = d & 15;
        float a = -INFINITY, b = INFINITY;
        for (int q = 0; q < RPP; ++q) {
          a = fmaxf(a, shf[i * stride + q * NB + cc]);
          b = fminf(b, shf[(16 + i) * stride + q * NB + cc]);
        }
        publish(&p.pmax[pb + d], a, done);
        publish(&p.pmin[pb + d], b, done);
      }
    } else {
      float am = 0.0f;
#pragma unroll
      for (int k = 0; k < BPT; ++k) {
        if (!valid(k)) continue;
        float x[16];
        unpack16(buf[k][0], buf[k][1], x);
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
      }
      am = wave_max(am);
      __syncthreads();
      if ((tid & 63) == 0) shw[tid >> 6] = am;
      __syncthreads();
      if (tid == 0) {
        float a = 0.0f;
        for (int q = 0; q < kFusedThreads / 64; ++q) a = fmaxf(a, shw[q]);
        publish(&p.pv[((size_t)c * p.H + h) * p.WPH + j], a, done);
      }
    }

    // ---- publish: the last workgroup of the head reduces it, the last head
    // of the unit sets the tensor scales and raises the ready flag.  Both
    // reductions spread their loads over all threads (issued in batches
    // before use), since every load after an acquire misses in L2.
    wait_published(done);
    __syncthreads();  // every thread's exchanges completed before thread 0 counts
    if (tid == 0) sh_flag = add_agent(&p.cnt_head[(size_t)u * p.H + h], 1u) == (unsigned)(p.WPH - 1);
    __syncthreads();
    if (sh_flag) {
      float a = 0.0f;
      if (tau == 0) {
        constexpr int NSPLIT = kFusedThreads / D > 0 ? kFusedThreads / D : 1;
        const int d = tid % D, part = tid / D;
        double sum = 0.0;
        float mxv = -INFINITY, mnv = INFINITY;
        const size_t hb = ((size_t)c * p.H + h) * p.WPH;
        for (int jb = part; jb < p.WPH; jb += NSPLIT * 8) {
          double ps[8];
          float px[8], pn[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int jj = jb + q * NSPLIT;
            if (jj < p.WPH) {
              const size_t i = (hb + jj) * D + d;
              ps[q] = fetch(&p.psum[i]); px[q] = fetch(&p.pmax[i]); pn[q] = fetch(&p.pmin[i]);
            } else {
              ps[q] = 0.0; px[q] = -INFINITY; pn[q] = INFINITY;
            }
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) { sum += ps[q]; mxv = fmaxf(mxv, px[q]); mnv = fminf(mnv, pn[q]); }
        }
        // combine the NSPLIT parts of each channel in a fixed order
        const int stride = kFusedThreads + 1;
        float* shf = reinterpret_cast<float*>(sh + 2 * stride);
        sh[tid] = sum;
        shf[tid] = mxv;
        shf[stride + tid] = mnv;
        __syncthreads();
        if (tid < D) {
          double s2 = 0.0;
          float x2 = -INFINITY, n2 = INFINITY;
          for (int q = 0; q < NSPLIT; ++q) {
            s2 += sh[q * D + tid];
            x2 = fmaxf(x2, shf[q * D + tid]);
            n2 = fminf(n2, shf[stride + q * D + tid]);
          }
          const float m = (float)(s2 / (double)p.L);
          publish(&p.kmean[((size_t)c * p.H + h) * D + tid], m, done);
          const float up = x2 - m, dn = m - n2;  // each one fp32 rounding
          a = fmaxf(up, dn);
        }
      } else {
        for (int jj = tid; jj < p.WPH; jj += kFusedThreads) a = fmaxf(a, fetch(&p.pv[((size_t)c * p.H + h) * p.WPH + jj]));
      }
      a = wave_max(a);
      wait_published(done);  // this thread's k_mean exchanges
      __syncthreads();
      if ((tid & 63) == 0) shw[tid >> 6] = a;
      __syncthreads();
      if (tid == 0) {
        float hm = 0.0f;
        for (int q = 0; q < kFusedThreads / 64; ++q) hm = fmaxf(hm, shw[q]);
        uint32_t d0 = 0;
        publish(&p.hamax[(size_t)u * p.H + h], hm, d0);
        wait_published(d0);
        sh_flag = add_agent(&p.cnt_unit[u], 1u) == (unsigned)(p.H - 1);
      }
      __syncthreads();
      if (sh_flag) {  // last head of the unit: tensor scales and the ready flag
        float A = 0.0f;
        for (int hh = tid; hh < p.H; hh += kFusedThreads) A = fmaxf(A, fetch(&p.hamax[(size_t)u * p.H + hh]));
        A = wave_max(A);
        __syncthreads();
        if ((tid & 63) == 0) shw[tid >> 6] = A;
        __syncthreads();
        if (tid == 0) {
          float Am = 0.0f;
          for (int q = 0; q < kFusedThreads / 64; ++q) Am = fmaxf(Am, shw[q]);
          const float C = mode_constant(MODE);
          uint32_t d0 = 0;
          publish(&p.genc[u], Am > 0.0f ? C / Am : 0.0f, d0);
          p.tscale[tau][c] = Am / C;  // output only: visible at kernel end
          wait_published(d0);
          store_agent(&p.flag[u], 1u);
        }
      }
    }

    // ---- wait for the unit's tensor scale (bounded) -------------------------
    if (tid == 0) {
      unsigned ok = 1, it = 0;
      while (load_agent(&p.flag[u]) == 0u) {
        if (load_agent(p.err) != 0u || ++it > p.spin_limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      if (!ok) atomicOr(p.err, 1u);
      sh_flag = ok;
      // one lane reads the encode scale: a device-scope load of one word by
      // every lane of every workgroup would be serialized
      if (ok) sh_g = fetch(&p.genc[u]);
    }
    __syncthreads();
    if (!sh_flag) {  // time-out: results are invalid, the error word says so
      if (p.choice && tid == 0) *reinterpret_cast<uint4*>(p.tally + (size_t)w * 4) = make_uint4(0, 0, 0, 0);
      return;
    }
    const float g = sh_g;
    if (tau == 0) {  // the head's channel means, shared by the workgroup through LDS
      for (int d = tid; d < D; d += kFusedThreads) sh_mean[d] = fetch(&p.kmean[((size_t)c * p.H + h) * D + d]);
      __syncthreads();
    }

    // ---- encode the slice; refill each slot with the next unit ------------
    const bool has_next = u + 1 < U;
    uint8_t* codes = p.codes[tau];
    uint8_t* scales = p.scales[tau];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      if (valid(k)) {
        float z[16];
        unpack16(buf[k][0], buf[k][1], z);
        if (tau == 0) {
          const float4* mp = reinterpret_cast<const float4*>(sh_mean + col * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 mv = mp[q];
            z[4 * q] = z[4 * q] - mv.x;  // k' = fl(K - m)
            z[4 * q + 1] = z[4 * q + 1] - mv.y;
            z[4 * q + 2] = z[4 * q + 2] - mv.z;
            z[4 * q + 3] = z[4 * q + 3] - mv.w;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = z[i] * g;  // z = fl(k' * g_enc)
        const Block46 q = quant_block16<MODE>(z, sh_tab);
        const size_t blk = ((size_t)h * p.T + (size_t)c * p.L + (r0 + roff + k * RPP)) * NB + col;
        store_nt(codes + blk * 8, q.lo, q.hi);
        store_nt(scales + blk, (uint8_t)q.scale);
        n4[tau] += q.use4;
        nblk[tau] += 1;
        if (has_next) {
          const uint16_t* s = src_of(u + 1, k);
          buf[k][0] = load_nt(s);
          buf[k][1] = load_nt(s + 8);
        }
      }
    }
  }

  if (p.choice) {
    const unsigned t[4] = {n4[0], nblk[0], n4[1], nblk[1]};
    store_wg_tally(p.tally + (size_t)blockIdx.x * 4, t, reinterpret_cast<unsigned*>(sh));
  }
}

__global__ void fused_zero_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// ------------------------------------------------------------- host side ---

FusedLayout fused_layout(int H, int nc, int D, int WPH) {
  FusedLayout l;
  const int U = 2 * nc;
  const size_t part = (size_t)nc * H * WPH * D;
  size_t off = 0;
  l.psum = off;     off = align_up(off + part * sizeof(double), 256);
  l.pmax = off;     off = align_up(off + part * sizeof(float), 256);
  l.pmin = off;     off = align_up(off + part * sizeof(float), 256);
  l.pv = off;       off = align_up(off + (size_t)nc * H * WPH * sizeof(float), 256);
  l.hamax = off;    off = align_up(off + (size_t)U * H * sizeof(float), 256);
  l.genc = off;     off = align_up(off + (size_t)U * sizeof(float), 256);
  l.tally = off;    off = align_up(off + (size_t)kFusedMaxWG * 4 * sizeof(uint32_t), 256);
  l.counters = off;  // cnt_head [U][H], cnt_unit [U], flag [U], err [1]
  l.n_counters = U * H + U + U + 1;
  off = align_up(off + (size_t)l.n_counters * sizeof(unsigned), 256);
  l.total = off;
  return l;
}

size_t fused_workspace_bound(int H, int T, int D, int L) {
  if (D / 16 != 8 || H <= 0 || L <= 0) return 0;
  const int WPH = kFusedMaxWG / H;
  if (WPH == 0) return 0;
  return fused_layout(H, T / L, D, WPH).total;
}

template <int BPT>
static const void* fused_kernel_ptr(int mode) {
  switch (mode) {
    case kModeFixed6: return reinterpret_cast<const void*>(&kv_fused_kernel<8, BPT, kModeFixed6>);
    case kModeFixed4: return reinterpret_cast<const void*>(&kv_fused_kernel<8, BPT, kModeFixed4>);
    default: return reinterpret_cast<const void*>(&kv_fused_kernel<8, BPT, kMode4over6>);
  }
}

static const void* pick_fused(int bpt_needed, int mode, int* bpt) {
  if (bpt_needed <= 2) { *bpt = 2; return fused_kernel_ptr<2>(mode); }
  if (bpt_needed <= 4) { *bpt = 4; return fused_kernel_ptr<4>(mode); }
  if (bpt_needed <= 6) { *bpt = 6; return fused_kernel_ptr<6>(mode); }
  return nullptr;
}

// Returns NVFP4_OK after enqueueing, a positive value when the fused form does
// not apply to this shape/device (the caller then uses the multi-kernel form),
// or NVFP4_ERR_HIP.
int fused_try_launch(FusedParams p, int mode, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (p.D != 128 || p.H <= 0 || p.nc <= 0) return 1;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return NVFP4_ERR_HIP;
  int coop = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return 1;
  // workgroups per CU that can be resident at once for the chosen instantiation
  const int nwg_target = ncu * kFusedWgPerCu;
  if (nwg_target > kFusedMaxWG) return 1;
  const int WPH = nwg_target / p.H;
  if (WPH == 0) return 1;
  const int RPW = (p.L + WPH - 1) / WPH;
  const int need = (RPW * 8 + kFusedThreads - 1) / kFusedThreads;
  int bpt = 0;
  const void* kern = pick_fused(need, mode, &bpt);
  if (!kern) return 1;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kFusedThreads, 0) != hipSuccess) return NVFP4_ERR_HIP;
  if (occ < kFusedWgPerCu) return 1;
  const FusedLayout l = fused_layout(p.H, p.nc, p.D, WPH);
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
  p.WPH = WPH;
  p.RPW = RPW;
  fused_zero_kernel<<<(l.n_counters + 255) / 256, 256, 0, s>>>(cnt, l.n_counters);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  void* args[] = {&p};
  if (hipLaunchCooperativeKernel(kern, dim3(nwg_target), dim3(kFusedThreads), args, 0, s) != hipSuccess) {
    (void)hipGetLastError();
    return NVFP4_ERR_HIP;
  }
  if (p.choice) {
    launch_choice_reduce(p.tally, nwg_target, p.choice, s);
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  }
  return NVFP4_OK;
}

}  // namespace nvfp4
