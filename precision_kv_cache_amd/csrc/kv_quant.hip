// kv_quant.hip -- per-chunk K smoothing + NVFP4 4/6 quantization of a KV
// cache layer (two-pass form), and its dequantize (LongLive-2.0 summary
// page: inference pipeline, step 7; full-stack NVFP4).
//
// Data layout (all row-major):
//   K, V        bf16 [H, T, D]; chunk c of head h = rows c*L .. c*L+L-1 of
//               head h's [T, D] slab (contiguous, L*D*2 bytes).
//   codes       [H, T, D/2]; scales [H, T, D/16]; one 16-element block per
//               (h, t, D/16 column); one lane of a workgroup owns one block.
//   k_mean      [nc, H, D] fp32; tensor scales [nc] fp32 per tensor.
//
// Two passes, each one launch over all chunks of the layer (tens of
// thousands of workgroups, so the per-tile reduction latency of one
// workgroup hides behind the others' streaming):
//   kv_stats    per (chunk, tensor, head, row tile): K channel sum (fp64),
//               max, min, or V largest magnitude -> workspace; the last tile
//               of a head (atomic counter) reduces the head: mean
//               m = fp32(sum / L) and the head's largest |fl(K - m)| =
//               max(fl(max - m), fl(m - min)) (exact: rounded subtraction is
//               monotone), or the V head maximum.
//   kv_quant    per (chunk, tensor, head, row tile): tensor scale from the
//               heads' maxima, smoothing, the 4/6 block quantizer, stores.
// The two run as separate kernels so that the VALU-heavy quantize kernel
// keeps its own (small) register and LDS footprint and high occupancy.
// Thread mapping: NB * RP working threads (NB = D/16 blocks per row,
// RP = 256/NB rows per pass), rounded up to whole waves (the extra lanes
// only contribute identity values to the reductions); thread t owns column
// t % NB for all its rows, so its 16 channel means stay in registers, and
// consecutive threads read consecutive 32-byte blocks (2 KB contiguous per
// wave and pass).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "kv_overlap.hpp"
#include "kv_two_pass.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {

// ---------------------------------------------------------------- stats ---

template <bool NT>
__device__ void kv_stats_tile(const KVParams& p, int c, int tau, int h, int ts, double* sh, float* shw,
                              unsigned* sh_flag) {
  const int tid = threadIdx.x, col = tid % p.NB, roff = tid / p.NB;
  const bool active = roff < p.RP;
  const int r0 = ts * p.rows_s;
  const int r1 = active ? min(r0 + p.rows_s, p.L) : r0;  // idle lanes take no rows
  const uint16_t* base = p.x[tau] + ((size_t)h * p.T + (size_t)c * p.L) * p.D + (size_t)col * 16;
  const size_t hb = ((size_t)c * p.H + h) * p.nst;
  uint32_t done = 0;  // completion of this thread's published partials

  if (tau == 0) {
    double s[16];
    float mx[16], mn[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { s[i] = 0.0; mx[i] = -INFINITY; mn[i] = INFINITY; }
    for (int rb = r0 + roff; rb < r1; rb += kBatch * p.RP) {
      uint4 a[kBatch], b[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int r = rb + q * p.RP;
        if (r < r1) {
          a[q] = load16<NT>(base + (size_t)r * p.D);
          b[q] = load16<NT>(base + (size_t)r * p.D + 8);
        }
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (rb + q * p.RP >= r1) continue;
        float x[16];
        unpack16(a[q], b[q], x);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] += (double)x[i];
          mx[i] = fmaxf(mx[i], x[i]);
          mn[i] = fminf(mn[i], x[i]);
        }
      }
    }
    // cross-thread reduction through LDS ([slot][thread] + pad)
    const int stride = kMaxThreads + 1;
    const size_t pbase = (hb + ts) * p.D;
#pragma unroll
    for (int i = 0; i < 16; ++i) sh[i * stride + tid] = s[i];
    __syncthreads();
    for (int d = tid; d < p.D; d += blockDim.x) {
      const int cc = d >> 4, i = d & 15;
      double acc = 0.0;
      for (int q = 0; q < p.RP; ++q) acc += sh[i * stride + q * p.NB + cc];
      publish(&p.psum[pbase + d], acc, done);
    }
    __syncthreads();
    float* shf = reinterpret_cast<float*>(sh);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      shf[i * stride + tid] = mx[i];
      shf[(16 + i) * stride + tid] = mn[i];
    }
    __syncthreads();
    for (int d = tid; d < p.D; d += blockDim.x) {
      const int cc = d >> 4, i = d & 15;
      float a = -INFINITY, b = INFINITY;
      for (int q = 0; q < p.RP; ++q) {
        a = fmaxf(a, shf[i * stride + q * p.NB + cc]);
        b = fminf(b, shf[(16 + i) * stride + q * p.NB + cc]);
      }
      publish(&p.pmax[pbase + d], a, done);
      publish(&p.pmin[pbase + d], b, done);
    }
  } else {
    float am = 0.0f;
    for (int rb = r0 + roff; rb < r1; rb += kBatch * p.RP) {
      uint4 a[kBatch], b[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int r = rb + q * p.RP;
        if (r < r1) {
          a[q] = load16<NT>(base + (size_t)r * p.D);
          b[q] = load16<NT>(base + (size_t)r * p.D + 8);
        }
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (rb + q * p.RP >= r1) continue;
        float x[16];
        unpack16(a[q], b[q], x);
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
      }
    }
    am = wave_max(am);
    if ((tid & 63) == 0) shw[tid >> 6] = am;
    __syncthreads();
    if (tid == 0) {
      float a = 0.0f;
      for (int w = 0; w < (int)(blockDim.x / 64); ++w) a = fmaxf(a, shw[w]);
      publish(&p.pvabs[hb + ts], a, done);
    }
  }

  // The last tile of (chunk, tensor, head) reduces the head.
  wait_published(done);
  __syncthreads();  // every thread's exchanges completed before thread 0 counts
  if (tid == 0) *sh_flag = add_agent(&p.cnt[((size_t)c * 2 + tau) * p.H + h], 1u) == (unsigned)(p.nst - 1);
  __syncthreads();
  if (!*sh_flag) return;
  float a = 0.0f;
  if (tau == 0) {
    // thread t reduces channel t % D over tiles t / D, t / D + NSPLIT, ...
    // (loads issued in batches), then the parts are combined in order
    const int nsplit = (int)blockDim.x >= p.D ? (int)blockDim.x / p.D : 1;
    const int stride = kMaxThreads + 1;
    float* shf = reinterpret_cast<float*>(sh + 2 * stride);
    for (int d0 = 0; d0 < p.D; d0 += (int)blockDim.x) {
      const int d = d0 + tid % (p.D < (int)blockDim.x ? p.D : (int)blockDim.x);
      const int part = p.D < (int)blockDim.x ? tid / p.D : 0;
      double sum = 0.0;
      float mxv = -INFINITY, mnv = INFINITY;
      if (part < nsplit && d < p.D) {
        for (int jb = part; jb < p.nst; jb += nsplit * 8) {
          double ps[8];
          float px[8], pn[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int jj = jb + q * nsplit;
            if (jj < p.nst) {
              const size_t i = (hb + jj) * p.D + d;
              ps[q] = fetch(&p.psum[i]); px[q] = fetch(&p.pmax[i]); pn[q] = fetch(&p.pmin[i]);
            } else {
              ps[q] = 0.0; px[q] = -INFINITY; pn[q] = INFINITY;
            }
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) { sum += ps[q]; mxv = fmaxf(mxv, px[q]); mnv = fminf(mnv, pn[q]); }
        }
      }
      __syncthreads();
      sh[tid] = sum;
      shf[tid] = mxv;
      shf[stride + tid] = mnv;
      __syncthreads();
      const int nd = min((int)blockDim.x, p.D - d0);
      if (tid < nd) {
        const int dd = p.D < (int)blockDim.x ? tid : tid;
        double s2 = 0.0;
        float x2 = -INFINITY, n2 = INFINITY;
        const int width = p.D < (int)blockDim.x ? p.D : (int)blockDim.x;
        for (int q = 0; q < nsplit; ++q) {
          s2 += sh[q * width + dd];
          x2 = fmaxf(x2, shf[q * width + dd]);
          n2 = fminf(n2, shf[stride + q * width + dd]);
        }
        const float m = (float)(s2 / (double)p.L);
        p.kmean[((size_t)c * p.H + h) * p.D + d0 + dd] = m;
        const float up = x2 - m, dn = m - n2;  // each one fp32 rounding
        a = fmaxf(a, fmaxf(up, dn));
      }
    }
  } else {
    for (int jj = tid; jj < p.nst; jj += blockDim.x) a = fmaxf(a, fetch(&p.pvabs[hb + jj]));
  }
  a = wave_max(a);
  __syncthreads();
  if ((tid & 63) == 0) shw[tid >> 6] = a;
  __syncthreads();
  if (tid == 0) {
    float hm = 0.0f;
    for (int w = 0; w < (int)(blockDim.x / 64); ++w) hm = fmaxf(hm, shw[w]);
    p.hamax[((size_t)tau * p.nc + c) * p.H + h] = hm;
  }
}

// ---------------------------------------------------------------- quant ---

// Returns this thread's {blocks kept at +-4, blocks}.  Lane (roff, col)
// takes rows r0 + roff, r0 + roff + RP, ... of the tile.
template <int MODE, bool SMOOTH, bool NT, int NBC>
__device__ __forceinline__ uint2 kv_quant_body(const KVParams& p, int tau, int c, int h, int qt, float g,
                                               const float2* tab) {
  const int tid = threadIdx.x, col = tid % p.NB, roff = tid / p.NB;
  const bool active = roff < p.RP;
  float m[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) m[i] = 0.0f;
  if (SMOOTH && active) {
    const float4* mp = reinterpret_cast<const float4*>(p.kmean + ((size_t)c * p.H + h) * p.D + (size_t)col * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = mp[j];
      m[4 * j] = v.x; m[4 * j + 1] = v.y; m[4 * j + 2] = v.z; m[4 * j + 3] = v.w;
    }
  }
  const int r0 = qt * p.rows_q;
  const int r1 = active ? min(r0 + p.rows_q, p.L) : r0;  // idle lanes take no rows
  return quant_rows<MODE, SMOOTH, NT, kBatch, NBC>(p.x[tau], p.codes[tau], p.scales[tau],
                                                   (size_t)h * p.T + (size_t)c * p.L, r0 + roff, r1, p.RP,
                                                   p.NB, col, m, g, tab);
}

template <int MODE, bool NT, int NBC>
__device__ void kv_quant_tile(const KVParams& p, int c, int tau, int h, int qt, unsigned* sh_tally,
                              const float2* tab) {
  // tensor scale of (tau, chunk) from the heads' maxima
  float A = 0.0f;
  const float* ha = p.hamax + ((size_t)tau * p.nc + c) * p.H;
  for (int i = 0; i < p.H; ++i) A = fmaxf(A, ha[i]);
  const float C = mode_constant(MODE);
  const float g = A > 0.0f ? C / A : 0.0f;
  if (qt == 0 && h == 0 && threadIdx.x == 0) p.tscale[tau][c] = A / C;
  const uint2 n = tau == 0 ? kv_quant_body<MODE, true, NT, NBC>(p, tau, c, h, qt, g, tab)
                           : kv_quant_body<MODE, false, NT, NBC>(p, tau, c, h, qt, g, tab);
  if (p.choice) {
    const unsigned t[4] = {tau == 0 ? n.x : 0u, tau == 0 ? n.y : 0u, tau == 1 ? n.x : 0u, tau == 1 ? n.y : 0u};
    store_wg_tally(p.tally + ((((size_t)c * 2 + tau) * p.H + h) * p.nqt + qt) * 4, t, sh_tally);
  }
}

// Statistics of chunks [s0, s1): one workgroup per (chunk, tensor, head,
// tile), tile fastest, K and V interleaved.
__global__ __launch_bounds__(kMaxThreads) void kv_stats_kernel(KVParams p) {
  __shared__ double sh[16 * (kMaxThreads + 1)];
  __shared__ float shw[kMaxThreads / 64];
  __shared__ unsigned sh_flag;
  unsigned idx = blockIdx.x;
  const int ts = idx % p.nst;
  idx /= p.nst;
  const int h = idx % p.H;
  idx /= p.H;
  kv_stats_tile<true>(p, p.s0 + (int)(idx >> 1), (int)(idx & 1), h, ts, sh, shw, &sh_flag);
}

// Quantization of chunks [q0, q1): one workgroup per (chunk, tensor, head,
// tile).  About 1 KB of LDS (the scale table, the choice tally), so
// occupancy is set by registers.
// NBC: blocks per row fixed at compile time (8 for D = 128), or 0.
template <int MODE, int NBC>
__global__ __launch_bounds__(kMaxThreads) void kv_quant_kernel(KVParams p) {
  __shared__ unsigned sh_tally[4 * (kMaxThreads / 64)];
  __shared__ float2 sh_tab[128];
  fill_scale_table(sh_tab);
  __syncthreads();
  unsigned idx = blockIdx.x;
  const int qt = idx % p.nqt;
  idx /= p.nqt;
  const int h = idx % p.H;
  idx /= p.H;
  kv_quant_tile<MODE, true, NBC>(p, p.q0 + (int)(idx >> 1), (int)(idx & 1), h, qt, sh_tally, sh_tab);
}

__global__ void zero_counters_kernel(unsigned* cnt, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) cnt[i] = 0u;
}

// One workgroup adds up the per-workgroup tallies [nslots][4] in 64-bit and
// writes choice [2][2] = {K kept +-6, K kept +-4, V kept +-6, V kept +-4}.
__global__ __launch_bounds__(256) void choice_reduce_kernel(const uint32_t* tally, size_t nslots,
                                                            unsigned long long* choice) {
  __shared__ unsigned long long sh[4][256];
  const int tid = threadIdx.x;
  unsigned long long a[4] = {0ull, 0ull, 0ull, 0ull};
  for (size_t i = tid; i < nslots; i += 256) {
    const uint4 t = *reinterpret_cast<const uint4*>(tally + (size_t)i * 4);
    a[0] += t.x; a[1] += t.y; a[2] += t.z; a[3] += t.w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) sh[j][tid] = a[j];
  __syncthreads();
  if (tid < 4) {
    unsigned long long s = 0ull;
    for (int q = 0; q < 256; ++q) s += sh[tid][q];
    sh[tid][0] = s;
  }
  __syncthreads();
  if (tid < 2) {
    const unsigned long long n4 = sh[2 * tid][0], nb = sh[2 * tid + 1][0];
    choice[2 * tid + 0] = nb - n4;
    choice[2 * tid + 1] = n4;
  }
}

void launch_choice_reduce(const uint32_t* tally, size_t nslots, unsigned long long* choice, hipStream_t s) {
  choice_reduce_kernel<<<1, 256, 0, s>>>(tally, nslots, choice);
}

void launch_kv_zero_counters(unsigned* cnt, int n, hipStream_t s) {
  zero_counters_kernel<<<(n + 255) / 256, 256, 0, s>>>(cnt, n);
}

void launch_kv_stats(const KVParams& p, unsigned n_workgroups, int threads, hipStream_t s) {
  kv_stats_kernel<<<n_workgroups, threads, 0, s>>>(p);
}

// -------------------------------------------------------------- dequant ---

// Two lanes per 16-element block (each lane one 8-element half), so every
// 16-byte bf16 store of a wave lands in one contiguous 1 KB run.  Thread t
// owns half-column t % HB (HB = 2 * D/16 halves per row) for kDeqRows rows,
// RP rows apart; it issues all of their code and scale loads before the
// first store, so each lane keeps kDeqRows loads in flight.  The bf16 output
// is streamed out with non-temporal stores: nothing here reads it again.
constexpr int kDeqRows = 2;

struct DeqParams {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
  const float* mean;
  uint16_t* out;
  int H, T, D, L, HB, RP, rows_q;
};

struct DeqGeom {
  int HB, RP, threads, rows_q, nqt;
};

static DeqGeom deq_geom(int D, int L) {
  DeqGeom g;
  g.HB = D / 8;
  g.RP = g.HB >= kMaxThreads ? 1 : kMaxThreads / g.HB;
  g.threads = (g.HB * g.RP + 63) / 64 * 64;
  g.rows_q = g.RP * kDeqRows;
  g.nqt = (L + g.rows_q - 1) / g.rows_q;
  return g;
}

// HBC: halves per row fixed at compile time (16 for D = 128), or 0.
template <bool MEAN, int HBC>
__global__ __launch_bounds__(512) void dequant_kernel(DeqParams p) {
  const int HB = HBC > 0 ? HBC : p.HB;
  const int RP = HBC > 0 ? kMaxThreads / HBC : p.RP;
  const int qt = blockIdx.x, c = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, hc = tid % HB, roff = tid / HB;
  if (roff >= RP) return;
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.0f;
  if (MEAN) {
    const float4* mp = reinterpret_cast<const float4*>(p.mean + ((size_t)c * p.H + h) * p.D + (size_t)hc * 8);
    const float4 a = mp[0], b = mp[1];
    m[0] = a.x; m[1] = a.y; m[2] = a.z; m[3] = a.w; m[4] = b.x; m[5] = b.y; m[6] = b.z; m[7] = b.w;
  }
  const float g = p.tscale[c];
  const int r = qt * RP * kDeqRows + roff;  // this lane's first row of the chunk
  const int r1 = min((qt + 1) * RP * kDeqRows, p.L);
  const size_t half = ((size_t)h * p.T + (size_t)c * p.L + r) * HB + hc;  // index of this lane's first half
  const uint32_t* cp = reinterpret_cast<const uint32_t*>(p.codes) + half;
  const uint8_t* sp = p.scales + (half >> 1);
  uint16_t* op = p.out + half * 8;
  const size_t step = (size_t)RP * HB;  // halves from one of the lane's rows to the next
  uint32_t q[kDeqRows], sb[kDeqRows];
#pragma unroll
  for (int k = 0; k < kDeqRows; ++k) {
    if (r + k * RP < r1) {
      q[k] = cp[k * step];
      sb[k] = sp[k * (step >> 1)];
    }
  }
#pragma unroll
  for (int k = 0; k < kDeqRows; ++k) {
    if (r + k * RP >= r1) break;
    const float S = __builtin_amdgcn_cvt_f32_fp8((int)sb[k], 0);
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[k], 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[k], 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[k], 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[k], 1.0f, 3);
    const float v[8] = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = (v[2 * j] * S) * g, b = (v[2 * j + 1] * S) * g;
      if (MEAN) { a = a + m[2 * j]; b = b + m[2 * j + 1]; }
      w[j] = pack_bf16x2(a, b);
    }
    const u32x4 ov = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(ov, reinterpret_cast<u32x4*>(op + k * step * 8));
  }
}

}  // namespace nvfp4

using namespace nvfp4;

// ------------------------------------------------------------ C-ABI -------

extern "C" NVFP4KV_API size_t nvfp4_kv_workspace_bytes(int H, int T, int D, int chunk_len) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len) || H == 0 || T == 0) return 0;
  const size_t two_pass = kv_workspace_layout(kv_geom(H, T, D, chunk_len)).total;
  const size_t ov = overlap_workspace_bound(H, T, D, chunk_len);
  return two_pass > ov ? two_pass : ov;
}

extern "C" NVFP4KV_API long long nvfp4_kv_error_word_offset(int H, int T, int D, int chunk_len) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len) || H == 0 || T == 0) return -1;
  return 0;  // the first word of the header block, in both kernel forms' layouts
}

namespace nvfp4 {

// Argument checks of nvfp4_kv_smooth_quantize that do not involve the
// workspace (no HIP call): NVFP4_OK, or the status to return.
int kv_quantize_check(const uint16_t* k, const uint16_t* v, int H, int T, int D, int chunk_len, int mode,
                      const uint8_t* k_codes, const uint8_t* v_codes, const uint8_t* k_scales,
                      const uint8_t* v_scales, const float* k_tensor_scale, const float* v_tensor_scale,
                      const float* k_mean, const unsigned long long* choice_counts, const void* workspace,
                      size_t ws_range) {
  if (!kv_shape_ok(H, T, D, chunk_len)) return NVFP4_ERR_SHAPE;
  mode &= ~NVFP4_KV_TWO_PASS;
  if (mode < 0 || mode > 2) return NVFP4_ERR_MODE;
  if (H == 0 || T == 0) return NVFP4_OK;
  if (!k || !v || !k_codes || !v_codes || !k_scales || !v_scales || !k_tensor_scale || !v_tensor_scale || !k_mean)
    return NVFP4_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, 8) || !aligned(v_codes, 8) || !aligned(k_mean, 16) ||
      !aligned(k_tensor_scale, 4) || !aligned(v_tensor_scale, 4) || !aligned(choice_counts, 8))
    return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)H * T * D;
  const int nc = T / chunk_len;
  const Range in[2] = {range_of(k, n * 2), range_of(v, n * 2)};
  const Range out[9] = {range_of(k_codes, n / 2), range_of(v_codes, n / 2), range_of(k_scales, n / 16),
                        range_of(v_scales, n / 16), range_of(k_tensor_scale, (size_t)nc * 4),
                        range_of(v_tensor_scale, (size_t)nc * 4), range_of(k_mean, (size_t)nc * H * D * 4),
                        range_of(choice_counts, 32), range_of(workspace, ws_range)};
  if (any_alias(in, 2, out, 9)) return NVFP4_ERR_ALIAS;
  return NVFP4_OK;
}

// The kernels of nvfp4_kv_smooth_quantize on a checked call, with the
// workspace given (at least nvfp4_kv_workspace_bytes, 256-byte aligned);
// err_word: where a timed-out wait is also recorded (the workspace's first
// word for the ordinary entry point).
int kv_quantize_launch(const uint16_t* k, const uint16_t* v, int H, int T, int D, int chunk_len, int mode,
                       uint8_t* k_codes, uint8_t* v_codes, uint8_t* k_scales, uint8_t* v_scales,
                       float* k_tensor_scale, float* v_tensor_scale, float* k_mean,
                       unsigned long long* choice_counts, void* workspace, size_t workspace_bytes,
                       unsigned* err_word, hipStream_t s) {
  const bool two_pass = (mode & NVFP4_KV_TWO_PASS) != 0;
  mode &= ~NVFP4_KV_TWO_PASS;
  const KVGeom g = kv_geom(H, T, D, chunk_len);
  const KVWorkspace wl = kv_workspace_layout(g);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();  // start from a clean error state
  if (!two_pass && D == 128) {
    OverlapParams q;
    q.x[0] = k; q.x[1] = v;
    q.codes[0] = k_codes; q.codes[1] = v_codes;
    q.scales[0] = k_scales; q.scales[1] = v_scales;
    q.tscale[0] = k_tensor_scale; q.tscale[1] = v_tensor_scale;
    q.kmean = k_mean;
    q.H = H; q.T = T; q.L = chunk_len; q.nc = g.nc;
    const int rc = overlap_try_launch(q, mode, 4, workspace, workspace_bytes, choice_counts, err_word, s);
    if (rc <= 0) return rc;  // enqueued, or a launch error
  }
  KVParams p;
  p.x[0] = k; p.x[1] = v;
  p.codes[0] = k_codes; p.codes[1] = v_codes;
  p.scales[0] = k_scales; p.scales[1] = v_scales;
  p.tscale[0] = k_tensor_scale; p.tscale[1] = v_tensor_scale;
  p.kmean = k_mean;
  p.psum = reinterpret_cast<double*>(ws + wl.psum);
  p.pmax = reinterpret_cast<float*>(ws + wl.pmax);
  p.pmin = reinterpret_cast<float*>(ws + wl.pmin);
  p.pvabs = reinterpret_cast<float*>(ws + wl.pvabs);
  p.hamax = reinterpret_cast<float*>(ws + wl.hamax);
  p.cnt = reinterpret_cast<unsigned*>(ws + wl.counters);
  p.tally = reinterpret_cast<uint32_t*>(ws + wl.tally);
  p.choice = choice_counts;
  p.H = H; p.T = T; p.D = D; p.L = chunk_len; p.nc = g.nc; p.NB = g.NB; p.RP = g.RP;
  p.rows_s = g.rows_s; p.rows_q = g.rows_q; p.nst = g.nst; p.nqt = g.nqt;

  zero_counters_kernel<<<(wl.n_counters + 255) / 256, 256, 0, s>>>(p.cnt, wl.n_counters);
  // Chunks per launch: all of them unless the grid would get too large.
  const long long per_chunk_wgs = 2LL * H * (g.nst > g.nqt ? g.nst : g.nqt);
  int group = (int)(kMaxLaunchWGs / per_chunk_wgs);
  group = group < 1 ? 1 : (group > g.nc ? g.nc : group);
  // per group of chunks: the statistics kernel, then the quantize kernel
  for (int c0 = 0; c0 < g.nc; c0 += group) {
    p.s0 = p.q0 = c0;
    p.s1 = p.q1 = c0 + group < g.nc ? c0 + group : g.nc;
    const long long ns = (long long)(p.s1 - p.s0) * 2 * H * g.nst;
    const long long nq = (long long)(p.q1 - p.q0) * 2 * H * g.nqt;
    kv_stats_kernel<<<(unsigned)ns, g.threads, 0, s>>>(p);
    const bool d128 = D == 128;
    switch (mode) {
      case NVFP4_MODE_FIXED6:
        if (d128) kv_quant_kernel<kModeFixed6, 8><<<(unsigned)nq, g.threads, 0, s>>>(p);
        else kv_quant_kernel<kModeFixed6, 0><<<(unsigned)nq, g.threads, 0, s>>>(p);
        break;
      case NVFP4_MODE_FIXED4:
        if (d128) kv_quant_kernel<kModeFixed4, 8><<<(unsigned)nq, g.threads, 0, s>>>(p);
        else kv_quant_kernel<kModeFixed4, 0><<<(unsigned)nq, g.threads, 0, s>>>(p);
        break;
      default:
        if (d128) kv_quant_kernel<kMode4over6, 8><<<(unsigned)nq, g.threads, 0, s>>>(p);
        else kv_quant_kernel<kMode4over6, 0><<<(unsigned)nq, g.threads, 0, s>>>(p);
        break;
    }
  }
  if (choice_counts) launch_choice_reduce(p.tally, wl.n_tally, choice_counts, s);
  return launch_status();
}

}  // namespace nvfp4


extern "C" NVFP4KV_API int nvfp4_kv_smooth_quantize(const uint16_t* k, const uint16_t* v, int H, int T, int D,
                                                    int chunk_len, int mode, uint8_t* k_codes, uint8_t* v_codes,
                                                    uint8_t* k_scales, uint8_t* v_scales, float* k_tensor_scale,
                                                    float* v_tensor_scale, float* k_mean,
                                                    unsigned long long* choice_counts, void* workspace,
                                                    size_t workspace_bytes, void* stream) noexcept {
  const size_t ws_need = nvfp4_kv_workspace_bytes(H, T, D, chunk_len);
  int rc = kv_quantize_check(k, v, H, T, D, chunk_len, mode, k_codes, v_codes, k_scales, v_scales, k_tensor_scale,
                             v_tensor_scale, k_mean, choice_counts, nullptr, 0);
  if (rc != NVFP4_OK || H == 0 || T == 0) return rc;
  if (!workspace || workspace_bytes < ws_need) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  // the kernels may use every byte nvfp4_kv_workspace_bytes covers
  rc = kv_quantize_check(k, v, H, T, D, chunk_len, mode, k_codes, v_codes, k_scales, v_scales, k_tensor_scale,
                         v_tensor_scale, k_mean, choice_counts, workspace, ws_need);
  if (rc != NVFP4_OK) return rc;
  return kv_quantize_launch(k, v, H, T, D, chunk_len, mode, k_codes, v_codes, k_scales, v_scales, k_tensor_scale,
                            v_tensor_scale, k_mean, choice_counts, workspace, workspace_bytes,
                            static_cast<unsigned*>(workspace), as_stream(stream));
}

extern "C" NVFP4KV_API int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                            const float* mean, int H, int T, int D, int chunk_len, uint16_t* out,
                                            void* stream) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len)) return NVFP4_ERR_SHAPE;
  if (H == 0 || T == 0) return NVFP4_OK;
  if (!codes || !scales || !tensor_scale || !out) return NVFP4_ERR_NULL;
  if (!aligned(codes, 8) || !aligned(out, 16) || !aligned(tensor_scale, 4) || !aligned(mean, 16))
    return NVFP4_ERR_ALIGN;
  const KVGeom g = kv_geom(H, T, D, chunk_len);
  const size_t n = (size_t)H * T * D;
  const Range in[4] = {range_of(codes, n / 2), range_of(scales, n / 16), range_of(tensor_scale, (size_t)g.nc * 4),
                       range_of(mean, mean ? (size_t)g.nc * H * D * 4 : 0)};
  const Range outr[1] = {range_of(out, n * 2)};
  if (any_alias(in, 4, outr, 1)) return NVFP4_ERR_ALIAS;
  const DeqGeom dg = deq_geom(D, chunk_len);
  DeqParams p;
  p.codes = codes; p.scales = scales; p.tscale = tensor_scale; p.mean = mean; p.out = out;
  p.H = H; p.T = T; p.D = D; p.L = chunk_len; p.HB = dg.HB; p.RP = dg.RP; p.rows_q = dg.rows_q;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  // chunks before heads in the dispatch order: the resident workgroups then
  // sweep one head's rows (all its chunks, contiguous) as a single front
  // instead of touching one region per (chunk, head) at once
  const dim3 grid(dg.nqt, g.nc, H);
  if (D == 128) {
    if (mean) dequant_kernel<true, 16><<<grid, dg.threads, 0, s>>>(p);
    else dequant_kernel<false, 16><<<grid, dg.threads, 0, s>>>(p);
  } else {
    if (mean) dequant_kernel<true, 0><<<grid, dg.threads, 0, s>>>(p);
    else dequant_kernel<false, 0><<<grid, dg.threads, 0, s>>>(p);
  }
  return launch_status();
}
