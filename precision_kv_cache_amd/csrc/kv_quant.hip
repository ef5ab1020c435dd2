// kv_quant.hip -- per-chunk K smoothing + NVFP4 4/6 quantization of a KV
// cache layer, and its dequantize (LongLive-2.0 summary page: inference
// pipeline, step 7; full-stack NVFP4).
//
// Data layout (all row-major):
//   K, V        bf16 [H, T, D]; chunk c of head h = rows c*L .. c*L+L-1 of
//               head h's [T, D] slab (contiguous, L*D*2 bytes).
//   codes       [H, T, D/2]; scales [H, T, D/16]; one 16-element block per
//               (h, t, D/16 column); one lane of a workgroup owns one block.
//   k_mean      [nc, H, D] fp32; tensor scales [nc] fp32 per tensor.
//
// Three kernels per group of chunks (the group is sized so that its K and V
// stay in the 256 MB Infinity Cache between the first and the last pass):
//   kv_stats    per (chunk, head, row tile): K channel sum (fp64), max, min;
//               V largest magnitude.                      -> workspace
//   kv_finalize per (chunk, head): channel mean m = fp32(sum / L) and the
//               head's largest |fl(K - m)| = max(fl(max - m), fl(m - min))
//               (exact: rounded subtraction is monotone); V head maximum.
//   kv_quant    per (chunk, head, row tile): tensor scale from the heads'
//               maxima, then smoothing, the 4/6 block quantizer, stores.
// Thread mapping: NB * RP working threads (NB = D/16 blocks per row,
// RP = 256/NB rows per pass), rounded up to whole waves (the extra lanes
// only contribute identity values to the wave reductions); thread t owns
// column t % NB for all its rows, so its 16 channel means stay in
// registers, and consecutive threads read consecutive 32-byte blocks (2 KB
// contiguous per wave and pass).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {

constexpr int kMaxThreads = 256;
constexpr int kStatsPasses = 16;  // rows per stats tile = RP * kStatsPasses
constexpr int kQuantPasses = 4;   // rows per quant / dequant tile = RP * kQuantPasses
constexpr size_t kGroupBytes = size_t(96) << 20;  // K+V bytes per launch group

struct KVGeom {
  int H, T, D, L, nc;
  int NB, RP, threads;
  int rows_s, rows_q, nst, nqt;
};

static KVGeom kv_geom(int H, int T, int D, int L) {
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
  size_t psum, pmax, pmin, pvabs, hamax, total;  // byte offsets
};

static KVWorkspace kv_workspace_layout(const KVGeom& g) {
  KVWorkspace w;
  const size_t nch = (size_t)g.nc * g.H * g.nst * g.D;
  size_t off = 0;
  w.psum = off;  off = align_up(off + nch * sizeof(double), 256);
  w.pmax = off;  off = align_up(off + nch * sizeof(float), 256);
  w.pmin = off;  off = align_up(off + nch * sizeof(float), 256);
  w.pvabs = off; off = align_up(off + (size_t)g.nc * g.H * g.nst * sizeof(float), 256);
  w.hamax = off; off = align_up(off + (size_t)2 * g.nc * g.H * sizeof(float), 256);
  w.total = off;
  return w;
}

struct KVParams {
  const uint16_t* x[2];  // K, V
  uint8_t* codes[2];
  uint8_t* scales[2];
  float* tscale[2];
  float* kmean;
  double* psum;
  float* pmax;
  float* pmin;
  float* pvabs;
  float* hamax;  // [2][nc][H]
  unsigned long long* choice;
  int H, T, D, L, nc, NB, RP, rows_s, rows_q, nst;
  int chunk0;
};

// ---------------------------------------------------------------- stats ---

__global__ __launch_bounds__(kMaxThreads) void kv_stats_kernel(KVParams p) {
  // LDS for the cross-thread reduction: 16 channel slots x up to 256 threads,
  // transposed ([slot][thread], +1 pad) so both phases avoid bank conflicts.
  __shared__ double sh[16 * (kMaxThreads + 1)];
  const int ts = blockIdx.x, h = blockIdx.y, tau = blockIdx.z & 1, c = p.chunk0 + (int)(blockIdx.z >> 1);
  const int tid = threadIdx.x, col = tid % p.NB, roff = tid / p.NB;
  const bool active = roff < p.RP;
  const int r0 = ts * p.rows_s;
  const int r1 = active ? min(r0 + p.rows_s, p.L) : r0;  // idle lanes take no rows
  const uint16_t* base = p.x[tau] + ((size_t)h * p.T + (size_t)c * p.L) * p.D + (size_t)col * 16;

  if (tau == 0) {
    double s[16];
    float mx[16], mn[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { s[i] = 0.0; mx[i] = -INFINITY; mn[i] = INFINITY; }
    for (int r = r0 + roff; r < r1; r += p.RP) {
      const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)r * p.D);
      const uint4 a = src[0], b = src[1];
      float x[16];
      unpack16(a, b, x);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] += (double)x[i];
        mx[i] = fmaxf(mx[i], x[i]);
        mn[i] = fminf(mn[i], x[i]);
      }
    }
    const int stride = kMaxThreads + 1;
    const size_t pbase = (((size_t)c * p.H + h) * p.nst + ts) * p.D;
    // sums: thread d reduces channel d over the RP row groups, in order
#pragma unroll
    for (int i = 0; i < 16; ++i) sh[i * stride + tid] = s[i];
    __syncthreads();
    for (int d = tid; d < p.D; d += blockDim.x) {
      const int cc = d >> 4, i = d & 15;
      double acc = 0.0;
      for (int q = 0; q < p.RP; ++q) acc += sh[i * stride + q * p.NB + cc];
      p.psum[pbase + d] = acc;
    }
    __syncthreads();
    float* shf = reinterpret_cast<float*>(sh);
#pragma unroll
    for (int i = 0; i < 16; ++i) shf[i * stride + tid] = mx[i];
    __syncthreads();
    for (int d = tid; d < p.D; d += blockDim.x) {
      const int cc = d >> 4, i = d & 15;
      float acc = -INFINITY;
      for (int q = 0; q < p.RP; ++q) acc = fmaxf(acc, shf[i * stride + q * p.NB + cc]);
      p.pmax[pbase + d] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) shf[i * stride + tid] = mn[i];
    __syncthreads();
    for (int d = tid; d < p.D; d += blockDim.x) {
      const int cc = d >> 4, i = d & 15;
      float acc = INFINITY;
      for (int q = 0; q < p.RP; ++q) acc = fminf(acc, shf[i * stride + q * p.NB + cc]);
      p.pmin[pbase + d] = acc;
    }
  } else {
    float am = 0.0f;
    for (int r = r0 + roff; r < r1; r += p.RP) {
      const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)r * p.D);
      const uint4 a = src[0], b = src[1];
      float x[16];
      unpack16(a, b, x);
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
    }
    am = wave_max(am);
    float* shf = reinterpret_cast<float*>(sh);
    if ((tid & 63) == 0) shf[tid >> 6] = am;
    __syncthreads();
    if (tid == 0) {
      float a = 0.0f;
      for (int w = 0; w < (int)((blockDim.x + 63) / 64); ++w) a = fmaxf(a, shf[w]);
      p.pvabs[((size_t)c * p.H + h) * p.nst + ts] = a;
    }
  }
}

// ------------------------------------------------------------- finalize ---

__global__ __launch_bounds__(kMaxThreads) void kv_finalize_kernel(KVParams p) {
  __shared__ float shw[kMaxThreads / 64];
  const int h = blockIdx.x, c = p.chunk0 + (int)blockIdx.y, tau = blockIdx.z;
  const int tid = threadIdx.x;
  float a = 0.0f;
  if (tau == 0) {
    for (int d = tid; d < p.D; d += blockDim.x) {
      double s = 0.0;
      float mx = -INFINITY, mn = INFINITY;
      for (int ts = 0; ts < p.nst; ++ts) {
        const size_t i = (((size_t)c * p.H + h) * p.nst + ts) * p.D + d;
        s += p.psum[i];
        mx = fmaxf(mx, p.pmax[i]);
        mn = fminf(mn, p.pmin[i]);
      }
      const float m = (float)(s / (double)p.L);
      p.kmean[((size_t)c * p.H + h) * p.D + d] = m;
      const float up = mx - m, dn = m - mn;  // each one fp32 rounding
      a = fmaxf(a, fmaxf(up, dn));
    }
  } else {
    for (int ts = tid; ts < p.nst; ts += blockDim.x) a = fmaxf(a, p.pvabs[((size_t)c * p.H + h) * p.nst + ts]);
  }
  a = wave_max(a);
  if ((tid & 63) == 0) shw[tid >> 6] = a;
  __syncthreads();
  if (tid == 0) {
    float m = 0.0f;
    for (int w = 0; w < (int)((blockDim.x + 63) / 64); ++w) m = fmaxf(m, shw[w]);
    p.hamax[((size_t)tau * p.nc + c) * p.H + h] = m;
  }
}

// ---------------------------------------------------------------- quant ---

template <int MODE, bool SMOOTH>
__device__ __forceinline__ void kv_quant_body(const KVParams& p, int tau, int c, int h, int qt, float g) {
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
  const size_t row0 = (size_t)h * p.T + (size_t)c * p.L;
  const uint16_t* xb = p.x[tau];
  uint8_t* codes = p.codes[tau];
  uint8_t* scales = p.scales[tau];
  unsigned n4 = 0, nblk = 0;
  for (int r = r0 + roff; r < r1; r += p.RP) {
    const size_t blk = (row0 + r) * p.NB + col;
    const uint4* src = reinterpret_cast<const uint4*>(xb + blk * 16);
    const uint4 a = src[0], b = src[1];
    float z[16];
    unpack16(a, b, z);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float xs = SMOOTH ? z[i] - m[i] : z[i];  // k' = fl(K - m)
      z[i] = xs * g;                                  // z = fl(k' * g_enc)
    }
    const Block46 q = quant_block16<MODE>(z);
    *reinterpret_cast<uint2*>(codes + blk * 8) = make_uint2(q.lo, q.hi);
    scales[blk] = (uint8_t)q.scale;
    n4 += q.use4;
    nblk += 1;
  }
  if (p.choice) {
    n4 = wave_sum_u32(n4);
    nblk = wave_sum_u32(nblk);
    if ((tid & 63) == 0 && nblk) {
      atomicAdd(p.choice + 2 * tau + 1, (unsigned long long)n4);
      atomicAdd(p.choice + 2 * tau + 0, (unsigned long long)(nblk - n4));
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kMaxThreads) void kv_quant_kernel(KVParams p) {
  const int qt = blockIdx.x, h = blockIdx.y, tau = blockIdx.z & 1, c = p.chunk0 + (int)(blockIdx.z >> 1);
  // tensor scale of (tau, chunk) from the heads' maxima
  float A = 0.0f;
  const float* ha = p.hamax + ((size_t)tau * p.nc + c) * p.H;
  for (int i = 0; i < p.H; ++i) A = fmaxf(A, ha[i]);
  const float C = mode_constant(MODE);
  const float g = A > 0.0f ? C / A : 0.0f;
  if (qt == 0 && h == 0 && threadIdx.x == 0) p.tscale[tau][c] = A / C;
  if (tau == 0)
    kv_quant_body<MODE, true>(p, tau, c, h, qt, g);
  else
    kv_quant_body<MODE, false>(p, tau, c, h, qt, g);
}

__global__ void zero_u64_kernel(unsigned long long* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// -------------------------------------------------------------- dequant ---

struct DeqParams {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
  const float* mean;
  uint16_t* out;
  int H, T, D, L, NB, RP, rows_q;
};

template <bool MEAN>
__global__ __launch_bounds__(kMaxThreads) void dequant_kernel(DeqParams p) {
  const int qt = blockIdx.x, h = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x, col = tid % p.NB, roff = tid / p.NB;
  if (roff >= p.RP) return;
  float m[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) m[i] = 0.0f;
  if (MEAN) {
    const float4* mp = reinterpret_cast<const float4*>(p.mean + ((size_t)c * p.H + h) * p.D + (size_t)col * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = mp[j];
      m[4 * j] = v.x; m[4 * j + 1] = v.y; m[4 * j + 2] = v.z; m[4 * j + 3] = v.w;
    }
  }
  const float g = p.tscale[c];
  const int r0 = qt * p.rows_q;
  const int r1 = min(r0 + p.rows_q, p.L);
  const size_t row0 = (size_t)h * p.T + (size_t)c * p.L;
  for (int r = r0 + roff; r < r1; r += p.RP) {
    const size_t blk = (row0 + r) * p.NB + col;
    const uint2 q = *reinterpret_cast<const uint2*>(p.codes + blk * 8);
    const float S = __builtin_amdgcn_cvt_f32_fp8((int)p.scales[blk], 0);
    float v[16];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t w = half ? q.y : q.x;
      const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
      const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
      float* o = v + 8 * half;
      o[0] = v0[0]; o[1] = v0[1]; o[2] = v1[0]; o[3] = v1[1];
      o[4] = v2[0]; o[5] = v2[1]; o[6] = v3[0]; o[7] = v3[1];
    }
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = (v[2 * j] * S) * g, b = (v[2 * j + 1] * S) * g;
      if (MEAN) { a = a + m[2 * j]; b = b + m[2 * j + 1]; }
      w[j] = pack_bf16x2(a, b);
    }
    uint4* dst = reinterpret_cast<uint4*>(p.out + blk * 16);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

}  // namespace nvfp4

using namespace nvfp4;

// ------------------------------------------------------------ C-ABI -------

static bool kv_shape_ok(int H, int T, int D, int L) {
  if (H < 0 || T < 0 || D <= 0 || L <= 0) return false;
  if (D % 16 != 0 || D > NVFP4_KV_MAX_D) return false;
  if (T % L != 0) return false;
  // block indices and row counts stay in 31 bits
  if ((long long)H * T * (D / 16) >= (1LL << 31)) return false;
  return true;
}

extern "C" NVFP4KV_API size_t nvfp4_kv_workspace_bytes(int H, int T, int D, int chunk_len) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len) || H == 0 || T == 0) return 0;
  return kv_workspace_layout(kv_geom(H, T, D, chunk_len)).total;
}

extern "C" NVFP4KV_API int nvfp4_kv_smooth_quantize(const uint16_t* k, const uint16_t* v, int H, int T, int D,
                                                    int chunk_len, int mode, uint8_t* k_codes, uint8_t* v_codes,
                                                    uint8_t* k_scales, uint8_t* v_scales, float* k_tensor_scale,
                                                    float* v_tensor_scale, float* k_mean,
                                                    unsigned long long* choice_counts, void* workspace,
                                                    size_t workspace_bytes, void* stream) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len)) return NVFP4_ERR_SHAPE;
  if (mode < 0 || mode > 2) return NVFP4_ERR_MODE;
  if (H == 0 || T == 0) return NVFP4_OK;
  if (!k || !v || !k_codes || !v_codes || !k_scales || !v_scales || !k_tensor_scale || !v_tensor_scale || !k_mean)
    return NVFP4_ERR_NULL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, 8) || !aligned(v_codes, 8) || !aligned(k_mean, 16) ||
      !aligned(k_tensor_scale, 4) || !aligned(v_tensor_scale, 4) || !aligned(choice_counts, 8))
    return NVFP4_ERR_ALIGN;
  const KVGeom g = kv_geom(H, T, D, chunk_len);
  const KVWorkspace wl = kv_workspace_layout(g);
  if (!workspace || workspace_bytes < wl.total) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)H * T * D;
  const Range in[2] = {range_of(k, n * 2), range_of(v, n * 2)};
  const Range out[10] = {range_of(k_codes, n / 2), range_of(v_codes, n / 2), range_of(k_scales, n / 16),
                         range_of(v_scales, n / 16), range_of(k_tensor_scale, (size_t)g.nc * 4),
                         range_of(v_tensor_scale, (size_t)g.nc * 4), range_of(k_mean, (size_t)g.nc * H * D * 4),
                         range_of(choice_counts, 32), range_of(workspace, wl.total), Range{0, 0}};
  if (any_alias(in, 2, out, 9)) return NVFP4_ERR_ALIAS;

  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
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
  p.choice = choice_counts;
  p.H = H; p.T = T; p.D = D; p.L = chunk_len; p.nc = g.nc; p.NB = g.NB; p.RP = g.RP;
  p.rows_s = g.rows_s; p.rows_q = g.rows_q; p.nst = g.nst;

  (void)hipGetLastError();  // start from a clean error state
  if (choice_counts) zero_u64_kernel<<<1, 64, 0, s>>>(choice_counts, 4);
  const size_t chunk_bytes = (size_t)2 * H * chunk_len * D * sizeof(uint16_t);
  int group = (int)(kGroupBytes / (chunk_bytes > 0 ? chunk_bytes : 1));
  group = group < 1 ? 1 : (group > 16384 ? 16384 : group);
  for (int c0 = 0; c0 < g.nc; c0 += group) {
    const int gn = g.nc - c0 < group ? g.nc - c0 : group;
    p.chunk0 = c0;
    kv_stats_kernel<<<dim3(g.nst, H, 2 * gn), g.threads, 0, s>>>(p);
    kv_finalize_kernel<<<dim3(H, gn, 2), kMaxThreads, 0, s>>>(p);
    const dim3 qgrid(g.nqt, H, 2 * gn);
    switch (mode) {
      case NVFP4_MODE_FIXED6: kv_quant_kernel<kModeFixed6><<<qgrid, g.threads, 0, s>>>(p); break;
      case NVFP4_MODE_FIXED4: kv_quant_kernel<kModeFixed4><<<qgrid, g.threads, 0, s>>>(p); break;
      default: kv_quant_kernel<kMode4over6><<<qgrid, g.threads, 0, s>>>(p); break;
    }
  }
  return launch_status();
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
  DeqParams p;
  p.codes = codes; p.scales = scales; p.tscale = tensor_scale; p.mean = mean; p.out = out;
  p.H = H; p.T = T; p.D = D; p.L = chunk_len; p.NB = g.NB; p.RP = g.RP; p.rows_q = g.rows_q;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const dim3 grid(g.nqt, H, g.nc);
  if (mean)
    dequant_kernel<true><<<grid, g.threads, 0, s>>>(p);
  else
    dequant_kernel<false><<<grid, g.threads, 0, s>>>(p);
  return launch_status();
}
