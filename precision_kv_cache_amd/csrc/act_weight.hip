// act_weight.hip -- NVFP4 4/6 quantizers for the GEMM operands that the
// LongLive-2.0 summary page lists for its NVFP4 path (training pipeline,
// step 4): activations with 1D 16-element blocks after a 16-point
// random-sign Hadamard transform, and weights with 2D 16x16 tiles.
//
// Both need the tensor's largest magnitude before any block can be encoded,
// so each is two passes: an amax pass (every workgroup stores its partial
// maximum in its own workspace slot; a shared atomic would serialize
// thousands of workgroups) and the quantize pass, whose every workgroup
// first reduces those partials itself (a few KB from L2, cheaper than a
// separate reduction launch between the passes) and which recomputes the
// rotation in registers instead of storing it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {

constexpr int kAWThreads = 256;
constexpr int kAmaxMaxWG = 2048;  // workgroups of the amax pass (grid-stride)
// workspace: [0, 256) unused; [256, ...) the amax pass's partial maxima
constexpr size_t kAWWorkspace = 256 + (size_t)kAmaxMaxWG * sizeof(float);

// 16-point random-sign Hadamard transform of one block, in place, without
// its final factor 1/4: w = H16 (s * x).  The sign flips ride on the first
// butterfly stage: with t = s_i x_i (exact), the pair (i, i + 1) becomes
// (fl(t + s_{i+1} x_{i+1}), fl(t - s_{i+1} x_{i+1})), each one fused
// multiply-add whose product is exact, so the rounding is that of the plain
// sum and difference; strides 2, 4, 8 then turn (a, b) into (a + b, a - b).
// The callers apply the 1/4 where it is exact and free: u = w / 4 exactly
// (w is a multiple of 2^-133, so w / 4 cannot underflow), hence
// max|u| = max|w| / 4 and fl(u * g) = fl(w * (g / 4)) with g / 4 exact.
// sgn[j] is -1 where bit j of the sign mask is set, else +1.
__device__ __forceinline__ void rht16_unscaled(float (&u)[16], const float (&sgn)[16]) {
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const float t = u[i] * sgn[i];
    const float b = u[i + 1];
    u[i] = __builtin_fmaf(b, sgn[i + 1], t);
    u[i + 1] = __builtin_fmaf(b, -sgn[i + 1], t);
  }
#pragma unroll
  for (int h = 2; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = u[i], b = u[i + h];
      u[i] = a + b;
      u[i + h] = a - b;
    }
  }
}

__device__ __forceinline__ void sign_factors(uint32_t mask, float (&sgn)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) sgn[j] = ((mask >> j) & 1u) ? -1.0f : 1.0f;
}

constexpr int kAmaxUnroll = 4;  // segments whose loads a lane issues together

// Largest |value| over nseg 16-element segments (optionally rotated).
// Each lane takes segments f, f + G, f + 2G, f + 3G (G = the grid's lanes)
// per step, their loads issued together.
template <bool RHT>
__global__ __launch_bounds__(kAWThreads) void amax16_kernel(const uint16_t* x, long long nseg, uint32_t sign_mask,
                                                            float* partial) {
  __shared__ float shw[kAWThreads / 64];
  float sgn[16];
  sign_factors(sign_mask, sgn);
  float am = 0.0f;
  const long long G = (long long)gridDim.x * blockDim.x;
  for (long long f = blockIdx.x * (long long)blockDim.x + threadIdx.x; f < nseg; f += kAmaxUnroll * G) {
    uint4 a[kAmaxUnroll], b[kAmaxUnroll];
#pragma unroll
    for (int q = 0; q < kAmaxUnroll; ++q) {
      if (f + q * G < nseg) {
        const uint4* src = reinterpret_cast<const uint4*>(x + (f + q * G) * 16);
        a[q] = src[0];
        b[q] = src[1];
      }
    }
#pragma unroll
    for (int q = 0; q < kAmaxUnroll; ++q) {
      if (f + q * G >= nseg) continue;
      float u[16];
      unpack16(a[q], b[q], u);
      if (RHT) rht16_unscaled(u, sgn);
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(u[i]));
    }
  }
  am = wave_max(am);
  if ((threadIdx.x & 63) == 0) shw[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.0f;
    for (int w = 0; w < (int)(blockDim.x / 64); ++w) m = fmaxf(m, shw[w]);
    partial[blockIdx.x] = RHT ? m * 0.25f : m;  // the rotation's 1/4, exact
  }
}

// The tensor maximum from the amax pass's n partial maxima, reduced by the
// whole workgroup (at most 2048 floats, read from L2): every quantize
// workgroup does this itself instead of waiting for a separate reduction
// launch.  Ends with a barrier; shw is 4 floats of LDS.
__device__ __forceinline__ float wg_partial_max(const float* partial, int n, float* shw) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, partial[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) shw[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(shw[0], shw[1]), fmaxf(shw[2], shw[3]));
}

// 1D quantize pass: one lane per 16-element block of the row-major tensor.
template <int MODE, bool RHT>
__global__ __launch_bounds__(kAWThreads) void quant1d_kernel(const uint16_t* x, long long nblk, uint32_t sign_mask,
                                                             const float* partial, int npart, uint8_t* codes,
                                                             uint8_t* scales, float* tensor_scale) {
  __shared__ float2 sh_tab[128];
  __shared__ float shw[kAWThreads / 64];
  fill_scale_table(sh_tab);
  const float A = wg_partial_max(partial, npart, shw);  // its barrier also orders the table's fill
  const float C = mode_constant(MODE);
  const float g = A > 0.0f ? C / A : 0.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[0] = A / C;
  const float gz = RHT ? g * 0.25f : g;  // the rotation's 1/4 folded into the scale (exact)
  float sgn[16];
  sign_factors(sign_mask, sgn);
  for (long long f = blockIdx.x * (long long)blockDim.x + threadIdx.x; f < nblk;
       f += (long long)gridDim.x * blockDim.x) {
    // the block's last read (the amax pass left it in the Infinity Cache)
    // and its codes are streamed: non-temporal loads and stores
    const uint4 a = load_nt(x + f * 16), b = load_nt(x + f * 16 + 8);
    float z[16];
    unpack16(a, b, z);
    if (RHT) rht16_unscaled(z, sgn);
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = z[i] * gz;
    const Block46 q = quant_block16<MODE>(z, sh_tab);
    store_nt(codes + f * 8, q.lo, q.hi);
    store_nt(scales + f, (uint8_t)q.scale);
  }
}

// 2D quantize pass: 16 lanes per 16x16 tile (lane = tile row), 4 tiles per
// wave; the tile maximum and the tile error are butterfly reductions inside
// the 16-lane group, the error one pairwise tree over the tile rows.
template <int MODE>
__global__ __launch_bounds__(kAWThreads) void quant2d_kernel(const uint16_t* w, int rows, int cols,
                                                             const float* partial, int npart, uint8_t* codes,
                                                             uint8_t* scales, float* tensor_scale) {
  __shared__ float2 sh_tab[128];
  __shared__ float shw[kAWThreads / 64];
  fill_scale_table(sh_tab);
  const float A = wg_partial_max(partial, npart, shw);  // its barrier also orders the table's fill
  const float C = mode_constant(MODE);
  const float g = A > 0.0f ? C / A : 0.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[0] = A / C;
  const int ntc = cols / 16;
  const long long ntiles = (long long)(rows / 16) * ntc;
  const int lane = threadIdx.x & 63, r = lane & 15;
  const long long waves_total = (long long)gridDim.x * (blockDim.x / 64);
  for (long long wv = blockIdx.x * (long long)(blockDim.x / 64) + (threadIdx.x >> 6); wv * 4 < ntiles;
       wv += waves_total) {
    const long long tile = wv * 4 + (lane >> 4);
    const bool active = tile < ntiles;
    const long long tr = active ? tile / ntc : 0, tc = active ? tile % ntc : 0;
    const size_t row = (size_t)tr * 16 + r;
    float z[16];
    if (active) {
      const uint4* src = reinterpret_cast<const uint4*>(w + row * cols + tc * 16);
      const uint4 a = src[0], b = src[1];
      unpack16(a, b, z);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = z[i] * g;
    float t = block_absmax(z);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) t = fmaxf(t, __shfl_xor(t, o, 64));
    const uint32_t s = candidate_codes(t);
    uint32_t lo, hi, scale, use4;
    if (MODE == kModeFixed6 || MODE == kModeFixed4) {
      const float2 sc = sh_tab[MODE == kModeFixed6 ? (s & 0xffu) : (s >> 8)];
      const Encoded16 e = encode16(z, sc.x, sc.y);
      lo = e.lo; hi = e.hi;
      scale = MODE == kModeFixed6 ? (s & 0xffu) : (s >> 8);
      use4 = MODE == kModeFixed4;
    } else {
      const float2 c6 = sh_tab[s & 0xffu], c4 = sh_tab[s >> 8];
      const Encoded16 e6 = encode16(z, c6.x, c6.y);
      const Encoded16 e4 = encode16(z, c4.x, c4.y);
      float err6 = e6.err_lo + e6.err_hi, err4 = e4.err_lo + e4.err_hi;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {  // pairwise tree over the 16 tile rows
        err6 = err6 + __shfl_xor(err6, o, 64);
        err4 = err4 + __shfl_xor(err4, o, 64);
      }
      const bool u4 = err4 < err6;
      lo = u4 ? e4.lo : e6.lo;
      hi = u4 ? e4.hi : e6.hi;
      scale = u4 ? (s >> 8) : (s & 0xffu);
      use4 = u4;
    }
    (void)use4;
    if (active) {
      *reinterpret_cast<uint2*>(codes + row * (cols / 2) + tc * 8) = make_uint2(lo, hi);
      if (r == 0) scales[tr * ntc + tc] = (uint8_t)scale;
    }
  }
}

// Dequantize 2D tiles: one lane per 16-element row segment.
__global__ __launch_bounds__(kAWThreads) void dequant2d_kernel(const uint8_t* codes, const uint8_t* scales,
                                                               const float* tensor_scale, int rows, int cols,
                                                               uint16_t* out) {
  const int ntc = cols / 16;
  const long long nseg = (long long)rows * ntc;
  const float g = tensor_scale[0];
  for (long long f = blockIdx.x * (long long)blockDim.x + threadIdx.x; f < nseg;
       f += (long long)gridDim.x * blockDim.x) {
    const long long row = f / ntc, cb = f % ntc;
    const uint2 q = *reinterpret_cast<const uint2*>(codes + f * 8);
    const float S = __builtin_amdgcn_cvt_f32_fp8((int)scales[(row / 16) * ntc + cb], 0);
    uint32_t wds[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t wq = half ? q.y : q.x;
      const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq, 1.0f, 0);
      const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq, 1.0f, 1);
      const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq, 1.0f, 2);
      const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wq, 1.0f, 3);
      wds[4 * half + 0] = pack_bf16x2((v0[0] * S) * g, (v0[1] * S) * g);
      wds[4 * half + 1] = pack_bf16x2((v1[0] * S) * g, (v1[1] * S) * g);
      wds[4 * half + 2] = pack_bf16x2((v2[0] * S) * g, (v2[1] * S) * g);
      wds[4 * half + 3] = pack_bf16x2((v3[0] * S) * g, (v3[1] * S) * g);
    }
    uint4* dst = reinterpret_cast<uint4*>(out + f * 16);
    dst[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    dst[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
  }
}

static unsigned grid_for(long long n, int per_thread_items) {
  long long b = (n + (long long)kAWThreads * per_thread_items - 1) / ((long long)kAWThreads * per_thread_items);
  return (unsigned)(b < 1 ? 1 : (b > (1 << 20) ? (1 << 20) : b));
}

}  // namespace nvfp4

using namespace nvfp4;

static bool aw_shape_ok(int rows, int cols, bool tiles) {
  if (rows < 0 || cols <= 0 || cols % 16) return false;
  if (tiles && rows % 16) return false;
  return (long long)rows * cols < (1LL << 40);
}

extern "C" NVFP4KV_API size_t nvfp4_quantize_1d_workspace_bytes(int rows, int cols) noexcept {
  return aw_shape_ok(rows, cols, false) ? kAWWorkspace : 0;
}

extern "C" NVFP4KV_API size_t nvfp4_quantize_2d_workspace_bytes(int rows, int cols) noexcept {
  return aw_shape_ok(rows, cols, true) ? kAWWorkspace : 0;
}

// amax pass over nseg 16-element segments: one partial maximum per
// workgroup into the workspace; returns their count.
static int launch_amax(const uint16_t* x, long long nseg, bool rht, uint32_t sign_mask, void* workspace,
                       hipStream_t s) {
  float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + 256);
  const unsigned g0 = grid_for(nseg, 4 * kAmaxUnroll);
  const unsigned ga = g0 < (unsigned)kAmaxMaxWG ? g0 : (unsigned)kAmaxMaxWG;
  if (rht)
    amax16_kernel<true><<<ga, kAWThreads, 0, s>>>(x, nseg, sign_mask, partial);
  else
    amax16_kernel<false><<<ga, kAWThreads, 0, s>>>(x, nseg, sign_mask, partial);
  return (int)ga;
}

extern "C" NVFP4KV_API int nvfp4_quantize_1d(const uint16_t* x, int rows, int cols, int mode, int hadamard,
                                             uint32_t sign_mask, uint8_t* codes, uint8_t* scales,
                                             float* tensor_scale, void* workspace, size_t workspace_bytes,
                                             void* stream) noexcept {
  if (!aw_shape_ok(rows, cols, false)) return NVFP4_ERR_SHAPE;
  if (mode < 0 || mode > 2) return NVFP4_ERR_MODE;
  if (rows == 0) return NVFP4_OK;
  if (!x || !codes || !scales || !tensor_scale) return NVFP4_ERR_NULL;
  if (!workspace || workspace_bytes < kAWWorkspace) return NVFP4_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) || !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)rows * cols;
  const Range in[1] = {range_of(x, n * 2)};
  const Range out[4] = {range_of(codes, n / 2), range_of(scales, n / 16), range_of(tensor_scale, 4),
                        range_of(workspace, kAWWorkspace)};
  if (any_alias(in, 1, out, 4)) return NVFP4_ERR_ALIAS;
  hipStream_t s = as_stream(stream);
  const float* partial = reinterpret_cast<const float*>(static_cast<char*>(workspace) + 256);
  const long long nblk = (long long)(n / 16);
  (void)hipGetLastError();
  const int np = launch_amax(x, nblk, hadamard != 0, sign_mask, workspace, s);
  const unsigned gq = grid_for(nblk, 8);  // eight blocks per lane: fewer workgroups re-reducing the partials
#define NVFP4_Q1D(MODE)                                                                                      \
  (hadamard ? quant1d_kernel<MODE, true><<<gq, kAWThreads, 0, s>>>(x, nblk, sign_mask, partial, np, codes,   \
                                                                   scales, tensor_scale)                     \
            : quant1d_kernel<MODE, false><<<gq, kAWThreads, 0, s>>>(x, nblk, sign_mask, partial, np, codes,  \
                                                                    scales, tensor_scale))
  switch (mode) {
    case NVFP4_MODE_FIXED6: NVFP4_Q1D(kModeFixed6); break;
    case NVFP4_MODE_FIXED4: NVFP4_Q1D(kModeFixed4); break;
    default: NVFP4_Q1D(kMode4over6); break;
  }
#undef NVFP4_Q1D
  return launch_status();
}

extern "C" NVFP4KV_API int nvfp4_quantize_2d(const uint16_t* w, int rows, int cols, int mode, uint8_t* codes,
                                             uint8_t* scales, float* tensor_scale, void* workspace,
                                             size_t workspace_bytes, void* stream) noexcept {
  if (!aw_shape_ok(rows, cols, true)) return NVFP4_ERR_SHAPE;
  if (mode < 0 || mode > 2) return NVFP4_ERR_MODE;
  if (rows == 0) return NVFP4_OK;
  if (!w || !codes || !scales || !tensor_scale) return NVFP4_ERR_NULL;
  if (!workspace || workspace_bytes < kAWWorkspace) return NVFP4_ERR_WORKSPACE;
  if (!aligned(w, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) || !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)rows * cols;
  const Range in[1] = {range_of(w, n * 2)};
  const Range out[4] = {range_of(codes, n / 2), range_of(scales, n / 256), range_of(tensor_scale, 4),
                        range_of(workspace, kAWWorkspace)};
  if (any_alias(in, 1, out, 4)) return NVFP4_ERR_ALIAS;
  hipStream_t s = as_stream(stream);
  const float* partial = reinterpret_cast<const float*>(static_cast<char*>(workspace) + 256);
  (void)hipGetLastError();
  const int np = launch_amax(w, (long long)(n / 16), false, 0u, workspace, s);
  const long long ntiles = (long long)(rows / 16) * (cols / 16);
  const unsigned gq = grid_for((ntiles + 3) / 4 * 64, 1);
  switch (mode) {
    case NVFP4_MODE_FIXED6:
      quant2d_kernel<kModeFixed6><<<gq, kAWThreads, 0, s>>>(w, rows, cols, partial, np, codes, scales, tensor_scale);
      break;
    case NVFP4_MODE_FIXED4:
      quant2d_kernel<kModeFixed4><<<gq, kAWThreads, 0, s>>>(w, rows, cols, partial, np, codes, scales, tensor_scale);
      break;
    default:
      quant2d_kernel<kMode4over6><<<gq, kAWThreads, 0, s>>>(w, rows, cols, partial, np, codes, scales, tensor_scale);
      break;
  }
  return launch_status();
}

extern "C" NVFP4KV_API int nvfp4_dequantize_2d(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                                               int rows, int cols, uint16_t* out, void* stream) noexcept {
  if (!aw_shape_ok(rows, cols, true)) return NVFP4_ERR_SHAPE;
  if (rows == 0) return NVFP4_OK;
  if (!codes || !scales || !tensor_scale || !out) return NVFP4_ERR_NULL;
  if (!aligned(codes, 8) || !aligned(out, 16) || !aligned(tensor_scale, 4)) return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)rows * cols;
  const Range in[3] = {range_of(codes, n / 2), range_of(scales, n / 256), range_of(tensor_scale, 4)};
  const Range outr[1] = {range_of(out, n * 2)};
  if (any_alias(in, 3, outr, 1)) return NVFP4_ERR_ALIAS;
  (void)hipGetLastError();
  dequant2d_kernel<<<grid_for((long long)(n / 16), 2), kAWThreads, 0, as_stream(stream)>>>(codes, scales,
                                                                                        tensor_scale, rows, cols, out);
  return launch_status();
}
