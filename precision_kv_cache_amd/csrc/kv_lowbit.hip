// kv_lowbit.hip -- 3-bit and 2-bit KV cache: per-chunk K smoothing and the
// two-candidate block scale at 3 or 2 bits per element, and the matching
// dequantize (LongLive-2.0 summary page: directions to extend, item 6, a
// 3-bit / 2-bit KV cache; inference pipeline, step 7 for the smoothing and
// the cache; full-stack NVFP4 for the adaptive block scale).
//
// The page gives no format.  The one taken (shared with the CPU reference):
//   element  sign bit + E1M1 magnitude {0, 0.5, 1, 1.5} (3 bits), or sign
//            bit + E1M0 magnitude {0, 1} (2 bits); nearest magnitude, ties
//            to the even code, saturating, sign bit = the sign bit of y;
//   block    16 consecutive channels, one E4M3FN scale; one fp32 tensor
//            scale per (chunk, tensor), as the 4-bit cache;
//   choice   candidates t_b / c_a and t_b / c_b: c_a maps the block maximum
//            onto the largest magnitude, c_b = c_a / 1.5 (3 bits: 1.5, 1)
//            or c_a * 1.5 (2 bits: 1, 1.5); the lower fp32 error (two
//            8-element fused halves added) wins, ties keep c_a;
//   C        448 * the smallest divisor the mode uses;
//   codes    element i of a block at bits [b*i, b*i + b) of the block's
//            little-endian bit field: 6 bytes per block at 3 bits, 4 at 2.
//
// Kernels: the two-pass statistics kernel of the 4-bit path (its K mean,
// channel max and min, and V largest magnitude are the same), then a
// quantize kernel per (chunk, tensor, head, row tile) whose lanes each
// encode one 16-element block per row: there is no hardware conversion for
// these grids, so a magnitude is rint(2|y|) capped at 3 (3 bits) or
// |y| > 0.5 (2 bits), which is exactly round to nearest with ties to the
// even code.  The dequantize decodes half a block per lane, a fixed column
// of rows, like the 4-bit one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "kv_two_pass.hpp"
#include "kv_overlap.hpp"
#include "lowbit_device.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {
namespace {

// One (chunk, tensor, head, row tile) of the quantize: lane (roff, col)
// takes rows r0 + roff, + RP, ... of column block col.
template <int BITS, int MODE>
__global__ __launch_bounds__(kMaxThreads) void kv_lowbit_quant_kernel(KVParams p) {
  __shared__ unsigned sh_tally[4 * (kMaxThreads / 64)];
  __shared__ float2 sh_tab[128];
  fill_scale_table(sh_tab);
  __syncthreads();
  unsigned idx = blockIdx.x;
  const int qt = idx % p.nqt;
  idx /= p.nqt;
  const int h = idx % p.H;
  idx /= p.H;
  const int c = p.q0 + (int)(idx >> 1), tau = (int)(idx & 1);
  // tensor scale of (tau, chunk) from the heads' maxima
  float A = 0.0f;
  const float* ha = p.hamax + ((size_t)tau * p.nc + c) * p.H;
  for (int i = 0; i < p.H; ++i) A = fmaxf(A, ha[i]);
  const float C = lowbit_constant<BITS>(MODE);
  const float g = A > 0.0f ? C / A : 0.0f;
  if (qt == 0 && h == 0 && threadIdx.x == 0) p.tscale[tau][c] = A / C;

  const int tid = threadIdx.x, col = tid % p.NB, roff = tid / p.NB;
  const bool active = roff < p.RP;
  float m[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) m[i] = 0.0f;
  if (tau == 0 && active) {
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
  unsigned nb = 0, n = 0;
  // one row per step: two rows' loads in flight need 110+ VGPRs (4 waves
  // per SIMD instead of 8) and measured slower
  for (int r = r0 + roff; r < r1; r += p.RP) {
    const size_t blk = (row0 + r) * p.NB + col;
    const uint16_t* px = p.x[tau] + blk * 16;
    const uint4 a = load_nt(px), b = load_nt(px + 8);
    float z[16];
    unpack16(a, b, z);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float xs = tau == 0 ? z[i] - m[i] : z[i];  // k' = fl(K - m)
      z[i] = xs * g;                                   // z = fl(k' * g_enc)
    }
    const LowBitBlock q = lowbit_block16<BITS, MODE>(z, sh_tab);
    uint8_t* pc = p.codes[tau] + blk * LowBit<BITS>::bytes;
    if (BITS == 3) {  // 6 bytes, 2-byte aligned
      uint16_t* pw = reinterpret_cast<uint16_t*>(pc);
      __builtin_nontemporal_store((uint16_t)(q.lo & 0xffffu), pw);
      __builtin_nontemporal_store((uint16_t)(q.lo >> 16), pw + 1);
      __builtin_nontemporal_store((uint16_t)(q.hi & 0xffffu), pw + 2);
    } else {
      __builtin_nontemporal_store(q.lo, reinterpret_cast<uint32_t*>(pc));
    }
    store_nt(p.scales[tau] + blk, (uint8_t)q.scale);
    nb += q.useb;
    n += 1;
  }
  if (p.choice) {
    const unsigned t[4] = {tau == 0 ? nb : 0u, tau == 0 ? n : 0u, tau == 1 ? nb : 0u, tau == 1 ? n : 0u};
    store_wg_tally(p.tally + ((((size_t)c * 2 + tau) * p.H + h) * p.nqt + qt) * 4, t, sh_tally);
  }
}


struct LowBitDeq {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
  const float* mean;
  uint16_t* out;
  int H, T, D, L, NB, RP;
};

constexpr int kLbDeqRows = 4;  // rows per lane

// One workgroup per (tile of RP * kLbDeqRows rows, chunk, head); lane (roff,
// hc) decodes half-block hc (8 channels: block hc / 2, half hc % 2) of rows
// roff, roff + RP, ... (RP = 256 / (2 NB) rows per pass).  So its chunk's
// means are loaded once, and each wave-wide store writes one contiguous run
// of whole rows, 16 bytes per lane.  The two lanes of a block both load its
// code bytes and scale.  Workgroups of max(2 NB, 256) lanes (rounded up to
// whole waves): a row of up to 512 halves (D <= 4096) is one pass.
template <int BITS, bool MEAN>
__global__ __launch_bounds__(512) void kv_lowbit_dequant_kernel(LowBitDeq p) {
  const int HB = 2 * p.NB;
  const int tid = threadIdx.x, hc = tid % HB, roff = tid / HB;
  if (roff >= p.RP) return;
  const int c = blockIdx.y, h = blockIdx.z, half = hc & 1;
  const float g = p.tscale[c];
  float m[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) m[i] = 0.0f;
  if (MEAN) {
    const float4* mp = reinterpret_cast<const float4*>(p.mean + ((size_t)c * p.H + h) * p.D + (size_t)hc * 8);
    const float4 a = mp[0], b = mp[1];
    m[0] = a.x; m[1] = a.y; m[2] = a.z; m[3] = a.w; m[4] = b.x; m[5] = b.y; m[6] = b.z; m[7] = b.w;
  }
  const int r0 = blockIdx.x * p.RP * kLbDeqRows + roff;
  const int r1 = min((blockIdx.x + 1) * p.RP * kLbDeqRows, p.L);
  const size_t row0 = (size_t)h * p.T + (size_t)c * p.L + r0;  // this lane's first row
  const size_t b0 = row0 * p.NB + (hc >> 1);                   // its first block
  const size_t step = (size_t)p.RP * p.NB;                     // blocks to the lane's next row
  uint32_t lo[kLbDeqRows], hi[kLbDeqRows], sb[kLbDeqRows];
#pragma unroll
  for (int k = 0; k < kLbDeqRows; ++k) {  // every load of the lane before the first store
    if (r0 + k * p.RP < r1) {
      const size_t b = b0 + k * step;
      const uint8_t* pc = p.codes + b * LowBit<BITS>::bytes;
      if (BITS == 3) {
        const uint16_t* pw = reinterpret_cast<const uint16_t*>(pc);
        lo[k] = (uint32_t)pw[0] | ((uint32_t)pw[1] << 16);
        hi[k] = pw[2];
      } else {
        lo[k] = *reinterpret_cast<const uint32_t*>(pc);
        hi[k] = 0u;
      }
      sb[k] = p.scales[b];
    }
  }
#pragma unroll
  for (int k = 0; k < kLbDeqRows; ++k) {
    if (r0 + k * p.RP >= r1) break;
    const float S = __builtin_amdgcn_cvt_f32_fp8((int)sb[k], 0);
    // this half's 8 codes, element 0 at bit 0: bits [8 BITS half, 8 BITS half + 8 BITS)
    // of the block's field (48 bits at 3 bits per element, 32 at 2)
    const uint64_t field = ((uint64_t)hi[k] << 32) | lo[k];
    const uint32_t w = (uint32_t)(field >> (8 * BITS * half));
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float x2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t code = (w >> (BITS * (i + u))) & ((1u << BITS) - 1u);
        const uint32_t mag = code & ((1u << (BITS - 1)) - 1u);
        const float v = BITS == 3 ? (float)mag * 0.5f : (float)mag;
        const float vs = __uint_as_float(__float_as_uint(v) | ((code >> (BITS - 1)) << 31));
        float xh = (vs * S) * g;  // two fp32 roundings (v * S is exact)
        if (MEAN) xh = xh + m[i + u];
        x2[u] = xh;
      }
      o[i / 2] = pack_bf16x2(x2[0], x2[1]);
    }
    uint16_t* po = p.out + ((row0 + (size_t)k * p.RP) * p.D + (size_t)hc * 8);
    __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4*>(po));
  }
}

template <int BITS>
void launch_lowbit_quant(const KVParams& p, int mode, unsigned nq, int threads, hipStream_t s) {
  switch (mode) {
    case kModeFixed6: kv_lowbit_quant_kernel<BITS, kModeFixed6><<<nq, threads, 0, s>>>(p); break;
    case kModeFixed4: kv_lowbit_quant_kernel<BITS, kModeFixed4><<<nq, threads, 0, s>>>(p); break;
    default: kv_lowbit_quant_kernel<BITS, kMode4over6><<<nq, threads, 0, s>>>(p); break;
  }
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API int nvfp4_kv_smooth_quantize_lowbit(const uint16_t* k, const uint16_t* v, int H, int T, int D,
                                                           int chunk_len, int bits, int mode, uint8_t* k_codes,
                                                           uint8_t* v_codes, uint8_t* k_scales, uint8_t* v_scales,
                                                           float* k_tensor_scale, float* v_tensor_scale,
                                                           float* k_mean, unsigned long long* choice_counts,
                                                           void* workspace, size_t workspace_bytes,
                                                           void* stream) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len) || (bits != 3 && bits != 2)) return NVFP4_ERR_SHAPE;
  const bool two_pass = (mode & NVFP4_KV_TWO_PASS) != 0;
  mode &= ~NVFP4_KV_TWO_PASS;
  if (mode < 0 || mode > 2) return NVFP4_ERR_MODE;
  if (H == 0 || T == 0) return NVFP4_OK;
  if (!k || !v || !k_codes || !v_codes || !k_scales || !v_scales || !k_tensor_scale || !v_tensor_scale || !k_mean)
    return NVFP4_ERR_NULL;
  const size_t calign = bits == 3 ? 2 : 4;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_codes, calign) || !aligned(v_codes, calign) ||
      !aligned(k_mean, 16) || !aligned(k_tensor_scale, 4) || !aligned(v_tensor_scale, 4) ||
      !aligned(choice_counts, 8))
    return NVFP4_ERR_ALIGN;
  const KVGeom g = kv_geom(H, T, D, chunk_len);
  const KVWorkspace wl = kv_workspace_layout(g);
  // the kernels may use every byte nvfp4_kv_workspace_bytes covers
  const size_t ws_need = nvfp4_kv_workspace_bytes(H, T, D, chunk_len);
  if (!workspace || workspace_bytes < ws_need) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)H * T * D;
  const Range in[2] = {range_of(k, n * 2), range_of(v, n * 2)};
  const Range out[9] = {range_of(k_codes, n * bits / 8), range_of(v_codes, n * bits / 8),
                        range_of(k_scales, n / 16), range_of(v_scales, n / 16),
                        range_of(k_tensor_scale, (size_t)g.nc * 4), range_of(v_tensor_scale, (size_t)g.nc * 4),
                        range_of(k_mean, (size_t)g.nc * H * D * 4), range_of(choice_counts, 32),
                        range_of(workspace, ws_need)};
  if (any_alias(in, 2, out, 9)) return NVFP4_ERR_ALIAS;

  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  if (!two_pass && D == 128) {  // the single-launch overlapped kernel, as for NVFP4
    OverlapParams q;
    q.x[0] = k; q.x[1] = v;
    q.codes[0] = k_codes; q.codes[1] = v_codes;
    q.scales[0] = k_scales; q.scales[1] = v_scales;
    q.tscale[0] = k_tensor_scale; q.tscale[1] = v_tensor_scale;
    q.kmean = k_mean;
    q.H = H; q.T = T; q.L = chunk_len; q.nc = g.nc;
    const int rc = overlap_try_launch(q, mode, bits, workspace, workspace_bytes, choice_counts,
                                      static_cast<unsigned*>(workspace), s);
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
  launch_kv_zero_counters(p.cnt, wl.n_counters, s);
  const long long per_chunk_wgs = 2LL * H * (g.nst > g.nqt ? g.nst : g.nqt);
  int group = (int)(kMaxLaunchWGs / per_chunk_wgs);
  group = group < 1 ? 1 : (group > g.nc ? g.nc : group);
  for (int c0 = 0; c0 < g.nc; c0 += group) {
    p.s0 = p.q0 = c0;
    p.s1 = p.q1 = c0 + group < g.nc ? c0 + group : g.nc;
    const long long ns = (long long)(p.s1 - p.s0) * 2 * H * g.nst;
    const long long nq = (long long)(p.q1 - p.q0) * 2 * H * g.nqt;
    launch_kv_stats(p, (unsigned)ns, g.threads, s);
    if (bits == 3) launch_lowbit_quant<3>(p, mode, (unsigned)nq, g.threads, s);
    else launch_lowbit_quant<2>(p, mode, (unsigned)nq, g.threads, s);
  }
  if (choice_counts) launch_choice_reduce(p.tally, wl.n_tally, choice_counts, s);
  return launch_status();
}

extern "C" NVFP4KV_API int nvfp4_dequantize_lowbit(const uint8_t* codes, const uint8_t* scales,
                                                   const float* tensor_scale, const float* mean, int H, int T, int D,
                                                   int chunk_len, int bits, uint16_t* out, void* stream) noexcept {
  if (!kv_shape_ok(H, T, D, chunk_len) || (bits != 3 && bits != 2)) return NVFP4_ERR_SHAPE;
  if (H == 0 || T == 0) return NVFP4_OK;
  if (!codes || !scales || !tensor_scale || !out) return NVFP4_ERR_NULL;
  if (!aligned(codes, bits == 3 ? 2 : 4) || !aligned(out, 16) || !aligned(tensor_scale, 4) || !aligned(mean, 16))
    return NVFP4_ERR_ALIGN;
  const size_t n = (size_t)H * T * D;
  const int nc = T / chunk_len;
  const Range in[4] = {range_of(codes, n * bits / 8), range_of(scales, n / 16), range_of(tensor_scale, (size_t)nc * 4),
                       range_of(mean, mean ? (size_t)nc * H * D * 4 : 0)};
  const Range outr[1] = {range_of(out, n * 2)};
  if (any_alias(in, 4, outr, 1)) return NVFP4_ERR_ALIAS;
  LowBitDeq p;
  p.codes = codes; p.scales = scales; p.tscale = tensor_scale; p.mean = mean; p.out = out;
  p.H = H; p.T = T; p.D = D; p.L = chunk_len; p.NB = D / 16;
  const int HB = 2 * p.NB;                // half-blocks per row, at most 512
  p.RP = HB >= 256 ? 1 : 256 / HB;        // rows per pass
  const unsigned threads = (unsigned)((HB * p.RP + 63) / 64 * 64);
  // chunks before heads in the dispatch order (one contiguous front per head)
  const dim3 grid((unsigned)((chunk_len + p.RP * kLbDeqRows - 1) / (p.RP * kLbDeqRows)), (unsigned)nc, (unsigned)H);
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  if (bits == 3) {
    if (mean) kv_lowbit_dequant_kernel<3, true><<<grid, threads, 0, s>>>(p);
    else kv_lowbit_dequant_kernel<3, false><<<grid, threads, 0, s>>>(p);
  } else {
    if (mean) kv_lowbit_dequant_kernel<2, true><<<grid, threads, 0, s>>>(p);
    else kv_lowbit_dequant_kernel<2, false><<<grid, threads, 0, s>>>(p);
  }
  return launch_status();
}
