// kv_vt.hip -- V quantized with its 16-element blocks along the token axis
// (one block = 16 consecutive tokens of one channel), the layout an FP4
// P V product contracts over: the variant of the LongLive-2.0 summary page's
// NVFP4 V cache (inference pipeline, step 7) with the same 4/6 block scale
// (full-stack NVFP4 section) and the same tensor scale per (chunk, tensor).
//
// Three launches: a maximum pass (one partial |V| maximum per token tile, written,
// not accumulated, so nothing needs clearing), a per-chunk reduction that
// writes g_dec = A / C, and the quantize pass, which stages a tile of up to
// 128 tokens x 64 channels through LDS, so that each lane reads one
// channel's tokens, and runs the shared 4/6 block routine.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {
namespace {

constexpr int kVtThreads = 256;
constexpr int kVtTok = 128;  // tokens per tile
constexpr int kVtCh = 64;    // channels per tile
constexpr int kVtRow = kVtCh * 2;

struct VtGeom {
  int H, T, D, L, nc, tpc, ncg;  // tiles per chunk, channel groups
  long long ntiles;
};

// tile index -> (chunk, tile in chunk, head, channel group)
__device__ __forceinline__ void vt_tile(const VtGeom& g, long long i, int& c, int& j, int& h, int& cg) {
  cg = (int)(i % g.ncg);
  i /= g.ncg;
  h = (int)(i % g.H);
  i /= g.H;
  j = (int)(i % g.tpc);
  c = (int)(i / g.tpc);
}

__device__ __forceinline__ float wave_max_f(float m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// Partial maximum |V| per (chunk, 128-token tile, head): the tile's rows,
// all channels, are one contiguous run, streamed with 16-byte loads.
// partial[(c * tpc + j) * H + h].
__global__ __launch_bounds__(kVtThreads) void vt_max_kernel(const uint16_t* v, VtGeom g, float* partial) {
  __shared__ float shw[kVtThreads / 64];
  const int h = blockIdx.x % g.H, jc = blockIdx.x / g.H, j = jc % g.tpc, c = jc / g.tpc;
  const int t0 = c * g.L + j * kVtTok;
  const int ntok = min(kVtTok, (c + 1) * g.L - t0);
  const uint4* src = reinterpret_cast<const uint4*>(v + ((size_t)h * g.T + t0) * g.D);
  const int n16 = ntok * g.D / 8;  // 16-byte pieces of the run
  float m = 0.0f;
  // eight loads in flight per lane, then their maxima
  for (int base = 0; base < n16; base += 8 * kVtThreads) {
    uint4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kVtThreads + threadIdx.x;
      a[u] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(a[u].x)), fabsf(bf16_hi(a[u].x))),
                         fmaxf(fabsf(bf16_lo(a[u].y)), fabsf(bf16_hi(a[u].y)))));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(a[u].z)), fabsf(bf16_hi(a[u].z))),
                         fmaxf(fabsf(bf16_lo(a[u].w)), fabsf(bf16_hi(a[u].w)))));
    }
  }
  m = wave_max_f(m);
  if ((threadIdx.x & 63) == 0) shw[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(shw[0], shw[1]), fmaxf(shw[2], shw[3]));
}

// One workgroup per chunk: A = the chunk's largest |V|; writes its bits
// (for the quantize pass) and g_dec = A / C.
__global__ __launch_bounds__(kVtThreads) void vt_reduce_kernel(const float* partial, VtGeom g, float C,
                                                               uint32_t* amax_bits, float* tensor_scale) {
  __shared__ float shw[kVtThreads / 64];
  const long long per_chunk = (long long)g.tpc * g.H;
  const float* p = partial + blockIdx.x * per_chunk;
  float m = 0.0f;
  for (long long i = threadIdx.x; i < per_chunk; i += blockDim.x) m = fmaxf(m, p[i]);
  m = wave_max_f(m);
  if ((threadIdx.x & 63) == 0) shw[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float A = fmaxf(fmaxf(shw[0], shw[1]), fmaxf(shw[2], shw[3]));
    amax_bits[blockIdx.x] = __float_as_uint(A);
    tensor_scale[blockIdx.x] = A / C;
  }
}

// Quantize pass: the tile (up to 128 tokens x 64 channels) through LDS; lane
// t takes the channel pair 2 (t % 32), +1 and the 16-token block t / 32, so
// that one 4-byte LDS read serves two blocks.
template <int MODE>
__global__ __launch_bounds__(kVtThreads) void vt_quant_kernel(const uint16_t* v, VtGeom g,
                                                              const uint32_t* amax_bits, uint8_t* codes,
                                                              uint8_t* scales) {
  __shared__ float2 sh_tab[128];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kVtTok * kVtRow];
  fill_scale_table(sh_tab);
  int c, j, h, cg;
  vt_tile(g, blockIdx.x, c, j, h, cg);
  const int t0 = c * g.L + j * kVtTok;
  const int ntok = min(kVtTok, (c + 1) * g.L - t0);
  for (int r = threadIdx.x >> 3; r < ntok; r += kVtThreads / 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(v + ((size_t)h * g.T + t0 + r) * g.D + cg * kVtCh +
                                                    8 * (threadIdx.x & 7));
    *reinterpret_cast<uint4*>(tile + r * kVtRow + 16 * (threadIdx.x & 7)) = a;
  }
  __syncthreads();
  const int cp = threadIdx.x & 31, tb = threadIdx.x >> 5;  // channel pair, 16-token block
  if (16 * tb >= ntok) return;
  const float A = __uint_as_float(amax_bits[c]);
  const float gz = A > 0.0f ? mode_constant(MODE) / A : 0.0f;
  float z0[16], z1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + (16 * tb + i) * kVtRow + 4 * cp);
    z0[i] = bf16_lo(w) * gz;
    z1[i] = bf16_hi(w) * gz;
  }
  const size_t row = (size_t)h * g.D + cg * kVtCh + 2 * cp;  // output row (head, channel) of z0
  const size_t blk = row * (g.T / 16) + (t0 / 16) + tb;      // block index along that row
  const Block46 q0 = quant_block16<MODE>(z0, sh_tab);
  *reinterpret_cast<uint2*>(codes + blk * 8) = make_uint2(q0.lo, q0.hi);
  scales[blk] = (uint8_t)q0.scale;
  const Block46 q1 = quant_block16<MODE>(z1, sh_tab);
  const size_t blk1 = blk + g.T / 16;
  *reinterpret_cast<uint2*>(codes + blk1 * 8) = make_uint2(q1.lo, q1.hi);
  scales[blk1] = (uint8_t)q1.scale;
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API size_t nvfp4_kv_quantize_v_tblocks_workspace_bytes(int H, int T, int D,
                                                                          int chunk_len) noexcept {
  if (H < 1 || T < 1 || D < kVtCh || D % kVtCh || chunk_len < 16 || chunk_len % 16 || T % chunk_len) return 0;
  const long long nc = T / chunk_len, tpc = (chunk_len + kVtTok - 1) / kVtTok;
  const long long ntiles = nc * tpc * H * (D / kVtCh);
  return align_up((size_t)ntiles * 4, 256) + align_up((size_t)nc * 4, 256);
}

extern "C" NVFP4KV_API int nvfp4_kv_quantize_v_tblocks(const uint16_t* v, int H, int T, int D, int chunk_len,
                                                       int mode, uint8_t* codes, uint8_t* scales,
                                                       float* tensor_scale, void* workspace,
                                                       size_t workspace_bytes, void* stream) noexcept {
  if (H < 0 || T < 0 || D < kVtCh || D % kVtCh || D > NVFP4_KV_MAX_D || chunk_len < 16 || chunk_len % 16)
    return NVFP4_ERR_SHAPE;
  if (T % chunk_len != 0 || (long long)H * T * D > (1LL << 40)) return NVFP4_ERR_SHAPE;
  if (mode < kMode4over6 || mode > kModeFixed4) return NVFP4_ERR_MODE;
  if (H == 0 || T == 0) return NVFP4_OK;
  if (!v || !codes || !scales || !tensor_scale || !workspace) return workspace ? NVFP4_ERR_NULL : NVFP4_ERR_WORKSPACE;
  if (!aligned(v, 16) || !aligned(codes, 8) || !aligned(tensor_scale, 4) || !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  const size_t need = nvfp4_kv_quantize_v_tblocks_workspace_bytes(H, T, D, chunk_len);
  if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  const size_t n = (size_t)H * T * D;
  VtGeom g{};
  g.H = H; g.T = T; g.D = D; g.L = chunk_len; g.nc = T / chunk_len;
  g.tpc = (chunk_len + kVtTok - 1) / kVtTok;
  g.ncg = D / kVtCh;
  g.ntiles = (long long)g.nc * g.tpc * H * g.ncg;
  if (g.ntiles >= (1LL << 31)) return NVFP4_ERR_SHAPE;
  const Range in[1] = {range_of(v, n * 2)};
  const Range outr[4] = {range_of(codes, n / 2), range_of(scales, n / 16), range_of(tensor_scale, (size_t)g.nc * 4),
                         range_of(workspace, need)};
  if (any_alias(in, 1, outr, 4)) return NVFP4_ERR_ALIAS;
  float* partial = static_cast<float*>(workspace);
  uint32_t* amax = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + align_up((size_t)g.ntiles * 4, 256));
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  vt_max_kernel<<<dim3((unsigned)(g.ntiles / g.ncg)), dim3(kVtThreads), 0, s>>>(v, g, partial);
  vt_reduce_kernel<<<dim3((unsigned)g.nc), dim3(kVtThreads), 0, s>>>(partial, g, mode_constant(mode), amax,
                                                                      tensor_scale);
  switch (mode) {
    case kModeFixed6:
      vt_quant_kernel<kModeFixed6><<<dim3((unsigned)g.ntiles), dim3(kVtThreads), 0, s>>>(v, g, amax, codes, scales);
      break;
    case kModeFixed4:
      vt_quant_kernel<kModeFixed4><<<dim3((unsigned)g.ntiles), dim3(kVtThreads), 0, s>>>(v, g, amax, codes, scales);
      break;
    default:
      vt_quant_kernel<kMode4over6><<<dim3((unsigned)g.ntiles), dim3(kVtThreads), 0, s>>>(v, g, amax, codes, scales);
      break;
  }
  return launch_status();
}
