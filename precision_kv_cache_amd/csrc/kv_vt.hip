// kv_vt.hip -- V quantized with its 16-element blocks along the token axis
// (one block = 16 consecutive tokens of one channel), the layout an FP4
// P V product contracts over: the variant of the LongLive-2.0 summary page's
// NVFP4 V cache (inference pipeline, step 7) with the same 4/6 block scale
// (full-stack NVFP4 section) and the same tensor scale per (chunk, tensor).
//
// One launch.  A chunk's tensor scale needs its largest |V| before any of its
// blocks can be encoded, so each chunk is read twice: by statistics tiles
// (512 rows of one head each, largest magnitude, published per tile; the
// last tile of the chunk reduces them, writes g_dec = A / C and raises the
// chunk's ready words) and by quantize tiles (up to 128 tokens x 64 channels
// of one head, staged through LDS so that each lane reads one channel's
// tokens, then the shared 4/6 block routine).  The grid is a sequence of
// segments, segment s holding the statistics tiles of chunk s and then the
// quantize tiles of chunk s - depth, so the second read comes mostly from
// the Infinity Cache and the statistics of later chunks run beside the
// encoding of earlier ones.  A quantize tile waits only for statistics tiles of an earlier
// segment (lower workgroup index), and statistics tiles never wait; with
// in-order dispatch those are resident or finished whenever the quantize
// tile runs, so the waits cannot cycle.  They are bounded all the same: on
// time-out the error word (the first word of the workspace) is raised and
// the tile leaves.  Hand-off between workgroups as in nvfp4_device.hpp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {
namespace {

constexpr int kVtThreads = 256;
constexpr int kVtTok = 128;   // tokens per quantize tile
constexpr int kVtCh = 64;     // channels per quantize tile
constexpr int kVtRow = kVtCh * 2;
constexpr int kVsRows = 512;  // token rows per statistics tile
constexpr int kVtDepth = 1;   // segments between a chunk's statistics and its quantization
constexpr int kVtReplicas = 32;
constexpr int kVtReplicaStride = 32;  // 64-bit words between ready words (256 B)
constexpr unsigned kVtSpinLimit = 1u << 22;

struct VtParams {
  const uint16_t* v;
  uint8_t* codes;
  uint8_t* scales;
  float* tscale;
  float* partial;             // [nc][H][nst] largest |V| per statistics tile
  unsigned long long* ready;  // [kVtReplicas][nc], 256 B apart: 1 << 32 | encode-scale bits once ready
  unsigned* err;              // [1 + nc]: this call's error word, then per-chunk finished statistics tiles
  unsigned* err_sticky;       // the workspace's first word: set on a time-out too, never cleared here
  float C;
  int H, T, D, L, nc, tpc, ncg, nst, depth;
  unsigned spin_limit;
};

// Workspace: a 256-byte header (the sticky error word first), this call's
// error word and counters, ready words, partial maxima.
struct VtLayout {
  size_t err, ready, partial, total;
  size_t n_zero_words;  // this call's error word .. end of the ready words, cleared before the launch
};

constexpr size_t kVtHeader = 256;

VtLayout vt_layout(int H, int nc, int nst) {
  VtLayout l;
  l.err = kVtHeader;
  size_t off = kVtHeader + align_up((size_t)(1 + nc) * sizeof(unsigned), 256);
  l.ready = off;
  off += (size_t)kVtReplicas * nc * kVtReplicaStride * sizeof(unsigned long long);
  l.n_zero_words = (off - l.err) / sizeof(unsigned);
  l.partial = off;
  off = align_up(off + (size_t)nc * H * nst * sizeof(float), 256);
  l.total = off;
  return l;
}

struct VtTile {
  int stats;          // 1: statistics tile, 0: quantize tile
  int c, h, j, cg;    // chunk, head, tile within (chunk, head), channel group
};

// Workgroup index -> tile.  Segment s holds H * nst statistics tiles of
// chunk s (if s < nc), then tpc * H * ncg quantize tiles of chunk s - depth.
__device__ __forceinline__ VtTile vt_decode(const VtParams& p, unsigned b) {
  const unsigned NS = (unsigned)p.H * p.nst, NQ = (unsigned)p.tpc * p.H * p.ncg;
  int s;
  segment_of(b, p.nc, p.depth, NS, NQ, s, b);  // b: the offset in segment s from here on
  const unsigned ns = s < p.nc ? NS : 0u;
  VtTile t;
  t.stats = b < ns;
  if (t.stats) {
    t.c = s; t.h = (int)(b / p.nst); t.j = (int)(b % p.nst); t.cg = 0;
  } else {
    unsigned i = b - ns;
    t.c = s - p.depth;
    t.cg = (int)(i % p.ncg); i /= p.ncg;
    t.h = (int)(i % p.H);
    t.j = (int)(i / p.H);
  }
  return t;
}

// Statistics tile: the largest |V| of rows j * 512 .. of head h in chunk c
// (one contiguous run, 16-byte loads, eight in flight per lane).  The last
// tile of the chunk sets the tensor scales and raises the ready words.
__device__ void vt_stats_tile(const VtParams& p, int c, int h, int j, float* shw, unsigned* sh_flag) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r0 = j * kVsRows;
  const int nr = min(kVsRows, p.L - r0);
  const uint4* src = reinterpret_cast<const uint4*>(p.v + ((size_t)h * p.T + (size_t)c * p.L + r0) * p.D);
  const int n16 = nr * p.D / 8;
  float m = 0.0f;
  for (int base = 0; base < n16; base += 8 * kVtThreads) {
    uint4 a[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kVtThreads + tid;
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
  m = wave_max(m);
  if (lane == 0) shw[wv] = m;
  __syncthreads();
  const unsigned per_chunk = (unsigned)p.H * p.nst;
  if (tid == 0) {
    uint32_t done = 0;
    publish(&p.partial[((size_t)c * p.H + h) * p.nst + j], fmaxf(fmaxf(shw[0], shw[1]), fmaxf(shw[2], shw[3])), done);
    wait_published(done);
    *sh_flag = add_agent(&p.err[1 + c], 1u) == per_chunk - 1;
  }
  __syncthreads();
  if (!*sh_flag) return;
  float A = 0.0f;
  for (unsigned i = tid; i < per_chunk; i += kVtThreads) A = fmaxf(A, fetch(&p.partial[(size_t)c * per_chunk + i]));
  A = wave_max(A);
  if (lane == 0) shw[wv] = A;
  __syncthreads();
  if (tid < kVtReplicas) {
    const float Am = fmaxf(fmaxf(shw[0], shw[1]), fmaxf(shw[2], shw[3]));
    const float g = Am > 0.0f ? p.C / Am : 0.0f;
    if (tid == 0) p.tscale[c] = Am / p.C;  // output only: visible at kernel end
    (void)__hip_atomic_exchange(p.ready + ((size_t)tid * p.nc + c) * kVtReplicaStride,
                                (1ull << 32) | __float_as_uint(g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Quantize tile: the tile (up to 128 tokens x 64 channels) through LDS --
// staged before the wait for the chunk's scale, since V is an input; then
// lane t takes the channel pair 2 (t % 32), +1 and the 16-token block t / 32,
// so that one 4-byte LDS read serves two blocks.
template <int MODE>
__device__ void vt_quant_tile(const VtParams& p, int c, int j, int h, int cg, uint8_t* tile, const float2* tab,
                              float* shw, unsigned* sh_flag) {
  const int tid = threadIdx.x;
  const int t0 = c * p.L + j * kVtTok;
  const int ntok = min(kVtTok, (c + 1) * p.L - t0);
  for (int r = tid >> 3; r < ntok; r += kVtThreads / 8) {
    const uint4 a = *reinterpret_cast<const uint4*>(p.v + ((size_t)h * p.T + t0 + r) * p.D + cg * kVtCh +
                                                    8 * (tid & 7));
    *reinterpret_cast<uint4*>(tile + r * kVtRow + 16 * (tid & 7)) = a;
  }
  if (tid == 0) {
    const unsigned long long* rw = p.ready + ((size_t)(blockIdx.x % kVtReplicas) * p.nc + c) * kVtReplicaStride;
    unsigned long long w = __hip_atomic_load(rw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      w = __hip_atomic_load(rw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *sh_flag = ok ? 1u : 0u;
    shw[0] = __uint_as_float((uint32_t)w);
  }
  __syncthreads();  // the tile, the scale table and the chunk's scale
  if (!*sh_flag) return;
  const int cp = tid & 31, tb = tid >> 5;  // channel pair, 16-token block
  if (16 * tb >= ntok) return;
  const float gz = shw[0];
  float z0[16], z1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + (16 * tb + i) * kVtRow + 4 * cp);
    z0[i] = bf16_lo(w) * gz;
    z1[i] = bf16_hi(w) * gz;
  }
  const size_t row = (size_t)h * p.D + cg * kVtCh + 2 * cp;  // output row (head, channel) of z0
  const size_t blk = row * (p.T / 16) + (t0 / 16) + tb;      // block index along that row
  const Block46 q0 = quant_block16<MODE>(z0, tab);
  *reinterpret_cast<uint2*>(p.codes + blk * 8) = make_uint2(q0.lo, q0.hi);
  p.scales[blk] = (uint8_t)q0.scale;
  const Block46 q1 = quant_block16<MODE>(z1, tab);
  const size_t blk1 = blk + p.T / 16;
  *reinterpret_cast<uint2*>(p.codes + blk1 * 8) = make_uint2(q1.lo, q1.hi);
  p.scales[blk1] = (uint8_t)q1.scale;
}

template <int MODE>
__global__ __launch_bounds__(kVtThreads) void vt_kernel(VtParams p) {
  __shared__ float2 sh_tab[128];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kVtTok * kVtRow];
  __shared__ float shw[kVtThreads / 64];
  __shared__ unsigned sh_flag;
  const VtTile t = vt_decode(p, blockIdx.x);
  if (t.stats) {
    vt_stats_tile(p, t.c, t.h, t.j, shw, &sh_flag);
  } else {
    fill_scale_table(sh_tab);
    vt_quant_tile<MODE>(p, t.c, t.j, t.h, t.cg, tile, sh_tab, shw, &sh_flag);
  }
}

// grid-stride, so that any count is cleared by a bounded grid
__global__ void vt_zero_kernel(unsigned* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API size_t nvfp4_kv_quantize_v_tblocks_workspace_bytes(int H, int T, int D,
                                                                          int chunk_len) noexcept {
  if (H < 1 || T < 1 || D < kVtCh || D % kVtCh || chunk_len < 16 || chunk_len % 16 || T % chunk_len) return 0;
  const int nc = T / chunk_len, nst = (chunk_len + kVsRows - 1) / kVsRows;
  return vt_layout(H, nc, nst).total;
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
  VtParams p{};
  p.H = H; p.T = T; p.D = D; p.L = chunk_len; p.nc = T / chunk_len;
  p.tpc = (chunk_len + kVtTok - 1) / kVtTok;
  p.ncg = D / kVtCh;
  p.nst = (chunk_len + kVsRows - 1) / kVsRows;
  p.depth = kVtDepth;
  p.spin_limit = kVtSpinLimit;
  p.C = mode_constant(mode);
  // work-items of the launch and tile indices stay in 32 bits; a statistics
  // run (512 rows) in 31-bit element offsets
  const long long grid = (long long)p.nc * H * ((long long)p.nst + (long long)p.tpc * p.ncg);
  if (grid >= (1LL << 24) || (long long)kVsRows * D >= (1LL << 31)) return NVFP4_ERR_SHAPE;
  const Range in[1] = {range_of(v, n * 2)};
  const Range outr[4] = {range_of(codes, n / 2), range_of(scales, n / 16), range_of(tensor_scale, (size_t)p.nc * 4),
                         range_of(workspace, need)};
  if (any_alias(in, 1, outr, 4)) return NVFP4_ERR_ALIAS;
  const VtLayout l = vt_layout(H, p.nc, p.nst);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.v = v; p.codes = codes; p.scales = scales; p.tscale = tensor_scale;
  p.err = reinterpret_cast<unsigned*>(ws + l.err);
  p.err_sticky = reinterpret_cast<unsigned*>(ws);
  p.ready = reinterpret_cast<unsigned long long*>(ws + l.ready);
  p.partial = reinterpret_cast<float*>(ws + l.partial);
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  const size_t zb = (l.n_zero_words + 255) / 256;
  vt_zero_kernel<<<dim3((unsigned)(zb < 4096 ? zb : 4096)), dim3(256), 0, s>>>(p.err, l.n_zero_words);
  switch (mode) {
    case kModeFixed6: vt_kernel<kModeFixed6><<<dim3((unsigned)grid), dim3(kVtThreads), 0, s>>>(p); break;
    case kModeFixed4: vt_kernel<kModeFixed4><<<dim3((unsigned)grid), dim3(kVtThreads), 0, s>>>(p); break;
    default: vt_kernel<kMode4over6><<<dim3((unsigned)grid), dim3(kVtThreads), 0, s>>>(p); break;
  }
  return launch_status();
}
