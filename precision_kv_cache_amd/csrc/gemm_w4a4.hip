// gemm_w4a4.hip -- the W4A4 GEMM on NVFP4 operands that the LongLive-2.0
// summary page runs its linear layers with (training pipeline, step 4: 2D
// block scales for weights, 1D for activations, RHT against outliers;
// inference pipeline, step 6: a W4A4 model).
//
//   out[m][n] = bf16( g_A g_W sum_k (v S)_A[m][k] (v S)_W[n][k] )
//
// NVFP4 values v * S have at most 6 significant bits and lie in
// [2^-10, 2688], so each operand decodes exactly to fp16 (one conversion of
// two E2M1 codes and one packed fp16 multiply by the E4M3 scale per two
// elements); the products are exact in fp32 and accumulate in fp32 on
// v_mfma_f32_16x16x32_f16; the two tensor scales multiply the result once.
// gfx950's scaled FP4 matrix instructions take E8M0 scales per 32 elements,
// not NVFP4's E4M3 scales per 16, hence decode on load.
//
// One workgroup (8 waves) computes a 256 x 256 output tile.  K advances in
// tiles of 64: the workgroup decodes the A and W tiles once into double-
// buffered LDS ([row][k], 144-byte rows), and each wave, owning 128 rows of
// M and 64 columns of N, computes C^T = W A^T with W as the matrix
// instruction's A operand, so that a lane ends with 4 consecutive output
// columns of one row.  The codes of tile k + 2 are loaded while tile k is
// multiplied, two lanes per row (32 contiguous bytes), and the decode of tile
// k + 1 is interleaved with tile k's matrix instructions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {
namespace {

constexpr int kGThreads = 512;
constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kRow = kTK * 2 + 16;  // LDS bytes per operand row (padded: 8 rows hit distinct banks)
constexpr int kOpBytes = 256 * kRow;
constexpr int kGBuf = 2 * kOpBytes;  // A then W
constexpr int kXcds = 8;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GemmParams {
  const uint8_t *ac, *as, *wc, *ws;
  const float *ag, *wg;
  uint16_t* out;
  int M, N, K, w2d;
  int ntm, ntn, total, per_xcd;
};

// One decode unit: 32 codes (two 16-element blocks) of one operand row and
// their two scale bytes.
struct Unit {
  uint4 c;
  uint32_t s;
};

// Thread t's unit of a tile: row t / 2, block pair t % 2 (the two lanes of
// a row read its 32 contiguous code bytes).  Rows past the operand's end
// re-read its last row; their products land in outputs that are not stored.
__device__ __forceinline__ Unit load_unit(const uint8_t* codes, const uint8_t* scales, int rows, int row0, int K,
                                          int k0, bool s2d, int t) {
  const int bp = t & 1;
  const int row = min(row0 + (t >> 1), rows - 1);
  Unit u;
  u.c = *reinterpret_cast<const uint4*>(codes + (size_t)row * (K / 2) + k0 / 2 + 16 * bp);
  const size_t si = (s2d ? (size_t)(row / 16) : (size_t)row) * (K / 16) + k0 / 16 + 2 * bp;
  u.s = *reinterpret_cast<const uint16_t*>(scales + si);
  return u;
}

// Two E2M1 codes (byte SEL of w) times the scale S, as packed fp16.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_scaled(uint32_t w, f16x2 S) {
  const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL) * S;
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// v * S of the unit's 32 codes (exact in fp16) into row t / 2 of the operand
// tile at op.
__device__ __forceinline__ void store_unit(uint8_t* op, const Unit& u, int t) {
  const uint32_t w[4] = {u.c.x, u.c.y, u.c.z, u.c.w};
  uint8_t* dst = op + (t >> 1) * kRow + 64 * (t & 1);
  const f16x2 S = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u.s, 1.0f, false);  // the two E4M3 scales
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 Sj = j < 2 ? f16x2{S.x, S.x} : f16x2{S.y, S.y};
    *reinterpret_cast<u32x4*>(dst + 16 * j) = u32x4{fp4x2_scaled<0>(w[j], Sj), fp4x2_scaled<1>(w[j], Sj),
                                                    fp4x2_scaled<2>(w[j], Sj), fp4x2_scaled<3>(w[j], Sj)};
  }
}

__device__ __forceinline__ f16x8 frag(const uint8_t* p) { return *reinterpret_cast<const f16x8*>(p); }

__global__ __launch_bounds__(kGThreads) void gemm_w4a4_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kGBuf];

  // consecutive slots of one XCD take consecutive N tiles of one M tile, so
  // that they share that XCD's L2 for the A rows
  const int w = (int)(blockIdx.x % kXcds) * p.per_xcd + (int)(blockIdx.x / kXcds);
  if (w >= p.total) return;
  const int m0 = (w / p.ntn) * kTM, n0 = (w % p.ntn) * kTN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;  // this wave: rows m0 + 128 wm .., columns n0 + 64 wn ..
  const bool w2 = p.w2d != 0;

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile 0 decoded, tile 1 (clamped to the last) loaded
  const int nk = p.K / kTK;
  Unit ua = load_unit(p.ac, p.as, p.M, m0, p.K, 0, false, t);
  Unit uw = load_unit(p.wc, p.ws, p.N, n0, p.K, 0, w2, t);
  store_unit(lds, ua, t);
  store_unit(lds + kOpBytes, uw, t);
  ua = load_unit(p.ac, p.as, p.M, m0, p.K, min(1, nk - 1) * kTK, false, t);
  uw = load_unit(p.wc, p.ws, p.N, n0, p.K, min(1, nk - 1) * kTK, w2, t);
  __syncthreads();

  // Iteration kt multiplies tile kt, decodes tile kt + 1 into the other
  // buffer (free since the previous barrier; after the last tile the decode
  // is of a clamped repeat that nothing reads) and loads tile kt + 2.  No
  // branches in the body, so that the scheduling groups below span it.
  for (int kt = 0; kt < nk; ++kt) {
    const Unit ca = ua, cw = uw;
    const int kn = min(kt + 2, nk - 1) * kTK;
    ua = load_unit(p.ac, p.as, p.M, m0, p.K, kn, false, t);
    uw = load_unit(p.wc, p.ws, p.N, n0, p.K, kn, w2, t);
    const uint8_t* A = lds + (kt & 1) * kGBuf;
    const uint8_t* B = A + kOpBytes;
    uint8_t* nb = lds + ((kt + 1) & 1) * kGBuf;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 wf[4], af[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = frag(B + (64 * wn + 16 * i + l16) * kRow + 64 * ks + 16 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) af[j] = frag(A + (128 * wm + 16 * j + l16) * kRow + 64 * ks + 16 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
    store_unit(nb, ca, t);
    store_unit(nb + kOpBytes, cw, t);
    // schedule: the loads, the first fragments, then each matrix instruction
    // followed by a decode instruction (and the second fragments, then the
    // LDS writes, spread among them)
    __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);   // global loads
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      if ((i & 3) == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS writes
    }
    __syncthreads();
  }

  // acc[i][j][e] = C^T[n0 + 64 wn + 16 i + 4 g + e][m0 + 128 wm + 16 j + l16]
  const float gaw = p.ag[0] * p.wg[0];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + 128 * wm + 16 * j + l16;
    if (m >= p.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 64 * wn + 16 * i + 4 * g;
      if (n >= p.N) continue;
      const f32x4 v = acc[i][j];
      *reinterpret_cast<u32x2*>(p.out + (size_t)m * p.N + n) =
          u32x2{pack_bf16x2(v[0] * gaw, v[1] * gaw), pack_bf16x2(v[2] * gaw, v[3] * gaw)};
    }
  }
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API int nvfp4_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales,
                                           const float* a_tensor_scale, int M, int K, const uint8_t* w_codes,
                                           const uint8_t* w_scales, const float* w_tensor_scale, int N, int w_2d,
                                           uint16_t* out, void* stream) noexcept {
  if (M < 0 || N < 0 || K < 0 || K % kTK != 0 || N % 16 != 0) return NVFP4_ERR_SHAPE;
  if ((long long)M * K > (1LL << 40) || (long long)N * K > (1LL << 40)) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_tensor_scale || !w_codes || !w_scales || !w_tensor_scale || !out)
    return NVFP4_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 2) || !aligned(w_scales, 2) ||
      !aligned(out, 8) || !aligned(a_tensor_scale, 4) || !aligned(w_tensor_scale, 4))
    return NVFP4_ERR_ALIGN;
  const size_t nw_s = w_2d ? (size_t)(N / 16) * (K / 16) : (size_t)N * (K / 16);
  const Range in[6] = {range_of(a_codes, (size_t)M * K / 2), range_of(a_scales, (size_t)M * K / 16),
                       range_of(a_tensor_scale, 4), range_of(w_codes, (size_t)N * K / 2), range_of(w_scales, nw_s),
                       range_of(w_tensor_scale, 4)};
  const Range outr[1] = {range_of(out, (size_t)M * N * 2)};
  if (any_alias(in, 6, outr, 1)) return NVFP4_ERR_ALIAS;
  if (K == 0) return NVFP4_ERR_SHAPE;

  GemmParams p{};
  p.ac = a_codes; p.as = a_scales; p.wc = w_codes; p.ws = w_scales;
  p.ag = a_tensor_scale; p.wg = w_tensor_scale; p.out = out;
  p.M = M; p.N = N; p.K = K; p.w2d = w_2d != 0;
  p.ntm = (M + kTM - 1) / kTM;
  p.ntn = (N + kTN - 1) / kTN;
  const long long total = (long long)p.ntm * p.ntn;
  if (total > (1LL << 28)) return NVFP4_ERR_SHAPE;
  p.total = (int)total;
  p.per_xcd = (p.total + kXcds - 1) / kXcds;
  (void)hipGetLastError();
  gemm_w4a4_kernel<<<dim3(kXcds * p.per_xcd), dim3(kGThreads), 0, as_stream(stream)>>>(p);
  return launch_status();
}
