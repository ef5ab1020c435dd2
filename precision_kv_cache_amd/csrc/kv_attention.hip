// kv_attention.hip -- softmax attention of bf16 queries over key ranges of
// one layer's NVFP4 KV cache, decoding the cache tile by tile into LDS (in
// each workgroup, or once per call in the staged form below).  This is the
// consumer of the cache that the LongLive-2.0 summary page builds in its
// inference pipeline (step 7: smoothed K and V in NVFP4 per chunk) and reads
// through a global sink, a shot sink and the recent window (step 9).
//
// One workgroup (8 waves) takes 256 queries of one head; each wave holds 32
// queries as the B operand of v_mfma_f32_16x16x32_bf16.  Keys stream in tiles
// of 64: the workgroup decodes each tile once into LDS (K as [key][dim], V
// transposed to [dim][key]) and every wave then computes
//   S^T = K~ Q^T         (4 key blocks x 2 query blocks x 4 dim steps),
//   online softmax in the base-2 domain, lane-local per query,
//   O^T += V~^T P^T      (8 dim blocks x 2 query blocks x 2 key steps),
// where the S^T accumulators, rounded to bf16, are the P^T operand as they
// stand: the V tile's key order in LDS is permuted to match them.
//
// Decode on load: v comes from the E2M1 conversion instruction (scale 1,
// exact), then one fp32 multiply by the block scale S.  For K, v * S has at
// most 6 significant bits, so K~ = v * S is exact in bf16 and the logits are
// exact up to fp32 accumulation: the per-chunk factor g_K * scale * log2(e)
// multiplies the accumulated dot product inside the fused multiply-add that
// feeds exp2, and the smoothing mean enters as the bias
// scale * log2(e) * (q . m_c), one value per (query, chunk).  For V the
// factor S * g_V is applied before one rounding to bf16.  Tiles never cross a
// chunk edge, so the factors and the bias are uniform over a tile.
//
// With a workspace, the host may split each query block's key list into up
// to four parts of about equal tile counts, one workgroup each, when that
// fills the CUs in fewer rounds; each part stores its unnormalized O, its
// reference maximum and its weight sum, and a small kernel merges the parts
// per query row in a fixed order.
//
// Staged form: when the workspace also holds, after the room of every split,
// the decoded image of every key tile (the LDS bytes the decode would write,
// 35 KB per tile and cache head), a staging kernel decodes each tile once per
// call, and the attention workgroups copy the images into LDS with
// direct-to-LDS loads instead of decoding every tile in each of the head's
// query blocks: four image buffers, the copies a pair of tiles ahead, one
// barrier per pair.  The images hold the same bytes and the per-tile steps
// are shared, so the results are bit-identical to the decode-on-load form.
#include <hip/hip_runtime.h>
#include <math.h>
#include <algorithm>
#include <stdint.h>

#include "host_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4kv.h"

namespace nvfp4 {
namespace {

constexpr int kD = 128;              // head dimension of this kernel
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;              // queries per wave
constexpr int kQB = kWaves * kQW;    // queries per workgroup
constexpr int kKT = 64;              // keys per tile
constexpr int kKRow = kD * 2 + 16;   // LDS bytes per K row (padded: 16 rows hit distinct banks)
constexpr int kVRow = kKT * 2 + 16;  // LDS bytes per V^T row
constexpr int kKBytes = kKT * kKRow;
constexpr int kVBytes = kD * kVRow;
constexpr int kBuf = kKBytes + kVBytes;
constexpr int kXcds = 8;
constexpr int kMaxSplit = 4;  // key splits per query block at most

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct AttnParams {
  const uint16_t* q;
  const uint8_t *kc, *ks, *vc, *vs;
  const float *kg, *vg, *km;
  uint16_t* out;
  float* lse;
  int H, Tq, group, Hkv, T, L;
  long long hstride, cstride;  // cache rows between heads / between chunks (head-major: T, L; chunk-major: L, H_kv L)
  int nr;
  int rstart[NVFP4_ATTN_MAX_RANGES], rlen[NVFP4_ATTN_MAX_RANGES];
  float sigma;  // softmax scale * log2(e)
  int nqb;      // query blocks per head
  int hq;       // H * nqb
  int total;    // hq * ksplit
  int per_xcd;  // workgroup slots per XCD
  // Key splits: workgroup (j, h, qb) takes split_tiles[j] tiles of the key
  // list from the cursor (split_r[j], split_pos[j]).  With ksplit > 1 it
  // writes its unnormalized O, its reference maximum M (base-2 logits) and
  // its weight sum l to part_o / part_ml, and a combine kernel merges them.
  int ksplit;
  int split_r[kMaxSplit], split_pos[kMaxSplit], split_tiles[kMaxSplit];
  float* part_o;   // [ksplit][H][Tq][D]
  float* part_ml;  // [ksplit][H][Tq][2]
  // Staged form: img holds the decoded LDS image of tile t of cache head kvh
  // at (kvh * ntiles + t) * kBuf; split j starts at tile split_t0[j].
  const uint8_t* img;
  uint8_t* img_out;  // the same buffer, written by the staging kernel
  long long ntiles;
  int split_t0[kMaxSplit];
};

// Next tile of the key list: [start, start + n), n <= 64, inside one range
// and one chunk.  (r, pos) is the cursor; all of it is workgroup-uniform.
__device__ __forceinline__ bool next_tile(const AttnParams& p, int& r, int& pos, int& start, int& n) {
  while (r < p.nr && pos >= p.rstart[r] + p.rlen[r]) {
    ++r;
    if (r < p.nr) pos = p.rstart[r];
  }
  if (r >= p.nr) return false;
  const int end = p.rstart[r] + p.rlen[r];
  const int cend = pos - pos % p.L + min(p.L, end - (pos - pos % p.L));  // min(chunk end, range end)
  start = pos;
  n = min(kKT, cend - pos);
  pos += n;
  return true;
}

// next_tile within a split's budget of tiles.
__device__ __forceinline__ bool take_tile(const AttnParams& p, int& r, int& pos, int& start, int& n, int& left) {
  if (left <= 0) return false;
  --left;
  return next_tile(p, r, pos, start, n);
}

// Raw cache bytes of one tile, held in registers between the global loads
// and the decode into LDS.
struct TileRegs {
  uint32_t k0, k1;  // K: 16 codes of one (key, block)
  uint32_t kscale;  // its E4M3 scale byte
  uint32_t v[4];    // V: 4 codes (2 bytes) of 4 keys
  uint32_t vscale[4];
};

// Thread roles for a tile.  K -- key tid / 8, block tid % 8 (16 dims): the
// eight lanes of a key read its 64 contiguous code bytes, and a wave covers
// eight consecutive keys.  V -- keys 4 (tid % 16) .. +3, dims 4 (tid / 16)
// .. +3, so that sixteen lanes write the sixteen 8-byte slots of one V^T row
// (distinct banks).  Keys past the tile's end (n >= 1) load the tile's last
// key instead, so the loads need no branches; those keys' logits are set to
// -inf and their weights to 0 after the products, and their values are
// finite, so they add nothing.
__device__ __forceinline__ void load_tile(const AttnParams& p, int kvh, int start, int n, TileRegs& t) {
  const int tid = threadIdx.x;
  const size_t row0 = (size_t)kvh * p.hstride + (size_t)(start / p.L) * p.cstride + start % p.L;
  {
    const int kk = min(tid >> 3, n - 1), b = tid & 7;
    const uint2 c = *reinterpret_cast<const uint2*>(p.kc + (row0 + kk) * (kD / 2) + 8 * b);
    t.k0 = c.x;
    t.k1 = c.y;
    t.kscale = p.ks[(row0 + kk) * (kD / 16) + b];
  }
  {
    const int a = tid & 15, c = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = min(4 * a + i, n - 1);
      t.v[i] = *reinterpret_cast<const uint16_t*>(p.vc + (row0 + kk) * (kD / 2) + 2 * c);
      t.vscale[i] = p.vs[(row0 + kk) * (kD / 16) + (c >> 2)];
    }
  }
}

// Two E2M1 codes (byte `sel` of w) -> fp32, exact (scale operand 1).
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Decode the tile's registers into LDS buffer `buf`: K~ = v * S (exact in
// bf16), V~ = bf16(v * S * gv).
__device__ __forceinline__ void store_tile(uint8_t* buf, const TileRegs& t, float gv) {
  const int tid = threadIdx.x;
  {
    const int kk = tid >> 3, b = tid & 7;
    const float f = __builtin_amdgcn_cvt_f32_fp8(t.kscale, 0);
    f32x2 x[8];
    x[0] = fp4x2<0>(t.k0); x[1] = fp4x2<1>(t.k0); x[2] = fp4x2<2>(t.k0); x[3] = fp4x2<3>(t.k0);
    x[4] = fp4x2<0>(t.k1); x[5] = fp4x2<1>(t.k1); x[6] = fp4x2<2>(t.k1); x[7] = fp4x2<3>(t.k1);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = pack_bf16x2(x[i].x * f, x[i].y * f);
    uint8_t* dst = buf + kk * kKRow + 32 * b;
    *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(dst + 16) = u32x4{w[4], w[5], w[6], w[7]};
  }
  {
    const int a = tid & 15, c = tid >> 4;
    float val[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = __builtin_amdgcn_cvt_f32_fp8(t.vscale[i], 0) * gv;
      const f32x2 lo = fp4x2<0>(t.v[i]), hi = fp4x2<1>(t.v[i]);
      val[i][0] = lo.x * f;
      val[i][1] = lo.y * f;
      val[i][2] = hi.x * f;
      val[i][3] = hi.y * f;
    }
    // key 4a + i sits at column 32 (a / 8) + 8 (a % 4) + 4 ((a % 8) / 4) + i of
    // the V^T rows: the order in which the S^T accumulators hold the keys.
    const int col = 32 * (a >> 3) + 8 * (a & 3) + 4 * ((a & 7) >> 2);
    uint8_t* vbuf = buf + kKBytes;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      uint8_t* dst = vbuf + (4 * c + dd) * kVRow + 2 * col;
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(val[0][dd], val[1][dd]), pack_bf16x2(val[2][dd], val[3][dd])};
    }
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ float bf(const bf16x8& v, int i) { return (float)v[i]; }

// Largest x over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes that
// hold one query), by two VALU lane swaps.
__device__ __forceinline__ float max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Cursor (range, position) at which tile `at` of the key list starts: the
// walk of next_tile, counted in closed form per chunk piece.
__device__ bool tile_cursor(const AttnParams& p, long long at, int& cr, int& cpos) {
  long long t = 0;
  for (int r = 0; r < p.nr; ++r) {
    long long pos = p.rstart[r];
    const long long end = pos + p.rlen[r];
    while (pos < end) {
      const long long cend = min(end, (pos / p.L + 1) * (long long)p.L);  // this chunk piece's end
      const long long nt = (cend - pos + kKT - 1) / kKT;
      if (at < t + nt) {
        cr = r;
        cpos = (int)(pos + (at - t) * kKT);
        return true;
      }
      t += nt;
      pos = cend;
    }
  }
  return false;
}

// Staging kernel: decodes tile blockIdx.x of cache head blockIdx.y's key
// list into LDS exactly as the decode-on-load path does (store_tile), then
// copies the 35 KB image out in whole 16-byte rows per lane, so the workspace
// receives full cache lines (the pad bytes carry whatever LDS held; nothing
// reads them).  WIDE: the tile's code rows (64 contiguous bytes per key) and
// scale rows (8 bytes) are first copied into LDS with 16- and 8-byte loads,
// and the decode reads its bytes from there; else the decode-on-load path's
// own narrow loads (load_tile), for caches whose codes are not 16-byte or
// whose scales are not 8-byte aligned.
template <bool WIDE>
__global__ __launch_bounds__(kThreads) void attention_stage_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t img[kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t raw[2][kKT * (kD / 2 + kD / 16)];  // K, V: codes then scales
  const int kvh = blockIdx.y;
  const long long ti = blockIdx.x;
  int r = 0, pos = 0, start = 0, n = 0;
  if (!tile_cursor(p, ti, r, pos) || !next_tile(p, r, pos, start, n)) return;
  TileRegs regs;
  if constexpr (WIDE) {
    const int tid = threadIdx.x;
    const size_t row0 = (size_t)kvh * p.hstride + (size_t)(start / p.L) * p.cstride + start % p.L;
    constexpr int kCodeRow = kD / 2, kScaleRow = kD / 16, kScales = kKT * kCodeRow;
    {  // codes: 4 x 16 bytes per key, threads 0-255 for K, 256-511 for V
      const int op = tid >> 8, ch = tid & 255, kk = ch >> 2;
      if (kk < n) {
        const uint8_t* src = (op == 0 ? p.kc : p.vc) + (row0 + kk) * kCodeRow + 16 * (ch & 3);
        *reinterpret_cast<u32x4*>(raw[op] + 16 * ch) = *reinterpret_cast<const u32x4*>(src);
      }
    }
    if (tid < 2 * kKT) {  // scales: 8 bytes per key
      const int op = tid / kKT, kk = tid % kKT;
      if (kk < n) {
        const uint8_t* src = (op == 0 ? p.ks : p.vs) + (row0 + kk) * kScaleRow;
        *reinterpret_cast<u32x2*>(raw[op] + kScales + 8 * kk) = *reinterpret_cast<const u32x2*>(src);
      }
    }
    __syncthreads();
    {  // the fields load_tile would read, from LDS (keys past the end: the last key)
      const int kk = min(tid >> 3, n - 1), b = tid & 7;
      const uint2 c = *reinterpret_cast<const uint2*>(raw[0] + kk * kCodeRow + 8 * b);
      regs.k0 = c.x;
      regs.k1 = c.y;
      regs.kscale = raw[0][kScales + kk * kScaleRow + b];
    }
    {
      const int a = tid & 15, c = tid >> 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = min(4 * a + i, n - 1);
        regs.v[i] = *reinterpret_cast<const uint16_t*>(raw[1] + kk * kCodeRow + 2 * c);
        regs.vscale[i] = raw[1][kScales + kk * kScaleRow + (c >> 2)];
      }
    }
  } else {
    load_tile(p, kvh, start, n, regs);
  }
  store_tile(img, regs, p.vg[start / p.L]);
  __syncthreads();
  u32x4* dst = reinterpret_cast<u32x4*>(p.img_out + ((size_t)kvh * p.ntiles + ti) * kBuf);
  const u32x4* src = reinterpret_cast<const u32x4*>(img);
  for (int i = threadIdx.x; i < kBuf / 16; i += kThreads) dst[i] = src[i];
}

constexpr int kImageRounds = kBuf / 1024;  // rounds of 64 lanes x 16 bytes per image
static_assert(kBuf % 1024 == 0, "the image is whole rounds of 64 x 16 bytes (and 256-byte aligned)");

// Copies the image of tile ti of cache head kvh into LDS buffer `buf` by
// direct-to-LDS loads, the rounds spread over the waves.  The caller waits
// for them (vmcnt) before its barrier.
__device__ __forceinline__ void copy_image(const AttnParams& p, int kvh, long long ti, uint8_t* buf) {
  const uint8_t* src = p.img + ((size_t)kvh * p.ntiles + ti) * kBuf + (threadIdx.x & 63) * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int wi = wave; wi < kImageRounds; wi += kWaves)
    __builtin_amdgcn_global_load_lds(src + (size_t)wi * 1024, (__attribute__((address_space(3))) void*)(buf + wi * 1024),
                                     16, 0, 0);
}

// ---- the per-tile steps of a wave (32 queries), shared by both kernels ----

// Q^T fragments: lane holds query qw0 + 16 nt + l16, dims 32 ks + 8 g .. +7.
__device__ __forceinline__ void load_queries(const AttnParams& p, int h, int qw0, int l16, int g, bf16x8 (&bq)[2][4]) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = qw0 + 16 * nt + l16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (qi < p.Tq)
        bq[nt][ks] = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)h * p.Tq + qi) * kD + 32 * ks + 8 * g);
      else
        bq[nt][ks] = bf16x8{};
    }
  }
}

// A tile of chunk c: logit factor kf = g_K * sigma and, per query, the bias
// beta = sigma * (q . m_c).
__device__ __forceinline__ void chunk_factors(const AttnParams& p, int kvh, int c, const bf16x8 (&bq)[2][4], int g,
                                              float& kf, float (&beta)[2]) {
  kf = p.kg[c] * p.sigma;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float part = 0.f;
    if (p.km) {
      const float* mc = p.km + ((size_t)c * p.Hkv + kvh) * kD + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 m0 = *reinterpret_cast<const float4*>(mc + 32 * ks);
        const float4 m1 = *reinterpret_cast<const float4*>(mc + 32 * ks + 4);
        const bf16x8& qv = bq[nt][ks];
        part = __builtin_fmaf(bf(qv, 0), m0.x, part);
        part = __builtin_fmaf(bf(qv, 1), m0.y, part);
        part = __builtin_fmaf(bf(qv, 2), m0.z, part);
        part = __builtin_fmaf(bf(qv, 3), m0.w, part);
        part = __builtin_fmaf(bf(qv, 4), m1.x, part);
        part = __builtin_fmaf(bf(qv, 5), m1.y, part);
        part = __builtin_fmaf(bf(qv, 6), m1.z, part);
        part = __builtin_fmaf(bf(qv, 7), m1.w, part);
      }
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    beta[nt] = part * p.sigma;
  }
}

// S^T = K~ Q^T: s[mt][nt][i] = q . (v S) of key 16 mt + 4 g + i, query 16 nt + l16.
__device__ __forceinline__ void tile_scores(const uint8_t* kb, const bf16x8 (&bq)[2][4], int l16, int g,
                                            f32x4 (&s)[4][2]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) s[mt][0] = s[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const bf16x8 a = lds_frag(kb + (16 * mt + l16) * kKRow + 64 * ks + 16 * g);
      s[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[0][ks], s[mt][0], 0, 0, 0);
      s[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[1][ks], s[mt][1], 0, 0, 0);
    }
  }
}

// Online softmax of a tile of t_n keys, base 2: logit = s * kf + beta (kf >=
// 0, so the largest s gives the largest logit).  The reference M moves only
// when a logit exceeds it by more than 8, so the weights stay below 2^8 and
// the O rescale is rare.  Leaves the weights, rounded to bf16, in pb: the P^T
// fragments, keys 32 k2 + 8 g + j (j < 4: block 2 k2, j >= 4: block 2 k2 + 1).
__device__ __forceinline__ void tile_softmax(f32x4 (&s)[4][2], int t_n, float kf, const float (&beta)[2],
                                             float (&M)[2], float (&lsum)[2], f32x4 (&o)[8][2], bf16x8 (&pb)[2][2],
                                             int g) {
  if (t_n < kKT) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * mt + 4 * g + i >= t_n) s[mt][0][i] = s[mt][1][i] = -INFINITY;
  }
  float alpha[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float mx = s[0][nt][0];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][nt][i]);
    mx = max4(mx);
    const float cand = __builtin_fmaf(mx, kf, beta[nt]);
    const float mnew = cand > M[nt] + 8.0f ? cand : M[nt];
    alpha[nt] = __builtin_amdgcn_exp2f(M[nt] - mnew);
    const float c0 = beta[nt] - mnew;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[mt][nt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][i], kf, c0));
    if (t_n < kKT) {  // keys past the tile's end weigh 0 (also when kf == 0)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * mt + 4 * g + i >= t_n) s[mt][nt][i] = 0.f;
    }
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rs += s[mt][nt][i];
    lsum[nt] = __builtin_fmaf(lsum[nt], alpha[nt], rs);
    M[nt] = mnew;
  }
  if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f) != 0) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) o[m][nt] *= alpha[nt];
  }
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const f32x4 a = s[2 * k2][nt], b = s[2 * k2 + 1][nt];
      const u32x4 u{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                    pack_bf16x2(b[2], b[3])};
      pb[k2][nt] = __builtin_bit_cast(bf16x8, u);
    }
}

// O^T += V~^T P^T
__device__ __forceinline__ void tile_pv(const uint8_t* vb, const bf16x8 (&pb)[2][2], int l16, int g,
                                        f32x4 (&o)[8][2]) {
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const bf16x8 a = lds_frag(vb + (16 * m + l16) * kVRow + 64 * k2 + 16 * g);
      o[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[k2][0], o[m][0], 0, 0, 0);
      o[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[k2][1], o[m][1], 0, 0, 0);
    }
  }
}

// O = O^T / l, rows of 4 dims per lane; lse = ln 2 * (M + log2 l).  A key
// split stores its O, M and l for the combine kernel instead.  The lane's
// indices are recomputed here rather than kept live across the tile loop.
__device__ __forceinline__ void store_rows(const AttnParams& p, int js, int h, int qb, const f32x4 (&o)[8][2],
                                           const float (&M)[2], const float (&lsum)[2]) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g = lane >> 4;
  const int qw0 = qb * kQB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kQW;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float l = lsum[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int qi = qw0 + 16 * nt + l16;
    if (qi >= p.Tq) continue;
    if (p.ksplit > 1) {
      const size_t row = ((size_t)js * p.H + h) * p.Tq + qi;
      float* dst = p.part_o + row * kD + 4 * g;
#pragma unroll
      for (int m = 0; m < 8; ++m) *reinterpret_cast<f32x4*>(dst + 16 * m) = o[m][nt];
      if (g == 0) *reinterpret_cast<f32x2*>(p.part_ml + row * 2) = f32x2{M[nt], l};
      continue;
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    uint16_t* dst = p.out + ((size_t)h * p.Tq + qi) * kD + 4 * g;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f32x4 v = o[m][nt];
      *reinterpret_cast<u32x2*>(dst + 16 * m) = u32x2{pack_bf16x2(v[0] * inv, v[1] * inv),
                                                      pack_bf16x2(v[2] * inv, v[3] * inv)};
    }
    if (p.lse && g == 0) p.lse[(size_t)h * p.Tq + qi] = (M[nt] + __log2f(l)) * 0.69314718055994531f;
  }
}

// The workgroup's (key split, head, query block).  Workgroups are dispatched
// round-robin over the XCDs; the slots of one XCD take consecutive query
// blocks of the same head so that they share that XCD's L2 for the head's
// cache.
struct Work {
  int js, h, kvh, qb;
};
__device__ __forceinline__ bool work_of(const AttnParams& p, Work& wk) {
  const int w = (int)(blockIdx.x % kXcds) * p.per_xcd + (int)(blockIdx.x / kXcds);
  if (w >= p.total) return false;
  wk.js = w / p.hq;
  const int hqi = w % p.hq;
  wk.h = hqi / p.nqb;
  wk.qb = hqi % p.nqb;
  wk.kvh = wk.h / p.group;
  return true;
}

// Decode on load: the workgroup decodes each tile into one of two LDS
// buffers (the next tile's bytes load while the current tile is computed),
// one barrier per tile.
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBuf];
  Work wk;
  if (!work_of(p, wk)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int qw0 = wk.qb * kQB + wave * kQW;
  bf16x8 bq[2][4];
  load_queries(p, wk.h, qw0, l16, g, bq);
  f32x4 o[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m][0] = o[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f}, beta[2] = {0.f, 0.f};
  float kf = 0.f;
  int cur_chunk = -1;

  int r = p.split_r[wk.js], pos = p.split_pos[wk.js], left = p.split_tiles[wk.js];
  int t_start = 0, t_n = 0;
  bool have = take_tile(p, r, pos, t_start, t_n, left);
  TileRegs regs;
  if (have) {
    load_tile(p, wk.kvh, t_start, t_n, regs);
    store_tile(lds, regs, p.vg[t_start / p.L]);
  }
  __syncthreads();
  int cur = 0;
  while (have) {
    int n_start = 0, n_n = 0;
    const bool nhave = take_tile(p, r, pos, n_start, n_n, left);
    if (nhave) load_tile(p, wk.kvh, n_start, n_n, regs);
    const int c = t_start / p.L;
    if (c != cur_chunk) {
      cur_chunk = c;
      chunk_factors(p, wk.kvh, c, bq, g, kf, beta);
    }
    const uint8_t* kb = lds + cur * kBuf;
    f32x4 s[4][2];
    bf16x8 pb[2][2];
    tile_scores(kb, bq, l16, g, s);
    tile_softmax(s, t_n, kf, beta, M, lsum, o, pb, g);
    tile_pv(kb + kKBytes, pb, l16, g, o);
    // the next tile into the other buffer, last read before the previous barrier
    if (nhave) store_tile(lds + (cur ^ 1) * kBuf, regs, p.vg[n_start / p.L]);
    __syncthreads();
    cur ^= 1;
    t_start = n_start;
    t_n = n_n;
    have = nhave;
  }
  store_rows(p, wk.js, wk.h, wk.qb, o, M, lsum);
}

// Staged form: four image buffers and one barrier per pair of tiles.  At the
// barrier before tiles t, t + 1 (t even from the split's first tile) both
// are in LDS; right after it every wave issues its share of the copies of
// tiles t + 2, t + 3 into the buffers of tiles t - 2, t - 1 (read before
// this barrier), then computes t and t + 1 with no barrier between them, so
// the waves may drift apart within a pair.
__global__ __launch_bounds__(kThreads) void attention_staged_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kBuf];
  Work wk;
  if (!work_of(p, wk)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int qw0 = wk.qb * kQB + wave * kQW;
  bf16x8 bq[2][4];
  load_queries(p, wk.h, qw0, l16, g, bq);
  f32x4 o[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m][0] = o[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f}, beta[2] = {0.f, 0.f};
  float kf = 0.f;
  int cur_chunk = -1;

  int r = p.split_r[wk.js], pos = p.split_pos[wk.js], left = p.split_tiles[wk.js];
  long long ti = p.split_t0[wk.js];  // tile index of the pair's first tile
  int c0s = 0, c0n = 0, c1s = 0, c1n = 0;  // the pair's tiles: start, count
  bool h0 = take_tile(p, r, pos, c0s, c0n, left);
  bool h1 = h0 && take_tile(p, r, pos, c1s, c1n, left);
  if (h0) copy_image(p, wk.kvh, ti, lds);
  if (h1) copy_image(p, wk.kvh, ti + 1, lds + kBuf);
  int b = 0;  // buffer of the pair's first tile: 0 or 2
  f32x4 s[4][2];
  bf16x8 pb[2][2];
  while (h0) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the pair are in LDS
    __builtin_amdgcn_s_barrier();
    int n0s = 0, n0n = 0, n1s = 0, n1n = 0;
    const bool g0 = h1 && take_tile(p, r, pos, n0s, n0n, left);
    const bool g1 = g0 && take_tile(p, r, pos, n1s, n1n, left);
    uint8_t* nb = lds + (b ^ 2) * kBuf;
    if (g0) copy_image(p, wk.kvh, ti + 2, nb);
    if (g1) copy_image(p, wk.kvh, ti + 3, nb + kBuf);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && !h1) break;
      const int ts = k == 0 ? c0s : c1s, tn = k == 0 ? c0n : c1n;
      const uint8_t* kb = lds + (b + k) * kBuf;
      const int c = ts / p.L;
      if (c != cur_chunk) {
        cur_chunk = c;
        chunk_factors(p, wk.kvh, c, bq, g, kf, beta);
      }
      tile_scores(kb, bq, l16, g, s);
      tile_softmax(s, tn, kf, beta, M, lsum, o, pb, g);
      tile_pv(kb + kKBytes, pb, l16, g, o);
    }
    c0s = n0s; c0n = n0n; c1s = n1s; c1n = n1n;
    h0 = g0;
    h1 = g1;
    b ^= 2;
    ti += 2;
  }
  store_rows(p, wk.js, wk.h, wk.qb, o, M, lsum);
}

// Merges the key splits of each query row: M* = max_j M_j, w_j = 2^(M_j - M*)
// (0 for a split without keys), out = sum_j w_j O_j / sum_j w_j l_j, lse =
// ln 2 (M* + log2 sum_j w_j l_j); in a fixed split order.  32 lanes per row,
// 4 dims each.
__global__ __launch_bounds__(256) void attention_combine_kernel(const float* part_o, const float* part_ml, int ksplit,
                                                                long long rows, uint16_t* out, float* lse) {
  const long long row = (long long)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const int d = 4 * (threadIdx.x & 31);
  float Mj[kMaxSplit], lj[kMaxSplit];
  float Ms = -INFINITY;
  for (int j = 0; j < ksplit; ++j) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(part_ml + ((size_t)j * rows + row) * 2);
    Mj[j] = ml[0];
    lj[j] = ml[1];
    Ms = fmaxf(Ms, ml[0]);
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int j = 0; j < ksplit; ++j) {
    if (Mj[j] == -INFINITY) continue;  // no keys in this split
    const float wj = __builtin_amdgcn_exp2f(Mj[j] - Ms);
    const f32x4 oj = *reinterpret_cast<const f32x4*>(part_o + ((size_t)j * rows + row) * kD + d);
    acc += oj * wj;
    L = __builtin_fmaf(lj[j], wj, L);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<u32x2*>(out + (size_t)row * kD + d) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (lse && d == 0) lse[row] = (Ms + __log2f(L)) * 0.69314718055994531f;
}

}  // namespace

// Host replica of the kernel's tile walk: the number of tiles of the key
// list, and the cursor (range, position) at which tile `at` starts.  Tiles
// are at most 64 keys and never cross a chunk or range edge.
static long long host_tiles(const AttnParams& p, long long at, int* cur_r, int* cur_pos) {
  long long t = 0;
  for (int r = 0; r < p.nr; ++r) {
    long long pos = p.rstart[r];
    const long long end = pos + p.rlen[r];
    while (pos < end) {
      const long long cend = std::min(end, (pos / p.L + 1) * (long long)p.L);  // this chunk piece's end
      const long long nt = (cend - pos + kKT - 1) / kKT;
      if (at >= t && at < t + nt) {
        *cur_r = r;
        *cur_pos = (int)(pos + (at - t) * kKT);
        return t;
      }
      t += nt;
      pos = cend;
    }
  }
  return t;
}

// Workspace bytes of k key splits over `rows` query rows: the partial O,
// then (M, l) per row.
static size_t split_bytes(int k, size_t rows) {
  return align_up((size_t)k * rows * kD * 4, 256) + align_up((size_t)k * rows * 8, 256);
}

// Bytes of the decoded tile images of a key list of ntiles tiles.
static size_t image_bytes(int H_kv, long long ntiles) { return (size_t)H_kv * (size_t)ntiles * kBuf; }

constexpr long long kMaxPieces = 1 << 16;        // chunk pieces of a key list that splits and staging walk
// Tiles of a staged key list: the staging grid's work-items (tiles x 512)
// stay below 2^32, as a launch counts them in 32 bits.
constexpr long long kMaxImageTiles = (1LL << 32) / kThreads - 1;
// Workgroups of an attention launch, every split included, for the same reason.
constexpr long long kMaxAttnGroups = (1LL << 32) / kThreads - kXcds;

// Chunk pieces of the key list (each range cut at chunk edges).
static long long count_pieces(const AttnParams& p) {
  long long pieces = 0;
  for (int r = 0; r < p.nr; ++r)
    pieces += ((long long)p.rstart[r] + p.rlen[r] - 1) / p.L - p.rstart[r] / p.L + 1;
  return pieces;
}

// Key splits per query block: the count (at most kMaxSplit) that minimizes
// the rounds of the grid over the CUs, per unit of work, when the workspace
// holds it and every split gets at least 4 tiles.
static int choose_ksplit(int hq, long long ntiles, size_t rows, size_t ws_bytes) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return 1;
  int best = 1;
  double best_t = 1e30;
  for (int k = 1; k <= kMaxSplit; ++k) {
    if (k > 1 && (ntiles < 4LL * k || split_bytes(k, rows) > ws_bytes || (long long)hq * k > kMaxAttnGroups)) break;
    const double rounds = (double)(((long long)hq * k + ncu - 1) / ncu) / k;
    if (rounds < best_t - 1e-9) {
      best_t = rounds;
      best = k;
    }
  }
  return best;
}

// Shared host path of the two layouts.
static int attention_launch(const uint16_t* q, int H, int Tq, int D, const uint8_t* k_codes, const uint8_t* k_scales,
                     const float* k_tensor_scale, const float* k_mean, const uint8_t* v_codes,
                     const uint8_t* v_scales, const float* v_tensor_scale, int H_kv, int T, int chunk_len,
                     const int* key_ranges, int n_ranges, float softmax_scale, uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, void* stream, bool chunk_major) {
  if (H < 0 || Tq < 0 || T < 0 || H_kv < 1 || chunk_len < 1 || D != kD) return NVFP4_ERR_SHAPE;
  if (H % H_kv != 0 || T % chunk_len != 0) return NVFP4_ERR_SHAPE;
  if (n_ranges < 0 || n_ranges > NVFP4_ATTN_MAX_RANGES || !(softmax_scale > 0.f && softmax_scale <= 3.0e38f))
    return NVFP4_ERR_SHAPE;
  if (n_ranges > 0 && !key_ranges) return NVFP4_ERR_NULL;
  for (int i = 0; i < n_ranges; ++i) {
    const long long a = key_ranges[2 * i], n = key_ranges[2 * i + 1];
    if (a < 0 || n < 0 || a + n > T) return NVFP4_ERR_SHAPE;
  }
  if (H == 0 || Tq == 0) return NVFP4_OK;
  if (!q || !out) return NVFP4_ERR_NULL;
  if (T > 0 && (!k_codes || !k_scales || !k_tensor_scale || !v_codes || !v_scales || !v_tensor_scale))
    return NVFP4_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 8) || !aligned(k_codes, 8) || !aligned(v_codes, 2) ||
      !aligned(k_mean, 16) || !aligned(k_tensor_scale, 4) || !aligned(v_tensor_scale, 4) || !aligned(lse, 4) ||
      !aligned(workspace, 256))
    return NVFP4_ERR_ALIGN;
  const size_t nq = (size_t)H * Tq * kD, nkv = (size_t)H_kv * T * kD, nc = (size_t)(T / chunk_len);
  const Range in[8] = {range_of(q, nq * 2),
                       range_of(k_codes, nkv / 2),
                       range_of(k_scales, nkv / 16),
                       range_of(k_tensor_scale, nc * 4),
                       range_of(k_mean, k_mean ? nc * H_kv * kD * 4 : 0),
                       range_of(v_codes, nkv / 2),
                       range_of(v_scales, nkv / 16),
                       range_of(v_tensor_scale, nc * 4)};
  const Range outr[3] = {range_of(out, nq * 2), range_of(lse, lse ? (size_t)H * Tq * 4 : 0),
                         range_of(workspace, workspace ? workspace_bytes : 0)};
  if (any_alias(in, 8, outr, 3)) return NVFP4_ERR_ALIAS;

  AttnParams p{};
  p.q = q;
  p.kc = k_codes; p.ks = k_scales; p.vc = v_codes; p.vs = v_scales;
  p.kg = k_tensor_scale; p.vg = v_tensor_scale; p.km = k_mean;
  p.out = out; p.lse = lse;
  p.H = H; p.Tq = Tq; p.group = H / H_kv; p.Hkv = H_kv; p.T = T; p.L = chunk_len;
  p.hstride = chunk_major ? chunk_len : T;
  p.cstride = chunk_major ? (long long)H_kv * chunk_len : chunk_len;
  p.nr = 0;
  for (int i = 0; i < n_ranges; ++i) {
    if (key_ranges[2 * i + 1] == 0) continue;
    p.rstart[p.nr] = key_ranges[2 * i];
    p.rlen[p.nr] = key_ranges[2 * i + 1];
    ++p.nr;
  }
  p.sigma = softmax_scale * 1.4426950408889634f;
  p.nqb = (Tq + kQB - 1) / kQB;
  const long long hq = (long long)H * p.nqb;
  if (hq > kMaxAttnGroups) return NVFP4_ERR_SHAPE;
  p.hq = (int)hq;
  // one split: the whole key list from its start, no tile budget
  p.ksplit = 1;
  p.split_r[0] = 0;
  p.split_pos[0] = p.nr > 0 ? p.rstart[0] : 0;
  p.split_tiles[0] = 0x7fffffff;
  p.split_t0[0] = 0;
  const size_t rows = (size_t)H * Tq;
  // Key splits and staging need the tile walk on the host (and the staging
  // kernel repeats it per workgroup), so both are skipped for key lists of
  // very many chunk pieces.
  const bool walkable = count_pieces(p) <= kMaxPieces;
  int cr = 0, cpos = 0;
  const long long ntiles = walkable ? host_tiles(p, -1, &cr, &cpos) : 0;
  if (workspace && walkable && workspace_bytes >= split_bytes(2, rows)) {
    const int k = choose_ksplit(p.hq, ntiles, rows, workspace_bytes);
    if (k > 1) {
      p.ksplit = k;
      for (int j = 0; j < k; ++j) {
        const long long t0 = ntiles * j / k, t1 = ntiles * (j + 1) / k;
        host_tiles(p, t0, &p.split_r[j], &p.split_pos[j]);
        p.split_tiles[j] = (int)(t1 - t0);
        p.split_t0[j] = (int)t0;
      }
      p.part_o = static_cast<float*>(workspace);
      p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up((size_t)k * rows * kD * 4, 256));
    }
  }
  // Staged form when the workspace holds, after the room of every key split,
  // every tile image (the size nvfp4_kv_attention_staged_workspace_bytes
  // gives): a smaller workspace keeps the decode on load.
  bool staged = false;
  const size_t img_off = split_bytes(kMaxSplit, rows);
  if (workspace && ntiles > 0 && ntiles <= kMaxImageTiles && H_kv <= 65535 &&
      img_off + image_bytes(H_kv, ntiles) <= workspace_bytes) {
    staged = true;
    p.ntiles = ntiles;
    p.img_out = static_cast<uint8_t*>(workspace) + img_off;
    p.img = p.img_out;
  }
  p.total = p.hq * p.ksplit;
  p.per_xcd = (p.total + kXcds - 1) / kXcds;
  hipStream_t s = as_stream(stream);
  (void)hipGetLastError();
  if (staged) {
    const dim3 sg((unsigned)p.ntiles, (unsigned)H_kv);
    if (aligned(k_codes, 16) && aligned(v_codes, 16) && aligned(k_scales, 8) && aligned(v_scales, 8))
      attention_stage_kernel<true><<<sg, dim3(kThreads), 0, s>>>(p);
    else
      attention_stage_kernel<false><<<sg, dim3(kThreads), 0, s>>>(p);
    attention_staged_kernel<<<dim3(kXcds * p.per_xcd), dim3(kThreads), 0, s>>>(p);
  } else {
    attention_kernel<<<dim3(kXcds * p.per_xcd), dim3(kThreads), 0, s>>>(p);
  }
  if (p.ksplit > 1) {
    const long long nb = ((long long)rows + 7) / 8;
    attention_combine_kernel<<<dim3((unsigned)nb), dim3(256), 0, s>>>(p.part_o, p.part_ml, p.ksplit, (long long)rows,
                                                                     out, lse);
  }
  return launch_status();
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" NVFP4KV_API size_t nvfp4_kv_attention_workspace_bytes(int H, int Tq, int D) noexcept {
  if (H < 1 || Tq < 1 || D != kD) return 0;
  return split_bytes(kMaxSplit, (size_t)H * Tq);
}

extern "C" NVFP4KV_API size_t nvfp4_kv_attention_staged_workspace_bytes(int H, int Tq, int D, int H_kv, int T,
                                                                       int chunk_len, const int* key_ranges,
                                                                       int n_ranges) noexcept {
  if (H < 1 || Tq < 1 || D != kD || H_kv < 1 || T < 0 || chunk_len < 1 || H % H_kv != 0 || T % chunk_len != 0)
    return 0;
  if (n_ranges < 0 || n_ranges > NVFP4_ATTN_MAX_RANGES || (n_ranges > 0 && !key_ranges)) return 0;
  AttnParams p{};
  p.L = chunk_len;
  for (int i = 0; i < n_ranges; ++i) {
    const long long a = key_ranges[2 * i], n = key_ranges[2 * i + 1];
    if (a < 0 || n < 0 || a + n > T) return 0;
    if (n == 0) continue;
    p.rstart[p.nr] = (int)a;
    p.rlen[p.nr] = (int)n;
    ++p.nr;
  }
  const size_t splits = split_bytes(kMaxSplit, (size_t)H * Tq);
  if (count_pieces(p) > kMaxPieces) return splits;  // such a key list runs unstaged
  int cr = 0, cpos = 0;
  const long long ntiles = host_tiles(p, -1, &cr, &cpos);
  if (ntiles > kMaxImageTiles || H_kv > 65535) return splits;
  return splits + image_bytes(H_kv, ntiles);
}

extern "C" NVFP4KV_API int nvfp4_kv_attention(const uint16_t* q, int H, int Tq, int D, const uint8_t* k_codes,
                                              const uint8_t* k_scales, const float* k_tensor_scale,
                                              const float* k_mean, const uint8_t* v_codes, const uint8_t* v_scales,
                                              const float* v_tensor_scale, int H_kv, int T, int chunk_len,
                                              const int* key_ranges, int n_ranges, float softmax_scale,
                                              uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                                              void* stream) noexcept {
  return attention_launch(q, H, Tq, D, k_codes, k_scales, k_tensor_scale, k_mean, v_codes, v_scales, v_tensor_scale,
                          H_kv, T, chunk_len, key_ranges, n_ranges, softmax_scale, out, lse, workspace,
                          workspace_bytes, stream, false);
}

extern "C" NVFP4KV_API int nvfp4_kv_attention_chunked(const uint16_t* q, int H, int Tq, int D,
                                                      const uint8_t* k_codes, const uint8_t* k_scales,
                                                      const float* k_tensor_scale, const float* k_mean,
                                                      const uint8_t* v_codes, const uint8_t* v_scales,
                                                      const float* v_tensor_scale, int H_kv, int T, int chunk_len,
                                                      const int* key_ranges, int n_ranges, float softmax_scale,
                                                      uint16_t* out, float* lse, void* workspace,
                                                      size_t workspace_bytes, void* stream) noexcept {
  return attention_launch(q, H, Tq, D, k_codes, k_scales, k_tensor_scale, k_mean, v_codes, v_scales, v_tensor_scale,
                          H_kv, T, chunk_len, key_ranges, n_ranges, softmax_scale, out, lse, workspace,
                          workspace_bytes, stream, true);
}
