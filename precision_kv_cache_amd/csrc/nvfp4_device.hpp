// nvfp4_device.hpp -- gfx950 device building blocks of the NVFP4 4/6
// quantizer: bf16 unpacking, the two candidate block scales, the exact
// reciprocal, the 16-element E2M1 encode with its fp32 error, and the 4/6
// choice (full-stack NVFP4 section of the LongLive-2.0 summary page).
//
// Every conversion uses a CDNA4 hardware instruction whose rounding matches
// the format definitions (round to nearest even, E2M1 saturating at 6 with
// the sign kept, E4M3FN with subnormals); the test suite sweeps them against
// the CPU reference.  All arithmetic is fp32, one rounding per operation;
// the fused multiply-adds below are written out where the result is
// identical to the unfused form (an exact product) or where the error sum
// is defined as fused.  Built with -ffp-contract=off so that the compiler
// adds no other contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));

enum { kMode4over6 = 0, kModeFixed6 = 1, kModeFixed4 = 2 };

// Tensor-scale constant: the encode scale maps the largest magnitude to C, so
// a block's candidate scale t_b / c stays within the E4M3 range (448) for
// every candidate the mode uses.
__host__ __device__ constexpr float mode_constant(int mode) { return mode == kModeFixed6 ? 2688.0f : 1792.0f; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bf16 values (two 16-byte loads) -> fp32.
__device__ __forceinline__ void unpack16(const uint4& a, const uint4& b, float (&x)[16]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = bf16_lo(w[j]);
    x[2 * j + 1] = bf16_hi(w[j]);
  }
}

// fl(t / 6) for t >= 0 without a division: the product with fl(1/6), its
// exact residual by a fused multiply-add, and one correction.  Equal to the
// IEEE quotient for every normal t; for subnormal t (t / 6 < 2^-126) it may
// differ by an ulp, but both round to the E4M3 code 0.
__device__ __forceinline__ float div6(float t) {
  const float inv6 = 0x1.555556p-3f;  // fl(1/6)
  const float q = t * inv6;
  const float r = __builtin_fmaf(-q, 6.0f, t);
  return __builtin_fmaf(r, inv6, q);
}

// fl(1 / S) for an E4M3 value S, 0 for S = 0: the hardware reciprocal (1 ulp)
// plus one Newton step whose residual is exact; equal to the IEEE quotient
// for all 126 positive finite E4M3 values.
__device__ __forceinline__ float recip_e4m3(float S) {
  const float r = __builtin_amdgcn_rcpf(S);
  const float e = __builtin_fmaf(-S, r, 1.0f);
  const float r2 = __builtin_fmaf(e, r, r);
  return S > 0.0f ? r2 : 0.0f;
}

// (S, fl(1/S)) for every E4M3FN byte 0 .. 127 (R = 0 for S = 0; byte 0x7F,
// a NaN, is never a candidate).  One LDS read then replaces a candidate's
// decode and reciprocal.  Filled by the first 128 threads of a workgroup;
// the caller synchronizes before the first use.
__device__ __forceinline__ void fill_scale_table(float2* tab) {
  const int i = threadIdx.x;
  if (i < 128) {
    const float S = __builtin_amdgcn_cvt_f32_fp8(i, 0);
    tab[i] = make_float2(S, recip_e4m3(S));
  }
}

// Both candidate scales of a block with largest |z| = t: byte 0 = E4M3(t/6),
// byte 1 = E4M3(t/4).
__device__ __forceinline__ uint32_t candidate_codes(float t) {
  // the conversion writes the low 16 bits and keeps the rest of its first
  // operand, which is masked off: passing t (dead here) saves zeroing a register
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(div6(t), t * 0.25f, __float_as_int(t), false) & 0xffffu;
}


// Encode 8 values z[0..7] (already in the encode domain) with reciprocal R:
// one word of 8 E2M1 codes, element 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t encode8(const float* z, float R) {
  // the four conversions write all four bytes of w, so its starting value is
  // irrelevant: starting from y0 (dead after the first one) saves zeroing it
  const float y0 = z[0] * R;
  uint32_t w = __float_as_uint(y0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y0, z[1] * R, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[2] * R, z[3] * R, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[4] * R, z[5] * R, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[6] * R, z[7] * R, 1.0f, 3);
  return w;
}

// Sum over the 8 elements of (z - v * S)^2, sequential fused accumulation
// from 0 in element order; v * S is exact, so fma(-v, S, z) is the rounded
// difference.
__device__ __forceinline__ float half_error(const float* z, uint32_t w, float S) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2 v;
    switch (j) {  // the byte selector is an instruction immediate
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    const float e0 = __builtin_fmaf(-v[0], S, z[2 * j]);
    acc = __builtin_fmaf(e0, e0, acc);
    const float e1 = __builtin_fmaf(-v[1], S, z[2 * j + 1]);
    acc = __builtin_fmaf(e1, e1, acc);
  }
  return acc;
}

struct Encoded16 {
  uint32_t lo, hi;  // codes of elements 0..7 and 8..15
  float err_lo, err_hi;
};

__device__ __forceinline__ Encoded16 encode16(const float (&z)[16], float S, float R) {
  Encoded16 r;
  r.lo = encode8(z, R);
  r.hi = encode8(z + 8, R);
  r.err_lo = half_error(z, r.lo, S);
  r.err_hi = half_error(z + 8, r.hi, S);
  return r;
}

__device__ __forceinline__ float block_absmax(const float (&z)[16]) {
  float t = fabsf(z[0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) t = fmaxf(t, fabsf(z[i]));
  return t;
}

struct Block46 {
  uint32_t lo, hi;  // 16 packed codes
  uint32_t scale;   // E4M3 byte
  uint32_t use4;    // 1 when the +-4 candidate was kept
};

// Four-Over-Six on one 16-element block in the encode domain: both
// candidates, each block's fp32 error (two halves added), keep +-4 only when
// its error is strictly lower.  The fixed modes evaluate one candidate.
// tab: the scale table of fill_scale_table (in LDS).
template <int MODE>
__device__ __forceinline__ Block46 quant_block16(const float (&z)[16], const float2* tab) {
  const float t = block_absmax(z);
  const uint32_t s = candidate_codes(t);
  Block46 out;
  if (MODE == kModeFixed6) {
    const float2 c = tab[s & 0xffu];
    const Encoded16 e = encode16(z, c.x, c.y);
    out.lo = e.lo; out.hi = e.hi; out.scale = s & 0xffu; out.use4 = 0;
  } else if (MODE == kModeFixed4) {
    const float2 c = tab[s >> 8];
    const Encoded16 e = encode16(z, c.x, c.y);
    out.lo = e.lo; out.hi = e.hi; out.scale = s >> 8; out.use4 = 1;
  } else {
    const float2 c6 = tab[s & 0xffu], c4 = tab[s >> 8];
    const Encoded16 e6 = encode16(z, c6.x, c6.y);
    const Encoded16 e4 = encode16(z, c4.x, c4.y);
    const float err6 = e6.err_lo + e6.err_hi;
    const float err4 = e4.err_lo + e4.err_hi;
    const bool use4 = err4 < err6;
    out.lo = use4 ? e4.lo : e6.lo;
    out.hi = use4 ? e4.hi : e6.hi;
    out.scale = use4 ? (s >> 8) : (s & 0xffu);
    out.use4 = use4 ? 1u : 0u;
  }
  return out;
}

// Two fp32 -> packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v = {a, b};
  b2 h = __builtin_convertvector(v, b2);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming 16-byte load / stores (non-temporal: the data is used once).
__device__ __forceinline__ uint4 load_nt(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// NT = false: an ordinary load, which allocates in the Infinity Cache so
// that a second read of the same data soon after is served from there.
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  if (NT) return load_nt(p);
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store_nt(uint8_t* p, uint32_t lo, uint32_t hi) {
  const u32x2 v = {lo, hi};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_nt(uint8_t* p, uint8_t b) { __builtin_nontemporal_store(b, p); }

// The quantize loop of one lane: rows r, r + step, ..., r + (BATCH - 1) *
// step (their loads issued together), then the same BATCH * step rows
// further on, and so on while below r_end, of a slab of rows of NB blocks
// whose first row is row0 (absolute row of the [H, T] row space), column
// block col.  With step = the workgroup's rows per pass, every load and
// store instruction of a wave covers whole consecutive rows.  One pointer per
// stream is advanced by a uniform offset per row, with no per-row index
// arithmetic.  NBC: blocks per row when known at compile time (then nb is
// ignored), else 0.  m: the channel means subtracted first when SMOOTH (the
// K path), g: the encode scale, tab: the scale table (LDS).  Returns
// {blocks kept at +-4, blocks}.
template <int MODE, bool SMOOTH, bool NT, int BATCH, int NBC>
__device__ __forceinline__ uint2 quant_rows(const uint16_t* xb, uint8_t* codes, uint8_t* scales, size_t row0,
                                            int r, int r_end, int step, int nb, int col, const float (&m)[16],
                                            float g, const float2* tab) {
  const int NB = NBC > 0 ? NBC : nb;
  const size_t blk = (row0 + r) * NB + col;
  const uint16_t* px = xb + blk * 16;
  uint8_t* pc = codes + blk * 8;
  uint8_t* ps = scales + blk;
  const size_t dq = (size_t)step * NB;  // blocks from one row of a batch to the next
  unsigned n4 = 0, nblk = 0;
  for (int rb = r; rb < r_end; rb += BATCH * step, px += BATCH * dq * 16, pc += BATCH * dq * 8, ps += BATCH * dq) {
    uint4 a[BATCH], b[BATCH];
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (rb + q * step < r_end) {
        a[q] = load16<NT>(px + q * dq * 16);
        b[q] = load16<NT>(px + q * dq * 16 + 8);
      }
    }
#pragma unroll
    for (int q = 0; q < BATCH; ++q) {
      if (rb + q * step >= r_end) continue;
      float z[16];
      unpack16(a[q], b[q], z);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float xs = SMOOTH ? z[i] - m[i] : z[i];  // k' = fl(K - m)
        z[i] = xs * g;                                  // z = fl(k' * g_enc)
      }
      const Block46 qb = quant_block16<MODE>(z, tab);
      store_nt(pc + q * dq * 8, qb.lo, qb.hi);
      store_nt(ps + q * dq, (uint8_t)qb.scale);
      n4 += qb.use4;
      nblk += 1;
    }
  }
  return make_uint2(n4, nblk);
}

// Full-tile form of quant_rows with the loads one row ahead: exactly ROWS
// rows per lane (r, r + step, ..., r + (ROWS - 1) step), and row q + 1's
// loads are issued before row q is encoded, so they are in flight during
// that encode.  Same arguments (NB fixed, no bound: every row exists) and
// result as quant_rows.
template <int MODE, bool SMOOTH, int ROWS, int NB>
__device__ __forceinline__ uint2 quant_rows_ahead(const uint16_t* xb, uint8_t* codes, uint8_t* scales, size_t row0,
                                                  int r, int step, int col, const float (&m)[16], float g,
                                                  const float2* tab) {
  const size_t blk = (row0 + r) * NB + col;
  const uint16_t* px = xb + blk * 16;
  uint8_t* pc = codes + blk * 8;
  uint8_t* ps = scales + blk;
  const size_t dq = (size_t)step * NB;  // blocks from one of the lane's rows to the next
  uint4 a[ROWS], b[ROWS];
  a[0] = load_nt(px);
  b[0] = load_nt(px + 8);
  unsigned n4 = 0;
#pragma unroll
  for (int q = 0; q < ROWS; ++q) {
    if (q + 1 < ROWS) {
      a[q + 1] = load_nt(px + (q + 1) * dq * 16);
      b[q + 1] = load_nt(px + (q + 1) * dq * 16 + 8);
    }
    __builtin_amdgcn_sched_barrier(0);  // the next row's loads go out before this row's arithmetic
    float z[16];
    unpack16(a[q], b[q], z);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float xs = SMOOTH ? z[i] - m[i] : z[i];  // k' = fl(K - m)
      z[i] = xs * g;                                  // z = fl(k' * g_enc)
    }
    const Block46 qb = quant_block16<MODE>(z, tab);
    store_nt(pc + q * dq * 8, qb.lo, qb.hi);
    store_nt(ps + q * dq, (uint8_t)qb.scale);
    n4 += qb.use4;
    __builtin_amdgcn_sched_barrier(0);
  }
  return make_uint2(n4, (unsigned)ROWS);
}

// Hand-off of small results between workgroups of one kernel.
//
// On this multi-XCD part every XCD has its own L2, and an agent-scope
// release / acquire fence writes back / invalidates that whole L2; with
// hundreds of workgroups publishing, those fences serialize and dominate.
// So results that other workgroups read inside the same kernel are written
// with agent-scope atomic exchanges, which are performed at the device's
// coherence point, and read with agent-scope atomic loads.  A writer waits
// for every exchange to return (completion at the coherence point) before
// the barrier after which one thread bumps the counter; a reader issues its
// loads only after it has seen the counter (the loads depend on the
// counter's value), so it observes the published values.
__device__ __forceinline__ unsigned add_agent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// publish: exchange, and fold the returned old value into `done` so the
// caller can make the exchange's completion explicit (see wait_published)
__device__ __forceinline__ void publish(float* p, float v, uint32_t& done) {
  done ^= __float_as_uint(__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void publish(double* p, double v, uint32_t& done) {
  const double o = __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  done ^= (uint32_t)__double_as_longlong(o);
}
// forces the wait for every exchange folded into `done` (its value is needed)
__device__ __forceinline__ void wait_published(uint32_t done) { asm volatile("" ::"v"(done)); }
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double fetch(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grids of segments (the single-launch kernels): segment s = 0 .. n - 1 +
// depth holds ns work items of unit s (when s < n), then nq items of unit
// s - depth (when 0 <= s - depth < n).  For the flat index b, the segment s
// and b's offset in it, in closed form: the segments are stats-only
// (s < min(depth, n)), then either both (depth <= s < n) and quantize-only
// (n <= s), or empty (n <= s < depth) and quantize-only.  ns, nq >= 1, and
// the caller keeps the grid below 2^32.
__device__ __forceinline__ void segment_of(unsigned b, int n, int depth, unsigned ns, unsigned nq, int& s,
                                           unsigned& off) {
  const unsigned a = (unsigned)(depth < n ? depth : n);
  if (b < a * ns) {
    s = (int)(b / ns);
    off = b % ns;
    return;
  }
  b -= a * ns;
  if (depth < n) {
    const unsigned both = ns + nq, m = (unsigned)(n - depth);
    if (b < m * both) {
      s = depth + (int)(b / both);
      off = b % both;
      return;
    }
    b -= m * both;
    s = n + (int)(b / nq);
  } else {
    s = depth + (int)(b / nq);
  }
  off = b % nq;
}

// Wave-level reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ unsigned wave_sum_u32(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 4/6 choice tallies without contended atomics: each workgroup sums its
// threads' counts {K kept +-4, K blocks, V kept +-4, V blocks} through LDS
// (sh: one entry of 4 per wave) and thread 0 stores them in the workgroup's
// own 16-byte slot; a one-workgroup kernel adds the slots up at the end.
// Every thread of the workgroup calls this (it holds two barriers).
__device__ __forceinline__ void store_wg_tally(uint32_t* slot, const unsigned (&t)[4], unsigned* sh) {
  const int tid = threadIdx.x, nw = (int)(blockDim.x + 63) / 64;
  unsigned w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = wave_sum_u32(t[j]);
  __syncthreads();
  if ((tid & 63) == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) sh[(tid >> 6) * 4 + j] = w[j];
  }
  __syncthreads();
  if (tid == 0) {
    unsigned a[4] = {0u, 0u, 0u, 0u};
    for (int q = 0; q < nw; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] += sh[q * 4 + j];
    *reinterpret_cast<uint4*>(slot) = make_uint4(a[0], a[1], a[2], a[3]);
  }
}

}  // namespace nvfp4
