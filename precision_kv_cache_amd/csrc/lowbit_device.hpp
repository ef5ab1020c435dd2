// lowbit_device.hpp -- the 3-bit / 2-bit KV block encoder, shared by the
// two-pass quantize kernel (kv_lowbit.hip) and the overlapped kernel
// (kv_overlap.hip).  The format: sign + E1M1 {0, .5, 1, 1.5} (3 bits) or sign
// + E1M0 {0, 1} (2 bits) elements, 16-element blocks with one E4M3FN scale
// chosen from two candidates t_b / c_a and t_b / c_b by the lower fp32 error
// (ties keep c_a), element i at bits [bits i, bits i + bits) of the block's
// 2 bits bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.hpp"

namespace nvfp4 {

template <int BITS>
struct LowBit {
  static constexpr float ca = BITS == 3 ? 1.5f : 1.0f;  // maps the block maximum onto the top magnitude
  static constexpr float cb = BITS == 3 ? 1.0f : 1.5f;  // the 3 : 2 companion
  static constexpr int bytes = 2 * BITS;                // code bytes per block
};

template <int BITS>
__host__ __device__ constexpr float lowbit_constant(int mode) {
  return 448.0f * (mode == kModeFixed6 ? LowBit<BITS>::ca
                                       : mode == kModeFixed4 ? LowBit<BITS>::cb
                                                             : (LowBit<BITS>::ca < LowBit<BITS>::cb ? LowBit<BITS>::ca
                                                                                                    : LowBit<BITS>::cb));
}

// One candidate on a block z (encode domain) with scale S and reciprocal R:
// the packed codes (lo: bits 0..31, hi: bits 32..47) and the fp32 error.
template <int BITS>
__device__ __forceinline__ float lowbit_candidate(const float (&z)[16], float S, float R, uint32_t& lo,
                                                  uint32_t& hi) {
  float elo = 0.0f, ehi = 0.0f;
  lo = 0u;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y = z[i] * R;
    const float a = fabsf(y);
    float k;  // magnitude index, as a float
    if (BITS == 3)
      k = fminf(__builtin_rintf(a * 2.0f), 3.0f);  // rint: nearest, ties to even
    else
      k = a > 0.5f ? 1.0f : 0.0f;                 // the tie 0.5 goes to the even code 0
    const float v = BITS == 3 ? k * 0.5f : k;      // magnitude value, exact
    const uint32_t neg = __float_as_uint(y) >> 31;
    const float vs = __uint_as_float(__float_as_uint(v) | (neg << 31));  // signed value (-0 kept)
    const float e = __builtin_fmaf(-vs, S, z[i]);  // v * S is exact: fl(z - v S)
    if (i < 8)
      elo = __builtin_fmaf(e, e, elo);
    else
      ehi = __builtin_fmaf(e, e, ehi);
    const uint32_t code = (uint32_t)k | (neg << (BITS - 1));
    const int pos = BITS * i;
    if (pos < 32) lo |= code << pos;
    if (pos + BITS > 32) hi |= code >> (32 - pos > 0 ? 32 - pos : 0) << (pos > 32 ? pos - 32 : 0);
  }
  return elo + ehi;
}

struct LowBitBlock {
  uint32_t lo, hi, scale, useb;
};

template <int BITS, int MODE>
__device__ __forceinline__ LowBitBlock lowbit_block16(const float (&z)[16], const float2* tab) {
  const float t = block_absmax(z);
  // both candidate scales in one conversion: byte 0 = E4M3(t / ca), byte 1 = E4M3(t / cb);
  // the division by 1.5 is the IEEE quotient (correctly rounded division)
  const float ra = LowBit<BITS>::ca == 1.0f ? t : t / LowBit<BITS>::ca;
  const float rb = LowBit<BITS>::cb == 1.0f ? t : t / LowBit<BITS>::cb;
  const uint32_t s = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, __float_as_int(t), false) & 0xffffu;
  LowBitBlock out;
  if (MODE == kModeFixed6) {
    const float2 c = tab[s & 0xffu];
    (void)lowbit_candidate<BITS>(z, c.x, c.y, out.lo, out.hi);
    out.scale = s & 0xffu;
    out.useb = 0;
  } else if (MODE == kModeFixed4) {
    const float2 c = tab[s >> 8];
    (void)lowbit_candidate<BITS>(z, c.x, c.y, out.lo, out.hi);
    out.scale = s >> 8;
    out.useb = 1;
  } else {
    const float2 c0 = tab[s & 0xffu], c1 = tab[s >> 8];
    uint32_t la, ha, lb, hb;
    const float ea = lowbit_candidate<BITS>(z, c0.x, c0.y, la, ha);
    const float eb = lowbit_candidate<BITS>(z, c1.x, c1.y, lb, hb);
    const bool useb = eb < ea;
    out.lo = useb ? lb : la;
    out.hi = useb ? hb : ha;
    out.scale = useb ? (s >> 8) : (s & 0xffu);
    out.useb = useb ? 1u : 0u;
  }
  return out;
}

// The quantize loop of one lane at 3 or 2 bits, as quant_rows: rows r, r +
// step, ... below r_end of a slab of rows of NB blocks whose first row is
// row0, column block col, one row per step (two rows' loads in flight need
// more registers than they save).  m: the channel means subtracted first
// when SMOOTH, g: the encode scale, tab: the scale table (LDS).  Returns
// {blocks keeping c_b, blocks}.
template <int BITS, int MODE, bool SMOOTH, int NBC>
__device__ __forceinline__ uint2 lowbit_quant_rows(const uint16_t* xb, uint8_t* codes, uint8_t* scales, size_t row0,
                                                   int r, int r_end, int step, int nb, int col,
                                                   const float (&m)[16], float g, const float2* tab) {
  const int NB = NBC > 0 ? NBC : nb;
  unsigned nbk = 0, n = 0;
  for (; r < r_end; r += step) {
    const size_t blk = (row0 + r) * NB + col;
    const uint16_t* px = xb + blk * 16;
    const uint4 a = load_nt(px), b = load_nt(px + 8);
    float z[16];
    unpack16(a, b, z);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float xs = SMOOTH ? z[i] - m[i] : z[i];  // k' = fl(K - m)
      z[i] = xs * g;                                  // z = fl(k' * g_enc)
    }
    const LowBitBlock q = lowbit_block16<BITS, MODE>(z, tab);
    uint8_t* pc = codes + blk * LowBit<BITS>::bytes;
    if (BITS == 3) {  // 6 bytes, 2-byte aligned
      uint16_t* pw = reinterpret_cast<uint16_t*>(pc);
      __builtin_nontemporal_store((uint16_t)(q.lo & 0xffffu), pw);
      __builtin_nontemporal_store((uint16_t)(q.lo >> 16), pw + 1);
      __builtin_nontemporal_store((uint16_t)(q.hi & 0xffffu), pw + 2);
    } else {
      __builtin_nontemporal_store(q.lo, reinterpret_cast<uint32_t*>(pc));
    }
    store_nt(scales + blk, (uint8_t)q.scale);
    nbk += q.useb;
    n += 1;
  }
  return make_uint2(nbk, n);
}

}  // namespace nvfp4
