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

// The sum, modulo 2^32, of 0x4B000000 << pos over the elements whose
// magnitude field lies in the low (hi = false) or high code word.
template <int BITS>
__host__ __device__ constexpr uint32_t lowbit_pack_bias(bool hi) {
  uint32_t b = 0u;
  for (int i = 0; i < 16; ++i) {
    const int pos = BITS * i;
    if (!hi && pos < 32) b += 0x4B000000u << pos;
    if (hi && pos >= 32) b += 0x4B000000u << (pos - 32);
  }
  return b;
}

// One candidate on a block z (encode domain) with scale S and reciprocal R:
// the packed magnitude fields of the codes (lo: bits 0..31, hi: bits
// 32..47; the sign bits are the block's, see lowbit_signs) and the fp32
// error.
//
// The magnitude index k (nearest grid point to |y|, y = fl(z R), ties to
// the even index, saturated at the top) comes from one fp32 rounding:
// 2|y| + 2^23 (3 bits) or |y| + 2^23 (2 bits) rounds to nearest even at a
// spacing of 1, i.e. to 2^23 + rint(2|y|) (or 2^23 + rint(|y|)), so after
// the clamp to 2^23 + top, k sits in the low bits of the sum and the
// magnitude value (k / 2, or k) is the sum minus 2^23, exactly.  The error
// needs no sign: y has z's sign (R >= 0) and v S is exact, so
// |fl(z - sign(z) v S)| = fl(|z| - v S) and the squares agree.
//
// CLAMP = false drops the saturation where it can never act: for the
// candidate that maps the block maximum t below the top magnitude (c = 1.0:
// c_b at 3 bits, c_a at 2 bits), S = E4M3(t) gives t / S <= 1.0625 for a
// normal S (RNE to 3 mantissa bits) and t / S < 1.5 for a subnormal one
// (S = k 2^-9, t in [(k - 1/2) 2^-9, (k + 1/2) 2^-9), ties going to even k),
// and R = fl(1 / S), so every |y| = fl(|z| R) <= fl(t R) stays below 1.5:
// 2|y| < 3 rounds to at most 3 = the 3-bit top index, |y| < 1.5 to at most
// 1 = the 2-bit top.  (S = 0 gives R = 0 and y = 0.)
template <int BITS, bool CLAMP = true>
__device__ __forceinline__ float lowbit_candidate(const float (&z)[16], float S, float R, uint32_t& lo,
                                                  uint32_t& hi) {
  constexpr float kMagic = 8388608.0f;  // 2^23
  constexpr float kTop = BITS == 3 ? 3.0f : 1.0f;
  float elo = 0.0f, ehi = 0.0f;
  lo = 0u;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y = z[i] * R;
    const float t0 = BITS == 3 ? __builtin_fmaf(fabsf(y), 2.0f, kMagic) : fabsf(y) + kMagic;
    const float t = CLAMP ? fminf(t0, kMagic + kTop) : t0;
    const float v = BITS == 3 ? __builtin_fmaf(t, 0.5f, -0.5f * kMagic) : t - kMagic;  // k / 2 or k, exact
    const float e = __builtin_fmaf(-v, S, fabsf(z[i]));
    if (i < 8)
      elo = __builtin_fmaf(e, e, elo);
    else
      ehi = __builtin_fmaf(e, e, ehi);
    // t's bits are 0x4B000000 + k (no carry: k <= top): the fields are added
    // with t's bits shifted in whole, and the shifted constant parts are
    // taken out once below
    const int pos = BITS * i;  // the magnitude field: bits pos .. pos + BITS - 2 (never across bit 32)
    if (pos < 32)
      lo += __float_as_uint(t) << pos;
    else
      hi += __float_as_uint(t) << (pos - 32);
  }
  lo -= lowbit_pack_bias<BITS>(false);
  hi -= lowbit_pack_bias<BITS>(true);
  return elo + ehi;
}

// The sign bits of a block's codes (bit BITS i + BITS - 1 = sign bit of
// z_i, which is y_i's for every candidate; -0 keeps its sign), split like
// the codes into lo (bits 0..31) and hi (bits 32..47).
template <int BITS>
__device__ __forceinline__ void lowbit_signs(const float (&z)[16], uint32_t& lo, uint32_t& hi) {
  lo = 0u;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t sb = __float_as_uint(z[i]) >> 31;
    const int pos = BITS * i + BITS - 1;
    if (pos < 32)
      lo |= sb << pos;
    else
      hi |= sb << (pos - 32);
  }
}

struct LowBitBlock {
  uint32_t lo, hi, scale, useb;
};

template <int BITS, int MODE>
__device__ __forceinline__ LowBitBlock lowbit_block16(const float (&z)[16], const float2* tab) {
  // At 3 bits the candidate whose constant is 1.0 (c_b) cannot saturate
  // (lowbit_candidate) and skips the clamp: 3-bit quantize 1-5 % faster.  The
  // same holds for c_a at 2 bits, but there the build without it measured
  // 0.6 % slower, so both 2-bit candidates keep it.
  constexpr bool kClampA = BITS == 2 || LowBit<BITS>::ca != 1.0f;
  constexpr bool kClampB = BITS == 2 || LowBit<BITS>::cb != 1.0f;
  const float t = block_absmax(z);
  // both candidate scales in one conversion: byte 0 = E4M3(t / ca), byte 1 = E4M3(t / cb);
  // the division by 1.5 is the IEEE quotient (correctly rounded division)
  const float ra = LowBit<BITS>::ca == 1.0f ? t : t / LowBit<BITS>::ca;
  const float rb = LowBit<BITS>::cb == 1.0f ? t : t / LowBit<BITS>::cb;
  const uint32_t s = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, __float_as_int(t), false) & 0xffffu;
  LowBitBlock out;
  uint32_t slo, shi;
  lowbit_signs<BITS>(z, slo, shi);
  if (MODE == kModeFixed6) {
    const float2 c = tab[s & 0xffu];
    (void)lowbit_candidate<BITS, kClampA>(z, c.x, c.y, out.lo, out.hi);
    out.scale = s & 0xffu;
    out.useb = 0;
  } else if (MODE == kModeFixed4) {
    const float2 c = tab[s >> 8];
    (void)lowbit_candidate<BITS, kClampB>(z, c.x, c.y, out.lo, out.hi);
    out.scale = s >> 8;
    out.useb = 1;
  } else {
    const float2 c0 = tab[s & 0xffu], c1 = tab[s >> 8];
    uint32_t la, ha, lb, hb;
    const float ea = lowbit_candidate<BITS, kClampA>(z, c0.x, c0.y, la, ha);
    const float eb = lowbit_candidate<BITS, kClampB>(z, c1.x, c1.y, lb, hb);
    const bool useb = eb < ea;
    out.lo = useb ? lb : la;
    out.hi = useb ? hb : ha;
    out.scale = useb ? (s >> 8) : (s & 0xffu);
    out.useb = useb ? 1u : 0u;
  }
  out.lo |= slo;
  out.hi |= shi;
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
