// Device arithmetic of the stochastic quantiser, shared by every kernel that packs messages, so that
// a row quantised after a gather is coded exactly as one quantised on its own.
//
// Method: SYLVIE guide, section 6 (scale = (max - min) / (2^b - 1), stochastic rounding of
// (h - min) / scale to an integer in [0, 2^b - 1], min kept as the zero-point).  Rounding draws come
// from Philox4x32-10 (Salmon et al., SC'11); feature j of row r uses the 16-bit half (j % 2) of
// word (j % 8) / 2 of the call with counter (node id, j / 8, epoch, stream id) and key (seed low,
// seed high), and rounds up when that number is below the fractional part times 2^16.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#pragma clang fp contract(off)

namespace qha {

// Philox4x32-10: ten rounds of the 4x32 S-box with the Weyl key schedule.  Each round's two
// three-way xors are one gfx950 three-input bit operation each (truth table 0x96 = a ^ b ^ c).
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3, k1, 0x96);
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ bool width_valid(uint32_t b) {
  return b == 1u || b == 2u || b == 4u || b == 8u || b == 32u;
}

// Per-row constants of a b-bit code (b < 32) from the row's exact min and max: the zero-point
// (min, with -0 made +0), scale = range / L and its reciprocal inv = L / range, both correctly
// rounded.  A row whose range is 0, or whose reciprocal overflows, is flat: scale 0, every code 0.
struct RowScale {
  float zp, sc, inv;
  uint32_t levels;     // L = 2^b - 1
  bool flat;
};

__device__ __forceinline__ RowScale row_scale(float mn, float mx, uint32_t b) {
  RowScale r;
  r.levels = (1u << b) - 1u;
  const float L = static_cast<float>(r.levels);
  r.zp = mn + 0.0f;
  const float range = mx - mn;
  float inv = __fdiv_rn(L, range);
  r.flat = (range == 0.0f) || isinf(inv);
  r.inv = r.flat ? 0.0f : inv;
  r.sc = r.flat ? 0.0f : __fdiv_rn(range, L);
  return r;
}

// The code of one value: q = floor(y) + [u16 < frac(y) * 2^16], clamped to L, for y = (v - min) * inv
// and the element's 16-bit draw u16.  Computed as (W + (65535 - u16)) >> 16 with W = ceil(y * 2^16):
// y >= +0 and y * 2^16 is exact (a power-of-two scale of a value below 2^9), so
// W = floor(y) * 2^16 + ceil(frac(y) * 2^16), and for an integer u16, u16 < frac(y) * 2^16 exactly
// when u16 < ceil(frac(y) * 2^16), which is when the low 16 bits of the sum carry.  A flat row has
// inv = 0, so y = W = 0 and its code is 0.
__device__ __forceinline__ uint32_t code_of(float v, float mn, const RowScale& r, uint32_t nu16) {
  const float y = (v - mn) * r.inv;
  const uint32_t w = static_cast<uint32_t>(__builtin_ceilf(y * 65536.0f));
  const uint32_t q = (w + nu16) >> 16;
  return q > r.levels ? r.levels : q;
}

// 65535 minus the 16-bit draw of feature j, from the four words of its group's Philox call.
__device__ __forceinline__ uint32_t draw16_c(const uint32_t (&w)[4], int j) {
  const uint32_t word = ~w[(j & 7) >> 1];
  return (j & 1) ? (word >> 16) : (word & 0xFFFFu);
}

}  // namespace qha
