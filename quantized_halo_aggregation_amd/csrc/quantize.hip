// Stochastic integer quantisation + bit packing of message rows, and the degree normalisation.
//
// Method: SYLVIE guide, section 6 (scale = (max - min) / (2^b - 1), stochastic rounding of
// (h - min) / scale, min travels as the zero-point).  Layout of a packed row: ceil(d*b/32)
// words, code j at bit j*b, LSB first (raw float32 words for b = 32).
//
// Mapping to gfx950: a row of d features is owned by d/8 lanes, each holding 8 consecutive
// features (two 16-byte loads).  One Philox4x32-10 call per lane yields the eight 16-bit rounding
// thresholds of its features, so the generator is paid once per 8 elements.  Row min/max come
// from a butterfly over the row's lanes; codes are packed in registers and neighbouring lanes'
// pieces are merged with lane shuffles (1- and 2-bit rows), so every word is written once.
// d = 128 gives 16 lanes per row and four rows per wavefront.
#include "qha_internal.hpp"
#include "quant_common.hpp"

#pragma clang fp contract(off)

namespace qha {
namespace {

template <int D>
__global__ __launch_bounds__(256) void quantize_pack_kernel(QuantArgs a) {
  constexpr int G = D / 8;      // lanes per row
  constexpr int RPW = 64 / G;   // rows per wavefront
  const int lane = threadIdx.x & 63;
  const int gl = lane % G;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int64_t r = wave * RPW + lane / G;
  const bool valid = r < a.n_rows;

  float v[8];
  uint32_t b = 0;
  uint32_t row_off = 0;
  if (valid) {
    const int64_t src = a.row_index ? static_cast<int64_t>(a.row_index[r]) : r;
    const float4* p = reinterpret_cast<const float4*>(a.x + src * a.ldx + gl * 8);
    const float4 lo = p[0];
    const float4 hi = p[1];
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    if (a.cls.n > 0) {
      // width-grouped buffer: the row's class, width and first word by arithmetic
      int32_t st = a.cls.start[0];
      uint32_t base = a.cls.base[0];
      b = static_cast<uint32_t>(a.cls.bits[0]);
#pragma unroll
      for (int c = 1; c < kMaxClasses; ++c) {
        if (c < a.cls.n && r >= a.cls.start[c]) {
          st = a.cls.start[c];
          base = a.cls.base[c];
          b = static_cast<uint32_t>(a.cls.bits[c]);
        }
      }
      const uint32_t words = (b == 32u) ? static_cast<uint32_t>(D) : (b * static_cast<uint32_t>(D) + 31u) >> 5;
      row_off = base + static_cast<uint32_t>(r - st) * words;
    } else {
      b = a.bits[r];
      row_off = a.word_offset[r];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }

  // exact min / max of the row: in-lane, then a butterfly over the row's G lanes
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off));
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }

  const bool active = valid && width_valid(b);
  const bool raw = b == 32u;
  uint32_t lo_w = 0, hi_w = 0;
  float sc = 0.0f, zp = 0.0f;
  if (active && !raw) {
    const RowScale rs = row_scale(mn, mx, b);
    zp = rs.zp;
    sc = rs.sc;
    uint32_t c0 = a.node_base + static_cast<uint32_t>(r);
    uint32_t c1 = static_cast<uint32_t>(gl);          // this lane's 8 features are group gl
    uint32_t c2 = a.epoch;
    uint32_t c3 = a.stream_id;
    philox4x32_10(c0, c1, c2, c3, a.seed_lo, a.seed_hi);
    const uint32_t w[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = code_of(v[i], mn, rs, draw16(w, i));
      const uint32_t pos = static_cast<uint32_t>(i) * b;       // < 64
      if (pos < 32u) lo_w |= q << pos;
      else hi_w |= q << (pos - 32u);
    }
  }

  // merge 8- and 16-bit lane pieces into whole words (all lanes take part in the shuffles)
  const uint32_t n1 = __shfl_down(lo_w, 1);
  const uint32_t n2 = __shfl_down(lo_w, 2);
  const uint32_t n3 = __shfl_down(lo_w, 3);
  if (!active) return;

  uint32_t* row_codes = a.codes + row_off;
  if (raw) {
#pragma unroll
    for (int i = 0; i < 8; ++i) row_codes[gl * 8 + i] = __float_as_uint(v[i]);
  } else if (b == 8u) {
    row_codes[2 * gl] = lo_w;
    row_codes[2 * gl + 1] = hi_w;
  } else if (b == 4u) {
    row_codes[gl] = lo_w;
  } else if (b == 2u) {
    if ((gl & 1) == 0) {
      const uint32_t up1 = (gl + 1 < G) ? n1 : 0u;
      row_codes[gl >> 1] = lo_w | (up1 << 16);
    }
  } else {  // b == 1
    if ((gl & 3) == 0) {
      uint32_t word = lo_w;
      if (gl + 1 < G) word |= n1 << 8;
      if (gl + 2 < G) word |= n2 << 16;
      if (gl + 3 < G) word |= n3 << 24;
      row_codes[gl >> 2] = word;
    }
  }
  if (gl == 0) *reinterpret_cast<float2*>(a.meta + 2 * r) = make_float2(zp, sc);   // (min, scale)
}

__global__ __launch_bounds__(256) void degree_norm_kernel(const int32_t* deg, int64_t n, int32_t kind,
                                                         float* out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t dg = deg[i];
  float v;
  if (kind == 0) {
    v = __fdiv_rn(1.0f, __fsqrt_rn(static_cast<float>(dg) + 1.0f));
  } else {
    v = dg > 0 ? __fdiv_rn(1.0f, static_cast<float>(dg)) : 0.0f;
  }
  out[i] = v;
}

template <int D>
hipError_t launch_quantize_d(const QuantArgs& a, hipStream_t s) {
  constexpr int RPB = 4 * (64 / (D / 8));   // rows per 256-thread block
  const int64_t blocks = (a.n_rows + RPB - 1) / RPB;
  hipLaunchKernelGGL(quantize_pack_kernel<D>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, int32_t d, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  switch (d) {
    case 16: return launch_quantize_d<16>(a, s);
    case 32: return launch_quantize_d<32>(a, s);
    case 64: return launch_quantize_d<64>(a, s);
    case 128: return launch_quantize_d<128>(a, s);
    case 256: return launch_quantize_d<256>(a, s);
    case 512: return launch_quantize_d<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_degree_norm(const int32_t* deg, int64_t n, int32_t kind, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(degree_norm_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, deg, n, kind, out);
  return hipGetLastError();
}

}  // namespace qha
