// Stochastic integer quantisation + bit packing of message rows, and the degree normalisation.
//
// Method: SYLVIE guide, section 6 (scale = (max - min) / (2^b - 1), stochastic rounding of
// (h - min) / scale, min travels as the zero-point).  Layout of a packed row: ceil(d*b/32)
// words, code j at bit j*b, LSB first (raw float32 words for b = 32).
//
// Mapping to gfx950: a row of d features is owned by d/16 lanes, each holding 16 consecutive
// features (four 16-byte loads).  Two Philox4x32-10 calls per lane yield the sixteen 16-bit
// rounding thresholds of its features, so the generator is paid once per 8 elements, and the
// per-row work every lane of a row repeats (the min / max butterfly, the scale's two rounded
// divisions, the width lookup) is shared by 16 features.  Codes are packed in registers (16 b
// bits a lane, whole words for b >= 2) and pairs of lanes' halves are merged with a lane shuffle
// for 1-bit rows, so every word is written once.  d = 128 gives 8 lanes per row and eight rows
// per wavefront.
#include "qha_internal.hpp"
#include "quant_common.hpp"

#pragma clang fp contract(off)

namespace qha {
namespace {

// min / max over the G lanes of a row (G = 1, 2, 4, 8, 16, 32; rows start at lanes that are
// multiples of G).  Lanes 1 and 2 apart through DPP quad permutes, then the mirrored lane of the
// half row (8 lanes) and of the row (16 lanes): after the quad steps every lane of a quad holds
// its quad's value, so the mirror pairs each lane with the other quad (half).  32 lanes: a swap
// of the two 16-lane halves.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int G>
__device__ __forceinline__ void row_min_max(float& mn, float& mx) {
  constexpr int kXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
  constexpr int kXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]
  constexpr int kHalfMirror = 0x141;
  constexpr int kMirror = 0x140;
  if constexpr (G >= 2) { mn = fminf(mn, dpp_f<kXor1>(mn)); mx = fmaxf(mx, dpp_f<kXor1>(mx)); }
  if constexpr (G >= 4) { mn = fminf(mn, dpp_f<kXor2>(mn)); mx = fmaxf(mx, dpp_f<kXor2>(mx)); }
  if constexpr (G >= 8) { mn = fminf(mn, dpp_f<kHalfMirror>(mn)); mx = fmaxf(mx, dpp_f<kHalfMirror>(mx)); }
  if constexpr (G >= 16) { mn = fminf(mn, dpp_f<kMirror>(mn)); mx = fmaxf(mx, dpp_f<kMirror>(mx)); }
  if constexpr (G >= 32) { mn = fminf(mn, __shfl_xor(mn, 16)); mx = fmaxf(mx, __shfl_xor(mx, 16)); }
}

template <int D>
__global__ __launch_bounds__(256) void quantize_pack_kernel(QuantArgs a) {
  constexpr int F = 16;          // features per lane: two Philox calls
  static_assert(D % F == 0 && D / F <= 32, "d = 16 .. 512");
  constexpr int G = D / F;       // lanes per row
  constexpr int RPW = 64 / G;    // rows per wavefront
  const int lane = threadIdx.x & 63;
  const int gl = lane % G;
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + wib) * RPW;   // wave's first row
  const int64_t r = r0 + lane / G;
  const bool valid = r < a.n_rows;

  // lanes past the last row work on the last row and store nothing
  const int64_t rc = valid ? r : a.n_rows - 1;
  float v[F];
  {
    const int64_t src = a.row_index ? static_cast<int64_t>(a.row_index[rc]) : rc;
    const float4* p = reinterpret_cast<const float4*>(a.x + src * a.ldx + gl * F);
#pragma unroll
    for (int q = 0; q < F / 4; ++q) {
      const float4 t = p[q];
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  }
  // The rounding draws depend only on the row's node id and the lane's groups, not on its values:
  // the two Philox calls (features 16 gl + 8 h .. + 7 are group 2 gl + h) run while the row's loads
  // are in flight.
  uint32_t w[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t c0 = a.node_base + static_cast<uint32_t>(r);
    uint32_t c1 = static_cast<uint32_t>(2 * gl + h);
    uint32_t c2 = a.epoch;
    uint32_t c3 = a.stream_id;
    philox4x32_10(c0, c1, c2, c3, a.seed_lo, a.seed_hi);
    // an empty statement that takes the four words as register operands: it keeps their computation
    // here, beside the row's loads, where the compiler would otherwise sink it past the branches below
    asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
    w[h][0] = c0;
    w[h][1] = c1;
    w[h][2] = c2;
    w[h][3] = c3;
  }
  uint32_t b, row_off;
  if (a.cls.n > 0) {
    // width-grouped buffer (fewer than 2^31 rows): the class of the wave's first row by selects over
    // the whole table (no branch waits on a table entry); a wave whose rows cross into the next
    // class looks its rows up one by one
    const int32_t w0 = static_cast<int32_t>(r0);
    const int32_t wl = w0 + (RPW - 1);
    int32_t st = a.cls.start[0];
    uint32_t base = a.cls.base[0];
    int32_t bb = a.cls.bits[0];
    bool straddle = false;
#pragma unroll
    for (int c = 1; c < kMaxClasses; ++c) {
      const bool in = c < a.cls.n;
      const int32_t sc = a.cls.start[c];
      const bool ge = in && w0 >= sc;
      st = ge ? sc : st;
      base = ge ? a.cls.base[c] : base;
      bb = ge ? a.cls.bits[c] : bb;
      straddle = straddle || (in && !ge && wl >= sc);
    }
    const int32_t r32 = static_cast<int32_t>(rc);
    if (straddle) {
#pragma unroll
      for (int c = 1; c < kMaxClasses; ++c) {
        const bool ge = c < a.cls.n && r32 >= a.cls.start[c];
        st = ge ? a.cls.start[c] : st;
        base = ge ? a.cls.base[c] : base;
        bb = ge ? a.cls.bits[c] : bb;
      }
    }
    b = static_cast<uint32_t>(bb);
    const uint32_t words = (b == 32u) ? static_cast<uint32_t>(D) : (b * static_cast<uint32_t>(D) + 31u) >> 5;
    row_off = base + static_cast<uint32_t>(r32 - st) * words;
  } else {
    b = a.bits[rc];
    row_off = a.word_offset[rc];
  }

  // exact min / max of the row: in-lane, then across the row's G lanes
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < F; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  row_min_max<G>(mn, mx);

  const bool active = valid && width_valid(b);
  const bool raw = b == 32u;
  const bool coded = active && !raw;
  // The lane's 16 codes in four groups: code 4k + i at bit i b of acc[k].  Every lane forms them
  // (rows that are raw or not written use width 1 and keep nothing), so that the draws, which every
  // lane uses, stay where they are computed: ahead of the wait for the row.
  const uint32_t bq = coded ? b : 1u;
  const RowScale rs = row_scale(mn, mx, bq);
  const float zp = coded ? rs.zp : 0.0f;
  const float sc = coded ? rs.sc : 0.0f;
  uint32_t acc[4] = {0u, 0u, 0u, 0u};
  {
    const uint32_t sh[4] = {0u, bq, 2u * bq, 3u * bq};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = 8 * h + i;
        const uint32_t q = code_of(v[j], mn, rs, draw16_c(w[h], i));
        acc[j >> 2] |= q << sh[j & 3];
      }
    }
  }
  // b = 4: words lo, hi; b <= 2: one word of 16 b bits (shifts wrap where the result is unused)
  const uint32_t t4 = (4u * b) & 31u;
  const uint32_t lo = acc[0] | (acc[1] << t4);
  const uint32_t hi = acc[2] | (acc[3] << t4);
  const uint32_t one = lo | (hi << ((2u * t4) & 31u));
  // 1-bit rows: a lane's codes fill half a word; the even lane takes its odd neighbour's half
  const uint32_t nb = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(one), 0xB1, 0xF, 0xF, true));
  if (!active) return;

  uint32_t* row_codes = a.codes + row_off;
  if (raw) {
#pragma unroll
    for (int i = 0; i < F; ++i) row_codes[gl * F + i] = __float_as_uint(v[i]);
  } else if (b == 8u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) row_codes[4 * gl + k] = acc[k];
  } else if (b == 4u) {
    row_codes[2 * gl] = lo;
    row_codes[2 * gl + 1] = hi;
  } else if (b == 2u) {
    row_codes[gl] = one;
  } else {  // b == 1
    if ((gl & 1) == 0) row_codes[gl >> 1] = one | ((gl + 1 < G) ? nb << 16 : 0u);
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
  constexpr int RPB = 4 * (64 / (D / 16));  // rows per 256-thread block
  const int64_t blocks = (a.n_rows + RPB - 1) / RPB;
  hipLaunchKernelGGL(quantize_pack_kernel<D>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, int32_t d, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.cls.n > 0 && a.n_rows > INT32_MAX) return hipErrorInvalidValue;   // class rows are 32-bit
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
