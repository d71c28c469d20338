// Normalised neighbour gather (SpMM over a CSR) with halo dequantisation fused into the loads.
//
// Method: SYLVIE guide, section 2 (z_v sums the neighbours' rows, each divided by
// sqrt(d_v d_u)) and section 6 (a received halo row is scale * q + min, restored to float32).
// The same kernel walks the transposed CSR for the embedding-gradient pass (sections 3 and 11).
//
// Mapping to gfx950: one wavefront owns one work item (a row, or a <= chunk-edge slice of a heavy
// row).  Its 64 lanes split the d features (d/64 contiguous floats per lane), so every neighbour
// costs one coalesced d*4-byte load.  The item's row bounds, column indices, edge weights and the
// halo metadata are wavefront-uniform and go through the scalar unit; only feature rows and packed
// code words use the vector memory pipe.  Edges are processed in batches of eight whose loads are
// all issued before the first is consumed, so each wavefront keeps eight rows in flight.  For a
// halo neighbour each lane fetches the one code word holding its features, shifts and masks its
// codes out and dequantises in float32 (scale * q + min, no contraction) before the weighted add.
// Accumulation is in float64: a float32 product w * x is exact in float64 and MI355X issues
// float64 FMAs at the rate of unpacked float32 ones, so in this memory-bound loop the wider sum
// costs no time and leaves the final rounding to float32 as the only error of the sum itself
// (sums over hub rows and columns with cancellation would otherwise lose digits).
// Heavy rows are split by the host-built plan; their slices write partial sums that a second
// kernel adds in slice order, so results do not depend on scheduling.  Widths below 64 put several
// items into one wavefront (d lanes each).
#include "qha_internal.hpp"

namespace qha {
namespace {

template <typename T>
using cptr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ cptr<T> cst(const T* p) {
  return (cptr<T>)(p);
}

constexpr int vec_of(int D) { return D >= 64 ? D / 64 : 1; }
constexpr int kBatch = 8;

__device__ __forceinline__ float dequant(float sc, uint32_t q, float zp) {
  return __fadd_rn(__fmul_rn(sc, static_cast<float>(q)), zp);
}

// Value of halo row k for this lane's VEC features (j0 = first feature of the lane).
template <int VEC>
__device__ __forceinline__ void load_halo(const GatherArgs& a, int64_t k, int j0, float (&xv)[VEC]) {
  const uint32_t b = cst(a.bits)[k];
  const uint32_t off = cst(a.word_offset)[k];
  const uint32_t* row = a.codes + off;
  if (b == 32u) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) xv[i] = __uint_as_float(row[j0 + i]);
    return;
  }
  if (!(b == 1u || b == 2u || b == 4u || b == 8u)) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) xv[i] = 0.0f;
    return;
  }
  const float sc = cst(a.scale)[k];
  const float zp = cst(a.zero_point)[k];
  const uint32_t mask = (1u << b) - 1u;
  const uint32_t pos = static_cast<uint32_t>(j0) * b;       // first bit of the lane's codes
  if (VEC * 8 <= 32 || b * VEC <= 32u) {
    const uint32_t word = row[pos >> 5] >> (pos & 31u);
#pragma unroll
    for (int i = 0; i < VEC; ++i) xv[i] = dequant(sc, (word >> (static_cast<uint32_t>(i) * b)) & mask, zp);
  } else {
    // VEC * b == 64: two consecutive words, four (b = 8) codes each
    const uint32_t w0 = row[pos >> 5];
    const uint32_t w1 = row[(pos >> 5) + 1];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const uint32_t p = static_cast<uint32_t>(i) * b;
      const uint32_t w = p < 32u ? (w0 >> p) : (w1 >> (p - 32u));
      xv[i] = dequant(sc, w & mask, zp);
    }
  }
}

template <int VEC>
__device__ __forceinline__ void load_inner(const GatherArgs& a, int64_t u, int j0, float (&xv)[VEC]) {
  const float* p = a.x + u * a.ldx + j0;
  if constexpr (VEC == 1) {
    xv[0] = p[0];
  } else if constexpr (VEC == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    xv[0] = t.x; xv[1] = t.y;
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const float4 t = reinterpret_cast<const float4*>(p)[q];
      xv[4 * q + 0] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
    }
  }
}

template <int D, bool HALO>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;      // lanes per item
  constexpr int IPW = 64 / G;     // items per wavefront
  const int lane = threadIdx.x & 63;
  const int j0 = (lane % G) * VEC;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t item = wave * IPW + (IPW == 1 ? 0 : lane / G);
  if (item >= a.n_items) return;

  int64_t row;
  int32_t e0, e1;
  bool split = false;
  if (a.item_row != nullptr) {
    row = cst(a.item_row)[item];
    e0 = cst(a.rowptr)[row];
    e1 = cst(a.rowptr)[row + 1];
    if (item < a.n_split_items) {
      e0 += cst(a.item_chunk)[item] * a.chunk;
      e1 = min(e1, e0 + a.chunk);
      split = true;
    }
  } else {
    row = item;
    e0 = cst(a.rowptr)[row];
    e1 = cst(a.rowptr)[row + 1];
  }
  const double rs = a.rs ? static_cast<double>(cst(a.rs)[row]) : 1.0;

  double acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0;

  for (int32_t e = e0; e < e1; e += kBatch) {
    const int cnt = min(kBatch, e1 - e);
    int32_t u[kBatch];
    double w[kBatch];
    float xv[kBatch][VEC];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) u[i] = (i < cnt) ? cst(a.colidx)[e + i] : 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < cnt) {
        w[i] = a.cs ? rs * static_cast<double>(cst(a.cs)[u[i]]) : rs;
        if (HALO && u[i] >= a.n_inner) {
          load_halo<VEC>(a, static_cast<int64_t>(u[i]) - a.n_inner, j0, xv[i]);
        } else {
          load_inner<VEC>(a, u[i], j0, xv[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < cnt) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = fma(w[i], static_cast<double>(xv[i][v]), acc[v]);
      }
    }
  }

  if (split) {
    double* p = a.partial + item * D + j0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) p[v] = acc[v];
    return;
  }
  float* dst = a.out + row * a.ldo + j0;
  float res[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(a.beta ? static_cast<double>(dst[v]) + acc[v] : acc[v]);
  if constexpr (VEC == 1) {
    dst[0] = res[0];
  } else if constexpr (VEC == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(res[0], res[1]);
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q)
      reinterpret_cast<float4*>(dst)[q] = make_float4(res[4 * q], res[4 * q + 1], res[4 * q + 2], res[4 * q + 3]);
  }
}

// Adds the partial sums of every split row in slice order and writes the row.
template <int D>
__global__ __launch_bounds__(256) void combine_split_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  constexpr int IPW = 64 / G;
  const int lane = threadIdx.x & 63;
  const int j0 = (lane % G) * VEC;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t m = wave * IPW + (IPW == 1 ? 0 : lane / G);
  if (m >= a.n_split_rows) return;
  const int64_t row = cst(a.split_row)[m];
  const int32_t i0 = cst(a.split_ptr)[m];
  const int32_t i1 = cst(a.split_ptr)[m + 1];
  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = a.partial[static_cast<int64_t>(i0) * D + j0 + v];
  for (int32_t i = i0 + 1; i < i1; ++i) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = acc[v] + a.partial[static_cast<int64_t>(i) * D + j0 + v];
  }
  float* dst = a.out + row * a.ldo + j0;
#pragma unroll
  for (int v = 0; v < VEC; ++v)
    dst[v] = static_cast<float>(a.beta ? static_cast<double>(dst[v]) + acc[v] : acc[v]);
}

template <int D>
hipError_t launch_gather_d(const GatherArgs& a, bool with_halo, hipStream_t s) {
  constexpr int IPW = 64 / (D / vec_of(D));
  constexpr int IPB = 4 * IPW;   // items per 256-thread block
  if (a.n_items > 0) {
    const int64_t blocks = (a.n_items + IPB - 1) / IPB;
    if (with_halo)
      hipLaunchKernelGGL((gather_kernel<D, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((gather_kernel<D, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_split_rows > 0) {
    const int64_t blocks = (a.n_split_rows + IPB - 1) / IPB;
    hipLaunchKernelGGL((combine_split_kernel<D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int32_t d, bool with_halo, hipStream_t s) {
  switch (d) {
    case 16: return launch_gather_d<16>(a, with_halo, s);
    case 32: return launch_gather_d<32>(a, with_halo, s);
    case 64: return launch_gather_d<64>(a, with_halo, s);
    case 128: return launch_gather_d<128>(a, with_halo, s);
    case 256: return launch_gather_d<256>(a, with_halo, s);
    case 512: return launch_gather_d<512>(a, with_halo, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qha
