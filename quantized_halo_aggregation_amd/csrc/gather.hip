// Normalised neighbour gather (SpMM over a CSR) with halo dequantisation fused into the loads.
//
// Method: SYLVIE guide, section 2 (z_v sums the neighbours' rows, each divided by
// sqrt(d_v d_u)) and section 6 (a received halo row is scale * q + min, restored to float32).
// The same kernel walks the transposed CSR for the embedding-gradient pass (sections 3 and 11).
//
// Mapping to gfx950: one wavefront owns one work item of the host-built plan -- a group of
// consecutive short rows, or one chunk of a heavy row -- and streams through the item's
// contiguous edge list in batches of B edges.  Its 64 lanes split the d features (d/64
// contiguous floats per lane), so every neighbour costs one coalesced d*4-byte load.  Column
// indices, edge weights and halo metadata are wavefront-uniform and come through the scalar unit;
// only feature rows and packed code words use the vector memory pipe.  A batch runs in phases:
// (1) scalar loads of the batch's weights and halo metadata, vector loads of its inner rows and
// the scalar load of the next batch's column indices, all in flight together; (2) after one wait,
// the code words of its halo rows (one word per lane holds all of its codes); (3) the sums.  Row
// boundaries inside a group are tracked with scalar compares against the group's row pointers,
// held one per lane and read with readlane, so crossing a row costs a store and no load.
// A halo value is dequantised in float32 (scale * q + min, no contraction); every product is then
// accumulated in float64 (a float32 product is exact there, and MI355X issues float64 FMAs at the
// rate of unpacked float32 ones, so in this memory-bound loop the wider sum is free) and rounded
// to float32 once.  Chunks of a heavy row write float64 partial sums that a second kernel adds in
// chunk order, so results do not depend on scheduling.
#include "../../include/qha.h"
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
constexpr int batch_of(int D, bool halo) { return (D >= 512 || halo) ? 8 : 16; }
constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }

__device__ __forceinline__ int rdlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float rdlanef(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ float dequant(float sc, uint32_t q, float zp) {
  return __fadd_rn(__fmul_rn(sc, static_cast<float>(q)), zp);
}

__device__ __forceinline__ bool width_ok(uint32_t b) {
  return b == 1u || b == 2u || b == 4u || b == 8u || b == 32u;
}

template <int VEC>
__device__ __forceinline__ void store_row(float* p, const float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    p[0] = v[0];
  } else if constexpr (VEC == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q)
      reinterpret_cast<float4*>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

template <int VEC>
__device__ __forceinline__ void load_row(const float* p, float (&xv)[VEC]) {
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

template <int D, bool HALO, bool BETA>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;           // lanes that own features
  constexpr int B = batch_of(D, HALO);
  constexpr int CW = (VEC * 8 > 32) ? 2 : 1;   // code words a lane may need (8-bit codes, VEC = 8)
  const int lane = threadIdx.x & 63;
  const int j0 = (G == 64 ? lane : (lane < G ? lane : 0)) * VEC;   // idle lanes shadow lane 0
  const bool owner = (G == 64) || lane < G;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (item >= a.n_items) return;

  int32_t row0, nrows, e0, e1;
  if (a.items != nullptr) {
    cptr<int32_t> it = cst(a.items) + 4 * item;
    row0 = it[0];
    nrows = it[1];
    e0 = it[2];
    e1 = it[3];
  } else {
    row0 = static_cast<int32_t>(item);
    nrows = 1;
    e0 = cst(a.rowptr)[item];
    e1 = cst(a.rowptr)[item + 1];
  }
  const bool split = item < a.n_split_items;

  // the group's row ends, row scales and output rows, one row per lane (rows of a group are
  // never empty, so each edge closes at most one row)
  const int li = lane < nrows ? lane : nrows - 1;
  const int32_t v_end = split ? 0x7FFFFFFF : a.rowptr[row0 + li + 1];
  const float v_rs = (a.rs != nullptr) ? a.rs[row0 + li] : 1.0f;
  const int32_t v_out = (a.row_ids != nullptr) ? a.row_ids[row0 + li] : row0 + li;

  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
  int cur = 0;                                  // row of the group being summed
  int32_t cur_end = rdlane(v_end, 0);

  auto flush = [&]() {                          // write row `cur` and start the next one
    const double r = static_cast<double>(rdlanef(v_rs, cur));
    const int64_t orow = rdlane(v_out, cur);
    float* dst = a.out + orow * a.ldo + j0;
    if (owner) {
      float res[VEC];
      if constexpr (BETA) {
        float old[VEC];
        load_row<VEC>(dst, old);
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(static_cast<double>(old[v]) + r * acc[v]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(r * acc[v]);
      }
      store_row<VEC>(dst, res);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
    ++cur;
    cur_end = rdlane(v_end, cur < nrows ? cur : nrows - 1);
  };

  int32_t u_next[B];
  if (e0 < e1) {
#pragma unroll
    for (int i = 0; i < B; ++i) u_next[i] = cst(a.colidx)[min(e0 + i, e1 - 1)];
  }

  for (int32_t e = e0; e < e1; e += B) {
    int32_t u[B];
#pragma unroll
    for (int i = 0; i < B; ++i) u[i] = u_next[i];

    // phase 1: weights, halo metadata and inner rows; the next batch's indices
    float cw[B];
    float xv[B][VEC];
    uint32_t woff[B], bw[B];
    float mn[B], sc[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      cw[i] = a.cs ? cst(a.cs)[u[i]] : 1.0f;
      if (HALO && u[i] >= a.n_inner) {
        const int64_t k = static_cast<int64_t>(u[i]) - a.n_inner;
        woff[i] = cst(a.word_offset)[k];
        if constexpr (D >= 32) {
          // the width follows from the row's word count (unique for d >= 32)
          bw[i] = ((cst(a.word_offset)[k + 1] - woff[i]) << 5) >> log2i(D);
        } else {
          bw[i] = cst(a.bits)[k];
        }
        mn[i] = cst(a.meta)[2 * k];
        sc[i] = cst(a.meta)[2 * k + 1];
      } else {
        load_row<VEC>(a.x + static_cast<int64_t>(u[i]) * a.ldx + j0, xv[i]);
      }
    }
    if (e + B < e1) {
#pragma unroll
      for (int i = 0; i < B; ++i) u_next[i] = cst(a.colidx)[min(e + B + i, e1 - 1)];
    }
    // phase 2: the code words of the halo rows
    uint32_t cwd[B][CW];
    if (HALO) {
#pragma unroll
      for (int i = 0; i < B; ++i) {
        if (u[i] >= a.n_inner) {
          const uint32_t b = bw[i];
          const uint32_t* row = a.codes + woff[i];
          if (b == 32u) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) xv[i][v] = __uint_as_float(row[j0 + v]);
          } else if (width_ok(b)) {
            const uint32_t pos = static_cast<uint32_t>(j0) * b;
            cwd[i][0] = row[pos >> 5];
            if (CW == 2) cwd[i][CW - 1] = (b * VEC > 32u) ? row[(pos >> 5) + 1] : 0u;
          }
        }
      }
    }
    // phase 3: dequantise and sum, closing the row whose last edge this is
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int32_t p = e + i;
      if (p < e1) {
        if (HALO && u[i] >= a.n_inner) {
          const uint32_t b = bw[i];
          if (b != 32u) {
            if (width_ok(b)) {
              const uint32_t mask = (1u << b) - 1u;
              const uint32_t sh = (static_cast<uint32_t>(j0) * b) & 31u;
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                const uint32_t bitpos = sh + static_cast<uint32_t>(v) * b;
                const uint32_t w = (CW == 2 && bitpos >= 32u) ? (cwd[i][CW - 1] >> (bitpos - 32u)) : (cwd[i][0] >> bitpos);
                xv[i][v] = dequant(sc[i], w & mask, mn[i]);
              }
            } else {
#pragma unroll
              for (int v = 0; v < VEC; ++v) xv[i][v] = 0.0f;
            }
          }
        }
        const double w = static_cast<double>(cw[i]);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = fma(w, static_cast<double>(xv[i][v]), acc[v]);
        if (p + 1 == cur_end) flush();
      }
    }
  }

  if (split) {
    double* p = a.partial + item * D + j0;
    if (owner) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) p[v] = acc[v];
    }
  } else if (e0 == e1) {
    flush();                                   // an empty row: zero, or left as it is (+0)
  }
}

// Adds the partial sums of every split row in chunk order, scales and writes the row.
template <int D>
__global__ __launch_bounds__(256) void combine_split_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 +
                    __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (m >= a.n_split_rows || lane >= G) return;
  const int j0 = lane * VEC;
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
  const double r = a.rs ? static_cast<double>(a.rs[row]) : 1.0;
  const int64_t orow = a.row_ids ? a.row_ids[row] : row;
  float* dst = a.out + orow * a.ldo + j0;
#pragma unroll
  for (int v = 0; v < VEC; ++v)
    dst[v] = static_cast<float>(a.beta ? static_cast<double>(dst[v]) + r * acc[v] : r * acc[v]);
}

template <int D>
hipError_t launch_gather_d(const GatherArgs& a, bool with_halo, hipStream_t s) {
  if (a.n_items > 0) {
    const dim3 grid(static_cast<unsigned>((a.n_items + 3) / 4));
    if (with_halo) {
      if (a.beta) hipLaunchKernelGGL((gather_kernel<D, true, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gather_kernel<D, true, false>), grid, dim3(256), 0, s, a);
    } else {
      if (a.beta) hipLaunchKernelGGL((gather_kernel<D, false, true>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gather_kernel<D, false, false>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_split_rows > 0) {
    const int64_t blocks = (a.n_split_rows + 3) / 4;
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
