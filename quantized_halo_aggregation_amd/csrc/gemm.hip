// Dense projection C = op(A) op(B) on fp32 matrix cores, with the ReLU epilogue of the forward
// and the ReLU-mask prologue of the backward.
//
// Method: SYLVIE guide, section 2 (z_v = W a_v, h_v = sigma(z_v)) and section 7 (the weight
// gradient sum_v (dL/dh_v * sigma'(z_v)) a_v^T).
//
// Mapping to gfx950: a 256-thread block owns a 64x128 tile of C; its four wavefronts own 32x64
// pieces, each held as two v_mfma_f32_32x32x2f32 accumulators (32 fp32 per lane) plus their
// float64 running sums.  K advances 32 at a time through LDS tiles that keep the operand's global layout
// (k-contiguous tiles are read with 16-byte LDS reads, the others with 4-byte reads), padded so
// neither the stores nor the fragment reads conflict on banks.  Within an 8-wide k slab, MFMA c
// of a lane in half h consumes k = 4h + c, which lets a single 16-byte read feed four MFMAs.
// The next tile's global loads are issued before the current tile is consumed.  Each 32-wide k
// step accumulates into fresh fp32 MFMA accumulators that are then added into float64 running
// sums, so a long dot product is rounded in float32 only over 32 terms at a time (for K = 512 this
// keeps near-zero outputs of cancelling sums within 1e-6).  Skinny reductions (the weight
// gradient, k = node count) are split over k into float64 partial tiles that a second kernel sums
// in fixed order.
#include "qha_internal.hpp"

namespace qha {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 64;
constexpr int BN = 128;
constexpr int BK = 32;
constexpr int PAD = 4;
constexpr int A_LOADS = BM * BK / 4 / 256;   // float4 loads per thread per k step
constexpr int B_LOADS = BN * BK / 4 / 256;

template <bool TA, bool TB, bool MASK, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  constexpr int A_ELEMS = TA ? BK * (BM + PAD) : BM * (BK + PAD);
  constexpr int B_ELEMS = TB ? BN * (BK + PAD) : BK * (BN + PAD);
  __shared__ __attribute__((aligned(16))) float As[A_ELEMS];
  __shared__ __attribute__((aligned(16))) float Bs[B_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1;        // 32-row half of the block tile
  const int wn = wid & 1;         // 64-column half
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.y) * BN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.z) * p.k_per_split;
  const int64_t kend = min(p.k, kbeg + p.k_per_split);

  double sum[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[j][r] = 0.0;

  float4 ra[A_LOADS], rb[B_LOADS];
  const float4 zero4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

  // global -> registers for the tile starting at k0
  auto load_tiles = [&](int64_t k0) {
#pragma unroll
    for (int s = 0; s < A_LOADS; ++s) {
      const int f = tid + 256 * s;
      int64_t gr, gc;     // storage row / column of the float4's first element
      bool ok;
      if (!TA) {          // A stored [m][k]
        const int row = f / (BK / 4), kq = f % (BK / 4);
        gr = m0 + row;
        gc = k0 + 4 * kq;
        ok = gr < p.m && gc < kend;
      } else {            // A stored [k][m]
        const int kr = f / (BM / 4), mq = f % (BM / 4);
        gr = k0 + kr;
        gc = m0 + 4 * mq;
        ok = gr < kend && gc < p.m;
      }
      float4 v = zero4;
      if (ok) {
        v = *reinterpret_cast<const float4*>(p.a + gr * p.lda + gc);
        if (MASK) {
          const float4 x = *reinterpret_cast<const float4*>(p.aux + gr * p.ld_aux + gc);
          v.x = x.x > 0.0f ? v.x : 0.0f;
          v.y = x.y > 0.0f ? v.y : 0.0f;
          v.z = x.z > 0.0f ? v.z : 0.0f;
          v.w = x.w > 0.0f ? v.w : 0.0f;
        }
      }
      ra[s] = v;
    }
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s) {
      const int f = tid + 256 * s;
      int64_t gr, gc;
      bool ok;
      if (TB) {           // B stored [n][k]
        const int row = f / (BK / 4), kq = f % (BK / 4);
        gr = n0 + row;
        gc = k0 + 4 * kq;
        ok = gr < p.n && gc < kend;
      } else {            // B stored [k][n]
        const int kr = f / (BN / 4), nq = f % (BN / 4);
        gr = k0 + kr;
        gc = n0 + 4 * nq;
        ok = gr < kend && gc < p.n;
      }
      rb[s] = ok ? *reinterpret_cast<const float4*>(p.b + gr * p.ldb + gc) : zero4;
    }
  };

  auto store_tiles = [&]() {
#pragma unroll
    for (int s = 0; s < A_LOADS; ++s) {
      const int f = tid + 256 * s;
      if (!TA) {
        const int row = f / (BK / 4), kq = f % (BK / 4);
        *reinterpret_cast<float4*>(&As[row * (BK + PAD) + 4 * kq]) = ra[s];
      } else {
        const int kr = f / (BM / 4), mq = f % (BM / 4);
        *reinterpret_cast<float4*>(&As[kr * (BM + PAD) + 4 * mq]) = ra[s];
      }
    }
#pragma unroll
    for (int s = 0; s < B_LOADS; ++s) {
      const int f = tid + 256 * s;
      if (TB) {
        const int row = f / (BK / 4), kq = f % (BK / 4);
        *reinterpret_cast<float4*>(&Bs[row * (BK + PAD) + 4 * kq]) = rb[s];
      } else {
        const int kr = f / (BN / 4), nq = f % (BN / 4);
        *reinterpret_cast<float4*>(&Bs[kr * (BN + PAD) + 4 * nq]) = rb[s];
      }
    }
  };

  if (kbeg < kend) {
    load_tiles(kbeg);
    store_tiles();
    __syncthreads();
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) load_tiles(k0 + BK);
    floatx16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
    for (int slab = 0; slab < BK / 8; ++slab) {
      const int kk = slab * 8 + 4 * h;
      float af[4], bf[2][4];
      const int row = wm * 32 + l32;
      if (!TA) {
        const float4 t = *reinterpret_cast<const float4*>(&As[row * (BK + PAD) + kk]);
        af[0] = t.x; af[1] = t.y; af[2] = t.z; af[3] = t.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) af[c] = As[(kk + c) * (BM + PAD) + row];
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = wn * 64 + ni * 32 + l32;
        if (TB) {
          const float4 t = *reinterpret_cast<const float4*>(&Bs[col * (BK + PAD) + kk]);
          bf[ni][0] = t.x; bf[ni][1] = t.y; bf[ni][2] = t.z; bf[ni][3] = t.w;
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) bf[ni][c] = Bs[(kk + c) * (BN + PAD) + col];
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[c], bf[ni][c], acc[ni], 0, 0, 0);
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[ni][r] += static_cast<double>(acc[ni][r]);
    __syncthreads();
    if (more) {
      store_tiles();
      __syncthreads();
    }
  }

  // accumulator element r of lane (h, l32) is C[8*(r/4) + 4*h + r%4][l32] of the 32x32 block
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t grow = m0 + wm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t gcol = n0 + wn * 64 + ni * 32 + l32;
      if (grow < p.m && gcol < p.n) {
        const double s = sum[ni][r];
        if (SPLIT) {
          p.ws[static_cast<int64_t>(blockIdx.z) * p.m * p.n + grow * p.n + gcol] = s;
        } else {
          float* dst = p.c + grow * p.ldc + gcol;
          float v = static_cast<float>(p.beta ? static_cast<double>(*dst) + s : s);
          if (p.epi == 1) v = v > 0.0f ? v : 0.0f;
          *dst = v;
        }
      }
    }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t mn = p.m * p.n;
  if (idx >= mn) return;
  double s = 0.0;
  for (int z = 0; z < p.splits; ++z) s += p.ws[z * mn + idx];
  const int64_t i = idx / p.n, j = idx % p.n;
  float* dst = p.c + i * p.ldc + j;
  float v = static_cast<float>(p.beta ? static_cast<double>(*dst) + s : s);
  if (p.epi == 1) v = v > 0.0f ? v : 0.0f;
  *dst = v;
}

template <bool TA, bool TB, bool MASK>
hipError_t launch_variant(const GemmArgs& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.m + BM - 1) / BM), static_cast<unsigned>((p.n + BN - 1) / BN),
                  static_cast<unsigned>(p.splits));
  if (p.splits > 1)
    hipLaunchKernelGGL((gemm_kernel<TA, TB, MASK, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<TA, TB, MASK, false>), grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits <= 1) return e;
  const int64_t mn = p.m * p.n;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>((mn + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

void gemm_split_rule(int64_t m, int64_t n, int64_t k, int32_t* splits, int64_t* k_per_split) {
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  int64_t s = 1;
  if (tiles < 256 && k > 8 * BK * 16) {
    s = (512 + tiles - 1) / tiles;                 // about two blocks per compute unit
    const int64_t max_s = (k + 16 * BK - 1) / (16 * BK);   // at least 16 k-steps per split
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
  }
  int64_t kps = (k + s - 1) / s;
  kps = ((kps + BK - 1) / BK) * BK;
  if (kps < BK) kps = BK;
  s = (k + kps - 1) / kps;
  if (s < 1) s = 1;
  *splits = static_cast<int32_t>(s);
  *k_per_split = s == 1 ? (k < 1 ? 1 : k) : kps;
}

hipError_t launch_gemm(const GemmArgs& p, hipStream_t s) {
  if (p.m == 0 || p.n == 0) return hipSuccess;
  const bool mask = p.pro == 1;
  if (!p.ta && p.tb && !mask) return launch_variant<false, true, false>(p, s);
  if (!p.ta && p.tb && mask) return launch_variant<false, true, true>(p, s);
  if (!p.ta && !p.tb && !mask) return launch_variant<false, false, false>(p, s);
  if (!p.ta && !p.tb && mask) return launch_variant<false, false, true>(p, s);
  if (p.ta && p.tb && !mask) return launch_variant<true, true, false>(p, s);
  if (p.ta && p.tb && mask) return launch_variant<true, true, true>(p, s);
  if (p.ta && !p.tb && !mask) return launch_variant<true, false, false>(p, s);
  return launch_variant<true, false, true>(p, s);
}

}  // namespace qha
