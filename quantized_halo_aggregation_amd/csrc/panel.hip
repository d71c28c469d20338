// Row-panel dense products for width 128 layers: the forward projection H = ReLU(A W^T) and the
// fused backward dZ = dH * [H > 0], dA = dZ W, dW = dZ^T A.
//
// Method: SYLVIE guide, section 2 (z_v = W a_v, h_v = sigma(z_v)) and section 7 (the weight
// gradient sums (dL/dh_v * sigma'(z_v)) a_v^T over the rows).
//
// Mapping to gfx950: the tall operands have m rows (a partition's nodes, 10^5..10^6) and 128
// columns; W is 128 x 128 (64 KB).  One 1024-thread block per compute unit keeps W in LDS for the
// whole launch and streams 64-row panels of the tall operands through LDS, loading the next
// panel into registers while the matrix cores work on the current one; sixteen wavefronts (four
// per SIMD) hide each other's LDS latency.  Each wavefront owns two 16 x 16 tiles of a panel's
// product (v_mfma_f32_16x16x4f32); in the backward it also owns one 32 x 32 tile of dW
// (v_mfma_f32_32x32x2f32), which stays in registers across all of the block's panels, so dH, H
// and A are each read once and dZ is formed once.  Operand reads: a lane that walks a row along
// the contraction takes four consecutive values with one 16-byte LDS read and feeds them to four
// consecutive MFMAs (the lane groups take interleaved k ranges); a lane that walks a column reads
// one float per MFMA, the lane groups far enough apart in rows that the 64 reads hit 64 banks
// (row strides of 136 and 132 floats, measured free of bank conflicts for these patterns).
// Precision: for the forward and dA each MFMA chain adds 32 products in fp32 and those partial
// sums are added in float64.  A block's dW tiles are fp32 MFMA sums over its panels' rows (about
// m/256 rows); a second kernel adds the blocks' partials in float64 in a fixed order, so results
// are deterministic.
#include "qha_internal.hpp"

namespace qha {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int PR = 64;             // rows per panel
constexpr int PD = 128;            // n = k = 128
// LDS row strides (floats), chosen by bank: a 16-byte read by lane (g, i) at row i, column 4g is
// conflict-free at a stride of 136; a 4-byte read whose lane groups sit 4 rows apart at column i
// (W in the backward) needs 132
constexpr int LS = PD + 8;
constexpr int LSW = PD + 4;
constexpr int NT = 1024;           // threads per block: 16 wavefronts, four per SIMD
constexpr int SV = PR * PD / 4 / NT;   // float4 per thread per staged panel array (2)
constexpr int WV = PD * PD / 4 / NT;   // float4 per thread for W (4)

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void zero(float __attribute__((ext_vector_type(N)))& v) {
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = 0.0f;
}

// Rows [r0, r0 + PR) of a [m x 128] row-major matrix, float4 f = tid + NT*s at (row f/32, col 4*(f%32));
// rows at or past m read as zero.
__device__ __forceinline__ void load_panel(const float* p, int64_t ld, int64_t m, int64_t r0, float4 (&v)[SV]) {
#pragma unroll
  for (int s = 0; s < SV; ++s) {
    const int f = static_cast<int>(threadIdx.x) + NT * s;
    const int64_t r = r0 + (f >> 5);
    v[s] = r < m ? *reinterpret_cast<const float4*>(p + r * ld + 4 * (f & 31)) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

__device__ __forceinline__ void store_panel(float* lds, const float4 (&v)[SV]) {
#pragma unroll
  for (int s = 0; s < SV; ++s) {
    const int f = static_cast<int>(threadIdx.x) + NT * s;
    *reinterpret_cast<float4*>(&lds[(f >> 5) * LS + 4 * (f & 31)]) = v[s];
  }
}

template <int STRIDE>
__device__ __forceinline__ void load_w(float* lds, const float* w, int64_t ldw) {
#pragma unroll
  for (int s = 0; s < WV; ++s) {
    const int f = static_cast<int>(threadIdx.x) + NT * s;
    *reinterpret_cast<float4*>(&lds[(f >> 5) * STRIDE + 4 * (f & 31)]) =
        *reinterpret_cast<const float4*>(w + static_cast<int64_t>(f >> 5) * ldw + 4 * (f & 31));
  }
}

// H = epi(A W^T): A [m x 128], W [128 x 128], H [m x 128].  Wavefront w owns panel rows
// 16*(w/4) .. +15 and output columns 32*(w%4) .. +31 as two 16 x 16 tiles (v_mfma_f32_16x16x4f32:
// lane (g, i) = (lane/16, lane%16) supplies row i of A and row i of W^T's column block at
// k = 16q + 4g + c for MFMA c of step q; its four accumulators are C[4g + r][i]).
__global__ __launch_bounds__(NT) void panel_fwd_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) float Ws[PD * LS];
  __shared__ __attribute__((aligned(16))) float As[PR * LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int i = lane & 15;
  const int rt = wid >> 2;      // 16-row block of the panel
  const int cp = wid & 3;       // 32-column block of the output
  const int64_t n_panels = (p.m + PR - 1) / PR;

  load_w<LS>(Ws, p.w, p.ldw);
  float4 st[SV];
  int64_t panel = blockIdx.x;
  if (panel < n_panels) load_panel(p.a, p.lda, p.m, panel * PR, st);
  const float* arow = &As[(16 * rt + i) * LS + 4 * g];
  const float* brow0 = &Ws[(32 * cp + i) * LS + 4 * g];
  const float* brow1 = brow0 + 16 * LS;
  for (; panel < n_panels; panel += gridDim.x) {
    __syncthreads();                       // the previous panel's reads are done
    store_panel(As, st);
    __syncthreads();
    if (panel + gridDim.x < n_panels) load_panel(p.a, p.lda, p.m, (panel + gridDim.x) * PR, st);

    double sum0[4], sum1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sum0[r] = sum1[r] = 0.0;
#pragma unroll
    for (int kc = 0; kc < PD / 32; ++kc) {
      floatx4 acc0, acc1;
      zero<4>(acc0);
      zero<4>(acc1);
#pragma unroll
      for (int q = 2 * kc; q < 2 * kc + 2; ++q) {
        const float4 av = *reinterpret_cast<const float4*>(arow + 16 * q);
        const float4 b0 = *reinterpret_cast<const float4*>(brow0 + 16 * q);
        const float4 b1 = *reinterpret_cast<const float4*>(brow1 + 16 * q);
        acc0 = mfma16(av.x, b0.x, acc0);
        acc1 = mfma16(av.x, b1.x, acc1);
        acc0 = mfma16(av.y, b0.y, acc0);
        acc1 = mfma16(av.y, b1.y, acc1);
        acc0 = mfma16(av.z, b0.z, acc0);
        acc1 = mfma16(av.z, b1.z, acc1);
        acc0 = mfma16(av.w, b0.w, acc0);
        acc1 = mfma16(av.w, b1.w, acc1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sum0[r] += static_cast<double>(acc0[r]);
        sum1[r] += static_cast<double>(acc1[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = panel * PR + 16 * rt + 4 * g + r;
      if (row < p.m) {
        float v0 = static_cast<float>(sum0[r]);
        float v1 = static_cast<float>(sum1[r]);
        if (p.relu) {
          v0 = v0 > 0.0f ? v0 : 0.0f;
          v1 = v1 > 0.0f ? v1 : 0.0f;
        }
        float* dst = p.out + row * p.ldo + 32 * cp + i;
        dst[0] = v0;
        dst[16] = v1;
      }
    }
  }
}

// dZ = dH * [H > 0]; dA = dZ W; per-block dW partial = dZ^T A to ws[block][128][128].
// Wavefront w: dA rows 16*(w/4) .. +15, columns 32*(w%4) .. +31 as two 16 x 16 tiles (contraction
// over n = 16q + 4g + c); dW tile rows 32*(w/4) .., columns 32*(w%4) .. (32 x 32, contraction over
// the panel's rows p = 16s + 8h + c, lane halves eight rows apart).
__global__ __launch_bounds__(NT) void panel_bwd_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) float Ws[PD * LSW];
  __shared__ __attribute__((aligned(16))) float Zs[PR * LS];
  __shared__ __attribute__((aligned(16))) float As[PR * LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;
  const int i = lane & 15;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int rt = wid >> 2;
  const int cp = wid & 3;
  const int64_t n_panels = (p.m + PR - 1) / PR;

  load_w<LSW>(Ws, p.w, p.ldw);
  floatx16 wacc;                 // the block's dW tile, over all of its panels
  zero<16>(wacc);

  float4 sg[SV], sh[SV], sa[SV];
  int64_t panel = blockIdx.x;
  if (panel < n_panels) {
    load_panel(p.dh, p.lddh, p.m, panel * PR, sg);
    load_panel(p.h, p.ldh, p.m, panel * PR, sh);
    load_panel(p.a, p.lda, p.m, panel * PR, sa);
  }
  const float* zrow = &Zs[(16 * rt + i) * LS + 4 * g];
  const float* wcol = &Ws[(4 * g) * LSW + 32 * cp + i];
  const float* zcol = &Zs[(4 * h) * LS + 32 * rt + l32];
  const float* acol = &As[(4 * h) * LS + 32 * cp + l32];
  for (; panel < n_panels; panel += gridDim.x) {
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SV; ++s) {
      float4 z;
      z.x = sh[s].x > 0.0f ? sg[s].x : 0.0f;
      z.y = sh[s].y > 0.0f ? sg[s].y : 0.0f;
      z.z = sh[s].z > 0.0f ? sg[s].z : 0.0f;
      z.w = sh[s].w > 0.0f ? sg[s].w : 0.0f;
      sg[s] = z;
    }
    store_panel(Zs, sg);
    store_panel(As, sa);
    __syncthreads();
    const int64_t next = panel + gridDim.x;
    if (next < n_panels) {
      load_panel(p.dh, p.lddh, p.m, next * PR, sg);
      load_panel(p.h, p.ldh, p.m, next * PR, sh);
      load_panel(p.a, p.lda, p.m, next * PR, sa);
    }

    // dA tiles
    double as0[4], as1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) as0[r] = as1[r] = 0.0;
#pragma unroll
    for (int nc = 0; nc < PD / 32; ++nc) {
      floatx4 acc0, acc1;
      zero<4>(acc0);
      zero<4>(acc1);
#pragma unroll
      for (int q = 2 * nc; q < 2 * nc + 2; ++q) {
        const float4 z = *reinterpret_cast<const float4*>(zrow + 16 * q);
        const float* wq = wcol + 16 * q * LSW;
        acc0 = mfma16(z.x, wq[0 * LSW], acc0);
        acc1 = mfma16(z.x, wq[0 * LSW + 16], acc1);
        acc0 = mfma16(z.y, wq[1 * LSW], acc0);
        acc1 = mfma16(z.y, wq[1 * LSW + 16], acc1);
        acc0 = mfma16(z.z, wq[2 * LSW], acc0);
        acc1 = mfma16(z.z, wq[2 * LSW + 16], acc1);
        acc0 = mfma16(z.w, wq[3 * LSW], acc0);
        acc1 = mfma16(z.w, wq[3 * LSW + 16], acc1);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        as0[r] += static_cast<double>(acc0[r]);
        as1[r] += static_cast<double>(acc1[r]);
      }
    }
    // stored before the dW work, which leaves that work to cover the stores' completion
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = panel * PR + 16 * rt + 4 * g + r;
      if (row < p.m) {
        float* dst = p.da + row * p.ldda + 32 * cp + i;
        dst[0] = static_cast<float>(as0[r]);
        dst[16] = static_cast<float>(as1[r]);
      }
    }

    // dW tile: lane half h takes the panel rows p = 8s + 4h + c
#pragma unroll
    for (int s = 0; s < PR / 8; ++s) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = (8 * s + c) * LS;
        wacc = mfma32(zcol[off], acol[off], wacc);
      }
    }
  }

  float* part = p.ws + static_cast<int64_t>(blockIdx.x) * PD * PD;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
    part[n * PD + 32 * cp + l32] = wacc[r];
  }
}

// dW = sum over blocks of the per-block partials in float64, in block order within four fixed
// ranges that are then added in order.  One block per 64 outputs.
__global__ __launch_bounds__(256) void panel_dw_reduce_kernel(const float* ws, int32_t n_blocks, float* dw,
                                                              int64_t lddw) {
  __shared__ double part[4][64];
  const int t = threadIdx.x;
  const int o = blockIdx.x * 64 + (t & 63);
  const int g = t >> 6;
  const int b0 = (n_blocks * g) / 4, b1 = (n_blocks * (g + 1)) / 4;
  const float* src = ws + o;
  double s = 0.0;
  int b = b0;
  for (; b + 8 <= b1; b += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[static_cast<int64_t>(b + j) * PD * PD];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += static_cast<double>(v[j]);
  }
  for (; b < b1; ++b) s += static_cast<double>(src[static_cast<int64_t>(b) * PD * PD]);
  part[g][t & 63] = s;
  __syncthreads();
  if (g == 0) {
    const double v = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    dw[static_cast<int64_t>(o / PD) * lddw + (o % PD)] = static_cast<float>(v);
  }
}

int32_t panel_grid(int64_t m) {
  const int64_t n_panels = (m + PR - 1) / PR;
  return static_cast<int32_t>(n_panels < kPanelBlocks ? n_panels : kPanelBlocks);
}

}  // namespace

bool panel_fits(int64_t n, int64_t k) { return n == PD && k == PD; }

size_t panel_bwd_workspace(int64_t m) {
  return static_cast<size_t>(panel_grid(m)) * PD * PD * sizeof(float);
}

hipError_t launch_panel_fwd(const PanelArgs& p, hipStream_t s) {
  if (p.m == 0) return hipSuccess;
  hipLaunchKernelGGL(panel_fwd_kernel, dim3(static_cast<unsigned>(panel_grid(p.m))), dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_panel_bwd(const PanelArgs& p, hipStream_t s) {
  if (p.m == 0) return hipSuccess;
  const int32_t grid = panel_grid(p.m);
  hipLaunchKernelGGL(panel_bwd_kernel, dim3(static_cast<unsigned>(grid)), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(panel_dw_reduce_kernel, dim3(PD * PD / 64), dim3(256), 0, s, static_cast<const float*>(p.ws),
                     grid, p.dw, p.lddw);
  return hipGetLastError();
}

}  // namespace qha
