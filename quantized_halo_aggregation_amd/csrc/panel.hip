// Row-panel dense products for width 128 layers: the forward projection H = ReLU(A W^T) and the
// fused backward dZ = dH * [H > 0], dA = dZ W, dW = dZ^T A.
//
// Method: SYLVIE guide, section 2 (z_v = W a_v, h_v = sigma(z_v)) and section 7 (the weight
// gradient sums (dL/dh_v * sigma'(z_v)) a_v^T over the rows).
//
// Mapping to gfx950: the tall operands have m rows (a partition's nodes, 10^5..10^6) and 128
// columns, W is 128 x 128 (64 KB).  One 512-thread block per compute unit keeps W in LDS for the
// whole launch and streams 64-row panels of the tall operands through LDS, loading the next
// panel into registers while the matrix cores work on the current one.  The eight wavefronts
// each own one 32 x 32 output tile of a panel's product (v_mfma_f32_32x32x2f32); the backward
// wavefronts also own two 32 x 32 tiles of dW, which stay in registers across all of the block's
// panels, so dH, H and A are each read once and dZ is formed once.  Operand reads: a lane that
// walks a row along the contraction takes four (or eight) consecutive values with one 16-byte
// LDS read and feeds them to consecutive MFMAs (the two lane halves take interleaved k ranges);
// a lane that walks a column reads one float per MFMA, its lane half eight rows away from the
// other so the 64 reads hit 64 different banks (LDS rows are padded to 132 floats).
// Precision: for the forward and dA each MFMA chain adds 32 products in fp32 and those partial
// sums are added in float64.  A block's dW tiles are fp32 MFMA sums over its panels' rows (about
// m/256 rows); a second kernel adds the blocks' partials in float64 in a fixed order, so results
// are deterministic.
#include "qha_internal.hpp"

namespace qha {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int PR = 64;             // rows per panel
constexpr int PD = 128;            // n = k = 128
constexpr int LS = PD + 4;         // LDS row stride (floats)
constexpr int NT = 512;            // threads per block
constexpr int SV = PR * PD / 4 / NT;   // float4 per thread per staged panel array (4)
constexpr int WV = PD * PD / 4 / NT;   // float4 per thread for W (8)

__device__ __forceinline__ floatx16 mfma(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.0f;
  return z;
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

__device__ __forceinline__ void load_w(float* lds, const float* w, int64_t ldw) {
#pragma unroll
  for (int s = 0; s < WV; ++s) {
    const int f = static_cast<int>(threadIdx.x) + NT * s;
    *reinterpret_cast<float4*>(&lds[(f >> 5) * LS + 4 * (f & 31)]) =
        *reinterpret_cast<const float4*>(w + static_cast<int64_t>(f >> 5) * ldw + 4 * (f & 31));
  }
}

// H = epi(A W^T): A [m x 128], W [128 x 128], H [m x 128].
__global__ __launch_bounds__(NT) void panel_fwd_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) float Ws[PD * LS];
  __shared__ __attribute__((aligned(16))) float As[PR * LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int rt = wid >> 2;      // 32-row half of the panel
  const int ct = wid & 3;       // 32-column quarter of the output
  const int64_t n_panels = (p.m + PR - 1) / PR;

  load_w(Ws, p.w, p.ldw);
  float4 st[SV];
  int64_t panel = blockIdx.x;
  if (panel < n_panels) load_panel(p.a, p.lda, p.m, panel * PR, st);
  const float* arow = &As[(32 * rt + l32) * LS + 4 * h];
  const float* brow = &Ws[(32 * ct + l32) * LS + 4 * h];
  for (; panel < n_panels; panel += gridDim.x) {
    __syncthreads();                       // the previous panel's reads are done
    store_panel(As, st);
    __syncthreads();
    if (panel + gridDim.x < n_panels) load_panel(p.a, p.lda, p.m, (panel + gridDim.x) * PR, st);

    double sum[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[r] = 0.0;
#pragma unroll
    for (int kc = 0; kc < PD / 32; ++kc) {
      floatx16 acc = zero16();
#pragma unroll
      for (int q = 4 * kc; q < 4 * kc + 4; ++q) {
        // lane half h contributes k = 8q + 4h + c to MFMA c of this quad
        const float4 av = *reinterpret_cast<const float4*>(arow + 8 * q);
        const float4 bv = *reinterpret_cast<const float4*>(brow + 8 * q);
        acc = mfma(av.x, bv.x, acc);
        acc = mfma(av.y, bv.y, acc);
        acc = mfma(av.z, bv.z, acc);
        acc = mfma(av.w, bv.w, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] += static_cast<double>(acc[r]);
    }
    // accumulator element r of lane (h, l32) is C[8*(r/4) + 4*h + r%4][l32] of the 32 x 32 tile
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = panel * PR + 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < p.m) {
        float v = static_cast<float>(sum[r]);
        if (p.relu) v = v > 0.0f ? v : 0.0f;
        p.out[row * p.ldo + 32 * ct + l32] = v;
      }
    }
  }
}

// dZ = dH * [H > 0]; dA = dZ W; per-block dW partial = dZ^T A to ws[block][128][128].
__global__ __launch_bounds__(NT) void panel_bwd_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) float Ws[PD * LS];
  __shared__ __attribute__((aligned(16))) float Zs[PR * LS];
  __shared__ __attribute__((aligned(16))) float As[PR * LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int rt = wid >> 2;          // dA tile: panel rows 32*rt ..
  const int ct = wid & 3;           //          dA columns 32*ct ..
  const int ni = wid >> 1;          // dW tiles: rows 32*ni .., columns 32*kj0 .. and 32*(kj0+1) ..
  const int kj0 = 2 * (wid & 1);
  const int64_t n_panels = (p.m + PR - 1) / PR;

  load_w(Ws, p.w, p.ldw);
  floatx16 w0 = zero16(), w1 = zero16();   // the block's dW tiles, over all of its panels

  float4 sg[SV], sh[SV], sa[SV];
  int64_t panel = blockIdx.x;
  if (panel < n_panels) {
    load_panel(p.dh, p.lddh, p.m, panel * PR, sg);
    load_panel(p.h, p.ldh, p.m, panel * PR, sh);
    load_panel(p.a, p.lda, p.m, panel * PR, sa);
  }
  const float* zrow = &Zs[(32 * rt + l32) * LS + 8 * h];
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

    // dA tile: contraction over n = 16q + 8h + c (lane halves eight rows of W apart)
    double asum[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) asum[r] = 0.0;
#pragma unroll
    for (int nc = 0; nc < PD / 32; ++nc) {
      floatx16 acc = zero16();
#pragma unroll
      for (int q = 2 * nc; q < 2 * nc + 2; ++q) {
        const float4 z0 = *reinterpret_cast<const float4*>(zrow + 16 * q);
        const float4 z1 = *reinterpret_cast<const float4*>(zrow + 16 * q + 4);
        const float* wcol = &Ws[(16 * q + 8 * h) * LS + 32 * ct + l32];
        acc = mfma(z0.x, wcol[0 * LS], acc);
        acc = mfma(z0.y, wcol[1 * LS], acc);
        acc = mfma(z0.z, wcol[2 * LS], acc);
        acc = mfma(z0.w, wcol[3 * LS], acc);
        acc = mfma(z1.x, wcol[4 * LS], acc);
        acc = mfma(z1.y, wcol[5 * LS], acc);
        acc = mfma(z1.z, wcol[6 * LS], acc);
        acc = mfma(z1.w, wcol[7 * LS], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) asum[r] += static_cast<double>(acc[r]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = panel * PR + 32 * rt + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < p.m) p.da[row * p.ldda + 32 * ct + l32] = static_cast<float>(asum[r]);
    }

    // dW tiles: contraction over the panel's rows p = 16s + 8h + c
#pragma unroll
    for (int s = 0; s < PR / 16; ++s) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int pr = 16 * s + 8 * h + c;
        const float za = Zs[pr * LS + 32 * ni + l32];
        w0 = mfma(za, As[pr * LS + 32 * kj0 + l32], w0);
        w1 = mfma(za, As[pr * LS + 32 * (kj0 + 1) + l32], w1);
      }
    }
  }

  float* part = p.ws + static_cast<int64_t>(blockIdx.x) * PD * PD;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = 32 * ni + 8 * (r >> 2) + 4 * h + (r & 3);
    part[n * PD + 32 * kj0 + l32] = w0[r];
    part[n * PD + 32 * (kj0 + 1) + l32] = w1[r];
  }
}

// dW = sum over blocks of the float64 partials, in block order within four fixed ranges that are
// then added in order.  One block per 64 outputs.
__global__ __launch_bounds__(256) void panel_dw_reduce_kernel(const float* ws, int32_t n_blocks, float* dw,
                                                              int64_t lddw) {
  __shared__ double part[4][64];
  const int t = threadIdx.x;
  const int o = blockIdx.x * 64 + (t & 63);
  const int g = t >> 6;
  const int b0 = (n_blocks * g) / 4, b1 = (n_blocks * (g + 1)) / 4;
  double s = 0.0;
  for (int b = b0; b < b1; ++b) s += static_cast<double>(ws[static_cast<int64_t>(b) * PD * PD + o]);
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
