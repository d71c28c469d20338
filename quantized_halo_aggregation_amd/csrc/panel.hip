// Row-panel dense products for width 128 layers: the forward projection H = ReLU(A W^T) and the
// fused backward dZ = dH * [H > 0], dA = dZ W, dW = dZ^T A.
//
// Method: SYLVIE guide, section 2 (z_v = W a_v, h_v = sigma(z_v)) and section 7 (the weight
// gradient sums (dL/dh_v * sigma'(z_v)) a_v^T over the rows).
//
// Mapping to gfx950: the tall operands have m rows (a partition's nodes, 10^5..10^6) and 128
// columns; W is 128 x 128 (64 KB).
// Forward (panel_fwd_x3_kernel): float32 products on the bf16 matrix cores.  Each operand is split
// into three bf16 parts and each product is rebuilt from the six part products that matter (the
// split and the error bound are at split3); W's parts stay in registers, A is streamed through LDS
// as three bf16 planes of 64-row panels, double-buffered, with v_mfma_f32_32x32x16_bf16.
// Backward (panel_bwd_kernel): one 1024-thread block per compute unit keeps W in LDS for the whole
// launch and streams 64-row panels of dH, H and A through LDS, loading the next panel into
// registers while the matrix cores work on the current one; sixteen wavefronts (four per SIMD)
// hide each other's LDS latency.  Each wavefront owns two 16 x 16 tiles of dA
// (v_mfma_f32_16x16x4f32) and one 32 x 32 tile of dW (v_mfma_f32_32x32x2f32), which stays in
// registers across all of the block's panels, so dH, H and A are each read once and dZ is formed
// once.  Operand reads: a lane that walks a row along the contraction takes four consecutive
// values with one 16-byte LDS read and feeds them to four consecutive MFMAs (the lane groups take
// interleaved k ranges); a lane that walks a column reads one float per MFMA, the lane groups far
// enough apart in rows that the reads hit distinct banks (row strides of 136 and 132 floats,
// measured free of bank conflicts for these patterns).
// Precision: for the forward and dA each MFMA chain adds 32 k-steps in float32 and those partial
// sums are added in float64.  A block's dW tiles are float32 MFMA sums over its panels' rows
// (about m/256 rows); a second kernel adds the blocks' partials in float64 in a fixed order, so
// results are deterministic.
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int X3_NT = 512;          // 8 wavefronts: 2 row blocks x 4 column blocks of 32 x 32
constexpr int X3_PR = 64;           // rows per panel
constexpr int X3_LS = 136;          // bf16 per staged row: the 32 x 32 operand reads hit distinct banks

// x = hi + mid + lo exactly, each a bf16 rounded to nearest (even): hi holds x's top 8 significant
// bits, mid the next 8, lo the last 8 (x - hi and then (x - hi) - mid are exact in float32).
__device__ __forceinline__ void split3(float x, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  const float r = x - static_cast<float>(hi);
  mid = static_cast<__bf16>(r);
  lo = static_cast<__bf16>(r - static_cast<float>(mid));
}

__device__ __forceinline__ floatx16 mfma32b(const bf16x8& a, const bf16x8& b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Stages 4 floats of a panel row (row r, columns c .. c + 3) as the three bf16 planes.
__device__ __forceinline__ void stage4(__bf16* planes, int r, int c, const float4& v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 h, m, l;
  const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    __bf16 a, b, d;
    split3(x[j], a, b, d);
    h[j] = a;
    m[j] = b;
    l[j] = d;
  }
  const int o = r * X3_LS + c;
  *reinterpret_cast<bf16x4*>(planes + o) = h;
  *reinterpret_cast<bf16x4*>(planes + X3_PR * X3_LS + o) = m;
  *reinterpret_cast<bf16x4*>(planes + 2 * X3_PR * X3_LS + o) = l;
}

// H = epi(A W^T) on the bf16 matrix cores.  Every float32 operand is split into three bf16 parts
// (split3) and each product a * w is formed from the six part products whose weight is at least
// 2^-16 of it, hi*hi + hi*mid + mid*hi + hi*lo + lo*hi + mid*mid (smallest first); the three
// dropped ones are below 2^-23 |a w| together, about the size of float32 rounding.  The 32 x 32
// MFMA accumulates in float32; each 32-k chain is folded into float64 as in the panel kernel.
// W's parts stay in registers for the whole launch (lane (h, l) of the wavefront owning output
// columns 32 cb .. +31 holds W[32 cb + l][16 s + 8 h .. +7] for the 8 k-steps s); A panels are
// staged in LDS as three bf16 planes, double-buffered, so each panel costs one barrier, and the
// next panel's rows are loaded into registers while the current one is multiplied.
__global__ __launch_bounds__(X3_NT) void panel_fwd_x3_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) __bf16 Ap[2][3 * X3_PR * X3_LS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int h = lane >> 5;
  const int l = lane & 31;
  const int cb = wid & 3;       // 32-column block of the output
  const int rb = wid >> 2;      // 32-row block of the panel
  const int64_t n_panels = (p.m + X3_PR - 1) / X3_PR;
  const int64_t stride = gridDim.x;
  int64_t panel = blockIdx.x;
  if (panel >= n_panels) return;

  bf16x8 wh[PD / 16], wm[PD / 16], wl[PD / 16];
  {
    const float* wr = p.w + static_cast<int64_t>(32 * cb + l) * p.ldw + 8 * h;
#pragma unroll
    for (int st = 0; st < PD / 16; ++st) {
      const float4 u0 = *reinterpret_cast<const float4*>(wr + 16 * st);
      const float4 u1 = *reinterpret_cast<const float4*>(wr + 16 * st + 4);
      const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __bf16 a, b, d;
        split3(x[j], a, b, d);
        wh[st][j] = a;
        wm[st][j] = b;
        wl[st][j] = d;
      }
    }
  }

  // staging: float4 f = tid + X3_NT * s of a panel is row f / 32, columns 4 (f % 32) .. +3
  constexpr int XV = X3_PR * PD / 4 / X3_NT;   // 4
  float4 sv[XV];
  auto load = [&](int64_t pn) {
#pragma unroll
    for (int s = 0; s < XV; ++s) {
      const int f = tid + X3_NT * s;
      const int64_t r = pn * X3_PR + (f >> 5);
      sv[s] = *reinterpret_cast<const float4*>(p.a + (r < p.m ? r : p.m - 1) * p.lda + 4 * (f & 31));
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int s = 0; s < XV; ++s) {
      const int f = tid + X3_NT * s;
      stage4(Ap[buf], f >> 5, 4 * (f & 31), sv[s]);
    }
  };
  load(panel);
  stage(0);
  __syncthreads();
  if (panel + stride < n_panels) load(panel + stride);

  for (int buf = 0; panel < n_panels; panel += stride, buf ^= 1) {
    const __bf16* ah = Ap[buf] + (32 * rb + l) * X3_LS + 8 * h;
    const __bf16* am = ah + X3_PR * X3_LS;
    const __bf16* al = am + X3_PR * X3_LS;
    double sum[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[r] = 0.0;
#pragma unroll
    for (int kc = 0; kc < PD / 32; ++kc) {
      floatx16 acc;
      zero<16>(acc);
#pragma unroll
      for (int st = 2 * kc; st < 2 * kc + 2; ++st) {
        const bf16x8 xh = *reinterpret_cast<const bf16x8*>(ah + 16 * st);
        const bf16x8 xm = *reinterpret_cast<const bf16x8*>(am + 16 * st);
        const bf16x8 xl = *reinterpret_cast<const bf16x8*>(al + 16 * st);
        acc = mfma32b(xm, wm[st], acc);
        acc = mfma32b(xl, wh[st], acc);
        acc = mfma32b(xh, wl[st], acc);
        acc = mfma32b(xm, wh[st], acc);
        acc = mfma32b(xh, wm[st], acc);
        acc = mfma32b(xh, wh[st], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] += static_cast<double>(acc[r]);
    }
    // the next panel goes to the other buffer, whose last readers finished before the previous
    // barrier; its rows were loaded during this panel's products
    const int64_t next = panel + stride;
    if (next < n_panels) {
      stage(buf ^ 1);
      if (next + stride < n_panels) load(next + stride);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = panel * X3_PR + 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < p.m) {
        float v = static_cast<float>(sum[r]);
        if (p.relu) v = v > 0.0f ? v : 0.0f;
        p.out[row * p.ldo + 32 * cb + l] = v;
      }
    }
    __syncthreads();
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
  const int64_t n_panels = (p.m + X3_PR - 1) / X3_PR;
  const unsigned grid = static_cast<unsigned>(n_panels < kPanelBlocks ? n_panels : kPanelBlocks);
  hipLaunchKernelGGL(panel_fwd_x3_kernel, dim3(grid), dim3(X3_NT), 0, s, p);
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
