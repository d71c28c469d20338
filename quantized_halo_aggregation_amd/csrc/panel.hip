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

#include <type_traits>

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

// The same rows, every lane loading: a row at or past m re-reads row m - 1 (for products whose
// rows are independent and whose rows past m are never stored).  The number of loads in flight
// is then the same on every path, so waits can count them.
__device__ __forceinline__ void load_panel_all(const float* p, int64_t ld, int64_t m, int64_t r0, float4 (&v)[SV]) {
#pragma unroll
  for (int s = 0; s < SV; ++s) {
    const int f = static_cast<int>(threadIdx.x) + NT * s;
    const int64_t r = r0 + (f >> 5);
    v[s] = *reinterpret_cast<const float4*>(p + (r < m ? r : m - 1) * ld + 4 * (f & 31));
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

// One panel of the forward: stage it from registers (s0, s1) into LDS, start loading the panel
// `ahead` into the same registers, then multiply and store.  FULL: every row of the panel exists,
// so the stores are unconditional and every step issues the same number of memory operations.
template <bool FULL>
__device__ __forceinline__ void panel_fwd_step(const PanelArgs& p, float* As, const float* arow, const float* brow0,
                                               const float* brow1, int64_t panel, int64_t ahead, float4& s0,
                                               float4& s1, int rt, int cp, int g, int i) {
  static_assert(SV == 2, "two staged float4 per thread");
  __syncthreads();                       // the previous panel's reads are done
  {
    const float4 v[SV] = {s0, s1};
    store_panel(As, v);
  }
  __syncthreads();
  {
    float4 v[SV];
    load_panel_all(p.a, p.lda, p.m, ahead * PR, v);
    s0 = v[0];
    s1 = v[1];
  }

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
    if (FULL || row < p.m) {
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

// H = epi(A W^T): A [m x 128], W [128 x 128], H [m x 128].  Wavefront w owns panel rows
// 16*(w/4) .. +15 and output columns 32*(w%4) .. +31 as two 16 x 16 tiles (v_mfma_f32_16x16x4f32:
// lane (g, i) = (lane/16, lane%16) supplies row i of A and row i of W^T's column block at
// k = 16q + 4g + c for MFMA c of step q; its four accumulators are C[4g + r][i]).  A block walks
// its panels with two register sets of staged rows taken in turn, so each panel's load has two
// panels of work to arrive in.
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
  const int64_t n_full = p.m / PR;
  const int64_t stride = gridDim.x;
  const int64_t first = blockIdx.x;
  if (first >= n_panels) return;

  load_w<LS>(Ws, p.w, p.ldw);
  const float* arow = &As[(16 * rt + i) * LS + 4 * g];
  const float* brow0 = &Ws[(32 * cp + i) * LS + 4 * g];
  const float* brow1 = brow0 + 16 * LS;
  auto clampp = [&](int64_t q) { return q < n_panels ? q : n_panels - 1; };

  float4 a0, a1, b0, b1;
  {
    float4 v[SV];
    load_panel_all(p.a, p.lda, p.m, first * PR, v);
    a0 = v[0];
    a1 = v[1];
    load_panel_all(p.a, p.lda, p.m, clampp(first + stride) * PR, v);
    b0 = v[0];
    b1 = v[1];
  }
  // the ragged last panel of the matrix, if it is this block's, ends the walk (past the last
  // panel the prefetch re-reads it, keeping the loads in flight path-independent)
  int64_t panel = first;
  for (;;) {
    if (panel >= n_full) {
      if (panel < n_panels)
        panel_fwd_step<false>(p, As, arow, brow0, brow1, panel, clampp(panel + 2 * stride), a0, a1, rt, cp, g, i);
      break;
    }
    panel_fwd_step<true>(p, As, arow, brow0, brow1, panel, clampp(panel + 2 * stride), a0, a1, rt, cp, g, i);
    panel += stride;
    if (panel >= n_full) {
      if (panel < n_panels)
        panel_fwd_step<false>(p, As, arow, brow0, brow1, panel, clampp(panel + 2 * stride), b0, b1, rt, cp, g, i);
      break;
    }
    panel_fwd_step<true>(p, As, arow, brow0, brow1, panel, clampp(panel + 2 * stride), b0, b1, rt, cp, g, i);
    panel += stride;
  }
}

#ifndef QHA_PANEL_X3
#define QHA_PANEL_X3 1             // the forward on bf16 matrix cores with a three-way split
#endif
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

#ifndef QHA_PANEL_FWD_RB
#define QHA_PANEL_FWD_RB 0          // the row-block forward (0: the panel forward)
#endif
constexpr int F2_NT = 512;          // 8 wavefronts: 4 row slots x 2 column halves
constexpr int F2_BLOCKS = 512;      // two blocks per compute unit

// H = epi(A W^T) without per-panel barriers: W stays in LDS (loaded once per block) and every
// wavefront then works alone on 16-row blocks.  It loads its rows' A fragments from global memory
// straight into registers (lane (g, i): row i, columns 16q + 4g .. +3 for q = 0..7, the operand
// layout of v_mfma_f32_16x16x4f32) and computes one half of the output columns, four 16 x 16
// tiles, folding each 32-k MFMA chain into float64.  The two wavefronts of a row slot take the two
// halves of the same rows, so the second read of A is served by the compute unit's cache.
__global__ __launch_bounds__(F2_NT, 4) void panel_fwd_rb_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) float Ws[PD * LS];
#pragma unroll
  for (int s = 0; s < PD * PD / 4 / F2_NT; ++s) {
    const int f = static_cast<int>(threadIdx.x) + F2_NT * s;
    *reinterpret_cast<float4*>(&Ws[(f >> 5) * LS + 4 * (f & 31)]) =
        *reinterpret_cast<const float4*>(p.w + static_cast<int64_t>(f >> 5) * p.ldw + 4 * (f & 31));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int i = lane & 15;
  const int ch = wid & 1;
  const int rs = wid >> 1;
  const int64_t n_rb = (p.m + 15) / 16;
  const float* wrow = &Ws[(64 * ch + i) * LS + 4 * g];
  for (int64_t rb = static_cast<int64_t>(blockIdx.x) * 4 + rs; rb < n_rb; rb += static_cast<int64_t>(gridDim.x) * 4) {
    const int64_t arow = rb * 16 + i;
    float4 a[PD / 16];
#pragma unroll
    for (int q = 0; q < PD / 16; ++q)
      a[q] = arow < p.m ? *reinterpret_cast<const float4*>(p.a + arow * p.lda + 16 * q + 4 * g)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    double sum[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[t][r] = 0.0;
#pragma unroll
    for (int kc = 0; kc < PD / 32; ++kc) {
      // keeps each 32-k step's W reads within the step, so their registers are reused
      __builtin_amdgcn_sched_barrier(0);
      floatx4 acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) zero<4>(acc[t]);
#pragma unroll
      for (int q = 2 * kc; q < 2 * kc + 2; ++q) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 b = *reinterpret_cast<const float4*>(wrow + 16 * t * LS + 16 * q);
          acc[t] = mfma16(a[q].x, b.x, acc[t]);
          acc[t] = mfma16(a[q].y, b.y, acc[t]);
          acc[t] = mfma16(a[q].z, b.z, acc[t]);
          acc[t] = mfma16(a[q].w, b.w, acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[t][r] += static_cast<double>(acc[t][r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = rb * 16 + 4 * g + r;
      if (row < p.m) {
        float* dst = p.out + row * p.ldo + 64 * ch + i;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float v = static_cast<float>(sum[t][r]);
          if (p.relu) v = v > 0.0f ? v : 0.0f;
          dst[16 * t] = v;
        }
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
  if (QHA_PANEL_X3) {
    const int64_t n_panels = (p.m + X3_PR - 1) / X3_PR;
    const unsigned grid = static_cast<unsigned>(n_panels < kPanelBlocks ? n_panels : kPanelBlocks);
    hipLaunchKernelGGL(panel_fwd_x3_kernel, dim3(grid), dim3(X3_NT), 0, s, p);
  } else if (QHA_PANEL_FWD_RB) {
    const int64_t slots = ((p.m + 15) / 16 + 3) / 4;
    const unsigned grid = static_cast<unsigned>(slots < F2_BLOCKS ? slots : F2_BLOCKS);
    hipLaunchKernelGGL(panel_fwd_rb_kernel, dim3(grid), dim3(F2_NT), 0, s, p);
  } else {
    hipLaunchKernelGGL(panel_fwd_kernel, dim3(static_cast<unsigned>(panel_grid(p.m))), dim3(NT), 0, s, p);
  }
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
