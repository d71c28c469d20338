// Row-panel dense products: for width 128 layers the forward projection H = ReLU(A W^T) and the
// fused backward dZ = dH * [H > 0], dA = dZ W, dW = dZ^T A; for wider layers the weight gradient
// dW alone (dw_panel_kernel, below).
//
// Method: SYLVIE guide, section 2 (z_v = W a_v, h_v = sigma(z_v)) and section 7 (the weight
// gradient sums (dL/dh_v * sigma'(z_v)) a_v^T over the rows).
//
// Mapping to gfx950: the tall operands have m rows (a partition's nodes, 10^5..10^6) and 128
// columns; W is 128 x 128 (64 KB).  Both kernels compute float32 products on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16): each float32 operand is split exactly into three bf16 parts
// and each product is rebuilt from the six part products that matter (the split and the error
// bound are at split3).  One block per compute unit, persistent over row panels staged in LDS.
// Forward (panel_fwd_x3_kernel): W's parts stay in registers; A is streamed through LDS as three
// bf16 planes of 64-row panels, double-buffered.
// Backward (panel_bwd_x3_kernel): dZ and A are staged per 32-row panel; four wavefronts form dA
// (W's parts in registers, as in the forward) while four form the block's dW partial, so dH, H
// and A are each read once and dZ is formed once.
// Weight gradient at wider layers (dw_panel_kernel): blocks of 128 x 256 outputs over row ranges,
// the width-128 backward's dW role on its own.
// Precision: for the forward and dA each MFMA chain adds 32 k-steps in float32 and those partial
// sums are added in float64.  A block's dW tiles are float32 matrix-core sums over its panels' rows
// (about m/256 rows at width 128, at most about 4096 rows at wider layers); a second kernel adds
// the blocks' partials in float64 in a fixed order, so results are deterministic.
#include "qha_internal.hpp"

namespace qha {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
constexpr int PR = 64;             // rows per grid unit: the backward's grid is min(ceil(m / 64), 256)
constexpr int PD = 128;            // n = k = 128

template <int N>
__device__ __forceinline__ void zero(float __attribute__((ext_vector_type(N)))& v) {
#pragma unroll
  for (int r = 0; r < N; ++r) v[r] = 0.0f;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data: out-of-range stores dropped
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

// split3 of a pair (a, b), as packed words (a in the low half): one packed conversion rounds the
// pair to bf16, and the pair's float values come back by a shift and a mask of the packed word.
// Bit for bit the same parts as split3.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& ph, uint32_t& pm, uint32_t& pl) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float floatx2 __attribute__((ext_vector_type(2)));
  ph = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){a, b}, bf16x2));
  const float ra = a - __uint_as_float(ph << 16);
  const float rb = b - __uint_as_float(ph & 0xFFFF0000u);
  pm = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){ra, rb}, bf16x2));
  const float la = ra - __uint_as_float(pm << 16);
  const float lb = rb - __uint_as_float(pm & 0xFFFF0000u);
  pl = __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){la, lb}, bf16x2));
}

__device__ __forceinline__ floatx16 mfma32b(const bf16x8& a, const bf16x8& b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Stages 4 floats of a panel row (row r, columns c .. c + 3) as the three bf16 planes of ROWS rows.
template <int ROWS = 64>
__device__ __forceinline__ void stage4(__bf16* planes, int r, int c, const float4& v) {
  uint2 h, m, l;
  split_pair(v.x, v.y, h.x, m.x, l.x);
  split_pair(v.z, v.w, h.y, m.y, l.y);
  const int o = r * X3_LS + c;
  *reinterpret_cast<uint2*>(planes + o) = h;
  *reinterpret_cast<uint2*>(planes + ROWS * X3_LS + o) = m;
  *reinterpret_cast<uint2*>(planes + 2 * ROWS * X3_LS + o) = l;
}

// Sixteen stores that the hardware drops (a buffer of no records).  Issued after the loads that
// enter a panel loop, they give the loop's entry the same order of pending memory operations as
// its back edge (the next panel's loads, then the sixteen output stores), so the compiler's wait
// before staging a panel counts the stores as still in flight instead of waiting for them.
__device__ __forceinline__ void dropped_stores16(const float* base) {
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0, kBufferWord3);
#pragma unroll
  for (int r = 0; r < 16; ++r) __builtin_amdgcn_raw_buffer_store_b32(0u, none, static_cast<uint32_t>(64 * r), 0, 0);
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
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  dropped_stores16(p.out);

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
    // range-checked buffer stores (rows past m dropped by the hardware): no branches, so the
    // next panel's load wait need not cover them
    {
      const int64_t row0 = panel * X3_PR + 32 * rb;
      const int64_t rows = p.m - row0 < 32 ? (p.m - row0 > 0 ? p.m - row0 : 0) : 32;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          p.out + row0 * p.ldo, 0, static_cast<int32_t>(rows * p.ldo * 4), kBufferWord3);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = static_cast<float>(sum[r]);
        if (p.relu) v = v > 0.0f ? v : 0.0f;
        const int pr = 8 * (r >> 2) + 4 * h + (r & 3);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs,
                                              static_cast<uint32_t>((pr * p.ldo + 32 * cb + l) * 4), 0, 0);
      }
    }
    __syncthreads();
  }
}

// Backward on the bf16 matrix cores (same split and the same six part products as the forward).
// One 512-thread block per compute unit, persistent over 32-row panels staged in double-buffered
// LDS: dZ = dH [H > 0] and A in float32 (row stride 140 floats, so that the 4-byte column reads
// of the dW operands hit distinct banks) and dZ's three bf16 planes for the dA operand.  Every
// thread loads its share of the next panel (dH, H, A) into registers during the products and
// stages it after the panel's one barrier.  The wavefronts split the products by role, one of
// each per SIMD:
//  - wavefronts 0-3 form dA = dZ W for 32 output columns each: W's parts for those columns stay
//    in registers (lane (h, l) holds W[16 s + 8 h + j][32 c + l]) and each 32-k chain is folded
//    into float64;
//  - wavefronts 4-7 form a 64 x 64 quarter of the block's dW partial = dZ^T A (four 32 x 32
//    tiles; operands read down the panel's float32 columns and split as they are read),
//    accumulated in float32 across the block's panels like the float32 kernel's.
constexpr int BX_PR = 32;           // rows per panel
constexpr int BX_LS = 140;          // floats per staged row
constexpr int BX_NT = 512;
constexpr int BX_SV = BX_PR * PD / 4 / BX_NT;   // float4 per thread per staged array (2)

// split3 of eight values, two at a time
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 wh, wm, wl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t a, b, d;
    split_pair(x[2 * k], x[2 * k + 1], a, b, d);
    wh[k] = a;
    wm[k] = b;
    wl[k] = d;
  }
  hi = __builtin_bit_cast(bf16x8, wh);
  mid = __builtin_bit_cast(bf16x8, wm);
  lo = __builtin_bit_cast(bf16x8, wl);
}

// c += a b over the six part products, smallest first
__device__ __forceinline__ floatx16 mfma6(const bf16x8& ah, const bf16x8& am, const bf16x8& al, const bf16x8& bh,
                                          const bf16x8& bm, const bf16x8& bl, floatx16 c) {
  c = mfma32b(am, bm, c);
  c = mfma32b(al, bh, c);
  c = mfma32b(ah, bl, c);
  c = mfma32b(am, bh, c);
  c = mfma32b(ah, bm, c);
  return mfma32b(ah, bh, c);
}

// Thread tid's share of panel pn: float4 f = tid + 512 s at (row f / 32, column 4 (f % 32)).  Rows
// at or past m are read from row m - 1 (no branches around the loads) and staged as zero.
__device__ __forceinline__ void bx_load(const float* dh, int64_t lddh, const float* hp, int64_t ldh, const float* ap,
                                        int64_t lda, int64_t m, int64_t pn, int tid, float4 (&g)[BX_SV],
                                        float4 (&hh)[BX_SV], float4 (&a)[BX_SV]) {
#pragma unroll
  for (int sv = 0; sv < BX_SV; ++sv) {
    const int f = tid + BX_NT * sv;
    int64_t r = pn * BX_PR + (f >> 5);
    r = r < m ? r : m - 1;
    const int c = 4 * (f & 31);
    g[sv] = *reinterpret_cast<const float4*>(dh + r * lddh + c);
    hh[sv] = *reinterpret_cast<const float4*>(hp + r * ldh + c);
    a[sv] = *reinterpret_cast<const float4*>(ap + r * lda + c);
  }
}

__device__ __forceinline__ void bx_stage(float* zs, float* as, __bf16* zp, int64_t m, int64_t pn, int tid, const float4 (&g)[BX_SV],
                                         const float4 (&hh)[BX_SV], const float4 (&a)[BX_SV]) {
#pragma unroll
  for (int sv = 0; sv < BX_SV; ++sv) {
    const int f = tid + BX_NT * sv;
    const int o = (f >> 5) * BX_LS + 4 * (f & 31);
    const bool in = pn * BX_PR + (f >> 5) < m;
    float4 z, x;
    z.x = in && hh[sv].x > 0.0f ? g[sv].x : 0.0f;
    z.y = in && hh[sv].y > 0.0f ? g[sv].y : 0.0f;
    z.z = in && hh[sv].z > 0.0f ? g[sv].z : 0.0f;
    z.w = in && hh[sv].w > 0.0f ? g[sv].w : 0.0f;
    x.x = in ? a[sv].x : 0.0f;
    x.y = in ? a[sv].y : 0.0f;
    x.z = in ? a[sv].z : 0.0f;
    x.w = in ? a[sv].w : 0.0f;
    *reinterpret_cast<float4*>(zs + o) = z;
    *reinterpret_cast<float4*>(as + o) = x;
    stage4<BX_PR>(zp, f >> 5, 4 * (f & 31), z);
  }
}

__global__ __launch_bounds__(BX_NT) void panel_bwd_x3_kernel(PanelArgs p) {
  __shared__ __attribute__((aligned(16))) float Zs[2][BX_PR * BX_LS];
  __shared__ __attribute__((aligned(16))) float As[2][BX_PR * BX_LS];
  __shared__ __attribute__((aligned(16))) __bf16 Zp[2][3 * BX_PR * X3_LS];   // dZ's bf16 planes
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l = lane & 31;
  const int64_t n_panels = (p.m + BX_PR - 1) / BX_PR;
  const int64_t grid = gridDim.x;
  int64_t panel = blockIdx.x;
  if (panel >= n_panels) return;

  // the first panel staged, the second in flight
  float4 pg[BX_SV], ph[BX_SV], pa[BX_SV];
  bx_load(p.dh, p.lddh, p.h, p.ldh, p.a, p.lda, p.m, panel, tid, pg, ph, pa);
  bx_stage(Zs[0], As[0], Zp[0], p.m, panel, tid, pg, ph, pa);
  if (panel + grid < n_panels) bx_load(p.dh, p.lddh, p.h, p.ldh, p.a, p.lda, p.m, panel + grid, tid, pg, ph, pa);
  int buf = 0;

  if (wid < 4) {
    // ---- dA role: output columns 32 cb .. 32 cb + 31
    const int cb = wid;
    bf16x8 wh[PD / 16], wm[PD / 16], wl[PD / 16];
#pragma unroll
    for (int st = 0; st < PD / 16; ++st) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = p.w[static_cast<int64_t>(16 * st + 8 * h + j) * p.ldw + 32 * cb + l];
      split8(x, wh[st], wm[st], wl[st]);
    }
    dropped_stores16(p.da);
    for (; panel < n_panels; panel += grid) {
      __syncthreads();
      const int64_t nxt = panel + grid;
      if (nxt < n_panels) {
        bx_stage(Zs[buf ^ 1], As[buf ^ 1], Zp[buf ^ 1], p.m, nxt, tid, pg, ph, pa);
        if (nxt + grid < n_panels) bx_load(p.dh, p.lddh, p.h, p.ldh, p.a, p.lda, p.m, nxt + grid, tid, pg, ph, pa);
      }
      const __bf16* zp = Zp[buf];
#pragma unroll
      for (int rb = 0; rb < BX_PR / 32; ++rb) {
        double sum[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sum[r] = 0.0;
#pragma unroll
        for (int kc = 0; kc < PD / 32; ++kc) {
          floatx16 acc;
          zero<16>(acc);
#pragma unroll
          for (int st = 2 * kc; st < 2 * kc + 2; ++st) {
            const __bf16* zr = zp + (32 * rb + l) * X3_LS + 16 * st + 8 * h;
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(zr);
            const bf16x8 xm = *reinterpret_cast<const bf16x8*>(zr + BX_PR * X3_LS);
            const bf16x8 xl = *reinterpret_cast<const bf16x8*>(zr + 2 * BX_PR * X3_LS);
            acc = mfma6(xh, xm, xl, wh[st], wm[st], wl[st], acc);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) sum[r] += static_cast<double>(acc[r]);
        }
        // range-checked buffer stores: rows at or past m are dropped by the hardware, so the
        // stores need no branches (and the next panel's load waits need not cover them)
        const int64_t row0 = panel * BX_PR + 32 * rb;
        const int64_t rows = p.m - row0 < 32 ? p.m - row0 : 32;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            p.da + row0 * p.ldda, 0, static_cast<int32_t>(rows * p.ldda * 4), kBufferWord3);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pr = 8 * (r >> 2) + 4 * h + (r & 3);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(static_cast<float>(sum[r])), rs,
                                                static_cast<uint32_t>((pr * p.ldda + 32 * cb + l) * 4), 0, 0);
        }
      }
      buf ^= 1;
    }
    return;
  }

  // ---- dW role: wavefront q forms the tiles (o-block 2 (q / 2) + ot, i-block 2 (q % 2) + it)
  const int q = wid - 4;
  const int ob0 = 2 * (q >> 1);
  const int ib0 = 2 * (q & 1);
  floatx16 wacc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) zero<16>(wacc[k]);
  for (; panel < n_panels; panel += grid) {
    __syncthreads();
    const int64_t nxt = panel + grid;
    if (nxt < n_panels) {
      bx_stage(Zs[buf ^ 1], As[buf ^ 1], Zp[buf ^ 1], p.m, nxt, tid, pg, ph, pa);
      if (nxt + grid < n_panels) bx_load(p.dh, p.lddh, p.h, p.ldh, p.a, p.lda, p.m, nxt + grid, tid, pg, ph, pa);
    }
    const float* zb = Zs[buf];
    const float* ab = As[buf];
#pragma unroll
    for (int ks = 0; ks < BX_PR / 16; ++ks) {
      // lane half h takes the panel rows 16 ks + 8 h .. + 7
      bf16x8 zh[2], zm[2], zl[2], ah[2], am[2], al[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float xz[8], xa[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int o = (16 * ks + 8 * h + j) * BX_LS + l;
          xz[j] = zb[o + 32 * (ob0 + u)];
          xa[j] = ab[o + 32 * (ib0 + u)];
        }
        split8(xz, zh[u], zm[u], zl[u]);
        split8(xa, ah[u], am[u], al[u]);
      }
      // the four tiles' products interleaved, so that consecutive MFMAs are independent (each
      // tile still takes its six products smallest first)
#define QHA_DW_STEP(ZA, AB)                                                         \
  _Pragma("unroll") for (int ot = 0; ot < 2; ++ot)                                  \
  _Pragma("unroll") for (int it = 0; it < 2; ++it)                                  \
      wacc[2 * ot + it] = mfma32b(ZA[ot], AB[it], wacc[2 * ot + it]);
      QHA_DW_STEP(zm, am)
      QHA_DW_STEP(zl, ah)
      QHA_DW_STEP(zh, al)
      QHA_DW_STEP(zm, ah)
      QHA_DW_STEP(zh, am)
      QHA_DW_STEP(zh, ah)
#undef QHA_DW_STEP
    }
    buf ^= 1;
  }
  float* part = p.ws + static_cast<int64_t>(blockIdx.x) * PD * PD;
#pragma unroll
  for (int ot = 0; ot < 2; ++ot)
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int o = 32 * (ob0 + ot) + 8 * (r >> 2) + 4 * h + (r & 3);
        part[o * PD + 32 * (ib0 + it) + l] = wacc[2 * ot + it][r];
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

// ---- weight gradient of the general widths: dW = dZ^T A, dZ = dH * [H > 0] ----
// One 512-thread block per (row range, 128 dZ columns, 256 A columns), persistent over the range's
// 32-row panels (panels rr, rr + R, rr + 2R, ...).  As in the width-128 backward's dW role, each
// panel is staged as float32 rows in double-buffered LDS (row strides 132 and 260 floats: the
// column reads of the two lane halves, 8 rows apart, hit distinct banks), one barrier per panel,
// the next panel loaded into registers during the products; every wavefront forms a 64 x 64 block
// of four 32 x 32 tiles, reading its operands down the staged columns and splitting them as it
// reads (six part products, smallest first, the four tiles interleaved).  The tiles accumulate in
// float32 over the block's range and each block writes its range's partial once; a second kernel
// adds the R partials of every output in float64 in range order.  The blocks that
// share a row range take the same block index modulo 8, so they run on one XCD and its L2 serves
// their common rows.  A block sums at most about DW_RANGE_ROWS rows in float32 (as the width-128
// backward's blocks sum theirs), so the number of ranges grows with m.
constexpr int DW_PR = 32;
constexpr int DW_ZC = 128;
constexpr int DW_AC = 256;
constexpr int DW_ZLS = 132;
constexpr int DW_ALS = 260;
constexpr int DW_RANGE_ROWS = 4096;
constexpr int DW_SZ = DW_PR * DW_ZC / 4 / 512;   // float4 of dH (and of H) per thread per panel
constexpr int DW_SA = DW_PR * DW_AC / 4 / 512;   // float4 of A per thread per panel

__global__ __launch_bounds__(512) void dw_panel_kernel(DwArgs p) {
  __shared__ __attribute__((aligned(16))) float Zs[2][DW_PR * DW_ZLS];
  __shared__ __attribute__((aligned(16))) float As[2][DW_PR * DW_ALS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l = lane & 31;
  const int g = p.groups_z * p.groups_a;
  const int b = static_cast<int>(blockIdx.x);
  const int j = (b >> 3) % g;
  const int64_t rr = 8 * static_cast<int64_t>((b >> 3) / g) + (b & 7);
  const int zc0 = DW_ZC * (j % p.groups_z);
  const int ac0 = DW_AC * (j / p.groups_z);
  const int ob0 = 2 * (wid & 1);      // o-blocks (32 dZ columns each) ob0, ob0 + 1 of 4
  const int ib0 = 2 * (wid >> 1);     // i-blocks (32 A columns each) ib0, ib0 + 1 of 8
  const int64_t n_panels = (p.m + DW_PR - 1) / DW_PR;
  const int64_t stride = p.ranges;

  floatx16 wacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) zero<16>(wacc[t]);

  // thread tid's share of a panel: dZ float4 f = tid + 512 s at (row f / 32, column 4 (f % 32)),
  // A float4 f at (row f / 64, column 4 (f % 64)); rows at or past m are read from row m - 1 (no
  // branches around the loads) and staged as zero
  float4 gz[DW_SZ], gh[DW_SZ], ga[DW_SA];
  auto load = [&](int64_t pn) {
#pragma unroll
    for (int s = 0; s < DW_SZ; ++s) {
      const int f = tid + 512 * s;
      int64_t r = pn * DW_PR + (f >> 5);
      r = r < p.m ? r : p.m - 1;
      gz[s] = *reinterpret_cast<const float4*>(p.dh + r * p.lddh + zc0 + 4 * (f & 31));
      gh[s] = *reinterpret_cast<const float4*>(p.h + r * p.ldh + zc0 + 4 * (f & 31));
    }
#pragma unroll
    for (int s = 0; s < DW_SA; ++s) {
      const int f = tid + 512 * s;
      int64_t r = pn * DW_PR + (f >> 6);
      r = r < p.m ? r : p.m - 1;
      ga[s] = *reinterpret_cast<const float4*>(p.a + r * p.lda + ac0 + 4 * (f & 63));
    }
  };
  auto stage = [&](int buf, int64_t pn) {
#pragma unroll
    for (int s = 0; s < DW_SZ; ++s) {
      const int f = tid + 512 * s;
      const bool in = pn * DW_PR + (f >> 5) < p.m;
      float4 z;
      z.x = in && gh[s].x > 0.0f ? gz[s].x : 0.0f;
      z.y = in && gh[s].y > 0.0f ? gz[s].y : 0.0f;
      z.z = in && gh[s].z > 0.0f ? gz[s].z : 0.0f;
      z.w = in && gh[s].w > 0.0f ? gz[s].w : 0.0f;
      *reinterpret_cast<float4*>(&Zs[buf][(f >> 5) * DW_ZLS + 4 * (f & 31)]) = z;
    }
#pragma unroll
    for (int s = 0; s < DW_SA; ++s) {
      const int f = tid + 512 * s;
      const bool in = pn * DW_PR + (f >> 6) < p.m;
      float4 x;
      x.x = in ? ga[s].x : 0.0f;
      x.y = in ? ga[s].y : 0.0f;
      x.z = in ? ga[s].z : 0.0f;
      x.w = in ? ga[s].w : 0.0f;
      *reinterpret_cast<float4*>(&As[buf][(f >> 6) * DW_ALS + 4 * (f & 63)]) = x;
    }
  };

  int64_t panel = rr;
  if (panel < n_panels) {
    load(panel);
    stage(0, panel);
    if (panel + stride < n_panels) load(panel + stride);
  }
  int buf = 0;
  for (; panel < n_panels; panel += stride) {
    __syncthreads();
    const int64_t nxt = panel + stride;
    if (nxt < n_panels) {
      stage(buf ^ 1, nxt);
      if (nxt + stride < n_panels) load(nxt + stride);
    }
    const float* zb = Zs[buf];
    const float* ab = As[buf];
#pragma unroll
    for (int ks = 0; ks < DW_PR / 16; ++ks) {
      // lane half h takes the panel rows 16 ks + 8 h .. + 7
      bf16x8 zh[2], zm[2], zl[2], ah[2], am[2], al[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float xz[8], xa[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int row = 16 * ks + 8 * h + q;
          xz[q] = zb[row * DW_ZLS + 32 * (ob0 + u) + l];
          xa[q] = ab[row * DW_ALS + 32 * (ib0 + u) + l];
        }
        split8(xz, zh[u], zm[u], zl[u]);
        split8(xa, ah[u], am[u], al[u]);
      }
#define QHA_DW_STEP(ZA, AB)                                                         \
  _Pragma("unroll") for (int ot = 0; ot < 2; ++ot)                                  \
  _Pragma("unroll") for (int it = 0; it < 2; ++it)                                  \
      wacc[2 * ot + it] = mfma32b(ZA[ot], AB[it], wacc[2 * ot + it]);
      QHA_DW_STEP(zm, am)
      QHA_DW_STEP(zl, ah)
      QHA_DW_STEP(zh, al)
      QHA_DW_STEP(zm, ah)
      QHA_DW_STEP(zh, am)
      QHA_DW_STEP(zh, ah)
#undef QHA_DW_STEP
    }
    buf ^= 1;
  }
  // this range's partial for the block's outputs (zero if the range holds no panel)
  float* part = p.ws + rr * static_cast<int64_t>(p.n) * p.k;
#pragma unroll
  for (int ot = 0; ot < 2; ++ot)
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t o = zc0 + 32 * (ob0 + ot) + 8 * (r >> 2) + 4 * h + (r & 3);
        part[o * p.k + ac0 + 32 * (ib0 + it) + l] = wacc[2 * ot + it][r];
      }
}

// dW[o][i] = the float64 sum of the R ranges' partials in range order; eight ranges' loads are
// issued together.  One thread per output.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const float* ws, int32_t ranges, int64_t nk, int32_t k,
                                                        float* dw, int64_t lddw) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= nk) return;
  const float* src = ws + idx;
  double s = 0.0;
  int z = 0;
  for (; z + 8 <= ranges; z += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = src[static_cast<int64_t>(z + u) * nk];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += static_cast<double>(t[u]);
  }
  for (; z < ranges; ++z) s += static_cast<double>(src[static_cast<int64_t>(z) * nk]);
  dw[(idx / k) * lddw + idx % k] = static_cast<float>(s);
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
  if (p.ldo >= (int64_t{1} << 24)) return hipErrorInvalidValue;   // 32-row store ranges in 32 bits
  const int64_t n_panels = (p.m + X3_PR - 1) / X3_PR;
  const unsigned grid = static_cast<unsigned>(n_panels < kPanelBlocks ? n_panels : kPanelBlocks);
  hipLaunchKernelGGL(panel_fwd_x3_kernel, dim3(grid), dim3(X3_NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_panel_bwd(const PanelArgs& p, hipStream_t s) {
  if (p.m == 0) return hipSuccess;
  if (p.ldda >= (int64_t{1} << 24)) return hipErrorInvalidValue;  // 32-row store ranges in 32 bits
  const int32_t grid = panel_grid(p.m);
  hipLaunchKernelGGL(panel_bwd_x3_kernel, dim3(static_cast<unsigned>(grid)), dim3(BX_NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(panel_dw_reduce_kernel, dim3(PD * PD / 64), dim3(256), 0, s, static_cast<const float*>(p.ws),
                     grid, p.dw, p.lddw);
  return hipGetLastError();
}


bool dw_panel_fits(int64_t m, int64_t n, int64_t k) {
  return m > 0 && n > 0 && k > 0 && n % DW_ZC == 0 && k % DW_AC == 0;
}

int32_t dw_panel_ranges(int64_t m, int64_t n, int64_t k) {
  // enough blocks for every compute unit, and at most about DW_RANGE_ROWS rows per range
  // (a whole number of rounds of kPanelBlocks blocks when the ranges outnumber one round)
  const int64_t g = (n / DW_ZC) * (k / DW_AC);
  int64_t fill = kPanelBlocks / g;
  fill = fill < 8 ? 8 : fill / 8 * 8;
  const int64_t len = (m + DW_RANGE_ROWS - 1) / DW_RANGE_ROWS;
  return static_cast<int32_t>((len + fill - 1) / fill * fill);
}

size_t dw_panel_workspace(int64_t m, int64_t n, int64_t k) {
  return static_cast<size_t>(dw_panel_ranges(m, n, k)) * static_cast<size_t>(n) * static_cast<size_t>(k) *
         sizeof(float);
}

hipError_t launch_dw_panel(const DwArgs& a, float* dw, int64_t lddw, hipStream_t s) {
  const int64_t g = static_cast<int64_t>(a.groups_z) * a.groups_a;
  const int64_t blocks = static_cast<int64_t>(a.ranges) * g;
  hipLaunchKernelGGL(dw_panel_kernel, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nk = static_cast<int64_t>(a.n) * a.k;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3(static_cast<unsigned>((nk + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(a.ws), a.ranges, nk, a.k, dw, lddw);
  return hipGetLastError();
}

}  // namespace qha
