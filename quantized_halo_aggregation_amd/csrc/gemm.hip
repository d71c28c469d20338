// Dense projection C = op(A) op(B) with float32 products on the bf16 matrix cores, with the ReLU
// epilogue of the forward and the ReLU-mask prologue of the backward.
//
// Method: SYLVIE guide, section 2 (z_v = W a_v, h_v = sigma(z_v)) and section 7 (the weight
// gradient sum_v (dL/dh_v * sigma'(z_v)) a_v^T).
//
// Mapping to gfx950: a block owns a 64x128 tile of C (256 threads), or 64x256 for outputs at least
// 512 wide (512 threads, so each A tile is staged once for twice the columns); its wavefronts own
// 32x64 pieces, each two 32x32 accumulators (32 fp32 per lane) plus their float64 running sums.  The
// float32 products run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16): every operand value is
// split exactly into three bf16 parts as its tile is staged in LDS (once per block), and each
// product is rebuilt from the six part products of weight >= 2^-16 of it (the dropped ones total
// below 2^-23 of the product, about one float32 rounding).  K advances 32 at a time; the tiles are
// staged k-contiguous ([row][k] for A, [column][k] for B, 40 bf16 per row so that the 16-byte
// operand reads and the 8-byte staging writes hit distinct banks); operands stored k-major are
// read four k at a time with coalesced 4-byte loads, which transposes them on the way in (range-
// checked buffer loads at 32-bit offsets when they span under 2 GiB, else 64-bit addresses).
// When A has many rows and the caller's workspace has room, B (the weights) is split once per call
// by split_b_kernel, in the order of the MFMA fragments, and gemm_bsplit_kernel runs the products:
// 64 x 128 block tiles whose wavefronts own 64 rows x 32 columns each and read their B fragments
// straight from the split parts (L2-resident, 1 KB per wavefront load), so LDS carries only A
// (the same parts and the same part products per accumulator, so the same bits).
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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data, range-checked against num_records

constexpr int BM = 64;
constexpr int BK = 32;
constexpr int KS = BK + 8;     // bf16 per staged row
// Block tile BM x BN with two wavefronts along m and BN / 64 along n (2 BN threads): BN = 256 for
// outputs at least 512 wide (each A tile is then staged once for twice the columns; measured
// faster there, slower at 256), else 128.
template <int BN>
struct Tile {
  static constexpr int NT = 2 * BN;
  static constexpr int A_LOADS = BM * BK / 4 / NT;   // float4 loads per thread per k step
  static constexpr int B_LOADS = BN * BK / 4 / NT;
};
int tile_n(int64_t n) { return n >= 512 ? 256 : 128; }
// B is split once per call (into the workspace) when A has at least this many rows: below it the
// per-tile split of B costs little and the extra launch would not pay
constexpr int64_t kBSplitMinRows = 16384;
constexpr int64_t kXcds = 8;        // accelerator complex dies of an MI355X, each with its own L2
#ifndef QHA_GEMM_ORDER
#define QHA_GEMM_ORDER 2
#endif

// x = hi + mid + lo exactly for a pair of values, as packed bf16 words (first value in the low
// half): each part is rounded to nearest even, and the remainders x - hi and (x - hi) - mid are
// exact in float32.
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

// Stages a float4 that runs along k (4 consecutive k of one row) into the three planes.
template <int ROWS>
__device__ __forceinline__ void stage_k4(__bf16* planes, int row, int k, const float4& v) {
  uint2 h, m, l;
  split_pair(v.x, v.y, h.x, m.x, l.x);
  split_pair(v.z, v.w, h.y, m.y, l.y);
  const int o = row * KS + k;
  *reinterpret_cast<uint2*>(planes + o) = h;
  *reinterpret_cast<uint2*>(planes + ROWS * KS + o) = m;
  *reinterpret_cast<uint2*>(planes + 2 * ROWS * KS + o) = l;
}

__device__ __forceinline__ floatx16 mfma6(const bf16x8& ah, const bf16x8& am, const bf16x8& al, const bf16x8& bh,
                                          const bf16x8& bm, const bf16x8& bl, floatx16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bm, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bm, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c, 0, 0, 0);
}

// global -> registers for the tiles starting at k0, as float4s that run along k: float4 s of a
// thread is (row, k0 + 4 kq .. + 3) of A (rows m0 + row) and B (columns n0 + row).  An operand
// stored k-contiguous is read with one 16-byte load per float4 (eight lanes per row); one stored
// k-major with four 4-byte loads whose lanes run along the rows (coalesced), which transposes it on
// the way in.  Values outside the operands (rows, columns, k) are zero; out-of-range loads read the
// operand's first element instead (no branch around the loads).  A k-contiguous operand has k a
// multiple of 4 (the entry points require it), so none of its float4s runs past the last k; a
// k-major operand's k (a row count) is arbitrary, and each of its four k is checked.
template <bool TRANS, int ROWS, int NL, int NT>
__device__ __forceinline__ void load_k4(const float* x, int64_t ld, const float* aux, int64_t ld_aux, bool mask,
                                        int64_t r0, int64_t rows, int64_t k0, int64_t kend, int tid, float4 (&v)[NL],
                                        bool buf32 = false) {
  if (TRANS && buf32) {
    // k-major operand within 2 GiB: range-checked buffer loads at 32-bit offsets.  The hardware
    // checks only the per-lane offset against a buffer's size (not the scalar offset), so each of
    // the four k of a float4 gets a buffer of its own: buffer j starts j rows further on and ends
    // at row kend, so a read of row gk + j >= kend returns 0 while every lane uses the same offset.
    // Lanes past the last column or past kend get an offset beyond every buffer.
    __amdgpu_buffer_rsrc_t rx[4], ra[4];
    const float* xa = mask ? aux : x;
    const int64_t lda_ = mask ? ld_aux : ld;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t left = kend - j > 0 ? kend - j : 0;
      rx[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x + j * ld), 0, static_cast<int32_t>(left * ld * 4),
                                               kBufferWord3);
      ra[j] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(xa + j * lda_), 0,
                                               static_cast<int32_t>(left * lda_ * 4), kBufferWord3);
    }
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int f = tid + NT * s;
      const int row = f % ROWS;
      const int kq = f / ROWS;
      const int64_t gr = r0 + row, gk = k0 + 4 * kq;
      const bool ok = gr < rows && gk < kend;
      const uint32_t ox = ok ? static_cast<uint32_t>((gk * ld + gr) * 4) : 0x80000000u;
      const uint32_t oa = ok ? static_cast<uint32_t>((gk * ld_aux + gr) * 4) : 0x80000000u;
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float t = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx[j], ox, 0, 0));
        if (mask) {
          const float a = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra[j], oa, 0, 0));
          t = a > 0.0f ? t : 0.0f;
        }
        e[j] = t;
      }
      v[s] = make_float4(e[0], e[1], e[2], e[3]);
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < NL; ++s) {
    const int f = tid + NT * s;
    const int row = TRANS ? f % ROWS : f / (BK / 4);
    const int kq = TRANS ? f / ROWS : f % (BK / 4);
    const int64_t gr = r0 + row, gk = k0 + 4 * kq;
    float e[4];
    if (!TRANS) {         // stored [row][k]
      const bool ok = gr < rows && gk < kend;
      const int64_t off = ok ? gr * ld + gk : 0;
      const float4 t = *reinterpret_cast<const float4*>(x + off);
      e[0] = t.x; e[1] = t.y; e[2] = t.z; e[3] = t.w;
      if (mask) {
        const float4 a = *reinterpret_cast<const float4*>(aux + (ok ? gr * ld_aux + gk : 0));
        e[0] = a.x > 0.0f ? e[0] : 0.0f;
        e[1] = a.y > 0.0f ? e[1] : 0.0f;
        e[2] = a.z > 0.0f ? e[2] : 0.0f;
        e[3] = a.w > 0.0f ? e[3] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = ok ? e[j] : 0.0f;
    } else {              // stored [k][row]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = gr < rows && gk + j < kend;
        float t = x[ok ? (gk + j) * ld + gr : 0];
        if (mask) t = aux[ok ? (gk + j) * ld_aux + gr : 0] > 0.0f ? t : 0.0f;
        e[j] = ok ? t : 0.0f;
      }
    }
    v[s] = make_float4(e[0], e[1], e[2], e[3]);
  }
}

template <int BN, bool TA, bool TB, bool MASK>
__device__ __forceinline__ void load_tiles(const GemmArgs& p, int tid, int64_t m0, int64_t n0, int64_t k0, int64_t kend,
                                           float4 (&ra)[Tile<BN>::A_LOADS], float4 (&rb)[Tile<BN>::B_LOADS]) {
  load_k4<TA, BM, Tile<BN>::A_LOADS, Tile<BN>::NT>(p.a, p.lda, p.aux, p.ld_aux, MASK, m0, p.m, k0, kend, tid, ra, p.buf32 != 0);
  load_k4<!TB, BN, Tile<BN>::B_LOADS, Tile<BN>::NT>(p.b, p.ldb, nullptr, 0, false, n0, p.n, k0, kend, tid, rb, p.buf32 != 0);
}

// registers -> the k-contiguous bf16 planes of the tiles
template <int BN, bool TA, bool TB>
__device__ __forceinline__ void store_tiles(__bf16* As, __bf16* Bs, int tid, const float4 (&ra)[Tile<BN>::A_LOADS],
                                            const float4 (&rb)[Tile<BN>::B_LOADS]) {
#pragma unroll
  for (int s = 0; s < Tile<BN>::A_LOADS; ++s) {
    const int f = tid + Tile<BN>::NT * s;
    if (!TA) stage_k4<BM>(As, f / (BK / 4), 4 * (f % (BK / 4)), ra[s]);
    else stage_k4<BM>(As, f % BM, 4 * (f / BM), ra[s]);
  }
#pragma unroll
  for (int s = 0; s < Tile<BN>::B_LOADS; ++s) {
    const int f = tid + Tile<BN>::NT * s;
    if (TB) stage_k4<BN>(Bs, f / (BK / 4), 4 * (f % (BK / 4)), rb[s]);
    else stage_k4<BN>(Bs, f % BN, 4 * (f / BN), rb[s]);
  }
}

// B's parts split once per call (hi, mid, lo of every value, by split_pair, so the same parts as the
// per-tile split), written in the order in which gemm_bsplit_kernel's wavefronts read them as MFMA
// fragments; columns padded to the 128-wide tile and k to BK with zeros, so no load needs a range
// check.
__global__ __launch_bounds__(256) void split_b_kernel(const float* b, int64_t ldb, int32_t tb, int64_t n, int64_t k,
                                                      uint32_t* planes, int64_t n_pad, int64_t k_pad) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // a pair (j, 2 kq .. + 1)
  const int64_t pairs = n_pad * (k_pad / 2);
  if (i >= pairs) return;
  const int64_t j = i / (k_pad / 2), kk = 2 * (i % (k_pad / 2));
  float v[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bool ok = j < n && kk + t < k;
    v[t] = ok ? b[tb ? j * ldb + kk + t : (kk + t) * ldb + j] : 0.0f;
  }
  uint32_t h, m, l;
  split_pair(v[0], v[1], h, m, l);
  // fragment order: for each 32-column tile and 16-k step, the three planes' fragments in lane
  // order (lane (hf, c) holds column 32 t + c, k = 16 s + 8 hf .. + 7, as 16 bytes), so that a
  // wavefront reads one fragment of one plane as 1 KB of consecutive memory
  const int64_t nks = k_pad / 16;
  const int64_t chunk = (((j / 32) * nks + kk / 16) * 3) * 64 + ((kk / 8) % 2) * 32 + j % 32;
  const int64_t w = (kk % 8) / 2;
  planes[(chunk + 0 * 64) * 4 + w] = h;
  planes[(chunk + 1 * 64) * 4 + w] = m;
  planes[(chunk + 2 * 64) * 4 + w] = l;
}

template <int BN, bool TA, bool TB, bool MASK, bool SPLIT>
__global__ __launch_bounds__(Tile<BN>::NT) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) __bf16 As[3 * BM * KS];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[3 * BN * KS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / (BN / 64);   // 32-row half of the block tile
  const int wn = wid % (BN / 64);   // 64-column slice
  const int h = lane >> 5;
  const int l32 = lane & 31;
  int64_t mbk = blockIdx.x, nbk = blockIdx.y, zk = blockIdx.z;
  if constexpr (SPLIT && QHA_GEMM_ORDER == 2) {
    // split reductions on a one-dimensional grid: the output tiles of one k range are consecutive
    // blocks of one XCD, so the rows of that range, which every tile reads, are shared in its L2
    const int64_t mb = (p.m + BM - 1) / BM, tiles = mb * ((p.n + BN - 1) / BN), b = blockIdx.x;
    const int64_t sl = b / kXcds, t = sl % tiles;
    zk = sl / tiles * kXcds + b % kXcds;
    if (zk >= p.splits) return;        // the padding of the last group of XCD splits
    mbk = t % mb;
    nbk = t / mb;
  }
  if constexpr (!SPLIT && QHA_GEMM_ORDER > 0) {
    // one-dimensional grid: the column tiles of a row tile are consecutive blocks (order 1), or
    // consecutive blocks of one XCD (order 2: blocks are dealt to the eight XCDs in turn), so that
    // A's rows, read once per column tile, come from cache the second time
    const int64_t nb = (p.n + BN - 1) / BN, b = blockIdx.x;
    if constexpr (QHA_GEMM_ORDER == 1) {
      nbk = b % nb;
      mbk = b / nb;
    } else {
      const int64_t sl = b / kXcds;
      nbk = sl % nb;
      mbk = sl / nb * kXcds + b % kXcds;
      if (mbk * BM >= p.m) return;     // the padding of the last group of XCD rows
    }
  }
  const int64_t m0 = mbk * BM;
  const int64_t n0 = nbk * BN;
  const int64_t kbeg = zk * p.k_per_split;
  const int64_t kend = min(p.k, kbeg + p.k_per_split);

  double sum[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[j][r] = 0.0;

  float4 ra[Tile<BN>::A_LOADS], rb[Tile<BN>::B_LOADS];

  if (kbeg < kend) {
    load_tiles<BN, TA, TB, MASK>(p, tid, m0, n0, kbeg, kend, ra, rb);
    store_tiles<BN, TA, TB>(As, Bs, tid, ra, rb);
    __syncthreads();
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
    const bool more = k0 + BK < kend;
    if (more) load_tiles<BN, TA, TB, MASK>(p, tid, m0, n0, k0 + BK, kend, ra, rb);
    floatx16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      // lane (h, l32) takes k = 16 ks + 8 h .. + 7 of row l32 (A) and of column l32 (B)
      const __bf16* ap = As + (wm * 32 + l32) * KS + 16 * ks + 8 * h;
      const bf16x8 xh = *reinterpret_cast<const bf16x8*>(ap);
      const bf16x8 xm = *reinterpret_cast<const bf16x8*>(ap + BM * KS);
      const bf16x8 xl = *reinterpret_cast<const bf16x8*>(ap + 2 * BM * KS);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const __bf16* bp = Bs + (wn * 64 + ni * 32 + l32) * KS + 16 * ks + 8 * h;
        const bf16x8 yh = *reinterpret_cast<const bf16x8*>(bp);
        const bf16x8 ym = *reinterpret_cast<const bf16x8*>(bp + BN * KS);
        const bf16x8 yl = *reinterpret_cast<const bf16x8*>(bp + 2 * BN * KS);
        acc[ni] = mfma6(xh, xm, xl, yh, ym, yl, acc[ni]);
      }
    }
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[ni][r] += static_cast<double>(acc[ni][r]);
    __syncthreads();
    if (more) {
      store_tiles<BN, TA, TB>(As, Bs, tid, ra, rb);
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
          p.ws[zk * p.m * p.n + grow * p.n + gcol] = s;
        } else {
          float* dst = p.c + grow * p.ldc + gcol;
          float v = static_cast<float>(p.beta ? static_cast<double>(*dst) + s : s);
          if (p.epi == 1) v = v > 0.0f ? v : 0.0f;
          *dst = v;
        }
      }
    }
}

// The products with B split once per call (A not transposed, k not split): the same part products
// as gemm_kernel in the same order per accumulator (so the same bits), with a different division of
// the block tile: each wavefront owns all BM = 64 rows and 32 columns, and reads its B fragments --
// 16 bytes of one plane for one column and 8 consecutive k, a contiguous piece of the split planes --
// straight from global memory (the planes stay in L2), one k step ahead, instead of through LDS.
// Only A's tile is staged, so LDS carries A's fragments (read by every wavefront) and no B tile:
// about half the LDS bytes per MFMA of the 32 x 64 wavefront tiles, which were bound by them.
template <int BN, bool TA, bool MASK>
__global__ __launch_bounds__(Tile<BN>::NT) void gemm_bsplit_kernel(GemmArgs p) {
  static_assert(!TA, "B split once is used with A not transposed");
  __shared__ __attribute__((aligned(16))) __bf16 Asb[2][3 * BM * KS];   // double-buffered A tile
  constexpr int NT = Tile<BN>::NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);   // 32-column slice of the block tile
  const int h = lane >> 5;
  const int l32 = lane & 31;
  int64_t mbk = blockIdx.x, nbk = blockIdx.y;
  if constexpr (QHA_GEMM_ORDER > 0) {
    // the unsplit kernels' order: the column tiles of a row tile are consecutive blocks (of one XCD)
    const int64_t nb = (p.n + BN - 1) / BN, b = blockIdx.x;
    if constexpr (QHA_GEMM_ORDER == 1) {
      nbk = b % nb;
      mbk = b / nb;
    } else {
      const int64_t sl = b / kXcds;
      nbk = sl % nb;
      mbk = sl / nb * kXcds + b % kXcds;
      if (mbk * BM >= p.m) return;
    }
  }
  const int64_t m0 = mbk * BM;
  const int64_t n0 = nbk * BN;
  const int64_t kend = p.k;

  double sum[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[j][r] = 0.0;

  // B's split parts in fragment order (split_b_kernel), padded with zeros to whole column tiles
  // and k steps: this wavefront's fragment of plane q at 16-k step s is 64 consecutive u32x4
  const int64_t nks = (p.k + BK - 1) / BK * (BK / 16);
  const u32x4* bsrc = reinterpret_cast<const u32x4*>(p.bsplit) + ((n0 / 32 + wn) * nks) * 3 * 64 + lane;
  auto load_b = [&](int64_t k0, u32x4 (&dst)[2][3]) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
      for (int q = 0; q < 3; ++q) dst[ks][q] = bsrc[((k0 / 16 + ks) * 3 + q) * 64];
  };
  // A's rows for the k step at k0: raw float4s (and the ReLU mask's beside them), with nothing
  // computed from them here, so that the loads stay in flight through the current step's products;
  // the range check and the mask are applied as the tile is staged
  constexpr int AL = Tile<BN>::A_LOADS;
  auto a_ok = [&](int s, int64_t k0, int64_t& off, int64_t& offm) {
    const int f = tid + NT * s;
    const int64_t gr = m0 + f / (BK / 4), gk = k0 + 4 * (f % (BK / 4));
    const bool ok = gr < p.m && gk < kend;
    off = ok ? gr * p.lda + gk : 0;
    offm = ok ? gr * p.ld_aux + gk : 0;
    return ok;
  };
  auto load_a = [&](int64_t k0, float4 (&ra)[AL], float4 (&rm)[MASK ? AL : 1]) {
#pragma unroll
    for (int s = 0; s < AL; ++s) {
      int64_t off, offm;
      a_ok(s, k0, off, offm);
      ra[s] = *reinterpret_cast<const float4*>(p.a + off);
      if constexpr (MASK) rm[s] = *reinterpret_cast<const float4*>(p.aux + offm);
    }
  };
  auto stage_a = [&](__bf16* As, int64_t k0, const float4 (&ra)[AL], const float4 (&rm)[MASK ? AL : 1]) {
#pragma unroll
    for (int s = 0; s < AL; ++s) {
      int64_t off, offm;
      const bool ok = a_ok(s, k0, off, offm);
      float4 v = ra[s];
      if constexpr (MASK) {
        v.x = rm[s].x > 0.0f ? v.x : 0.0f;
        v.y = rm[s].y > 0.0f ? v.y : 0.0f;
        v.z = rm[s].z > 0.0f ? v.z : 0.0f;
        v.w = rm[s].w > 0.0f ? v.w : 0.0f;
      }
      v = ok ? v : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      const int f = tid + NT * s;
      stage_k4<BM>(As, f / (BK / 4), 4 * (f % (BK / 4)), v);
    }
  };

  float4 ra[AL], rm[MASK ? AL : 1];
  u32x4 bq[2][3], bn[2][3];
  if (kend > 0) {
    load_a(0, ra, rm);
    load_b(0, bq);
    stage_a(Asb[0], 0, ra, rm);
    __syncthreads();
  }
  // one k step: the next step's A rows and B fragments are loaded (into nxt) while this step's
  // products run from cur and A's tile in As; two steps per loop trip, so the fragment sets
  // alternate without copies.  The next A tile is staged into the other buffer An after this
  // step's products, so one barrier per step orders both the reads and the writes.
  auto kstep = [&](int64_t k0, const __bf16* As, __bf16* An, const u32x4 (&cur)[2][3], u32x4 (&nxt)[2][3]) {
    const bool more = k0 + BK < kend;
    // the loads are issued whether or not a next step exists (past the last step A's rows read the
    // operand's first element and B's fragments this step's again, all unused): with no branch
    // around them the compiler waits for exactly the loads each use needs, and keeps them here
    load_a(k0 + BK, ra, rm);
    floatx16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8 yh = __builtin_bit_cast(bf16x8, cur[ks][0]);
      const bf16x8 ym = __builtin_bit_cast(bf16x8, cur[ks][1]);
      const bf16x8 yl = __builtin_bit_cast(bf16x8, cur[ks][2]);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        // lane (h, l32) takes k = 16 ks + 8 h .. + 7 of row 32 mi + l32
        const __bf16* ap = As + (32 * mi + l32) * KS + 16 * ks + 8 * h;
        const bf16x8 xh = *reinterpret_cast<const bf16x8*>(ap);
        const bf16x8 xm = *reinterpret_cast<const bf16x8*>(ap + BM * KS);
        const bf16x8 xl = *reinterpret_cast<const bf16x8*>(ap + 2 * BM * KS);
        acc[mi] = mfma6(xh, xm, xl, yh, ym, yl, acc[mi]);
      }
    }
    // the next step's B fragments are requested once this step's products have taken theirs (they
    // come from L2); requested before them, they would sit behind this step's A rows in the load
    // queue, and the compiler's wait for the fragments in use would also wait for those rows
    load_b(more ? k0 + BK : k0, nxt);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[mi][r] += static_cast<double>(acc[mi][r]);
    // staged whether or not a next step exists (past the last step the buffer is not read again):
    // a branch here would let the compiler sink the loads above into it, next to their use
    stage_a(An, k0 + BK, ra, rm);
    __syncthreads();
  };
  for (int64_t k0 = 0; k0 < kend; k0 += 2 * BK) {
    kstep(k0, Asb[0], Asb[1], bq, bn);
    if (k0 + BK < kend) kstep(k0 + BK, Asb[1], Asb[0], bn, bq);
  }

  // accumulator element r of lane (h, l32) is C[8*(r/4) + 4*h + r%4][l32] of the 32x32 block
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t grow = m0 + 32 * mi + 8 * (r >> 2) + 4 * h + (r & 3);
      const int64_t gcol = n0 + 32 * wn + l32;
      if (grow < p.m && gcol < p.n) {
        const double s = sum[mi][r];
        float* dst = p.c + grow * p.ldc + gcol;
        float v = static_cast<float>(p.beta ? static_cast<double>(*dst) + s : s);
        if (p.epi == 1) v = v > 0.0f ? v : 0.0f;
        *dst = v;
      }
    }
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t mn = p.m * p.n;
  if (idx >= mn) return;
  // the splits' partials are added one by one in split order; the loads of eight splits are issued
  // together, so the sum waits for memory once per eight splits instead of once per split
  const double* src = p.ws + idx;
  double s = 0.0;
  int z = 0;
  for (; z + 8 <= p.splits; z += 8) {
    double t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = src[static_cast<int64_t>(z + u) * mn];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += t[u];
  }
  for (; z < p.splits; ++z) s += src[static_cast<int64_t>(z) * mn];
  const int64_t i = idx / p.n, j = idx % p.n;
  float* dst = p.c + i * p.ldc + j;
  float v = static_cast<float>(p.beta ? static_cast<double>(*dst) + s : s);
  if (p.epi == 1) v = v > 0.0f ? v : 0.0f;
  *dst = v;
}

template <int BN, bool TA, bool TB, bool MASK>
hipError_t launch_tiled(const GemmArgs& p, hipStream_t s) {
  const int64_t mb = (p.m + BM - 1) / BM, nb = (p.n + BN - 1) / BN;
  if ((mb + kXcds) * nb * (p.splits + kXcds) > int64_t(0x7FFFFFFF)) return hipErrorInvalidValue;   // grid size
  const dim3 grid(static_cast<unsigned>(mb), static_cast<unsigned>(nb), static_cast<unsigned>(p.splits));
  // the unsplit kernels run on a one-dimensional grid in the order described in gemm_kernel
  const dim3 grid1(static_cast<unsigned>(QHA_GEMM_ORDER == 2 ? (mb + kXcds - 1) / kXcds * kXcds * nb : mb * nb));
  const dim3 gridu = QHA_GEMM_ORDER > 0 ? grid1 : grid;
  const dim3 grids = QHA_GEMM_ORDER == 2 ? dim3(static_cast<unsigned>((p.splits + kXcds - 1) / kXcds * kXcds * mb * nb))
                                         : grid;
  if constexpr (!TA) {
    if (p.bsplit != nullptr && p.splits == 1) {
      const int64_t n_pad = (p.n + BN - 1) / BN * BN, k_pad = (p.k + BK - 1) / BK * BK;
      const int64_t pairs = n_pad * (k_pad / 2);
      hipLaunchKernelGGL(split_b_kernel, dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), 0, s, p.b,
                         p.ldb, p.tb, p.n, p.k, p.bsplit, n_pad, k_pad);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gemm_bsplit_kernel<BN, TA, MASK>), gridu, dim3(Tile<BN>::NT), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.splits > 1)
    hipLaunchKernelGGL((gemm_kernel<BN, TA, TB, MASK, true>), grids, dim3(Tile<BN>::NT), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BN, TA, TB, MASK, false>), gridu, dim3(Tile<BN>::NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits <= 1) return e;
  const int64_t mn = p.m * p.n;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(static_cast<unsigned>((mn + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool TA, bool TB, bool MASK>
hipError_t launch_variant(const GemmArgs& p, hipStream_t s) {
  // with B split once every width takes 128-wide tiles: the products whose wavefronts read B's
  // fragments from memory ran faster with four wavefronts per block than with eight sharing A's tile
  if (!TA && p.bsplit != nullptr && p.splits == 1) return launch_tiled<128, TA, TB, MASK>(p, s);
  return tile_n(p.n) == 256 ? launch_tiled<256, TA, TB, MASK>(p, s) : launch_tiled<128, TA, TB, MASK>(p, s);
}

}  // namespace

void gemm_split_rule(int64_t m, int64_t n, int64_t k, int32_t* splits, int64_t* k_per_split) {
  const int bn = tile_n(n);
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + bn - 1) / bn);
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

size_t gemm_bsplit_bytes(int32_t ta, int64_t m, int64_t n, int64_t k) {
  int32_t splits;
  int64_t kps;
  gemm_split_rule(m, n, k, &splits, &kps);
  if (ta || splits != 1 || m < kBSplitMinRows || n <= 0 || k <= 0) return 0;
  const int64_t bn = 128;   // the tile width of the products that read B split once
  return static_cast<size_t>(3 * ((n + bn - 1) / bn * bn) * ((k + BK - 1) / BK * BK) * 2);
}

hipError_t launch_gemm(const GemmArgs& p0, hipStream_t s) {
  if (p0.m == 0 || p0.n == 0) return hipSuccess;
  // k-major operands (and the mask beside A) are read with 32-bit buffer offsets when every one
  // of them spans less than 2 GiB
  GemmArgs p = p0;
  const int64_t lim = int64_t(1) << 31;
  bool fits = true;
  if (p.ta) fits = fits && p.k * p.lda * 4 < lim && (p.pro != 1 || p.k * p.ld_aux * 4 < lim);
  if (!p.tb) fits = fits && p.k * p.ldb * 4 < lim;
  p.buf32 = fits ? 1 : 0;
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
