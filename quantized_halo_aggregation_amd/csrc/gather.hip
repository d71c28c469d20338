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
// indices and edge weights are wavefront-uniform and live in scalar registers while a batch is
// summed.  A batch runs in phases:
// (1) vector loads of its inner rows, of its halo rows' code words (one word per lane holds all of
// its codes) and (min, scale) pairs, and of the next batch's column indices and edge weights (one
// edge per lane, read out with readlane when that batch starts), all in flight together; (2) the
// sums.  When the received buffer is
// grouped by width (the guide's section 9 packing), a halo row's code offset is arithmetic on its
// index -- its class comes from one ballot against the class starts held one per lane -- so the
// code load needs no earlier load; with a per-row offset table the code words are fetched in an
// extra phase once the offsets have arrived.  Row
// boundaries inside a group are tracked with scalar compares against the group's row pointers,
// held one per lane and read with readlane, so crossing a row costs a store and no load.
// A halo value is dequantised in float32 (scale * q + min, no contraction); every product is then
// accumulated in float64 (a float32 product is exact there, and MI355X issues float64 FMAs at the
// rate of unpacked float32 ones, so in this memory-bound loop the wider sum is free) and rounded
// to float32 once.  Chunks of a heavy row write float64 partial sums that a second kernel adds in
// chunk order, so results do not depend on scheduling.
// Gathers whose every column is a plain float row (the transposed passes, and forward calls
// without halo columns) run a leaner kernel: column indices and weights come by scalar loads, and
// rows by range-checked buffer loads at 32-bit offsets, whenever x spans less than 4 GiB.
#include "../../include/qha.h"
#include "qha_internal.hpp"
#include "quant_common.hpp"

// the dequantisation scale * q + min is two roundings, as the message format defines it
#pragma clang fp contract(off)

namespace qha {
namespace {

template <typename T>
using cptr = const __attribute__((address_space(4))) T*;

template <typename T>
__device__ __forceinline__ cptr<T> cst(const T* p) {
  return (cptr<T>)(p);
}

constexpr int vec_of(int D) { return D >= 64 ? D / 64 : 1; }
#ifndef QHA_BATCH
#define QHA_BATCH 16        // edges per batch of the inner-row gather
#endif
#ifndef QHA_HALO_BATCH
#define QHA_HALO_BATCH 8    // edges per batch when halo rows are dequantised too
#endif
#ifndef QHA_ROWS_KERNEL
#define QHA_ROWS_KERNEL 1
#endif
#ifndef QHA_ROWS_BATCH
#define QHA_ROWS_BATCH 16   // edges per batch of the plain-row gather at d <= 128 (8 KB in flight)
#endif
constexpr int rows_batch_of(int D) { return D >= 512 ? QHA_ROWS_BATCH / 4 : (D >= 256 ? QHA_ROWS_BATCH / 2 : QHA_ROWS_BATCH); }
constexpr int batch_of(int D, bool halo) { return D >= 512 ? 8 : (halo ? QHA_HALO_BATCH : QHA_BATCH); }
constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }

__device__ __forceinline__ int rdlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float rdlanef(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// scale * q + min with two roundings.  Written with plain operators under this file's contract(off):
// the header forms of __fmul_rn / __fadd_rn are plain operators compiled with contraction allowed,
// and once inlined their product and sum may be fused into one FMA.
__device__ __forceinline__ float dequant(float sc, uint32_t q, float zp) {
  const float t = sc * static_cast<float>(q);
  return t + zp;
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

// VEC floats from an address that is only 4-byte aligned (a raw halo row inside a packed buffer);
// global memory on gfx950 serves unaligned multi-dword loads.
template <int VEC>
__device__ __forceinline__ void load_row_unaligned(const float* p, float (&xv)[VEC]) {
  typedef float f2u __attribute__((ext_vector_type(2), aligned(4)));
  typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
  if constexpr (VEC == 1) {
    xv[0] = p[0];
  } else if constexpr (VEC == 2) {
    const f2u t = *reinterpret_cast<const f2u*>(p);
    xv[0] = t.x; xv[1] = t.y;
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const f4u t = reinterpret_cast<const f4u*>(p)[q];
      xv[4 * q + 0] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
    }
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

// Width and first code word of halo row k of a width-grouped buffer; the class table is held one
// class per lane (v_cstart: first row, INT_MAX past the last class), so the class is the number of
// lanes whose class starts at or before k, minus one.
template <int D>
__device__ __forceinline__ void class_of(int32_t v_cstart, int32_t v_cbits, uint32_t v_cbase, int32_t k, uint32_t& b,
                                         uint32_t& off) {
  const int c = __popcll(__ballot(v_cstart <= k)) - 1;
  b = static_cast<uint32_t>(rdlane(v_cbits, c));
  const uint32_t words = (b == 32u) ? static_cast<uint32_t>(D) : (((b << log2i(D)) + 31u) >> 5);
  off = static_cast<uint32_t>(rdlane(static_cast<int>(v_cbase), c)) + static_cast<uint32_t>(k - rdlane(v_cstart, c)) * words;
}

// Quantises output row k of a gather, held VEC features per lane (lane l owns features l*VEC ..,
// idle lanes of narrow rows shadow lane 0), with the arithmetic of quantize_pack_kernel: exact
// row min / max, one Philox call per group of 8 features, codes packed least-significant first
// and the pieces of lanes that share a word merged with lane shuffles.  Every lane must call it.
template <int D>
__device__ __forceinline__ void quantize_out_row(const QuantOut& q, int64_t k, const float (&v)[vec_of(D)], int lane,
                                                 int j0, bool owner) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  uint32_t b, off;
  if (q.cls.n > 0) {
    int32_t st = q.cls.start[0];
    uint32_t base = q.cls.base[0];
    b = static_cast<uint32_t>(q.cls.bits[0]);
#pragma unroll
    for (int c = 1; c < kMaxClasses; ++c) {
      if (c < q.cls.n && k >= q.cls.start[c]) {
        st = q.cls.start[c];
        base = q.cls.base[c];
        b = static_cast<uint32_t>(q.cls.bits[c]);
      }
    }
    const uint32_t words = (b == 32u) ? static_cast<uint32_t>(D) : (b * static_cast<uint32_t>(D) + 31u) >> 5;
    off = base + static_cast<uint32_t>(k - st) * words;
  } else {
    b = q.bits[k];
    off = q.word_offset[k];
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < VEC; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (!width_valid(b)) return;              // a row of an unknown width is left untouched
  uint32_t* row = q.codes + off;
  if (b == 32u) {
    if (owner) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) row[j0 + i] = __float_as_uint(v[i]);
    }
    if (lane == 0) *reinterpret_cast<float2*>(q.meta + 2 * k) = make_float2(0.0f, 0.0f);
    return;
  }
  const RowScale rs = row_scale(mn, mx, b);
  uint32_t c0 = q.node_base + static_cast<uint32_t>(k);
  uint32_t c1 = static_cast<uint32_t>(j0 >> 3);
  uint32_t c2 = q.epoch;
  uint32_t c3 = q.stream_id;
  philox4x32_10(c0, c1, c2, c3, q.seed_lo, q.seed_hi);
  const uint32_t w[4] = {c0, c1, c2, c3};
  uint64_t piece = 0;
#pragma unroll
  for (int i = 0; i < VEC; ++i)
    piece |= static_cast<uint64_t>(code_of(v[i], mn, rs, draw16(w, j0 + i))) << (static_cast<uint32_t>(i) * b);
  const uint32_t lane_bits = static_cast<uint32_t>(VEC) * b;
  const uint32_t first = (static_cast<uint32_t>(j0) * b) >> 5;
  if (lane_bits <= 32u) {
    uint32_t word = static_cast<uint32_t>(piece) << ((static_cast<uint32_t>(j0) * b) & 31u);
    const uint32_t share = 32u / lane_bits;          // lanes whose pieces fill one word
    for (uint32_t o = 1; o < share; o <<= 1) word |= __shfl_xor(word, static_cast<int>(o));
    if (owner && (static_cast<uint32_t>(lane) & (share - 1u)) == 0u) row[first] = word;
  } else {
    if (owner) {
      row[first] = static_cast<uint32_t>(piece);
      row[first + 1] = static_cast<uint32_t>(piece >> 32);
    }
  }
  if (lane == 0) *reinterpret_cast<float2*>(q.meta + 2 * k) = make_float2(rs.zp, rs.sc);
}

template <int D, bool HALO, bool BETA, bool GROUPED, bool QUANT>
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

  // the group's row ends and output rows, one row per lane (rows of a group are never empty, so
  // each edge closes at most one row)
  const int li = lane < nrows ? lane : nrows - 1;
  const int32_t v_end = split ? 0x7FFFFFFF : a.rowptr[row0 + li + 1];
  const int32_t v_out = (a.row_ids != nullptr) ? a.row_ids[row0 + li] : row0 + li;

  // width classes of a grouped halo buffer, class i in lane i
  int32_t v_cstart = 0x7FFFFFFF, v_cbits = 0;
  uint32_t v_cbase = 0;
  if constexpr (HALO && GROUPED) {
#pragma unroll
    for (int c = 0; c < kMaxClasses; ++c) {
      if (lane == c && c < a.cls.n) {
        v_cstart = a.cls.start[c];
        v_cbits = a.cls.bits[c];
        v_cbase = a.cls.base[c];
      }
    }
  }

  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
  int cur = 0;                                  // row of the group being summed
  int32_t cur_end = rdlane(v_end, 0);

  auto flush = [&]() {                          // write row `cur` and start the next one
    const int64_t orow = rdlane(v_out, cur);
    if constexpr (QUANT) {
      float res[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
      quantize_out_row<D>(a.q, orow, res, lane, j0, owner);
    } else if (owner) {
      float* dst = a.out + orow * a.ldo + j0;
      float res[VEC];
      if constexpr (BETA) {
        float old[VEC];
        load_row<VEC>(dst, old);
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(static_cast<double>(old[v]) + acc[v]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
      }
      store_row<VEC>(dst, res);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
    ++cur;
    cur_end = rdlane(v_end, cur < nrows ? cur : nrows - 1);
  };

  // the next batch's column indices and weights, edge i of the batch in lane i (vector loads, so
  // the prefetch holds no scalar registers)
  int32_t v_u = 0;
  float v_w = 1.0f;
  const bool weighted = a.w != nullptr;
  auto fetch = [&](int32_t eb) {
    const int32_t ei = min(eb + lane, e1 - 1);
    v_u = a.colidx[ei];
    if (weighted) v_w = a.w[ei];
  };
  if (e0 < e1) fetch(e0);

  for (int32_t e = e0; e < e1; e += B) {
    int32_t u[B];
    float ww[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      u[i] = rdlane(v_u, i);
      ww[i] = rdlanef(v_w, i);
    }

    if constexpr (HALO && GROUPED) {
      // batch set-up, vectorised over the batch's edges (edge i in lane i): each edge's class,
      // width and code offset, and the two addresses its loads will use -- the value (an inner
      // row, the raw floats of a 32-bit halo row, or for a quantised halo row its (min, scale) pair
      // when each lane holds two features) and the code word row (the first word of the buffer for
      // edges without codes).
      constexpr bool META_IN_XV = VEC == 2;
      const int32_t vk = v_u - static_cast<int32_t>(a.n_inner);
      const bool vh = vk >= 0;
      uint32_t vb = 0, vst = 0, vcb = 0;
#pragma unroll
      for (int c = 0; c < kMaxClasses; ++c) {
        if (c < a.cls.n && vk >= a.cls.start[c]) {
          vb = static_cast<uint32_t>(a.cls.bits[c]);
          vst = static_cast<uint32_t>(a.cls.start[c]);
          vcb = a.cls.base[c];
        }
      }
      const bool vq = vh && vb != 32u;                           // a quantised halo row
      const uint32_t vlgb = vq ? static_cast<uint32_t>(__builtin_ctz(vb)) : 0u;
      // words per row, a power of two: ceil(d*b/32) for codes (d = 16 with 1-bit codes fills half a
      // word), d for raw rows
      const uint32_t vlgdb = static_cast<uint32_t>(log2i(D)) + vlgb;
      const uint32_t vlgw = (vb == 32u) ? static_cast<uint32_t>(log2i(D)) : (vlgdb > 5u ? vlgdb - 5u : 0u);
      const uint32_t voff = vh ? vcb + ((static_cast<uint32_t>(vk) - vst) << vlgw) : 0u;
      const uint64_t vval = !vh ? reinterpret_cast<uint64_t>(a.x + static_cast<int64_t>(v_u) * a.ldx)
                          : (vq && META_IN_XV) ? reinterpret_cast<uint64_t>(a.meta + 2 * static_cast<int64_t>(vk))
                                               : reinterpret_cast<uint64_t>(a.codes + voff);
      const uint64_t vcode = reinterpret_cast<uint64_t>(a.codes + (vq ? voff : 0u));
      const uint64_t vmeta = reinterpret_cast<uint64_t>(a.meta + 2 * static_cast<int64_t>(vq ? vk : 0));
      const uint32_t vkind = vq ? vb : (vh ? 32u : 0u);          // 0: inner, 32: raw halo, else width

      // phase 1: per edge, two (three when d >= 256) loads from the prepared addresses
      float xv[B][VEC];
      float2 mp[B];
      uint32_t cwd[B][CW];
      uint32_t kind[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        kind[i] = static_cast<uint32_t>(rdlane(static_cast<int>(vkind), i));
        const bool q = kind[i] != 0u && kind[i] != 32u;
        const uint64_t va = (static_cast<uint64_t>(static_cast<uint32_t>(rdlane(static_cast<int>(vval >> 32), i))) << 32) |
                            static_cast<uint32_t>(rdlane(static_cast<int>(vval), i));
        load_row_unaligned<VEC>(reinterpret_cast<const float*>(va) + (q ? 0 : j0), xv[i]);
        if constexpr (!META_IN_XV) {
          const uint64_t ma = (static_cast<uint64_t>(static_cast<uint32_t>(rdlane(static_cast<int>(vmeta >> 32), i))) << 32) |
                              static_cast<uint32_t>(rdlane(static_cast<int>(vmeta), i));
          mp[i] = *reinterpret_cast<const float2*>(ma);
        }
        const uint64_t ca = (static_cast<uint64_t>(static_cast<uint32_t>(rdlane(static_cast<int>(vcode >> 32), i))) << 32) |
                            static_cast<uint32_t>(rdlane(static_cast<int>(vcode), i));
        const uint32_t lgb = static_cast<uint32_t>(rdlane(static_cast<int>(vlgb), i));
        const uint32_t* crow = reinterpret_cast<const uint32_t*>(ca);
        const uint32_t cw0 = q ? ((static_cast<uint32_t>(j0) << lgb) >> 5) : 0u;
        cwd[i][0] = crow[cw0];
        if (CW == 2) cwd[i][CW - 1] = crow[cw0 + ((q && kind[i] * VEC > 32u) ? 1u : 0u)];
      }
      if (e + B < e1) fetch(e + B);
      // phase 2: dequantise and sum, closing the row whose last edge this is
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int32_t p = e + i;
        if (p < e1) {
          const double wt = static_cast<double>(ww[i]);
          const uint32_t b = kind[i];
          float val[VEC];
          if (b != 0u && b != 32u) {
            const float mn = META_IN_XV ? xv[i][0] : mp[i].x;
            const float sc = META_IN_XV ? xv[i][1 % VEC] : mp[i].y;
            const uint32_t mask = (1u << b) - 1u;
            const uint32_t sh = (static_cast<uint32_t>(j0) << __builtin_ctz(b)) & 31u;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const uint32_t bitpos = sh + static_cast<uint32_t>(v) * b;
              const uint32_t wd = (CW == 2 && bitpos >= 32u) ? (cwd[i][CW - 1] >> (bitpos - 32u)) : (cwd[i][0] >> bitpos);
              val[v] = dequant(sc, wd & mask, mn);
            }
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) val[v] = xv[i][v];
          }
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(val[v]), acc[v]);
          if (p + 1 == cur_end) flush();
        }
      }
    } else {
      // phase 1: inner rows (and with a per-row offset table: the halo rows' widths, offsets and
      // (min, scale) pairs)
      float xv[B][VEC];
      float2 ms[B];
      uint32_t cwd[B][CW];
      uint32_t woff[B], bw[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        if (HALO && u[i] >= a.n_inner) {
          const int32_t k = u[i] - static_cast<int32_t>(a.n_inner);
          woff[i] = cst(a.word_offset)[k];
          if constexpr (D >= 32) {
            // the width follows from the row's word count (unique for d >= 32)
            bw[i] = ((cst(a.word_offset)[k + 1] - woff[i]) << 5) >> log2i(D);
          } else {
            bw[i] = cst(a.bits)[k];
          }
          ms[i] = *reinterpret_cast<const float2*>(a.meta + 2 * static_cast<int64_t>(k));
        } else {
          load_row<VEC>(a.x + static_cast<int64_t>(u[i]) * a.ldx + j0, xv[i]);
        }
      }
      if (e + B < e1) fetch(e + B);
      // phase 2: the code words of the halo rows, once their offsets are in
      if constexpr (HALO) {
#pragma unroll
        for (int i = 0; i < B; ++i) {
          if (u[i] >= a.n_inner) {
            const uint32_t b = bw[i];
            const uint32_t* row = a.codes + woff[i];
            if (b == 32u) {
#pragma unroll
              for (int v = 0; v < VEC; ++v) xv[i][v] = __uint_as_float(row[j0 + v]);
            } else if (width_valid(b)) {
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
          const double wt = static_cast<double>(ww[i]);
          if (HALO && u[i] >= a.n_inner && bw[i] != 32u) {
            const uint32_t b = bw[i];
            float q[VEC];
            if (width_valid(b)) {
              const uint32_t mask = (1u << b) - 1u;
              const uint32_t sh = (static_cast<uint32_t>(j0) * b) & 31u;
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                const uint32_t bitpos = sh + static_cast<uint32_t>(v) * b;
                const uint32_t wd = (CW == 2 && bitpos >= 32u) ? (cwd[i][CW - 1] >> (bitpos - 32u)) : (cwd[i][0] >> bitpos);
                q[v] = dequant(ms[i].y, wd & mask, ms[i].x);
              }
            } else {
#pragma unroll
              for (int v = 0; v < VEC; ++v) q[v] = 0.0f;
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(q[v]), acc[v]);
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(xv[i][v]), acc[v]);
          }
          if (p + 1 == cur_end) flush();
        }
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

// VEC floats of one row by a range-checked buffer load (a lane past the buffer's end reads 0).
template <int VEC>
__device__ __forceinline__ void buffer_row(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&xv)[VEC]) {
  const int o = static_cast<int>(off);
  if constexpr (VEC == 1) {
    xv[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0));
  } else if constexpr (VEC == 2) {
    const auto t = __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
    xv[0] = __uint_as_float(t[0]);
    xv[1] = __uint_as_float(t[1]);
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(r, o + 16 * q, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) xv[4 * q + c] = __uint_as_float(t[c]);
    }
  }
}

constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw 32-bit buffer, range-checked against num_records

// Gather of plain float rows (every column is a row of x: the transposed gathers, and forward
// gathers without halo columns).  A batch's B column indices and edge weights are read by scalar
// loads straight into scalar registers, so no lane-to-scalar moves are needed and the wait for them
// does not include the wavefront's earlier row stores; each row load is a buffer load whose offset
// (column * row pitch + the lane's features) is 32-bit and range-checked by the hardware.
template <int D, bool BETA>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  constexpr int B = rows_batch_of(D);
  const int lane = threadIdx.x & 63;
  const int j0 = (G == 64 ? lane : (lane < G ? lane : 0)) * VEC;
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
  const int li = lane < nrows ? lane : nrows - 1;
  const int32_t v_end = split ? 0x7FFFFFFF : a.rowptr[row0 + li + 1];
  const int32_t v_out = (a.row_ids != nullptr) ? a.row_ids[row0 + li] : row0 + li;

  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.x), static_cast<short>(0), static_cast<int>(a.x_bytes),
                                        static_cast<int>(kBufferWord3));
  const uint32_t pitch = static_cast<uint32_t>(a.ldx) * 4u;
  const uint32_t lane_off = static_cast<uint32_t>(j0) * 4u;
  cptr<int32_t> ci = cst(a.colidx);
  cptr<float> cw = cst(a.w);
  const bool weighted = a.w != nullptr;

  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
  int cur = 0;
  int32_t cur_end = rdlane(v_end, 0);
  auto flush = [&]() {
    const int64_t orow = rdlane(v_out, cur);
    if (owner) {
      float* dst = a.out + orow * a.ldo + j0;
      float res[VEC];
      if constexpr (BETA) {
        float old[VEC];
        load_row<VEC>(dst, old);
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(static_cast<double>(old[v]) + acc[v]);
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
      }
      store_row<VEC>(dst, res);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
    ++cur;
    cur_end = rdlane(v_end, cur < nrows ? cur : nrows - 1);
  };

  for (int32_t e = e0; e < e1; e += B) {
    int32_t u[B];
    float ww[B];
    if (e + B <= e1) {
#pragma unroll
      for (int i = 0; i < B; ++i) u[i] = ci[e + i];
      if (weighted) {
#pragma unroll
        for (int i = 0; i < B; ++i) ww[i] = cw[e + i];
      } else {
#pragma unroll
        for (int i = 0; i < B; ++i) ww[i] = 1.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int32_t ei = min(e + i, e1 - 1);
        u[i] = ci[ei];
        ww[i] = weighted ? cw[ei] : 1.0f;
      }
    }
    float xv[B][VEC];
#pragma unroll
    for (int i = 0; i < B; ++i) buffer_row<VEC>(xr, static_cast<uint32_t>(u[i]) * pitch + lane_off, xv[i]);
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int32_t p = e + i;
      if (p < e1) {
        const double wt = static_cast<double>(ww[i]);
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(xv[i][v]), acc[v]);
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
    flush();
  }
}

// Adds the partial sums of every split row in chunk order and writes (or quantises) the row.
template <int D, bool QUANT>
__global__ __launch_bounds__(256) void combine_split_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 4 +
                    __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (m >= a.n_split_rows) return;
  const bool owner = lane < G;
  const int j0 = (owner ? lane : 0) * VEC;          // idle lanes shadow lane 0
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
  const int64_t orow = a.row_ids ? a.row_ids[row] : row;
  if constexpr (QUANT) {
    float res[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
    quantize_out_row<D>(a.q, orow, res, lane, j0, owner);
  } else if (owner) {
    float* dst = a.out + orow * a.ldo + j0;
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      dst[v] = static_cast<float>(a.beta ? static_cast<double>(dst[v]) + acc[v] : acc[v]);
  }
}

__global__ __launch_bounds__(256) void edge_weights_kernel(int64_t n_rows, const int32_t* rowptr,
                                                           const int32_t* colidx, const float* r, const float* c,
                                                           float* w) {
  // one wavefront per row: the row factor is read once, the column factors are gathered
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 +
                      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  if (row >= n_rows) return;
  const int lane = threadIdx.x & 63;
  const float rf = r ? r[row] : 1.0f;
  for (int32_t e = rowptr[row] + lane; e < rowptr[row + 1]; e += 64)
    w[e] = __fmul_rn(rf, c ? c[colidx[e]] : 1.0f);
}

template <int D, bool HALO, bool BETA>
void launch_variant(const GatherArgs& a, dim3 grid, hipStream_t s) {
  if (HALO && a.cls.n > 0)
    hipLaunchKernelGGL((gather_kernel<D, HALO, BETA, true, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gather_kernel<D, HALO, BETA, false, false>), grid, dim3(256), 0, s, a);
}

template <int D>
hipError_t launch_gather_d(const GatherArgs& a, bool with_halo, bool quantize_out, hipStream_t s) {
  // the plain-row kernel addresses x with 32-bit byte offsets
  const int64_t x_bytes = a.n_inner > 0 ? ((a.n_inner - 1) * a.ldx + D) * 4 : 0;
  const bool rows_ok = x_bytes <= static_cast<int64_t>(0xFFFFFFFFu) && QHA_ROWS_KERNEL;

  if (a.n_items > 0) {
    const dim3 grid(static_cast<unsigned>((a.n_items + 3) / 4));
    if (quantize_out) {
      hipLaunchKernelGGL((gather_kernel<D, false, false, false, true>), grid, dim3(256), 0, s, a);
    } else if (with_halo) {
      if (a.beta) launch_variant<D, true, true>(a, grid, s);
      else launch_variant<D, true, false>(a, grid, s);
    } else if (rows_ok) {
      GatherArgs r = a;
      r.x_bytes = static_cast<uint32_t>(x_bytes);
      if (a.beta) hipLaunchKernelGGL((gather_rows_kernel<D, true>), grid, dim3(256), 0, s, r);
      else hipLaunchKernelGGL((gather_rows_kernel<D, false>), grid, dim3(256), 0, s, r);
    } else {
      if (a.beta) launch_variant<D, false, true>(a, grid, s);
      else launch_variant<D, false, false>(a, grid, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_split_rows > 0) {
    const int64_t blocks = (a.n_split_rows + 3) / 4;
    if (quantize_out)
      hipLaunchKernelGGL((combine_split_kernel<D, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((combine_split_kernel<D, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int32_t d, bool with_halo, hipStream_t s, bool quantize_out) {
  switch (d) {
    case 16: return launch_gather_d<16>(a, with_halo, quantize_out, s);
    case 32: return launch_gather_d<32>(a, with_halo, quantize_out, s);
    case 64: return launch_gather_d<64>(a, with_halo, quantize_out, s);
    case 128: return launch_gather_d<128>(a, with_halo, quantize_out, s);
    case 256: return launch_gather_d<256>(a, with_halo, quantize_out, s);
    case 512: return launch_gather_d<512>(a, with_halo, quantize_out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_edge_weights(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* r,
                               const float* c, float* w, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(edge_weights_kernel, dim3(static_cast<unsigned>((n_rows + 3) / 4)), dim3(256), 0, s, n_rows,
                     rowptr, colidx, r, c, w);
  return hipGetLastError();
}

}  // namespace qha
