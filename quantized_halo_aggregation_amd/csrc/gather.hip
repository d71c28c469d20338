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
// Three kernels share this scheme.  gather_rows_kernel serves gathers whose every column is a
// plain float row (the transposed passes, forward calls without halo columns): column indices and
// weights come by scalar loads, rows by range-checked buffer loads at 32-bit offsets.
// gather_grouped_kernel serves halo gathers over a width-grouped message: per-edge set-up is
// lane-parallel, and when x, the codes and the (min, scale) pairs lie within 4 GiB of one base
// every load is that base plus a 32-bit offset, so an edge costs no scalar selects.  gather_kernel
// is the general form: per-row offset tables, 64-bit addresses, and the fused quantising epilogue.
#include "../../include/qha.h"
#include "qha_internal.hpp"
#include "quant_common.hpp"

#include <mutex>
#include <type_traits>

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
#ifndef QHA_HALO_BATCH_128
#define QHA_HALO_BATCH_128 16   // the grouped gather's at d = 128, whose one load form keeps 16 edges in 70 VGPRs
#endif
#ifndef QHA_SINGLE_BASE
#define QHA_SINGLE_BASE 1
#endif
#ifndef QHA_GROUPED_KERNEL
#define QHA_GROUPED_KERNEL 1
#endif
#ifndef QHA_ROWS_KERNEL
#define QHA_ROWS_KERNEL 1
#endif
#ifndef QHA_ROWS_BATCH
#define QHA_ROWS_BATCH 16   // edges per batch of the plain-row gather at d <= 128 (8 KB in flight)
#endif
constexpr int rows_batch_of(int D) { return D >= 512 ? QHA_ROWS_BATCH / 4 : (D >= 256 ? QHA_ROWS_BATCH / 2 : QHA_ROWS_BATCH); }
constexpr int batch_of(int D, bool halo) { return D >= 512 ? 8 : (halo ? QHA_HALO_BATCH : QHA_BATCH); }
// the width-grouped halo gather's batch
constexpr int grouped_batch_of(int D) { return D == 128 ? QHA_HALO_BATCH_128 : batch_of(D, true); }
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

// Quantises message row k of a gather, held VEC features per lane (lane l owns features l*VEC ..,
// idle lanes of narrow rows shadow lane 0), with the arithmetic of quantize_pack_kernel: exact row
// min / max, the lane's rounding draws taken from the four words w of its group's Philox call,
// codes packed least-significant first and the pieces of lanes that share a word merged with lane
// shuffles.  Every lane must call it.
// Cross-lane steps of a message row's coding by DPP within each row of 16 lanes: quad permutes
// for lanes 1 and 2 apart, then the mirrored lane of the half row and of the row (after the quad
// steps every lane of a quad holds its quad's value, so a mirror pairs the two quads, then the two
// halves).  They replace LDS-routed lane shuffles, which the coding of every row would wait for.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Exact min and max over the wavefront's 64 lanes (idle lanes shadow lane 0, so they do not change
// them): DPP within each row of 16 lanes, then the four rows' results read out.
__device__ __forceinline__ void wave_min_max(float& mn, float& mx) {
#define QHA_MM_STEP(C)                                              \
  mn = fminf(mn, __uint_as_float(dpp_u<C>(__float_as_uint(mn)))); \
  mx = fmaxf(mx, __uint_as_float(dpp_u<C>(__float_as_uint(mx))));
  QHA_MM_STEP(kDppXor1)
  QHA_MM_STEP(kDppXor2)
  QHA_MM_STEP(kDppHalfMirror)
  QHA_MM_STEP(kDppMirror)
#undef QHA_MM_STEP
  mn = fminf(fminf(rdlanef(mn, 0), rdlanef(mn, 16)), fminf(rdlanef(mn, 32), rdlanef(mn, 48)));
  mx = fmaxf(fmaxf(rdlanef(mx, 0), rdlanef(mx, 16)), fmaxf(rdlanef(mx, 32), rdlanef(mx, 48)));
}

// OR of the disjoint code pieces of each aligned group of `share` lanes (1 .. 32), left in every
// lane of the group.
__device__ __forceinline__ uint32_t group_or(uint32_t w, uint32_t share) {
  if (share >= 2u) w |= dpp_u<kDppXor1>(w);
  if (share >= 4u) w |= dpp_u<kDppXor2>(w);
  if (share >= 8u) w |= dpp_u<kDppHalfMirror>(w);
  if (share >= 16u) w |= dpp_u<kDppMirror>(w);
  if (share >= 32u) w |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(w), 16));
  return w;
}

// Width and first code word of message row k (of a buffer the gather writes, or of a received one),
// from the width classes (scalar compares) or the per-row arrays.
template <int D, typename M>
__device__ __forceinline__ void message_row_layout(const M& q, int64_t k, uint32_t& b, uint32_t& off) {
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
}

// The width classes held one per lane (class c in lane lane0 + c), for kernels that look rows up
// inside a loop: a lookup then costs a few lane reads instead of scalar registers kept live through
// it.  Two tables can share the registers (the second in lanes 8 ..), each seen through its own view.
struct LaneClasses {
  int32_t start = 0x7FFFFFFF, bits = 0;
  uint32_t base = 0;
  int n = 0;
  int lane0 = 0;
};

__device__ __forceinline__ LaneClasses lane_classes(const Classes& cls, int lane) {
  LaneClasses c;
  c.n = cls.n;
#pragma unroll
  for (int i = 0; i < kMaxClasses; ++i) {
    if (lane == i && i < cls.n) {
      c.start = cls.start[i];
      c.bits = cls.bits[i];
      c.base = cls.base[i];
    }
  }
  return c;
}

// Table `second` put in lanes kMaxClasses .. of the registers holding `first` (lane_classes(first));
// the result is the view of the second table.
__device__ __forceinline__ LaneClasses lane_classes_beside(const LaneClasses& first, const Classes& second,
                                                          int lane) {
  LaneClasses c = first;
  c.n = second.n;
  c.lane0 = kMaxClasses;
#pragma unroll
  for (int i = 0; i < kMaxClasses; ++i) {
    if (lane == kMaxClasses + i && i < second.n) {
      c.start = second.start[i];
      c.bits = second.bits[i];
      c.base = second.base[i];
    }
  }
  return c;
}

template <int D, typename M>
__device__ __forceinline__ void message_row_layout(const M& q, const LaneClasses& lc, int64_t k, uint32_t& b,
                                                   uint32_t& off) {
  if (lc.n > 0) {
    int32_t st = rdlane(lc.start, lc.lane0);
    int32_t bb = rdlane(lc.bits, lc.lane0);
    uint32_t base = static_cast<uint32_t>(rdlane(static_cast<int>(lc.base), lc.lane0));
    for (int c = 1; c < lc.n; ++c) {
      const int32_t sc = rdlane(lc.start, lc.lane0 + c);
      if (k >= sc) {                                   // k and the class starts are uniform
        st = sc;
        bb = rdlane(lc.bits, lc.lane0 + c);
        base = static_cast<uint32_t>(rdlane(static_cast<int>(lc.base), lc.lane0 + c));
      }
    }
    b = static_cast<uint32_t>(bb);
    const uint32_t words = (b == 32u) ? static_cast<uint32_t>(D) : (b * static_cast<uint32_t>(D) + 31u) >> 5;
    off = base + static_cast<uint32_t>(k - st) * words;
  } else {
    b = q.bits[k];
    off = q.word_offset[k];
  }
}

// Quantises message row k of a gather (width b, codes from word off), held VEC features per lane
// (lane l owns features l*VEC .., idle lanes of narrow rows shadow lane 0), with the arithmetic of
// quantize_pack_kernel: exact row min / max, the lane's rounding draws taken from the four words w
// of its group's Philox call, codes packed least-significant first and the pieces of lanes that
// share a word merged with lane shuffles.  Every lane must call it.
template <int D>
__device__ __forceinline__ void quantize_row_with_draws(const QuantOut& q, int64_t k, uint32_t b, uint32_t off,
                                                        const float (&v)[vec_of(D)], int lane, int j0, bool owner,
                                                        const uint32_t (&w)[4]) {
  constexpr int VEC = vec_of(D);
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < VEC; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  wave_min_max(mn, mx);
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
  uint64_t piece = 0;
#pragma unroll
  for (int i = 0; i < VEC; ++i)
    piece |= static_cast<uint64_t>(code_of(v[i], mn, rs, draw16_c(w, j0 + i))) << (static_cast<uint32_t>(i) * b);
  const uint32_t lane_bits = static_cast<uint32_t>(VEC) * b;
  const uint32_t first = (static_cast<uint32_t>(j0) * b) >> 5;
  if (lane_bits <= 32u) {
    uint32_t word = static_cast<uint32_t>(piece) << ((static_cast<uint32_t>(j0) * b) & 31u);
    const uint32_t share = 32u / lane_bits;          // lanes whose pieces fill one word
    word = group_or(word, share);
    if (owner && (static_cast<uint32_t>(lane) & (share - 1u)) == 0u) row[first] = word;
  } else {
    if (owner) {
      row[first] = static_cast<uint32_t>(piece);
      row[first + 1] = static_cast<uint32_t>(piece >> 32);
    }
  }
  if (lane == 0) *reinterpret_cast<float2*>(q.meta + 2 * k) = make_float2(rs.zp, rs.sc);
}

// The same, drawing the lane's Philox call for row k itself (counter: node id, the lane's group).
template <int D>
__device__ __forceinline__ void quantize_out_row(const QuantOut& q, int64_t k, const float (&v)[vec_of(D)], int lane,
                                                 int j0, bool owner) {
  uint32_t c0 = q.node_base + static_cast<uint32_t>(k);
  uint32_t c1 = static_cast<uint32_t>(j0 >> 3);
  uint32_t c2 = q.epoch;
  uint32_t c3 = q.stream_id;
  philox4x32_10(c0, c1, c2, c3, q.seed_lo, q.seed_hi);
  const uint32_t w[4] = {c0, c1, c2, c3};
  uint32_t b, off;
  message_row_layout<D>(q, k, b, off);
  quantize_row_with_draws<D>(q, k, b, off, v, lane, j0, owner, w);
}

// Rounding draws of 512 / D consecutive message rows from one Philox call per lane: lane l holds the
// call of row k0 + l / (D / 8), group l % (D / 8).  A gather that codes the consecutive rows of a
// work item one after another pays one call per lane for several rows instead of one per row.
struct DrawCache {
  uint32_t w[4];
  int64_t k0 = -(int64_t(1) << 62);     // no batch yet: every row is outside it
};

template <int D>
__device__ __forceinline__ void draws_of_row(const QuantOut& q, DrawCache& dc, int64_t k, int lane, int j0,
                                             uint32_t (&w)[4]) {
  constexpr int GPR = D / 8;                // Philox groups per row
  constexpr int RB = 64 / GPR;              // rows per batch
  if (k < dc.k0 || k >= dc.k0 + RB) {       // k is wavefront-uniform
    dc.k0 = k;
    uint32_t c0 = q.node_base + static_cast<uint32_t>(k + lane / GPR);
    uint32_t c1 = static_cast<uint32_t>(lane % GPR);
    uint32_t c2 = q.epoch;
    uint32_t c3 = q.stream_id;
    philox4x32_10(c0, c1, c2, c3, q.seed_lo, q.seed_hi);
    dc.w[0] = c0;
    dc.w[1] = c1;
    dc.w[2] = c2;
    dc.w[3] = c3;
  }
  const int src = static_cast<int>(k - dc.k0) * GPR + (j0 >> 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = static_cast<uint32_t>(__shfl(static_cast<int>(dc.w[i]), src));
}

// ---- received messages added to stored rows (the receiver's "dequantise and continue backward",
// guide section 11, folded into the gather that stores the rows) ----

// Width and first code word of message row k held per lane (k < 0: no row, b = 0), with the
// classes held one per lane: the received rows of a work item's stored rows, looked up once when
// the item starts.
template <int D, typename M>
__device__ __forceinline__ void lane_row_layout(const M& q, const LaneClasses& lc, int32_t k, uint32_t& b,
                                                uint32_t& off) {
  b = 0u;
  off = 0u;
  if (lc.n > 0) {
    int32_t st = rdlane(lc.start, lc.lane0);
    int32_t bb = rdlane(lc.bits, lc.lane0);
    uint32_t base = static_cast<uint32_t>(rdlane(static_cast<int>(lc.base), lc.lane0));
    for (int c = 1; c < lc.n; ++c) {
      const int32_t sc = rdlane(lc.start, lc.lane0 + c);
      const int32_t bc = rdlane(lc.bits, lc.lane0 + c);
      const uint32_t basec = static_cast<uint32_t>(rdlane(static_cast<int>(lc.base), lc.lane0 + c));
      if (k >= sc) {                                   // per lane
        st = sc;
        bb = bc;
        base = basec;
      }
    }
    if (k >= 0) {
      b = static_cast<uint32_t>(bb);
      const uint32_t words = (b == 32u) ? static_cast<uint32_t>(D) : (b * static_cast<uint32_t>(D) + 31u) >> 5;
      off = base + static_cast<uint32_t>(k - st) * words;
    }
  } else if (k >= 0) {
    b = q.bits[k];
    off = q.word_offset[k];
  }
}

// The lane's code words of message row (b, off), both wavefront-uniform: its VEC raw floats for
// b = 32, else the one or two words holding its VEC codes.
template <int VEC>
__device__ __forceinline__ void fetch_codes(const uint32_t* codes, uint32_t b, uint32_t off, int j0,
                                            uint32_t (&wd)[VEC]) {
  const uint32_t* row = codes + off;
  if (b == 32u) {
    float t[VEC];
    load_row_unaligned<VEC>(reinterpret_cast<const float*>(row + j0), t);
#pragma unroll
    for (int v = 0; v < VEC; ++v) wd[v] = __float_as_uint(t[v]);
  } else if (width_valid(b)) {
    const uint32_t pos = static_cast<uint32_t>(j0) * b;
    wd[0] = row[pos >> 5];
    if constexpr (VEC * 8 > 32) wd[1] = (b * VEC > 32u) ? row[(pos >> 5) + 1] : 0u;
  }
}

// The lane's VEC features of a message row from its code words: scale * q + min (the raw float for
// b = 32; 0 for a width outside {1, 2, 4, 8, 32}).
template <int VEC>
__device__ __forceinline__ void dequant_lane(uint32_t b, float zp, float sc, int j0, const uint32_t (&wd)[VEC],
                                             float (&q)[VEC]) {
  if (b == 32u) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = __uint_as_float(wd[v]);
  } else if (width_valid(b)) {
    const uint32_t mask = (1u << b) - 1u;
    const uint32_t sh = (static_cast<uint32_t>(j0) * b) & 31u;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const uint32_t bit = sh + static_cast<uint32_t>(v) * b;
      uint32_t word = wd[0] >> (bit & 31u);
      if constexpr (VEC * 8 > 32) {
        if (bit >= 32u) word = wd[1] >> (bit - 32u);
      }
      q[v] = dequant(sc, word & mask, zp);
    }
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v) q[v] = 0.0f;
  }
}

// racc += the lane's features of the dequantised received rows idx[p0 .. p1), in list order, each
// added in float64 as the neighbour gather adds a halo row of weight 1 (the list is
// wavefront-uniform; rows are looked up as they come).
template <int D>
__device__ __forceinline__ void add_received_rows(const RecvAdd& r, const LaneClasses& lr, int32_t p0, int32_t p1,
                                                  int j0, double (&racc)[vec_of(D)]) {
  constexpr int VEC = vec_of(D);
  for (int32_t i = p0; i < p1; ++i) {
    const int32_t k = cst(r.idx)[i];
    uint32_t b, off;
    message_row_layout<D>(r, lr, k, b, off);
    cptr<float> m = cst(r.meta) + 2 * static_cast<int64_t>(k);
    const float zp = m[0], sc = m[1];
    uint32_t wd[VEC];
    fetch_codes<VEC>(r.codes, b, off, j0, wd);
    float q[VEC];
    dequant_lane<VEC>(b, zp, sc, j0, wd, q);
#pragma unroll
    for (int v = 0; v < VEC; ++v) racc[v] = fma(1.0, static_cast<double>(q[v]), racc[v]);
  }
}

template <int D, bool HALO, bool BETA, bool QUANT, bool RECV = false>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  static_assert(!RECV || QUANT, "received rows are added by the quantising gathers");
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

  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
  int cur = 0;                                  // row of the group being summed
  int32_t cur_end = rdlane(v_end, 0);

  const LaneClasses lr = RECV ? lane_classes(a.r.cls, lane) : LaneClasses();
  auto flush = [&]() {                          // write row `cur` and start the next one
    const int64_t orow = rdlane(v_out, cur);
    if (QUANT && orow >= a.q.first) {
      float res[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
      quantize_out_row<D>(a.q, orow - a.q.first, res, lane, j0, owner);
    } else {
      double racc[VEC];
      bool recv = false;
      if constexpr (RECV) {
        const int32_t p0 = cst(a.r.ptr)[orow], p1 = cst(a.r.ptr)[orow + 1];
        recv = p1 > p0;
#pragma unroll
        for (int v = 0; v < VEC; ++v) racc[v] = 0.0;
        add_received_rows<D>(a.r, lr, p0, p1, j0, racc);
      }
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
        if (recv) {                               // the row as stored, then its received rows added
#pragma unroll
          for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(static_cast<double>(res[v]) + racc[v]);
        }
        store_row<VEC>(dst, res);
      }
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
#ifndef QHA_QUANT_ROWS_BATCH
#define QHA_QUANT_ROWS_BATCH 8    // edges per batch when the gather also codes message rows (its epilogue is inlined per edge)
#endif
template <int D, bool BETA, bool QUANT, bool RECV = false>
__global__ __launch_bounds__(256) void gather_rows_kernel(GatherArgs a) {
  static_assert(!RECV || QUANT, "received rows are added by the quantising gathers");
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  constexpr int B = QUANT ? (rows_batch_of(D) * QHA_QUANT_ROWS_BATCH / QHA_ROWS_BATCH) : rows_batch_of(D);
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
  DrawCache dc;
  LaneClasses lc = QUANT ? lane_classes(a.q.cls, lane) : LaneClasses();

  // Received rows of the item's stored rows, one row per lane: the first received row of each (-1:
  // none), its width (with bit 8 set when the list holds more rows), first code word and (min,
  // scale).  The code words of the next row that takes one are loaded when the row before it closes
  // (those of the first row here), so adding them waits for nothing; further rows of a list (a node
  // with several copies) are looked up and loaded as the row closes.
  const LaneClasses lr = RECV ? lane_classes_beside(lc, a.r.cls, lane) : LaneClasses();
  if constexpr (RECV) {          // both tables in one set of registers
    lc.start = lr.start;
    lc.bits = lr.bits;
    lc.base = lr.base;
  }
  int32_t v_rk = -1;
  uint32_t v_rb = 0u, v_roff = 0u;
  float v_rzp = 0.0f, v_rsc = 0.0f;
  uint32_t pre[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) pre[v] = 0u;
  auto prefetch = [&](int row) {                // row < nrows
    if (rdlane(v_rk, row) >= 0)
      fetch_codes<VEC>(a.r.codes, static_cast<uint32_t>(rdlane(static_cast<int>(v_rb), row)) & 0xFFu,
                       static_cast<uint32_t>(rdlane(static_cast<int>(v_roff), row)), j0, pre);
  };
  if constexpr (RECV) {
    if (!split) {
      bool more = false;
      if (v_out < a.q.first) {
        const int32_t p0 = a.r.ptr[v_out], p1 = a.r.ptr[v_out + 1];
        if (p1 > p0) v_rk = a.r.idx[p0];
        more = p1 - p0 > 1;
      }
      lane_row_layout<D>(a.r, lr, v_rk, v_rb, v_roff);
      if (more) v_rb |= 0x100u;
      if (v_rk >= 0) {
        const float2 m = *reinterpret_cast<const float2*>(a.r.meta + 2 * static_cast<int64_t>(v_rk));
        v_rzp = m.x;
        v_rsc = m.y;
      }
      prefetch(0);
    }
  }

  auto flush = [&]() {
    const int64_t orow = rdlane(v_out, cur);
    if (QUANT && orow >= a.q.first) {
      // a message row: coded in place of being stored
      const int64_t k = orow - a.q.first;
      float res[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
      uint32_t w[4], b, off;
      draws_of_row<D>(a.q, dc, k, lane, j0, w);
      message_row_layout<D>(a.q, lc, k, b, off);
      quantize_row_with_draws<D>(a.q, k, b, off, res, lane, j0, owner, w);
    } else {
      double racc[VEC];
      bool recv = false;
      if constexpr (RECV) {
        if (rdlane(v_rk, cur) >= 0) {
          recv = true;
          const uint32_t info = static_cast<uint32_t>(rdlane(static_cast<int>(v_rb), cur));
          float q[VEC];
          dequant_lane<VEC>(info & 0xFFu, rdlanef(v_rzp, cur), rdlanef(v_rsc, cur), j0, pre, q);
#pragma unroll
          for (int v = 0; v < VEC; ++v) racc[v] = fma(1.0, static_cast<double>(q[v]), 0.0);
          if (info & 0x100u)
            add_received_rows<D>(a.r, lr, cst(a.r.ptr)[orow] + 1, cst(a.r.ptr)[orow + 1], j0, racc);
        }
        if (cur + 1 < nrows) prefetch(cur + 1);
      }
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
        if (recv) {                               // the row as stored, then its received rows added
#pragma unroll
          for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(static_cast<double>(res[v]) + racc[v]);
        }
        store_row<VEC>(dst, res);
      }
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

template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

// VEC floats at byte offset off (32-bit, the same register in every lane or a per-lane one) from a
// global base held in scalar registers: one global load in its scalar-base form.
template <int VEC>
__device__ __forceinline__ void global_row(gptr<char> base, uint32_t off, float (&xv)[VEC]) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef float v4f __attribute__((ext_vector_type(4)));
  gptr<char> p = base + off;
  if constexpr (VEC == 1) {
    xv[0] = *reinterpret_cast<gptr<float>>(p);
  } else if constexpr (VEC == 2) {
    const v2f t = *reinterpret_cast<gptr<v2f>>(p);
    xv[0] = t.x; xv[1] = t.y;
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const v4f t = reinterpret_cast<gptr<v4f>>(p)[q];
      xv[4 * q + 0] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
    }
  }
}

// Halo gather over a width-grouped message (rows ordered by width, the guide's section 9 packing).
// A batch's set-up runs one edge per lane: the column's class (a scan of the few class starts),
// width, code-row offset, and the 32-bit byte offset of the edge's value load -- the inner row,
// the raw row of a 32-bit halo, or the (min, scale) pair of a quantised one.  Each edge then moves
// three words to scalar registers (kind and width, value offset, code offset) and issues exactly
// two loads, with the value's base chosen by scalar selects: the value, and the code word that
// holds the lane's features (a word of the buffer's first row for edges without codes), so every
// edge's loads are counted alike and the sums can consume them one edge at a time.  Dequantisation
// branches once per edge on its width, with that width's lane shifts precomputed.
template <int D, bool BETA, bool SB>
__global__ __launch_bounds__(256) void gather_grouped_kernel(GatherArgs a) {
  constexpr int VEC = vec_of(D);
  constexpr int G = D / VEC;
  constexpr int B = grouped_batch_of(D);
  constexpr int CW = (VEC * 8 > 32) ? 2 : 1;
  constexpr int LGD = log2i(D);
  constexpr uint32_t LGV = static_cast<uint32_t>(log2i(VEC));
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

  // the class table, class c in lane c
  int32_t v_cstart = 0x7FFFFFFF, v_cbits = 0;
  uint32_t v_cbase = 0;
#pragma unroll
  for (int c = 0; c < kMaxClasses; ++c) {
    if (lane == c && c < a.cls.n) {
      v_cstart = a.cls.start[c];
      v_cbits = a.cls.bits[c];
      v_cbase = a.cls.base[c];
    }
  }
  const int ncls = a.cls.n;
  // per width b = 2^lgb: the lane's first code bit within its word
  uint32_t v_sh[4];
#pragma unroll
  for (int lgb = 0; lgb < 4; ++lgb) v_sh[lgb] = (static_cast<uint32_t>(j0) << lgb) & 31u;
  const uint32_t lane_eff = static_cast<uint32_t>(j0) >> LGV;

  // with one base (SB) every load is that base plus a 32-bit offset, and offsets carry the
  // buffers' own distances from it
  gptr<char> xb = SB ? (gptr<char>)(a.base) : (gptr<char>)(a.x);
  gptr<char> cb = SB ? (gptr<char>)(a.base) : (gptr<char>)(a.codes);
  gptr<char> mb = SB ? (gptr<char>)(a.base) : (gptr<char>)(a.meta);
  const uint32_t x_off = SB ? a.x_off : 0u;
  const uint32_t codes_off = SB ? a.codes_off : 0u;
  const uint32_t meta_off = SB ? a.meta_off : 0u;
  const uint32_t pitch = static_cast<uint32_t>(a.ldx) * 4u;
  const uint32_t lane_off = static_cast<uint32_t>(j0) * 4u;
  const int32_t n_inner = static_cast<int32_t>(a.n_inner);

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
    // set-up, edge i in lane i
    const int32_t vk = v_u - n_inner;
    const bool vh = vk >= 0;
    int32_t vst = rdlane(v_cstart, 0);
    uint32_t vb = static_cast<uint32_t>(rdlane(v_cbits, 0));
    uint32_t vcb = static_cast<uint32_t>(rdlane(static_cast<int>(v_cbase), 0));
    for (int c = 1; c < ncls; ++c) {
      const int32_t st = rdlane(v_cstart, c);
      const uint32_t bc = static_cast<uint32_t>(rdlane(v_cbits, c));
      const uint32_t cbc = static_cast<uint32_t>(rdlane(static_cast<int>(v_cbase), c));
      const bool ge = vk >= st;
      vst = ge ? st : vst;
      vb = ge ? bc : vb;
      vcb = ge ? cbc : vcb;
    }
    const bool vq = vh && vb != 32u;
    const uint32_t vlgb = static_cast<uint32_t>(__builtin_ctz(vb));             // 5 for raw rows
    const uint32_t vlgw = vb == 32u ? static_cast<uint32_t>(LGD) : (LGD + vlgb > 5u ? LGD + vlgb - 5u : 0u);
    const uint32_t vrow = vcb + (static_cast<uint32_t>(vk - vst) << vlgw);     // code-row word offset
    const uint32_t vvo = !vh ? x_off + static_cast<uint32_t>(v_u) * pitch
                             : (vq ? meta_off + static_cast<uint32_t>(vk) * 8u : codes_off + vrow * 4u);
    const uint32_t vco = codes_off + (vq ? vrow * 4u : 0u);
    // kind (0 inner, 32 raw halo, else the code width) | lane shift of the code word << 8: the word
    // holding a lane's first code is lane * VEC * b / 32, i.e. lane >> (5 - log2(VEC * b)); edges
    // without codes take shift 6, so every lane reads the buffer's first word
    const uint32_t vsh = vq ? (LGV + vlgb <= 5u ? 5u - LGV - vlgb : 0u) : 6u;
    const uint32_t vpk = (vh ? (vq ? vb : 32u) : 0u) | (vsh << 8) | ((vq ? vlgb : 0u) << 16);

    // phase 1: two loads per edge
    float xv[B][VEC];
    float mp[B][2];                    // (min, scale) when a lane holds one feature
    uint32_t cwd[B][CW];
    uint32_t pk[B];
    float ww[B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      pk[i] = static_cast<uint32_t>(rdlane(static_cast<int>(vpk), i));
      ww[i] = rdlanef(v_w, i);
      const uint32_t kind = pk[i] & 0xFFu;
      const uint32_t wsh = (pk[i] >> 8) & 0xFFu;
      const uint32_t vo = static_cast<uint32_t>(rdlane(static_cast<int>(vvo), i));
      const uint32_t co = static_cast<uint32_t>(rdlane(static_cast<int>(vco), i));
      const bool q = kind != 0u && kind != 32u;
      if (SB && VEC == 2) {
        // one load form for every edge: a quantised row's (min, scale) pair is read by all lanes
        global_row<VEC>(xb, vo + (lane_off & (q ? 0u : 0xFFFFFFFFu)), xv[i]);
      } else if (q) {
        float pr[2];
        global_row<2>(mb, vo, pr);
        if constexpr (VEC >= 2) {
          xv[i][0] = pr[0];
          xv[i][1] = pr[1];
        } else {
          mp[i][0] = pr[0];
          mp[i][1] = pr[1];
        }
      } else {
        global_row<VEC>(kind == 0u ? xb : cb, vo + lane_off, xv[i]);
      }
      // the byte offset of the word holding the lane's first code (8-bit codes at VEC = 8 take two
      // words a lane: lane * 2)
      uint32_t wofs = (lane_eff >> wsh) << 2;
      if constexpr (LGV + 3 > 5) {
        if (kind == 8u) wofs = lane_eff << 3;
      }
      gptr<uint32_t> crow = reinterpret_cast<gptr<uint32_t>>(cb + (co + wofs));
      cwd[i][0] = crow[0];
      if constexpr (CW == 2) cwd[i][1] = crow[kind * VEC > 32u && q ? 1 : 0];
    }
    if (e + B < e1) fetch(e + B);

    // phase 2: dequantise and sum, closing the row whose last edge this is
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int32_t p = e + i;
      if (p < e1) {
        const double wt = static_cast<double>(ww[i]);
        const uint32_t kind = pk[i] & 0xFFu;
        if (kind == 0u || kind == 32u) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(xv[i][v]), acc[v]);
        } else if constexpr (SB) {
          // the width as a run-time field: one branch per edge
          const float mn = VEC >= 2 ? xv[i][0] : mp[i][0];
          const float sc = VEC >= 2 ? xv[i][1 % VEC] : mp[i][1];
          const uint32_t b = kind;
          const uint32_t lgb = pk[i] >> 16;
          const uint32_t bit0 = (static_cast<uint32_t>(j0) << lgb) & 31u;
          float qv[VEC];
          if constexpr (CW == 1) {
            // a lane's VEC * b <= 32 bits of codes start at a multiple of VEC * b in one word:
            // shifted down once, code v is the field at bit v * b (a scalar offset)
            const uint32_t w0 = cwd[i][0] >> bit0;
#pragma unroll
            for (int v = 0; v < VEC; ++v)
              qv[v] = dequant(sc, __builtin_amdgcn_ubfe(w0, static_cast<uint32_t>(v) * b, b), mn);
          } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const uint32_t vb_ = static_cast<uint32_t>(v) * b;
              const uint32_t word = vb_ >= 32u ? cwd[i][CW - 1] : cwd[i][0];
              const uint32_t code = __builtin_amdgcn_ubfe(word, (bit0 + vb_) & 31u, b);
              qv[v] = dequant(sc, code, mn);
            }
          }
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(qv[v]), acc[v]);
        } else {
          const float mn = VEC >= 2 ? xv[i][0] : mp[i][0];
          const float sc = VEC >= 2 ? xv[i][1 % VEC] : mp[i][1];
          auto body = [&](auto bc) {
            constexpr uint32_t b = decltype(bc)::value;
            constexpr uint32_t lg = static_cast<uint32_t>(log2i(static_cast<int>(b)));
            float q[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const uint32_t word = (CW == 2 && (static_cast<uint32_t>(v) * b) >= 32u) ? cwd[i][CW - 1] : cwd[i][0];
              const uint32_t bit = (v_sh[lg] + static_cast<uint32_t>(v) * b) & 31u;
              q[v] = dequant(sc, (word >> bit) & ((1u << b) - 1u), mn);
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = fma(wt, static_cast<double>(q[v]), acc[v]);
          };
          if (kind == 4u) body(std::integral_constant<uint32_t, 4>{});
          else if (kind == 8u) body(std::integral_constant<uint32_t, 8>{});
          else if (kind == 2u) body(std::integral_constant<uint32_t, 2>{});
          else body(std::integral_constant<uint32_t, 1>{});
        }
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
template <int D, bool QUANT, bool RECV = false>
__global__ __launch_bounds__(256) void combine_split_kernel(GatherArgs a) {
  static_assert(!RECV || QUANT, "received rows are added by the quantising gathers");
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
  // the partials are added one by one in chunk order; the loads of U chunks (8, or 4 at d = 512)
  // are issued together, so a row waits for memory once per U chunks instead of once per chunk.
  // The last, partial batch reloads the row's last chunk in place of the chunks past it and adds
  // nothing from them.
  constexpr int U = VEC >= 8 ? 4 : 8;
  const double* pp = a.partial + j0;
  double acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = pp[static_cast<int64_t>(i0) * D + v];
  int32_t i = i0 + 1;
  for (; i + U <= i1; i += U) {
    double t[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) t[u][v] = pp[static_cast<int64_t>(i + u) * D + v];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = acc[v] + t[u][v];
    }
  }
  if (i < i1) {
    double t[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = i + u < i1 ? i + u : i1 - 1;
#pragma unroll
      for (int v = 0; v < VEC; ++v) t[u][v] = pp[c * D + v];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u < i1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = acc[v] + t[u][v];
      }
    }
  }
  const int64_t orow = a.row_ids ? a.row_ids[row] : row;
  if (QUANT && orow >= a.q.first) {
    float res[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) res[v] = static_cast<float>(acc[v]);
    quantize_out_row<D>(a.q, orow - a.q.first, res, lane, j0, owner);
  } else {
    double racc[VEC];
    bool recv = false;
    if constexpr (RECV) {
      const LaneClasses lr = lane_classes(a.r.cls, lane);
      const int32_t p0 = cst(a.r.ptr)[orow], p1 = cst(a.r.ptr)[orow + 1];
      recv = p1 > p0;
#pragma unroll
      for (int v = 0; v < VEC; ++v) racc[v] = 0.0;
      add_received_rows<D>(a.r, lr, p0, p1, j0, racc);
    }
    if (owner) {
      float* dst = a.out + orow * a.ldo + j0;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float res = static_cast<float>(a.beta ? static_cast<double>(dst[v]) + acc[v] : acc[v]);
        if (recv) res = static_cast<float>(static_cast<double>(res) + racc[v]);
        dst[v] = res;
      }
    }
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

template <int D>
hipError_t launch_gather_d(const GatherArgs& a, bool with_halo, bool quantize_out, hipStream_t s) {
  // received rows are added to the stored rows of quantising gathers only
  if (a.r.ptr != nullptr && !quantize_out) return hipErrorInvalidValue;
  const bool recv = a.r.ptr != nullptr;
  // the plain-row kernel addresses x with 32-bit byte offsets
  const int64_t x_bytes = a.n_inner > 0 ? ((a.n_inner - 1) * a.ldx + D) * 4 : 0;
  const bool rows_ok = x_bytes <= static_cast<int64_t>(0xFFFFFFFFu) && QHA_ROWS_KERNEL;
  // the grouped halo kernel addresses x, the codes and the (min, scale) pairs with 32-bit offsets
  bool grouped_ok = false, single_base = false;
  uintptr_t lo = 0;
  if (with_halo && a.cls.n > 0 && QHA_GROUPED_KERNEL) {
    const int c = a.cls.n - 1;
    const int64_t b = a.cls.bits[c];
    const int64_t words = b == 32 ? D : (D * b + 31) / 32;
    const int64_t code_bytes = (static_cast<int64_t>(a.cls.base[c]) + (a.cls.start[c + 1] - a.cls.start[c]) * words) * 4;
    grouped_ok = x_bytes <= static_cast<int64_t>(0xFFFFFFFFu) && code_bytes <= static_cast<int64_t>(0xFFFFFFFFu) &&
                 a.n_halo * 8 <= static_cast<int64_t>(0xFFFFFFFFu);
    // the span from the lowest to the highest byte of x, codes and meta
    const uintptr_t c0 = reinterpret_cast<uintptr_t>(a.codes), m0 = reinterpret_cast<uintptr_t>(a.meta);
    lo = c0 < m0 ? c0 : m0;
    uintptr_t hi = c0 + static_cast<uintptr_t>(code_bytes);
    const uintptr_t mh = m0 + static_cast<uintptr_t>(a.n_halo * 8);
    hi = mh > hi ? mh : hi;
    if (a.x != nullptr && x_bytes > 0) {
      const uintptr_t x0 = reinterpret_cast<uintptr_t>(a.x);
      lo = x0 < lo ? x0 : lo;
      const uintptr_t xh = x0 + static_cast<uintptr_t>(x_bytes);
      hi = xh > hi ? xh : hi;
    }
    single_base = QHA_SINGLE_BASE && hi - lo <= 0xFFFFFFFFull;
  }

  if (a.n_items > 0) {
    const dim3 grid(static_cast<unsigned>((a.n_items + 3) / 4));
    if (quantize_out && rows_ok) {
      GatherArgs r = a;
      r.x_bytes = static_cast<uint32_t>(x_bytes);
      if (recv) {
        if (a.beta) hipLaunchKernelGGL((gather_rows_kernel<D, true, true, true>), grid, dim3(256), 0, s, r);
        else hipLaunchKernelGGL((gather_rows_kernel<D, false, true, true>), grid, dim3(256), 0, s, r);
      } else {
        if (a.beta) hipLaunchKernelGGL((gather_rows_kernel<D, true, true>), grid, dim3(256), 0, s, r);
        else hipLaunchKernelGGL((gather_rows_kernel<D, false, true>), grid, dim3(256), 0, s, r);
      }
    } else if (quantize_out) {
      if (recv) {
        if (a.beta) hipLaunchKernelGGL((gather_kernel<D, false, true, true, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((gather_kernel<D, false, false, true, true>), grid, dim3(256), 0, s, a);
      } else {
        if (a.beta) hipLaunchKernelGGL((gather_kernel<D, false, true, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((gather_kernel<D, false, false, true>), grid, dim3(256), 0, s, a);
      }
    } else if (with_halo && grouped_ok) {
      GatherArgs r = a;
      if (single_base) {
        r.base = reinterpret_cast<const char*>(lo);
        r.x_off = a.x ? static_cast<uint32_t>(reinterpret_cast<uintptr_t>(a.x) - lo) : 0u;
        r.codes_off = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(a.codes) - lo);
        r.meta_off = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(a.meta) - lo);
        if (a.beta) hipLaunchKernelGGL((gather_grouped_kernel<D, true, true>), grid, dim3(256), 0, s, r);
        else hipLaunchKernelGGL((gather_grouped_kernel<D, false, true>), grid, dim3(256), 0, s, r);
      } else {
        if (a.beta) hipLaunchKernelGGL((gather_grouped_kernel<D, true, false>), grid, dim3(256), 0, s, r);
        else hipLaunchKernelGGL((gather_grouped_kernel<D, false, false>), grid, dim3(256), 0, s, r);
      }
    } else if (with_halo) {
      // the per-row offset table (also the way for width classes beyond 32-bit offsets)
      if (a.word_offset == nullptr || (D < 32 && a.bits == nullptr)) return hipErrorInvalidValue;
      if (a.beta) hipLaunchKernelGGL((gather_kernel<D, true, true, false>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gather_kernel<D, true, false, false>), grid, dim3(256), 0, s, a);
    } else if (rows_ok) {
      GatherArgs r = a;
      r.x_bytes = static_cast<uint32_t>(x_bytes);
      if (a.beta) hipLaunchKernelGGL((gather_rows_kernel<D, true, false>), grid, dim3(256), 0, s, r);
      else hipLaunchKernelGGL((gather_rows_kernel<D, false, false>), grid, dim3(256), 0, s, r);
    } else {
      if (a.beta) hipLaunchKernelGGL((gather_kernel<D, false, true, false>), grid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gather_kernel<D, false, false, false>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.n_split_rows > 0) {
    const int64_t blocks = (a.n_split_rows + 3) / 4;
    if (recv)
      hipLaunchKernelGGL((combine_split_kernel<D, true, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else if (quantize_out)
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

// Scratch of the allocation-free aggregation: the float64 partial rows of split heavy rows.  Each GPU
// the library is loaded on holds its own copy until the process ends.  In host code this name is a
// stand-in, not a device address: the kernels get the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) unsigned char scratch[QHA_NOALLOC_SCRATCH_BYTES];

void* noalloc_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

hipError_t launch_edge_weights(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* r,
                               const float* c, float* w, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(edge_weights_kernel, dim3(static_cast<unsigned>((n_rows + 3) / 4)), dim3(256), 0, s, n_rows,
                     rowptr, colidx, r, c, w);
  return hipGetLastError();
}

}  // namespace qha
