// Internal launch interface between the C ABI (abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace qha {

// Status helpers of the C ABI (the message is kept per thread for qha_last_error).
int fail(int status, const char* fmt, ...);
int ok();

constexpr int kMaxClasses = 8;

// Width classes of a width-grouped packed buffer (copied into kernel arguments); n == 0 means
// the per-row bits / word_offset arrays describe the layout instead.
struct Classes {
  int32_t n;
  int32_t bits[kMaxClasses];
  int32_t start[kMaxClasses + 1];
  uint32_t base[kMaxClasses];
};

struct QuantArgs {
  const float* x;
  int64_t ldx;
  const int32_t* row_index;
  int64_t n_rows;
  const uint8_t* bits;
  const uint32_t* word_offset;
  Classes cls;
  uint32_t seed_lo, seed_hi, epoch, stream_id, node_base;
  uint32_t* codes;
  float* meta;          // (min, scale) per row
};

// Quantised output of a gather: each output row r >= first is coded like qha_quantize_pack row
// r - first (node id node_base + r - first) instead of being stored; rows below first are stored.
struct QuantOut {
  int64_t first;
  uint32_t* codes;
  float* meta;
  const uint8_t* bits;
  const uint32_t* word_offset;
  Classes cls;
  uint32_t seed_lo, seed_hi, epoch, stream_id, node_base;
};

// Received messages added to the stored rows of a quantising gather (ptr == nullptr: none).  Stored
// row r gets, after its own rounding, the float64 sum of the dequantised message rows
// idx[ptr[r] .. ptr[r + 1]) in that order, rounded to float32 once more.
struct RecvAdd {
  const int32_t* ptr;
  const int32_t* idx;
  const uint32_t* codes;
  const float* meta;
  const uint8_t* bits;
  const uint32_t* word_offset;
  Classes cls;
};

// One gather over a CSR: out[row_ids[i]] (+)= sum_e w[e] * value(col_e).  value() is a float32
// row of x for col < n_inner and a dequantised halo message for col >= n_inner.
struct GatherArgs {
  int64_t n_rows;
  const int32_t* rowptr;
  const int32_t* colidx;
  const int32_t* row_ids;
  // work plan (items == nullptr: item i is row i alone)
  int64_t n_items;
  int64_t n_split_items;
  const int32_t* items;       // int32[4] per item: first row, row count, first edge, end edge
  int64_t n_split_rows;
  const int32_t* split_row;
  const int32_t* split_ptr;
  const float* w;             // per-edge weights (nullptr: 1)
  // values
  const float* x;
  int64_t ldx;
  int64_t n_inner;
  uint32_t x_bytes;           // readable bytes of x (set by the launcher for range-checked loads)
  const uint32_t* codes;
  uint32_t codes_bytes;       // bound on the readable bytes of codes (set by the launcher)
  // one base under x, codes and meta with every byte of them within 4 GiB of it (set by the
  // launcher when that holds): the grouped halo gather then addresses all three from one register
  const char* base;
  uint32_t x_off, codes_off, meta_off;
  const uint32_t* word_offset;
  const uint8_t* bits;
  Classes cls;
  const float* meta;
  int64_t n_halo;
  // output
  int32_t beta;
  float* out;
  int64_t ldo;
  double* partial;            // [n_split_items, d] float64 partial sums of split rows
  QuantOut q;                 // with launch_gather(..., quantize_out = true)
  RecvAdd r;                  // with quantize_out: messages added to the stored rows
};

struct GemmArgs {
  int32_t ta, tb;
  int64_t m, n, k;
  const float* a;
  int64_t lda;
  const float* b;
  int64_t ldb;
  int32_t beta;
  float* c;
  int64_t ldc;
  int32_t pro;
  const float* aux;
  int64_t ld_aux;
  int32_t epi;
  double* ws;          // float64 split-k partials [splits, m, n]
  int32_t splits;
  int64_t k_per_split;
  uint32_t* bsplit;    // workspace for B's three bf16 parts, split once per call (nullptr: B is
                       // split as its tiles are staged); used when A is not transposed and k is not split
  int32_t buf32;       // set by the launcher: k-major operands are read with 32-bit buffer offsets
};

// Row-panel products of width-128 layers (W's split parts held on chip, row panels streamed).
constexpr int kPanelBlocks = 256;    // one block per compute unit of an MI355X
struct PanelArgs {
  int64_t m;
  const float* a;      // [m x 128]: the forward input, or the backward's A (for dW)
  int64_t lda;
  const float* w;      // W [128 x 128]
  int64_t ldw;
  float* out;          // forward: H [m x 128]
  int64_t ldo;
  int32_t relu;
  const float* dh;     // backward: dH [m x 128]
  int64_t lddh;
  const float* h;      // backward: the forward output H (ReLU mask) [m x 128]
  int64_t ldh;
  float* da;           // backward: dA [m x 128]
  int64_t ldda;
  float* dw;           // backward: dW [128 x 128]
  int64_t lddw;
  float* ws;           // backward: per-block dW partials [blocks][128][128]
};
bool panel_fits(int64_t n, int64_t k);

// Weight gradient of the general widths: dW [n x k] = dZ^T A over m rows, dZ = dH * [H > 0], for n a
// multiple of 128 and k a multiple of 256 (row-panel blocks, one float32 partial per row range).
struct DwArgs {
  int64_t m;
  int32_t n, k;
  const float* dh;
  int64_t lddh;
  const float* h;
  int64_t ldh;
  const float* a;
  int64_t lda;
  float* ws;           // [ranges][n][k] partials
  int32_t ranges;      // row ranges R (a multiple of 8)
  int32_t groups_z;    // n / 128
  int32_t groups_a;    // k / 256
};
bool dw_panel_fits(int64_t m, int64_t n, int64_t k);
int32_t dw_panel_ranges(int64_t m, int64_t n, int64_t k);
size_t dw_panel_workspace(int64_t m, int64_t n, int64_t k);
hipError_t launch_dw_panel(const DwArgs& a, float* dw, int64_t lddw, hipStream_t s);
size_t panel_bwd_workspace(int64_t m);
hipError_t launch_panel_fwd(const PanelArgs& p, hipStream_t s);
hipError_t launch_panel_bwd(const PanelArgs& p, hipStream_t s);

// Split-k rule shared by the workspace query and the launcher.
void gemm_split_rule(int64_t m, int64_t n, int64_t k, int32_t* splits, int64_t* k_per_split);
// Bytes of B's split parts when splitting B once per call pays (A not transposed, k not split and
// enough rows of A), else 0.
size_t gemm_bsplit_bytes(int32_t ta, int64_t m, int64_t n, int64_t k);

hipError_t launch_degree_norm(const int32_t* deg, int64_t n, int32_t kind, float* out, hipStream_t s);
hipError_t launch_edge_weights(int64_t n_rows, const int32_t* rowptr, const int32_t* colidx, const float* r,
                               const float* c, float* w, hipStream_t s);
hipError_t launch_quantize(const QuantArgs& a, int32_t d, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, int32_t d, bool with_halo, hipStream_t s, bool quantize_out = false);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// Device address of the allocation-free aggregation's scratch (QHA_NOALLOC_SCRATCH_BYTES bytes) on
// the current device, looked up once per device; nullptr, with *err set, if the lookup fails.
void* noalloc_scratch(hipError_t* err);

}  // namespace qha
