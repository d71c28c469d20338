// Host-side width control: the Graph Extractor's mask levels, the Quant Orchestrator's per-epoch
// widths and the Coordinator's base-width / execution-mode rule.
//
// Method: SYLVIE guide, section 7 (importance from the global in-degree percentile of the boundary
// pool, equal degrees equal importance, the largest degree 1), section 9 (the epoch's base width
// shifts every level's width up, clipped at the top candidate; Figure 7) and section 8 (Eq. 3-5:
// mean partition loss, its exponential average, the loss descent rate per unit time, and the
// doubling / halving rule between b_min and b_max, plus the matching sync / async choice of the
// pipeline).  All decisions are exact: levels are integer arithmetic on the percentile count.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "../../include/qha.h"
#include "qha_internal.hpp"

#pragma clang fp contract(off)

namespace {

bool pow2_width(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }

}  // namespace

extern "C" {

int qha_mask_levels(const int32_t* deg, int64_t n, int32_t n_levels, uint8_t* level, double* importance) {
  if (n < 0) return qha::fail(QHA_ERR_INVALID_ARG, "bad n");
  if (n_levels < 1 || n_levels > QHA_MAX_LEVELS) return qha::fail(QHA_ERR_INVALID_ARG, "n_levels = %d", n_levels);
  if (n == 0) return qha::ok();
  if (!deg || !level) return qha::fail(QHA_ERR_INVALID_ARG, "deg / level is NULL");
  std::vector<int32_t> sorted(deg, deg + n);
  std::sort(sorted.begin(), sorted.end());
  for (int64_t i = 0; i < n; ++i) {
    // nodes of the pool whose degree is at most this node's: p = count / n
    const int64_t count = std::upper_bound(sorted.begin(), sorted.end(), deg[i]) - sorted.begin();
    level[i] = static_cast<uint8_t>((count * n_levels + n - 1) / n - 1);    // ceil(p * L) - 1
    if (importance) importance[i] = static_cast<double>(count) / static_cast<double>(n);
  }
  return qha::ok();
}

int qha_node_bits(const uint8_t* level, int64_t n, int32_t base_bits, int32_t max_bits, uint8_t* bits) {
  if (n < 0) return qha::fail(QHA_ERR_INVALID_ARG, "bad n");
  if (!pow2_width(base_bits) || !pow2_width(max_bits) || base_bits > max_bits)
    return qha::fail(QHA_ERR_INVALID_ARG, "base %d / max %d widths", base_bits, max_bits);
  if (n == 0) return qha::ok();
  if (!level || !bits) return qha::fail(QHA_ERR_INVALID_ARG, "level / bits is NULL");
  for (int64_t i = 0; i < n; ++i) {
    if (level[i] >= QHA_MAX_LEVELS) return qha::fail(QHA_ERR_INVALID_ARG, "level %d at %lld", level[i], (long long)i);
    const int32_t b = base_bits << level[i];
    bits[i] = static_cast<uint8_t>(b < max_bits ? b : max_bits);
  }
  return qha::ok();
}

int qha_level_order(const uint8_t* level, int64_t n, int32_t* order) {
  if (n < 0 || n > 2147483647LL) return qha::fail(QHA_ERR_INVALID_ARG, "bad n");
  if (n == 0) return qha::ok();
  if (!level || !order) return qha::fail(QHA_ERR_INVALID_ARG, "level / order is NULL");
  std::vector<int32_t> idx(static_cast<size_t>(n));
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return level[a] > level[b]; });
  std::memcpy(order, idx.data(), static_cast<size_t>(n) * sizeof(int32_t));
  return qha::ok();
}

int qha_coordinator_init(qha_coordinator* c, double lambda, int32_t delta, int32_t b_min, int32_t b_max,
                         int32_t descent_magnitude) {
  if (!c) return qha::fail(QHA_ERR_INVALID_ARG, "coordinator is NULL");
  if (!(lambda >= 0.0 && lambda <= 1.0)) return qha::fail(QHA_ERR_INVALID_ARG, "lambda outside [0, 1]");
  if (delta < 1 || delta > QHA_LDR_MAX_DELTA) return qha::fail(QHA_ERR_INVALID_ARG, "delta = %d", delta);
  if (!pow2_width(b_min) || !pow2_width(b_max) || b_min > b_max)
    return qha::fail(QHA_ERR_INVALID_ARG, "b_min %d / b_max %d", b_min, b_max);
  std::memset(c, 0, sizeof(*c));
  c->lambda = lambda;
  c->delta = delta;
  c->b_min = b_min;
  c->b_max = b_max;
  c->sign = descent_magnitude ? -1.0 : 1.0;
  c->bits = b_min;
  c->sync = 1;
  return qha::ok();
}

int qha_coordinator_step(qha_coordinator* c, const double* losses, int32_t n_partitions, double epoch_time,
                         int32_t* next_bits, int32_t* next_sync) {
  if (!c || !losses || n_partitions < 1) return qha::fail(QHA_ERR_INVALID_ARG, "coordinator / losses");
  if (!(epoch_time > 0.0)) return qha::fail(QHA_ERR_INVALID_ARG, "epoch time must be positive");
  const int64_t t = c->t;
  double sum = 0.0;
  for (int32_t i = 0; i < n_partitions; ++i) sum += losses[i];
  const double l_t = sum / static_cast<double>(n_partitions);
  const double f_before = t == 0 ? l_t : c->f_prev;
  const double f_t = c->lambda * f_before + (1.0 - c->lambda) * l_t;
  const double ldr_t = c->sign * (f_t - f_before) / epoch_time;
  const int32_t ring = c->delta + 1;
  c->ldr[t % ring] = ldr_t;
  if (t == 0) {
    c->bits = c->b_min;
  } else if (t > c->delta) {
    const double past = c->ldr[(t - c->delta) % ring];
    if (ldr_t < past) {
      if (c->bits < c->b_max) c->bits *= 2;
      c->sync = 1;
    } else {
      if (c->bits > c->b_min) c->bits /= 2;
      c->sync = 0;
    }
  }
  c->f_prev = f_t;
  c->last_ldr = ldr_t;
  c->t = t + 1;
  if (next_bits) *next_bits = c->bits;
  if (next_sync) *next_sync = c->sync;
  return qha::ok();
}

}  // extern "C"
