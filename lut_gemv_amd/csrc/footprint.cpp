// Storage footprint of a BCQ matrix and the search for group sizes that meet a
// storage target (Elamur card "LUT-GEMM -- paper by Park et al. (2022)", section
// "Interesting ideas: Group size as a separate hyper-parameter": bit width q and
// group size g are separate knobs chosen together for a target compression,
// and the scales must be counted in the storage).
#include <stdint.h>

#include "layout.h"
#include "lutgemm.h"

using namespace lutgemm;

namespace {

// q sign bits per weight, one fp16 scale per (plane, row, group) and one fp16
// offset per (row, group) when present.
uint64_t footprint(uint64_t N, uint64_t K, uint64_t q, uint64_t g, bool off) {
  const uint64_t groups = N * (K / g);
  return q * N * K + 16 * q * groups + (off ? 16 * groups : 0);
}

}  // namespace

extern "C" {

int bcq_footprint_bits(const lutgemm_shape* s, uint64_t* bits) {
  const int st = check_shape(s);
  if (st) return st;
  if (!bits) return LUTGEMM_ERR_NULL;
  *bits = s->K == 0 ? 0 : footprint((uint64_t)s->N, (uint64_t)s->K, (uint64_t)s->q,
                                    (uint64_t)s->g, s->has_offset != 0);
  return LUTGEMM_OK;
}

int bcq_search_group_sizes(int64_t N, int64_t K, int32_t has_offset, double max_bits_per_weight,
                           int32_t* out_g, uint64_t* out_bits) {
  if (!out_g || !out_bits) return LUTGEMM_ERR_NULL;
  if (N < 1 || K < 8 || K % 8 || N >= kMaxDim || K >= kMaxDim) return LUTGEMM_ERR_SHAPE;
  if (has_offset != 0 && has_offset != 1) return LUTGEMM_ERR_SHAPE;
  if (!(max_bits_per_weight > 0.0) || max_bits_per_weight > 1e6) return LUTGEMM_ERR_VALUE;
  const long double budget = (long double)max_bits_per_weight * (long double)N * (long double)K;
  for (int q = 1; q <= 8; ++q) {
    out_g[q - 1] = 0;
    out_bits[q - 1] = 0;
    // the footprint falls as g grows: the first divisor that fits is the finest
    for (int64_t g = 8; g <= K; g += 8) {
      if (K % g) continue;
      const uint64_t b = footprint((uint64_t)N, (uint64_t)K, (uint64_t)q, (uint64_t)g, has_offset);
      if ((long double)b <= budget) {
        out_g[q - 1] = (int32_t)g;
        out_bits[q - 1] = b;
        break;
      }
    }
  }
  return LUTGEMM_OK;
}

}  // extern "C"
