// Internal definitions shared by the host packer and the device launcher:
// shape validation and the geometry of the packed device format.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lutgemm.h"

namespace lutgemm {

constexpr int kRowTile = 16;     // output rows per row tile (one 16-byte load per lane and plane)
constexpr int kChunkTile = 64;   // 8-input chunks per input tile (one chunk per lane of a wave)
constexpr int kMaxDim = 1 << 30;
constexpr int kMaxBatch = 65535;

struct Geometry {
  int64_t N, K, q, g;
  bool has_offset;
  int64_t RT;    // row tiles
  int64_t Npad;  // RT * 16
  int64_t C;     // chunks (K / 8)
  int64_t KT;    // input tiles
  int64_t G;     // groups per row
  size_t bits_bytes, alpha_count, offset_count;
};

inline int check_shape(const lutgemm_shape* s) {
  if (!s) return LUTGEMM_ERR_NULL;
  if (s->N < 0 || s->K < 0 || s->N >= kMaxDim || s->K >= kMaxDim) return LUTGEMM_ERR_SHAPE;
  if (s->K % 8) return LUTGEMM_ERR_SHAPE;
  if (s->q < 1 || s->q > 8) return LUTGEMM_ERR_SHAPE;
  if (s->g < 8 || s->g % 8) return LUTGEMM_ERR_SHAPE;
  if (s->K > 0 && s->K % s->g) return LUTGEMM_ERR_SHAPE;
  if (s->has_offset != 0 && s->has_offset != 1) return LUTGEMM_ERR_SHAPE;
  return LUTGEMM_OK;
}

inline Geometry geometry(const lutgemm_shape* s) {
  Geometry g{};
  g.N = s->N;
  g.K = s->K;
  g.q = s->q;
  g.g = s->g;
  g.has_offset = s->has_offset != 0;
  g.RT = (g.N + kRowTile - 1) / kRowTile;
  g.Npad = g.RT * kRowTile;
  g.C = g.K / 8;
  g.KT = (g.C + kChunkTile - 1) / kChunkTile;
  g.G = g.K > 0 ? g.K / g.g : 0;
  g.bits_bytes = (size_t)g.RT * g.KT * g.q * kChunkTile * kRowTile;
  g.alpha_count = (size_t)g.q * g.Npad * g.G;
  g.offset_count = g.has_offset ? (size_t)g.Npad * g.G : 0;
  return g;
}

}  // namespace lutgemm
