// Host-side half of the C ABI: status strings, size queries and the packers
// that turn a BCQ (or uniform int-q) matrix into the device format.
//
// Packing is plain index arithmetic on the CPU; it runs once per weight
// matrix, not per product, so it is written for clarity and determinism.
#include <math.h>
#include <string.h>

#include <new>
#include <thread>
#include <vector>

#include "host_util.h"
#include "layout.h"
#include "lutgemm.h"

using namespace lutgemm;
using namespace lutgemm::host;

namespace {

int check_outputs(const Geometry& G, uint8_t* ob, size_t obn, uint16_t* oa, size_t oan,
                  uint16_t* oo, size_t oon) {
  if (G.bits_bytes && !ob) return LUTGEMM_ERR_NULL;
  if (G.alpha_count && !oa) return LUTGEMM_ERR_NULL;
  if (G.offset_count && !oo) return LUTGEMM_ERR_NULL;
  if (obn < G.bits_bytes || oan < G.alpha_count || (G.has_offset && oon < G.offset_count))
    return LUTGEMM_ERR_BUFFER;
  return LUTGEMM_OK;
}

// Offset of (row r, chunk c) inside one 1024-byte (row tile, input tile, plane)
// block: 64 lane blocks of 16 bytes, lane block 16*(r/4) + c/4 holding rows
// r/4*4 .. +3 and chunks c/4*4 .. +3 at byte 4*(r%4) + c%4.
inline int64_t in_block(int64_t r, int64_t c) {
  return ((r >> 2) * 16 + (c >> 2)) * 16 + (r & 3) * 4 + (c & 3);
}

// Byte offset of the 1024-byte block of (input tile kt, row tile rt, plane i):
// blocks are ordered input tile first, so the blocks of all row tiles for one
// input tile are contiguous.
inline size_t block_offset(const Geometry& G, int64_t kt, int64_t rt, int64_t i) {
  return (((size_t)kt * G.RT + rt) * G.q + i) * (size_t)(kChunkTile * kRowTile);
}

// Zero the blocks of row tile rt (all input tiles, all planes).
void clear_row_tile(const Geometry& G, int64_t rt, uint8_t* out) {
  for (int64_t kt = 0; kt < G.KT; ++kt)
    memset(out + block_offset(G, kt, rt, 0), 0, (size_t)G.q * kChunkTile * kRowTile);
}

// Scatter logical sign bytes bits[i][j][c] into the packed order; padding stays zero.
void pack_bits(const Geometry& G, const uint8_t* bits, uint8_t* out) {
  parallel_for(G.RT, [&](int64_t rt0, int64_t rt1) {
    for (int64_t rt = rt0; rt < rt1; ++rt) {
      clear_row_tile(G, rt, out);
      const int64_t rows = (G.N - rt * kRowTile) < kRowTile ? (G.N - rt * kRowTile) : kRowTile;
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t j = rt * kRowTile + r;
        for (int64_t i = 0; i < G.q; ++i) {
          const uint8_t* src = bits + ((size_t)i * G.N + j) * G.C;
          for (int64_t c = 0; c < G.C; ++c) {
            const int64_t kt = c / kChunkTile, cl = c % kChunkTile;
            out[block_offset(G, kt, rt, i) + in_block(r, cl)] = src[c];
          }
        }
      }
    }
  });
}

}  // namespace

extern "C" {

int lutgemm_abi_version(void) { return LUTGEMM_ABI_VERSION; }

const char* lutgemm_status_string(int status) {
  switch (status) {
    case LUTGEMM_OK: return "ok";
    case LUTGEMM_ERR_NULL: return "a required pointer is NULL";
    case LUTGEMM_ERR_SHAPE: return "invalid shape (N, K, q, g, has_offset or m)";
    case LUTGEMM_ERR_VALUE: return "invalid value (code or zero-point out of range, non-finite or overflowing scale)";
    case LUTGEMM_ERR_BUFFER: return "buffer or workspace too small";
    case LUTGEMM_ERR_ALIGN: return "device pointer misaligned";
    case LUTGEMM_ERR_UNSUPPORTED: return "unsupported device (gfx950 required) or feature not in this build";
    case LUTGEMM_ERR_HIP: return "HIP runtime error";
    case LUTGEMM_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

int lutgemm_check_shape(const lutgemm_shape* s) { return check_shape(s); }

int lutgemm_packed_sizes(const lutgemm_shape* s, size_t* bits_bytes, size_t* alpha_count,
                         size_t* offset_count) {
  int st = check_shape(s);
  if (st) return st;
  Geometry G = geometry(s);
  if (bits_bytes) *bits_bytes = G.bits_bytes;
  if (alpha_count) *alpha_count = G.alpha_count;
  if (offset_count) *offset_count = G.offset_count;
  return LUTGEMM_OK;
}

int bcq_pack(const lutgemm_shape* s, const uint8_t* bits, const uint16_t* alpha,
             const uint16_t* offset, uint8_t* out_bits, size_t out_bits_bytes,
             uint16_t* out_alpha, size_t out_alpha_count, uint16_t* out_offset,
             size_t out_offset_count) {
  try {
    int st = check_shape(s);
    if (st) return st;
    Geometry G = geometry(s);
    const size_t n_in_bits = (size_t)G.q * G.N * G.C;
    const size_t n_in_alpha = (size_t)G.q * G.N * G.G;
    const size_t n_in_off = (size_t)G.N * G.G;
    if ((n_in_bits && !bits) || (n_in_alpha && !alpha)) return LUTGEMM_ERR_NULL;
    if (G.has_offset && n_in_off && !offset) return LUTGEMM_ERR_NULL;
    st = check_outputs(G, out_bits, out_bits_bytes, out_alpha, out_alpha_count, out_offset,
                       out_offset_count);
    if (st) return st;
    for (size_t t = 0; t < n_in_alpha; ++t)
      if (!f16_is_finite(alpha[t])) return LUTGEMM_ERR_VALUE;
    if (G.has_offset)
      for (size_t t = 0; t < n_in_off; ++t)
        if (!f16_is_finite(offset[t])) return LUTGEMM_ERR_VALUE;

    if (G.bits_bytes) pack_bits(G, bits, out_bits);
    // alpha: [rt][grp][i][r]  <-  alpha[i][16 rt + r][grp]
    if (G.alpha_count) memset(out_alpha, 0, G.alpha_count * sizeof(uint16_t));
    for (int64_t j = 0; j < G.N; ++j) {
      const int64_t rt = j / kRowTile, r = j % kRowTile;
      for (int64_t grp = 0; grp < G.G; ++grp)
        for (int64_t i = 0; i < G.q; ++i)
          out_alpha[((rt * G.G + grp) * G.q + i) * kRowTile + r] =
              alpha[((size_t)i * G.N + j) * G.G + grp];
    }
    if (G.has_offset && G.offset_count) {
      memset(out_offset, 0, G.offset_count * sizeof(uint16_t));
      for (int64_t j = 0; j < G.N; ++j) {
        const int64_t rt = j / kRowTile, r = j % kRowTile;
        for (int64_t grp = 0; grp < G.G; ++grp)
          out_offset[(rt * G.G + grp) * kRowTile + r] = offset[(size_t)j * G.G + grp];
      }
    }
    return LUTGEMM_OK;
  } catch (const std::bad_alloc&) {
    return LUTGEMM_ERR_INTERNAL;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

int bcq_pack_uniform(const lutgemm_shape* s, const uint8_t* codes, const uint16_t* scale,
                     const uint8_t* zero, uint8_t* out_bits, size_t out_bits_bytes,
                     uint16_t* out_alpha, size_t out_alpha_count, uint16_t* out_offset,
                     size_t out_offset_count, size_t* n_rounded) {
  try {
    int st = check_shape(s);
    if (st) return st;
    if (!s->has_offset) return LUTGEMM_ERR_SHAPE;
    Geometry G = geometry(s);
    const size_t n_codes = (size_t)G.N * G.K;
    const size_t n_grp = (size_t)G.N * G.G;
    if ((n_codes && !codes) || (n_grp && (!scale || !zero))) return LUTGEMM_ERR_NULL;
    st = check_outputs(G, out_bits, out_bits_bytes, out_alpha, out_alpha_count, out_offset,
                       out_offset_count);
    if (st) return st;

    // ---- validate everything first: nothing is written on error
    const unsigned limit = 1u << G.q;
    for (size_t t = 0; t < n_codes; ++t)
      if (codes[t] >= limit) return LUTGEMM_ERR_VALUE;
    std::vector<uint16_t> a16((size_t)G.q * n_grp), o16(n_grp);
    size_t rounded = 0;
    for (size_t t = 0; t < n_grp; ++t) {
      if (!f16_is_finite(scale[t]) || zero[t] >= limit) return LUTGEMM_ERR_VALUE;
      const double sc = f16_to_f64(scale[t]);
      bool inexact = false;
      for (int64_t i = 0; i < G.q; ++i) {
        const double exact = ldexp(sc, (int)i - 1);  // s * 2^(i-1), exact in binary64
        const uint16_t h = f64_to_f16_rne(exact);
        if (!f16_is_finite(h)) return LUTGEMM_ERR_VALUE;
        inexact |= f16_to_f64(h) != exact;
        a16[(size_t)i * n_grp + t] = h;
      }
      // s * ((2^q - 1)/2 - z): a half-integer times an fp16 value, exact in binary64
      const double exact_o = sc * ((double)(limit - 1) * 0.5 - (double)zero[t]);
      const uint16_t ho = f64_to_f16_rne(exact_o);
      if (!f16_is_finite(ho)) return LUTGEMM_ERR_VALUE;
      inexact |= f16_to_f64(ho) != exact_o;
      o16[t] = ho;
      rounded += inexact ? 1 : 0;
    }

    // ---- sign planes: plane i holds bit i of each code
    if (G.bits_bytes) {
      parallel_for(G.RT, [&](int64_t rt0, int64_t rt1) {
        for (int64_t rt = rt0; rt < rt1; ++rt) {
          clear_row_tile(G, rt, out_bits);
          const int64_t rows = (G.N - rt * kRowTile) < kRowTile ? (G.N - rt * kRowTile) : kRowTile;
          for (int64_t r = 0; r < rows; ++r) {
            const uint8_t* row = codes + (size_t)(rt * kRowTile + r) * G.K;
            for (int64_t c = 0; c < G.C; ++c) {
              const int64_t kt = c / kChunkTile, cl = c % kChunkTile;
              for (int64_t i = 0; i < G.q; ++i) {
                unsigned byte = 0;
                for (int t = 0; t < 8; ++t) byte |= ((row[8 * c + t] >> i) & 1u) << t;
                out_bits[block_offset(G, kt, rt, i) + in_block(r, cl)] = (uint8_t)byte;
              }
            }
          }
        }
      });
    }
    if (G.alpha_count) memset(out_alpha, 0, G.alpha_count * sizeof(uint16_t));
    if (G.offset_count) memset(out_offset, 0, G.offset_count * sizeof(uint16_t));
    for (int64_t j = 0; j < G.N; ++j) {
      const int64_t rt = j / kRowTile, r = j % kRowTile;
      for (int64_t grp = 0; grp < G.G; ++grp) {
        const size_t t = (size_t)j * G.G + grp;
        for (int64_t i = 0; i < G.q; ++i)
          out_alpha[((rt * G.G + grp) * G.q + i) * kRowTile + r] = a16[(size_t)i * n_grp + t];
        out_offset[(rt * G.G + grp) * kRowTile + r] = o16[t];
      }
    }
    if (n_rounded) *n_rounded = rounded;
    return LUTGEMM_OK;
  } catch (const std::bad_alloc&) {
    return LUTGEMM_ERR_INTERNAL;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

}  // extern "C"
