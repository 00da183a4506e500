// lutgemv.hip -- host side of the BCQ LUT-GEMV library: argument checks,
// choice of kernel instance and work split, launch, and the C entry points
// declared in lutgemm.h. The kernels are in lutgemv_kernel.h (tables) and
// sign_mfma_kernel.h (the sign planes on the matrix cores).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "layout.h"
#include "lutgemm.h"
#include "lutgemv_kernel.h"
#include "sign_mfma_kernel.h"

namespace lutgemm {

// ------------------------------------------------------------------ scratch
// Device memory of lutgemm_run_noalloc: the split reduction's arrival counters
// (first kCounterBytes) and fp32 partial sums, in a file-scope array that every
// GPU the library runs on holds until the process ends. In host code the name
// `scratch` is only a stand-in: its device address is fetched per device with
// hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void zero_fill_kernel(uint16_t* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

__global__ void zero_bytes_kernel(uint8_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// ------------------------------------------------------------------ dispatch

// ring: >= 3 asks for the deeper ring where an instance has one, 0 for the
// default; xl: the variant with x staged in LDS (batch 1); pr: 1 paired tables,
// 2 half paired tables, 3 split paired tables; ei: the early-issue ring of the x-in-LDS variant; once:
// read-once (non-temporal) sign-plane loads at batch 1 without x in LDS.
KernelFn pick_kernel(int q, int rpw, int mc, bool gq, bool off, int w, int ring, bool xl,
                     int pr = 0, bool ei = false, bool once = false) {
  switch (q) {
    case 1: return kernels_of_q<1>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 2: return kernels_of_q<2>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 3: return kernels_of_q<3>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 4: return kernels_of_q<4>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 5: return kernels_of_q<5>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 6: return kernels_of_q<6>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 7: return kernels_of_q<7>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    case 8: return kernels_of_q<8>(rpw, mc, gq, off, w, ring, xl, pr, ei, once);
    default: return nullptr;
  }
}

// The nibble-table unit kernel for q planes: upw units per wave, ring depth nr
// (0: the deepest built for upw), or nullptr.
KernelFn pick_nibble(int q, bool off, int upw, int nr) {
  switch (q) {
    case 1: return nibble_kernel_of_q<1>(off, upw, nr);
    case 2: return nibble_kernel_of_q<2>(off, upw, nr);
    case 3: return nibble_kernel_of_q<3>(off, upw, nr);
    case 4: return nibble_kernel_of_q<4>(off, upw, nr);
    case 5: return nibble_kernel_of_q<5>(off, upw, nr);
    case 6: return nibble_kernel_of_q<6>(off, upw, nr);
    case 7: return nibble_kernel_of_q<7>(off, upw, nr);
    case 8: return nibble_kernel_of_q<8>(off, upw, nr);
    default: return nullptr;
  }
}


// The sign-plane MFMA kernel for q planes, cg groups of 16 batch rows, an
// offset term, w waves, non-temporal sign loads and x staged once per item
// (xi), or nullptr.
KernelFn pick_sign_mfma(int q, int cg, bool off, int w, bool nt, bool xi = false) {
  switch (q) {
    case 1: return sign_mfma_kernel_of_q<1>(cg, off, w, nt, xi);
    case 2: return sign_mfma_kernel_of_q<2>(cg, off, w, nt, xi);
    case 3: return sign_mfma_kernel_of_q<3>(cg, off, w, nt, xi);
    case 4: return sign_mfma_kernel_of_q<4>(cg, off, w, nt, xi);
    case 5: return sign_mfma_kernel_of_q<5>(cg, off, w, nt, xi);
    case 6: return sign_mfma_kernel_of_q<6>(cg, off, w, nt, xi);
    case 7: return sign_mfma_kernel_of_q<7>(cg, off, w, nt, xi);
    case 8: return sign_mfma_kernel_of_q<8>(cg, off, w, nt, xi);
    default: return nullptr;
  }
}

struct Config {
  int RPW, MC, S, W;
  int RI;                // row tiles per row block (<= W * RPW)
  int ring;              // >= 3: the deeper ring; 0: the instance's default
  bool xl;               // x staged in LDS
  int pr;                // 1: paired tables (two batch rows per table entry), 2: half
                         // paired tables, 3: split paired tables (both double-buffered),
                         // 4: paired tables built by MFMA, 0: none of these
  bool ei;               // early-issue ring (x in LDS, two register sets)
  bool once;             // batch 1 without x in LDS: non-temporal sign-plane loads
  bool us;               // the nibble-table unit kernel (batch 1, few row tiles per CU)
  int upw, nr;           // its units per wave and ring depth
  bool mf;               // the sign-plane MFMA kernel (MC = 16 or 32 batch rows per item)
  int64_t n_rb, n_bg;
  bool gq;
  size_t ws_bytes;
};

// Workspace of a launch whose input dimension is split S ways: the arrival
// counters, then fp32 partial sums [S][m][Npad].
size_t split_ws_bytes(const Geometry& G, int64_t m, int64_t S) {
  return kCounterBytes + (size_t)S * (size_t)m * (size_t)G.Npad * sizeof(float);
}

struct TileOverride {
  int rpw = 0, s = 0, w = 0, mc = 0, ring = 0, ri = 0, xl = -1, pr = -1, ei = -1, us = -1;
};

// Optional tuning override "RPW,S[,W[,MC[,ring[,RI[,XL[,PR[,EI[,US]]]]]]]]" (LUTGEMM_TILE);
// never needed for correctness. XL: 1 stages x in LDS where possible, 0 never
// (default: where possible). PR: 1 paired tables, 2 half paired tables, 3
// split paired tables, 4 paired tables built by MFMA, each where an instance
// has them, 5 the sign-plane MFMA kernel (with W waves, MC = 16 or 32 batch rows
// per item and split S, 0 for its own choice; scale groups of whole 128-input
// step groups), 0 never (default: the dispatcher's choice). EI: 1 the early-issue ring where
// x is staged in LDS with the default ring, 0 never (the default). US: 1 the
// nibble-table unit kernel where it applies (batch 1, scale groups dividing or
// multiples of 512 inputs, x in LDS) with RI row tiles per workgroup (default:
// ceil(row tiles / CUs)) and ring depth `ring` (0: its default), 0 never, -1
// the dispatcher's choice. With US = 1 the other fields are ignored.
bool tile_override(TileOverride* o) {
  const char* e = getenv("LUTGEMM_TILE");
  if (!e || !*e) return false;
  const int n = sscanf(e, "%d,%d,%d,%d,%d,%d,%d,%d,%d,%d", &o->rpw, &o->s, &o->w, &o->mc,
                       &o->ring, &o->ri, &o->xl, &o->pr, &o->ei, &o->us);
  return n >= 2;
}

// The sign-plane MFMA launch (scale groups of whole 128-input step groups):
// w waves of one row tile each per row block, cg groups of 16 batch rows per
// item, and the split of the input tiles s_force, or (s_force < 1) the split
// that gives the busiest CU the fewest tile steps, each item also paying about
// one tile step for its pipeline fill and a split two more for its reduction
// (measured on 12288 x 12288 at m = 4: 85.3 us unsplit on 48 CUs, splits 2, 3,
// 4, 5, 8: 49.8, 37.1, 30.8, 28.7, 36.4 us; on 49152 x 12288 at m = 4, splits
// 1, 2, 4, 5: 84.6, 89.5, 74.9, 77.6 us. A charge of two steps per item had
// kept 49152 x 12288 unsplit on 192 of the 256 CUs; with one it takes split 4
// there, 74.1 against 84.9 us at m = 4, 81.8 against 86.7 at m = 16, and
// 12288 x 12288 at m = 32 split 5, 42.6 against 44.1 us).
// Sign loads are non-temporal when one batch group reads the weights once.
bool mfma_config(const Geometry& G, int64_t m, int cus, size_t max_ws, int w, int cg,
                 int64_t s_force, Config* out) {
  if (G.g % 128 != 0 || cg < 1 || cg > 2) return false;
  const int mc = 16 * cg;
  const int64_t n_bg = (m + mc - 1) / mc;
  if (!pick_sign_mfma((int)G.q, cg, G.has_offset, w, n_bg == 1)) return false;
  const int64_t n_rb = (G.RT + w - 1) / w;
  int64_t best_s = 1;
  if (s_force >= 1) {
    best_s = s_force < G.KT ? s_force : G.KT;
    if ((uint64_t)best_s * (uint64_t)m * (uint64_t)G.Npad * 4u > 0xFFFFFFFFull) best_s = 1;
  } else {
    double best = 1e300;
    const int64_t smax = G.KT < 64 ? G.KT : 64;
    for (int64_t s = 1; s <= smax; ++s) {
      // (the kernel addresses its partials with 32-bit offsets)
      if (s > 1 && (split_ws_bytes(G, m, s) > max_ws ||
                    (uint64_t)s * (uint64_t)m * (uint64_t)G.Npad * 4u > 0xFFFFFFFFull))
        break;
      const int64_t items = n_rb * n_bg * s;
      const int64_t per_cu = (items + cus - 1) / cus;
      const int64_t tiles = (G.KT + s - 1) / s;
      const double cost = (double)per_cu * ((double)tiles + 1.0) + (s > 1 ? 2.0 : 0.0);
      if (cost < best - 1e-9) {
        best = cost;
        best_s = s;
      }
    }
  }
  Config c{};
  c.mf = true;
  c.gq = true;
  c.W = w;
  c.RPW = 1;
  c.MC = mc;
  c.RI = w;
  c.n_rb = n_rb;
  c.n_bg = n_bg;
  c.S = (int)best_s;
  *out = c;
  return true;
}

// Pick waves, rows per wave, batch rows per item, row tiles per item, the
// split of the input tiles and the ring depth. The kernel is persistent (one
// workgroup per CU, LDS-bound), so each of the `cus` compute units works
// through ceil(items / cus) items. Splits whose workspace would exceed
// `max_ws` bytes are not considered (no split needs none).
//
// Batch 1 with grouped scales (the HBM-bound case): when the matrix has
// between 8 and 16 row tiles per CU, each CU takes one row block of
// ceil(row tiles / CUs) row tiles over the whole input dimension, with 16
// waves, x staged in LDS and the early-issue 2-deep ring (or, when x does not
// fit, x from L2 and a 3-deep ring). All CUs then stream the same input tile
// window in step (the best access pattern measured), with no split reduction.
// (The early-issue ring is slower where a CU has several items or the input
// dimension is split, so it is used on this path only.)
//
// Otherwise a cost estimate charges each item its tiles, weighted by the row
// tiles it covers and its batch rows (a tile step of 16 row tiles is one unit;
// 8-wave instances pay for their lower latency hiding), plus a small cost per
// item and one for the split reduction.
Config choose_config(const Geometry& G, int64_t m, int cus, size_t max_ws,
                     bool allow_units = true) {
  Config c{};
  c.gq = (G.g % 32) == 0;
  c.W = 0;   // stays 0 if no instance fits (reported as an internal error)
  c.ring = 0;
  c.xl = false;
  c.pr = 0;
  c.ei = false;
  c.once = false;
  const int q = (int)G.q;
  const bool off = G.has_offset;
  // batch 1 with x small enough: stage it in LDS (16-wave instances)
  const bool xl_ok = m == 1 && G.KT * kChunkTile <= kXChunks;
  const int64_t ri1 = (G.RT + cus - 1) / cus;
  // x in LDS with the 2-deep ring, else the 3-deep ring with x from L2
  const bool xl1 = xl_ok && pick_kernel(q, 1, 1, true, off, 16, 0, true) != nullptr;
  const KernelFn deep = pick_kernel(q, 1, 1, true, off, 16, 3, false);
  const bool has_deep = deep && deep != pick_kernel(q, 1, 1, true, off, 16, 0, false);
  // The nibble-table unit kernel: batch 1, scale groups that divide an input
  // tile or are whole input tiles, x in LDS, and a workgroup of ri1 row tiles
  // with at most 8 (row tile, plane) units (half its waves) over at most 16
  // input tiles (one phase of tables). Measured against the split launch on 14
  // shapes (4096..28672 rows, 512..12288 inputs, q = 1..4): it won or tied
  // on every shape inside these bounds and lost by 5-70% on every shape
  // outside them (more units or a second phase), where the 4-input lookups
  // (two reads and four address operations per weight byte) cost more than
  // the table builds they save.
  const int upw1 = (int)((ri1 * q + 15) / 16);
  const bool us_g = c.gq && (512 % G.g == 0 || G.g % 512 == 0);
  const bool us1 = allow_units && m == 1 && us_g && xl_ok && ri1 * q <= 8 &&
                   G.KT <= kPhaseTiles && pick_nibble(q, off, upw1, 0) != nullptr;
  if (us1) {
    c.us = true;
    c.W = 16;
    c.RPW = 1;
    c.MC = 1;
    c.RI = (int)ri1;
    c.upw = upw1;
    c.nr = 0;
    c.xl = true;
    c.n_rb = (G.RT + ri1 - 1) / ri1;
    c.n_bg = 1;
    c.S = 1;
  } else if (m == 1 && c.gq && ri1 >= 8 && ri1 <= 16 && (xl1 || has_deep)) {
    c.W = 16;
    c.RPW = 1;
    c.MC = 1;
    c.RI = (int)ri1;
    c.ring = xl1 ? 0 : 3;
    c.xl = xl1;
    c.ei = xl1 && pick_kernel(q, 1, 1, true, off, 16, 0, true, false, true) != nullptr;
    c.n_rb = (G.RT + ri1 - 1) / ri1;
    c.n_bg = 1;
    c.S = 1;
  } else {
    double best = 1e300;
    // eff: cost of one input tile per unit of (row tiles x batch rows) / 16;
    // bar: cost of one input tile per batch row of the item (barriers and
    // table builds that serialise); min_m: smallest batch the candidate is
    // considered for. 16-wave paired tables (two batch rows per item, the
    // weights read once for both) are considered from m = 2: with the split
    // this model picks they measured 9-27% faster than 16 waves x 1 row at
    // m = 2..10 (12288 x 12288: 24.9 -> 22.2 us at m = 2, 39.5 -> 34.6 at 4,
    // 68.3 -> 53.8 at 8; 49152 x 12288 at m = 4: 130.2 -> 103.1), the same at
    // m = 16, and the model keeps 16 x 1 at odd m = 3, 5. Their tables are
    // built by MFMA (pr 4): 2.3-5.8% faster than the vector-ALU build at
    // m = 2..32 on 12288 x 12288, with 26% fewer VALU instructions at m = 32.
    struct Cand { int w, rpw, mc; double eff, bar; int pr; int min_m; };
    const Cand cands[] = {
        {16, 2, 1, 1.0, 0.0, false, 1},    {16, 1, 1, 1.0, 0.0, false, 1},
        {16, 1, 2, 0.5, 0.28, 4, 2},      {8, 2, 4, 0.5, 0.425, true, 8},
        {8, 1, 4, 0.5, 0.425, true, 8},    {8, 2, 2, 0.5, 0.425, true, 8},
        {8, 1, 2, 0.5, 0.425, true, 8},    {8, 2, 4, 0.71, 0.31, false, 4},
        {8, 1, 4, 0.71, 0.31, false, 4},   {8, 2, 2, 0.71, 0.31, false, 2},
        {8, 1, 2, 0.71, 0.31, false, 2},   {8, 2, 1, 1.3, 0.0, false, 1},
        {8, 1, 1, 1.3, 0.0, false, 1}};
    double best_eff = 1.0;
    for (const Cand& v : cands) {
      if (m < v.min_m) continue;
      if (!pick_kernel(q, v.rpw, v.mc, c.gq, off, v.w, 0, false, v.pr)) continue;
      const int64_t rows = (int64_t)v.w * v.rpw;            // row tiles per item
      const int64_t n_rb = (G.RT + rows - 1) / rows;
      const int64_t n_bg = (m + v.mc - 1) / v.mc;
      const int64_t smax = G.KT < 64 ? G.KT : 64;
      for (int64_t s = 1; s <= smax; ++s) {
        if (s > 1 && split_ws_bytes(G, m, s) > max_ws) break;
        const int64_t items = n_rb * n_bg * s;
        const int64_t per_cu = (items + cus - 1) / cus;
        const int64_t tiles = (G.KT + s - 1) / s;
        const double unit = v.eff * (double)rows * v.mc / 16.0;
        const double step = unit + v.bar * v.mc;
        // per item: filling and draining the pipeline, about one tile step for
        // several batch rows (measured: short batched items lose to long ones)
        const double fix = v.mc > 1 ? step : 0.3 * unit;
        const double cost = (double)per_cu * (tiles * step + fix) + (s > 1 ? 2.0 : 0.0);
        if (cost < best - 1e-9) {
          best = cost;
          best_eff = v.eff;
          c.W = v.w;
          c.RPW = v.rpw;
          c.MC = v.mc;
          c.pr = v.pr;
          c.RI = (int)rows;
          c.n_rb = n_rb;
          c.n_bg = n_bg;
          c.S = (int)s;
        }
      }
    }
    // Batch 1: a row block of 8 to 16 row tiles on 16 waves, sized so that the
    // items of a split just fill the compute units (waves past the block's row
    // tiles only help build the tables). Compared with the choice above by the
    // same cost with a fixed cost per tile step added (0.6 of a 16-row-tile
    // step: the latency of a step that does not depend on its bytes), which
    // the choice above leaves out. Measured: on 6144 x 12288 with the bytes
    // per CU held fixed, 3 steps of 12 row tiles 11.4 us against 6 steps of 6
    // 13.6 us; on 12288 x 12288, 5 steps of 16 row tiles (240 items) 15.9 us
    // against 6 steps of 12 (256 items) 16.3 us. Chosen by it: 22016 x 4096
    // (q = 3) 12.8 against 14.0 us, 28672 x 8192 (q = 4, g = 32) 32.6 against
    // 36.1, 6144 x 12288 11.5 against 11.9, 12288 x 4096 9.7 against 9.9.
    if (m == 1 && c.W > 0 && !c.pr && c.MC == 1 &&
        pick_kernel(q, 1, 1, c.gq, off, 16, 0, false, 0) != nullptr) {
      constexpr double kStepFix = 0.6;
      auto cost_of = [&](int64_t rows, int64_t s, double eff) {
        const int64_t items = ((G.RT + rows - 1) / rows) * s;
        const int64_t per_cu = (items + cus - 1) / cus;
        const int64_t tiles = (G.KT + s - 1) / s;
        const double unit = eff * (double)rows / 16.0;
        return (double)per_cu * (tiles * (unit + kStepFix) + 0.3 * unit) + (s > 1 ? 2.0 : 0.0);
      };
      double best2 = cost_of(c.RI, c.S, best_eff);
      const int64_t smax = G.KT < 64 ? G.KT : 64;
      for (int64_t s = 1; s <= smax && s <= cus; ++s) {
        if (s > 1 && split_ws_bytes(G, m, s) > max_ws) break;
        const int64_t per_s = cus / s;
        int64_t ri = (G.RT + per_s - 1) / per_s;
        ri = ri < 8 ? 8 : (ri > 16 ? 16 : ri);
        const int64_t n_rb = (G.RT + ri - 1) / ri;
        if (n_rb > kMaxCounters) continue;
        const double cost = cost_of(ri, s, 1.0);
        if (cost < best2 - 1e-9) {
          best2 = cost;
          c.W = 16;
          c.RPW = 1;
          c.MC = 1;
          c.pr = 0;
          c.RI = (int)ri;
          c.n_rb = n_rb;
          c.n_bg = 1;
          c.S = (int)s;
        }
      }
    }
    c.xl = !c.pr && xl_ok && pick_kernel(q, c.RPW, c.MC, c.gq, off, c.W, 0, true) != nullptr;
  }
  TileOverride o;
  const bool have_o = tile_override(&o);
  // the unit kernel declined: the choice without it (which applies the
  // override's other fields itself)
  if (have_o && o.us == 0 && c.us) return choose_config(G, m, cus, max_ws, false);
  if (have_o && o.us == 1) {
    const int64_t ri = (o.ri >= 1 && o.ri <= 64) ? o.ri : ri1;
    const int upw = (int)((ri * q + 15) / 16);
    if (m == 1 && us_g && xl_ok && pick_nibble(q, off, upw, o.ring)) {
      c = Config{};
      c.gq = true;
      c.us = true;
      c.W = 16;
      c.RPW = 1;
      c.MC = 1;
      c.RI = (int)ri;
      c.upw = upw;
      c.nr = o.ring;
      c.xl = true;
      c.n_rb = (G.RT + ri - 1) / ri;
      c.n_bg = 1;
      c.S = 1;
      c.ws_bytes = 0;
      return c;
    }
  } else if (have_o && o.pr == 5) {
    // the sign-plane MFMA kernel: W waves (default 16), MC = 16 or 32 batch
    // rows per item (default: 32 from m = 17 on), split S (0: its own choice)
    // (fields left at 0 fall back, in this order, to 8 waves and then to one
    // group of 16 batch rows where an instance with more is not built)
    Config f{};
    const int cg = o.mc ? (o.mc > 16 ? 2 : 1) : (m > 16 ? 2 : 1);
    bool ok = false;
    for (int k = 0; k < 4 && !ok; ++k) {
      const int w = k % 2 ? 8 : 16, g2 = k < 2 ? cg : 1;
      if ((o.w && w != o.w) || (o.mc && g2 != cg)) continue;
      ok = mfma_config(G, m, cus, max_ws, w, g2, o.s, &f);
    }
    if (ok) c = f;
  } else if (have_o) {
    const int w = o.w ? o.w : c.W;
    const int mc = o.mc ? o.mc : c.MC;
    const int pr = o.pr >= 1 && o.pr <= 4 ? o.pr : 0;
    const bool xl = pr ? false
                    : o.xl < 0 ? xl_ok && pick_kernel(q, o.rpw, mc, c.gq, off, w, o.ring, true)
                               : (o.xl > 0 && xl_ok);
    const bool ei = o.ei > 0 && xl && o.ring < 3 &&
                    pick_kernel(q, o.rpw, mc, c.gq, off, w, o.ring, xl, pr, true) != nullptr;
    if (pick_kernel(q, o.rpw, mc, c.gq, off, w, o.ring, xl, pr)) {
      c.us = false;
      c.W = w;
      c.RPW = o.rpw;
      c.MC = mc;
      c.ring = o.ring;
      c.xl = xl;
      c.pr = pr;
      c.ei = ei;
      c.RI = (o.ri >= 1 && o.ri <= c.W * c.RPW) ? o.ri : c.W * c.RPW;
      c.n_rb = (G.RT + c.RI - 1) / c.RI;
      c.n_bg = (m + c.MC - 1) / c.MC;
    }
    if (o.s >= 1) c.S = (int)(o.s < G.KT ? o.s : (G.KT > 0 ? G.KT : 1));
  }
  // With scale groups of whole 128-input step groups, the sign-plane MFMA
  // kernel (16 waves, 16 batch rows per item where built):
  // on 12288 x 12288 it measured 28.7 / 29.6 / 32.2 / 53.4 us at m = 4 / 8 /
  // 16 / 32 against 33.2 / 51.9 / 93.0 / 170.4 us for the best table launch;
  // at m = 2 the paired tables stay faster (21.2 against 28.1 us).
  // Past 16 batch rows, where 32-row items pad the batch no more than 16-row
  // ones and the 8-wave instance reads its operands a step ahead (at most 3
  // planes, the offset counted as one), 8 waves with 32 batch rows per item:
  // each sign vector then serves two MFMAs. Measured against 16 waves x 16
  // rows: 12288 x 12288 q = 3 at m = 24 / 32 / 64 43.1 / 44.2 / 75.8 against
  // 48.3 / 48.7 / 84.3 us, q = 2 at m = 32 36.2 against 40.2, 49152 x 12288
  // and 12288 x 49152 at m = 32 125.7 / 125.1 against 151.9 / 151.7; not at
  // m = 48 (75.6 against 66.0, the second group half empty) or q = 4 (58.8
  // against 58.0, no read-ahead).
  // From 3 batch rows on where the matrix holds at least 6144 (row tile,
  // input tile) units, and from 6 on always: on smaller matrices at m = 3..5
  // the table launches are faster (the sign table and the fill are fixed costs
  // that few tiles per CU do not amortise). Measured, tables against the
  // sign-plane MFMA kernel: at m = 3 4096 x 4096 9.8 / 13.5 us, 5120 x 5120
  // 11.6 / 14.9, 4096 x 11008 15.0 / 16.6, but 12288 x 4096 17.9 / 15.3,
  // 12288 x 12288 33.7 / 25.2, 49152 x 12288 107.7 / 85.0; at m = 4 4096 x
  // 11008 14.8 / 16.7, 4096 x 14336 18.8 / 17.7; at m = 6 and 8 4096 x 4096
  // within 2%, 4096 x 11008 19.0 / 16.8 and 21.1 / 17.0.
  if (!have_o && m >= 3 && (m >= 6 || G.RT * G.KT >= 6144)) {
    Config f{};
    const bool cg2 = m > 16 && (m + 31) / 32 * 32 <= (m + 15) / 16 * 16 &&
                     (q + (off ? 1 : 0)) * 2 <= 6;
    if ((cg2 && mfma_config(G, m, cus, max_ws, 8, 2, 0, &f)) ||
        mfma_config(G, m, cus, max_ws, 16, 1, 0, &f) || mfma_config(G, m, cus, max_ws, 8, 1, 0, &f))
      c = f;
  }
  if (c.S < 1) c.S = 1;
  if (c.S > 1 && split_ws_bytes(G, m, c.S) > max_ws) c.S = 1;
  if (c.n_rb * c.n_bg > kMaxCounters) c.S = 1;   // counters live in a fixed region
  // The sign-plane MFMA kernel stages x once per item instead of once per
  // input tile (no barrier in its tile loop) where the launch has one group of
  // 16 batch rows per item, no more items than compute units and at most
  // kXITiles input tiles per item; LUTGEMM_TILE field XL = 0 declines it.
  // 12288 x 12288 at m = 4 / 8 / 16 (split 5): see the kernel.
  if (c.mf) {
    const int64_t items = c.n_rb * c.n_bg * c.S;
    const int64_t tiles = (G.KT + c.S - 1) / c.S;
    c.xl = c.MC == 16 && items <= cus && tiles <= kXITiles && !(have_o && o.xl == 0) &&
           pick_sign_mfma(q, 1, off, c.W, c.n_bg == 1, true) != nullptr;
  }
  // batch 1 without x in LDS: each sign byte is still read once per product
  // (where a read-once instance exists for the choice, it differs from the
  // ordinary one)
  c.once = m == 1 && !c.xl && !c.pr && !c.mf && c.MC == 1 &&
           pick_kernel(q, c.RPW, c.MC, c.gq, off, c.W, c.ring, false, false, false, true) !=
               pick_kernel(q, c.RPW, c.MC, c.gq, off, c.W, c.ring, false, false, false, false);
  c.ws_bytes = c.S > 1 ? split_ws_bytes(G, m, c.S) : 0;
  return c;
}

std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[64];       // compute units of the device, 0 unknown

// The current device must be gfx950. LUTGEMM_FAKE_ARCH, a debugging aid,
// replaces the name the device reports (so the refusal path can be exercised
// on the real part); it is read on every call and bypasses the cache.
int check_device(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LUTGEMM_ERR_HIP;
  const bool cached = dev >= 0 && dev < 64;
  const char* fake = getenv("LUTGEMM_FAKE_ARCH");
  int known = (cached && !(fake && *fake)) ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
  int n = cached ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (known == 0 || n <= 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LUTGEMM_ERR_HIP;
    const char* name = (fake && *fake) ? fake : prop.gcnArchName;
    known = strncmp(name, "gfx950", 6) == 0 ? 1 : 2;
    n = prop.multiProcessorCount;
    if (n <= 0) return LUTGEMM_ERR_HIP;
    if (cached && !(fake && *fake)) {
      g_arch_ok[dev].store(known, std::memory_order_relaxed);
      g_cus[dev].store(n, std::memory_order_relaxed);
    }
  }
  *cus = n;
  return known == 1 ? LUTGEMM_OK : LUTGEMM_ERR_UNSUPPORTED;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The kernel addresses each input buffer with 32-bit offsets from its base
// (descriptor sizes are offset + extent, so the buffers stay below 4 GiB).
bool buffers_fit(const Geometry& G, int64_t m) {
  const uint64_t lim = 0xFFFFFFFFull;
  return G.bits_bytes <= lim && G.alpha_count * 2 <= lim && G.offset_count * 2 <= lim &&
         (uint64_t)m * (uint64_t)G.K * 2 <= lim;
}

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[64];     // device address of `scratch`, per device
std::atomic<int> g_scratch_zeroed[64];    // counters cleared on a stream not being captured

// The device address of this device's scratch, fetched once per device (with
// that device current); the first call also clears the arrival counters with
// a kernel on `strm`, so this call's launch, which follows on the same stream,
// finds them zero. A clear recorded into a graph being captured does not count:
// the next call outside a capture clears them again.
int device_scratch(int dev, hipStream_t strm, void** out) {
  if (dev < 0 || dev >= 64) return LUTGEMM_ERR_UNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr || !g_scratch_zeroed[dev].load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LUTGEMM_ERR_HIP;
      ptr = p;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    if (!g_scratch_zeroed[dev].load(std::memory_order_relaxed)) {
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(strm, &cap) != hipSuccess) {
        (void)hipGetLastError();               // unknown: clear again next time
        cap = hipStreamCaptureStatusActive;
      }
      hipLaunchKernelGGL(zero_bytes_kernel, dim3((unsigned)(kCounterBytes / 256)), dim3(256), 0,
                         strm, (uint8_t*)ptr, kCounterBytes);
      if (hipGetLastError() != hipSuccess) return LUTGEMM_ERR_HIP;
      if (cap == hipStreamCaptureStatusNone) g_scratch_zeroed[dev].store(1, std::memory_order_release);
    }
  }
  *out = ptr;
  return LUTGEMM_OK;
}

// Enqueue the product for a validated shape and configuration (K > 0): the
// kernel instance, its parameters and its persistent grid of min(items, cus)
// workgroups. `ws` is the workspace of a split launch (counters, then partials).
// Phase-trace buffer (traced builds only; see lutgemm_trace_attach).
std::atomic<unsigned long long*> g_trace{nullptr};
std::atomic<int64_t> g_trace_wgs{0};

int launch(const Geometry& G, int64_t m, const Config& c, int cus, const void* d_bits,
           const void* d_alpha, const void* d_offset, const void* d_x, void* d_y, void* ws,
           hipStream_t strm) {
  KernelFn fn = c.us ? pick_nibble((int)G.q, G.has_offset, c.upw, c.nr)
                : c.mf ? pick_sign_mfma((int)G.q, c.MC / 16, G.has_offset, c.W, c.n_bg == 1, c.xl)
                       : pick_kernel((int)G.q, c.RPW, c.MC, c.gq, G.has_offset, c.W, c.ring, c.xl,
                                     c.pr, c.ei, c.once);
  if (!fn) return LUTGEMM_ERR_INTERNAL;
  Params p{};
  p.trace = g_trace.load(std::memory_order_relaxed);
  p.trace_wgs = (int)g_trace_wgs.load(std::memory_order_relaxed);
  p.bits = (const uint8_t*)d_bits;
  p.alpha = (const uint32_t*)d_alpha;
  p.offset = G.has_offset ? (const uint32_t*)d_offset : nullptr;
  p.x = (const uint16_t*)d_x;
  p.y = (uint16_t*)d_y;
  p.counters = c.S > 1 ? (uint32_t*)ws : nullptr;
  p.partial = c.S > 1 ? (float*)((char*)ws + kCounterBytes) : nullptr;
  p.N = (int)G.N;
  p.K = (int)G.K;
  p.g = (int)G.g;
  p.m = (int)m;
  p.C = (int)G.C;
  p.KT = (int)G.KT;
  p.RT = (int)G.RT;
  p.G = (int)G.G;
  p.S = c.S;
  p.Npad = (int)G.Npad;
  p.n_rb = (int)c.n_rb;
  p.ri = c.RI;
  p.g_shift = -1;
  for (int b = 3; b < 31; ++b)
    if (((int64_t)1 << b) == G.g) p.g_shift = b;
  p.g_span = (int)((kChunkTile * 8 + G.g - 1) / G.g + 1);
  p.g_tile = (kChunkTile * 8) % G.g == 0 ? 1 : 0;
  p.n_bg = (int)c.n_bg;
  // Batch groups of one weight block side by side on one XCD (see decode_item):
  // measured 0.7-1.8 us faster at 2 and 3 batch groups of one-row items; at 4
  // it moved by -0.8..+0.3 us from one machine to another, and with paired tables at 4..16
  // groups it was slower (each round then streams few distinct blocks).
  p.xcd_bg = (!c.pr && !c.mf && c.n_bg > 1 && c.n_bg <= 3 && (c.n_rb * c.S) % 8 == 0) ? 1 : 0;
  const int64_t items = c.n_rb * c.n_bg * c.S;
  if (items > 0x7FFFFFFF - (int64_t)cus) return LUTGEMM_ERR_SHAPE;
  p.n_items = (int)items;
  // the unit kernel runs one item per workgroup; the others are persistent
  dim3 grid((unsigned)(c.us ? items : (items < cus ? items : cus)));
  void* args[] = {&p};
  if (hipLaunchKernel((const void*)fn, grid, dim3(64 * c.W), args, 0, strm) != hipSuccess)
    return LUTGEMM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
}

// y = 0 for an empty reduction (K = 0).
int launch_zero_y(void* d_y, size_t n, hipStream_t strm) {
  const size_t want = (n + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, strm, (uint16_t*)d_y, n);
  return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
}

// Checks shared by the entry points that run a product: shape, batch, buffer
// limits and the pointers and alignments of the operands (not the workspace).
// Returns LUTGEMM_OK with *nothing = 1 when there is no output to write.
int check_operands(const lutgemm_shape* s, int32_t m, const void* d_bits, const void* d_alpha,
                   const void* d_offset, const void* d_x, const void* d_y, Geometry* G,
                   int* nothing) {
  *nothing = 0;
  int st = check_shape(s);
  if (st) return st;
  if (m < 0 || m > kMaxBatch) return LUTGEMM_ERR_SHAPE;
  *G = geometry(s);
  if (!buffers_fit(*G, m)) return LUTGEMM_ERR_SHAPE;
  if (m == 0 || G->N == 0) {
    *nothing = 1;
    return LUTGEMM_OK;
  }
  if (!d_y) return LUTGEMM_ERR_NULL;
  if (!aligned(d_y, 2)) return LUTGEMM_ERR_ALIGN;
  if (G->K > 0) {
    if (!d_bits || !d_alpha || !d_x || (G->has_offset && !d_offset)) return LUTGEMM_ERR_NULL;
    if (!aligned(d_bits, 16) || !aligned(d_x, 16) || !aligned(d_alpha, 4) ||
        (G->has_offset && !aligned(d_offset, 4)))
      return LUTGEMM_ERR_ALIGN;
  }
  return LUTGEMM_OK;
}

}  // namespace
}  // namespace lutgemm

using namespace lutgemm;

extern "C" {

int lutgemm_workspace_size(const lutgemm_shape* s, int32_t m, size_t* bytes) {
  int st = check_shape(s);
  if (st) return st;
  if (!bytes) return LUTGEMM_ERR_NULL;
  if (m < 0 || m > kMaxBatch) return LUTGEMM_ERR_SHAPE;
  Geometry G = geometry(s);
  *bytes = 0;
  if (!buffers_fit(G, m)) return LUTGEMM_ERR_SHAPE;
  if (m == 0 || G.N == 0 || G.K == 0) return LUTGEMM_OK;
  const Config c = choose_config(G, m, kNominalCUs, SIZE_MAX);
  if (c.W == 0) return LUTGEMM_ERR_INTERNAL;
  *bytes = c.ws_bytes;
  return LUTGEMM_OK;
}

int lutgemm_workspace_init(void* d_workspace, size_t bytes, void* stream) {
  if (bytes == 0) return LUTGEMM_OK;
  if (!d_workspace) return LUTGEMM_ERR_NULL;
  const size_t want = (bytes + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(zero_bytes_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint8_t*)d_workspace, bytes);
  return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
}

int lutgemm_run(const lutgemm_shape* s, int32_t m, const void* d_bits, const void* d_alpha,
                const void* d_offset, const void* d_x, void* d_y, void* d_workspace,
                size_t workspace_bytes, void* stream) {
  try {
    Geometry G{};
    int nothing = 0;
    int st = check_operands(s, m, d_bits, d_alpha, d_offset, d_x, d_y, &G, &nothing);
    if (st || nothing) return st;
    // the workspace the size query promised for this shape (a full 256-CU part)
    Config c{};
    if (G.K > 0) {
      c = choose_config(G, m, kNominalCUs, SIZE_MAX);
      if (c.W == 0) return LUTGEMM_ERR_INTERNAL;
      if (c.ws_bytes) {
        if (!d_workspace) return LUTGEMM_ERR_NULL;
        if (workspace_bytes < c.ws_bytes) return LUTGEMM_ERR_BUFFER;
        if (!aligned(d_workspace, 16)) return LUTGEMM_ERR_ALIGN;
      }
    }
    int cus = 0;
    st = check_device(&cus);
    if (st) return st;
    hipStream_t strm = (hipStream_t)stream;
    if (G.K == 0) return launch_zero_y(d_y, (size_t)m * G.N, strm);
    // a device with another number of compute units gets its own choice, with
    // its split limited to the workspace passed
    if (cus != kNominalCUs) {
      c = choose_config(G, m, cus, d_workspace ? workspace_bytes : 0);
      if (c.W == 0) return LUTGEMM_ERR_INTERNAL;
    }
    return launch(G, m, c, cus, d_bits, d_alpha, d_offset, d_x, d_y, d_workspace, strm);
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

int lutgemm_trace_attach(void* d_buffer, size_t bytes) {
#ifdef LUTGEMM_PHASE_TRACE
  if (d_buffer && ((uintptr_t)d_buffer & 7)) return LUTGEMM_ERR_ALIGN;
  const size_t per_wg = (size_t)kTracePoints * sizeof(unsigned long long);
  const size_t wgs = d_buffer ? bytes / per_wg : 0;
  g_trace_wgs.store((int64_t)(wgs < 0x7FFFFFFF ? wgs : 0x7FFFFFFF), std::memory_order_relaxed);
  g_trace.store(d_buffer ? (unsigned long long*)d_buffer : nullptr, std::memory_order_relaxed);
  return LUTGEMM_OK;
#else
  (void)d_buffer;
  (void)bytes;
  return LUTGEMM_ERR_UNSUPPORTED;
#endif
}

int lutgemm_query_plan(const lutgemm_shape* s, int32_t m, int32_t cus, size_t workspace_bytes,
                       lutgemm_plan* out) {
  try {
    if (!s || !out) return LUTGEMM_ERR_NULL;
    int st = check_shape(s);
    if (st) return st;
    if (m < 0 || m > kMaxBatch || cus < 1) return LUTGEMM_ERR_SHAPE;
    const Geometry G = geometry(s);
    if (!buffers_fit(G, m)) return LUTGEMM_ERR_SHAPE;
    *out = lutgemm_plan{};
    if (m == 0 || G.N == 0 || G.K == 0) return LUTGEMM_OK;
    const Config c = choose_config(G, m, cus, workspace_bytes);
    if (c.W == 0) return LUTGEMM_ERR_INTERNAL;
    out->tables = c.us ? LUTGEMM_TABLES_NIBBLE
                  : c.mf ? LUTGEMM_TABLES_SIGN_MFMA
                  : c.pr == 3 ? LUTGEMM_TABLES_SPLIT
                  : c.pr == 4 ? LUTGEMM_TABLES_PAIRED_MFMA
                  : c.pr == 2 ? LUTGEMM_TABLES_HALF
                  : c.pr == 1 ? LUTGEMM_TABLES_PAIRED
                              : LUTGEMM_TABLES_SINGLE;
    out->waves = c.W;
    out->rows_per_wave = c.RPW;
    out->batch_rows = c.MC;
    out->row_tiles = c.RI;
    out->split = c.S;
    out->x_in_lds = c.xl ? 1 : 0;
    out->items = c.n_rb * c.n_bg * c.S;
    out->workgroups = c.us ? out->items : (out->items < cus ? out->items : cus);
    out->workspace_bytes = c.ws_bytes;
    return LUTGEMM_OK;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

int lutgemm_run_noalloc(const lutgemm_shape* s, int32_t m, const void* d_bits,
                        const void* d_alpha, const void* d_offset, const void* d_x, void* d_y,
                        void* stream) {
  try {
    Geometry G{};
    int nothing = 0;
    int st = check_operands(s, m, d_bits, d_alpha, d_offset, d_x, d_y, &G, &nothing);
    if (st || nothing) return st;
    // a split forced by the tuning override is refused, not changed, when its
    // workspace would not fit the scratch
    if (G.K > 0) {
      const Config forced = choose_config(G, m, kNominalCUs, SIZE_MAX);
      if (forced.W == 0) return LUTGEMM_ERR_INTERNAL;
      TileOverride o;
      if (tile_override(&o) && o.s > 1 && forced.ws_bytes > kScratchBytes) return LUTGEMM_ERR_BUFFER;
    }
    int cus = 0;
    st = check_device(&cus);
    if (st) return st;
    hipStream_t strm = (hipStream_t)stream;
    if (G.K == 0) return launch_zero_y(d_y, (size_t)m * G.N, strm);
    const Config c = choose_config(G, m, cus, kScratchBytes);
    if (c.W == 0) return LUTGEMM_ERR_INTERNAL;
    if (c.ws_bytes > kScratchBytes) return LUTGEMM_ERR_BUFFER;
    void* ws = nullptr;
    if (c.ws_bytes) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess) return LUTGEMM_ERR_HIP;
      st = device_scratch(dev, strm, &ws);
      if (st) return st;
    }
    return launch(G, m, c, cus, d_bits, d_alpha, d_offset, d_x, d_y, ws, strm);
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

size_t lutgemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
