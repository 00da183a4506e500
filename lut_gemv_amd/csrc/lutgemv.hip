// lutgemv.hip -- host side of the BCQ LUT-GEMV library: argument checks,
// choice of kernel instance and work split, launch, and the C entry points
// declared in lutgemm.h. The kernel itself is in lutgemv_kernel.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "layout.h"
#include "lutgemm.h"
#include "lutgemv_kernel.h"

namespace lutgemm {
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
// default; xl: the variant with x staged in LDS (batch 1); pr: paired tables;
// ei: the early-issue ring of the x-in-LDS variant; once: read-once
// (non-temporal) sign-plane loads at batch 1 without x in LDS.
KernelFn pick_kernel(int q, int rpw, int mc, bool gq, bool off, int w, int ring, bool xl,
                     bool pr = false, bool ei = false, bool once = false) {
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

struct Config {
  int RPW, MC, S, W;
  int RI;                // row tiles per row block (<= W * RPW)
  int ring;              // >= 3: the deeper ring; 0: the instance's default
  bool xl;               // x staged in LDS
  bool pr;               // paired tables (two batch rows per table entry)
  bool ei;               // early-issue ring (x in LDS, two register sets)
  bool once;             // batch 1 without x in LDS: non-temporal sign-plane loads
  int64_t n_rb, n_bg;
  bool gq;
  size_t ws_bytes;
};

struct TileOverride {
  int rpw = 0, s = 0, w = 0, mc = 0, ring = 0, ri = 0, xl = -1, pr = -1, ei = -1;
};

// Optional tuning override "RPW,S[,W[,MC[,ring[,RI[,XL[,PR[,EI]]]]]]]" (LUTGEMM_TILE);
// never needed for correctness. XL: 1 stages x in LDS where possible, 0 never
// (default: where possible). PR: 1 paired tables where an instance has them, 0
// never (default: the dispatcher's choice). EI: 1 the early-issue ring where
// x is staged in LDS with the default ring, 0 never (the default).
bool tile_override(TileOverride* o) {
  const char* e = getenv("LUTGEMM_TILE");
  if (!e || !*e) return false;
  const int n = sscanf(e, "%d,%d,%d,%d,%d,%d,%d,%d,%d", &o->rpw, &o->s, &o->w, &o->mc, &o->ring,
                       &o->ri, &o->xl, &o->pr, &o->ei);
  return n >= 2;
}

// Pick waves, rows per wave, batch rows per item, row tiles per item, the
// split of the input tiles and the ring depth. The kernel is persistent (one
// workgroup per CU, LDS-bound), so each CU works through ceil(items / kCUs)
// items.
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
Config choose_config(const Geometry& G, int64_t m) {
  Config c{};
  c.gq = (G.g % 32) == 0;
  c.W = 0;   // stays 0 if no instance fits (reported as an internal error)
  c.ring = 0;
  c.xl = false;
  c.pr = false;
  c.ei = false;
  c.once = false;
  const int q = (int)G.q;
  const bool off = G.has_offset;
  // batch 1 with x small enough: stage it in LDS (16-wave instances)
  const bool xl_ok = m == 1 && G.KT * kChunkTile <= kXChunks;
  const int64_t ri1 = (G.RT + kCUs - 1) / kCUs;
  // x in LDS with the 2-deep ring, else the 3-deep ring with x from L2
  const bool xl1 = xl_ok && pick_kernel(q, 1, 1, true, off, 16, 0, true) != nullptr;
  const KernelFn deep = pick_kernel(q, 1, 1, true, off, 16, 3, false);
  const bool has_deep = deep && deep != pick_kernel(q, 1, 1, true, off, 16, 0, false);
  if (m == 1 && c.gq && ri1 >= 8 && ri1 <= 16 && (xl1 || has_deep)) {
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
    // considered for. Measured on 12288 x 12288, m = 4..32: paired tables lost
    // to 16 waves x 1 row at m = 4, and 16-wave paired instances to 8-wave ones
    // at m = 8 (they win from m = 12 on).
    struct Cand { int w, rpw, mc; double eff, bar; bool pr; int min_m; };
    const Cand cands[] = {
        {16, 2, 1, 1.0, 0.0, false, 1},    {16, 1, 1, 1.0, 0.0, false, 1},
        {16, 1, 2, 0.5, 0.28, true, 12},   {8, 2, 4, 0.5, 0.425, true, 8},
        {8, 1, 4, 0.5, 0.425, true, 8},    {8, 2, 2, 0.5, 0.425, true, 8},
        {8, 1, 2, 0.5, 0.425, true, 8},    {8, 2, 4, 0.71, 0.31, false, 4},
        {8, 1, 4, 0.71, 0.31, false, 4},   {8, 2, 2, 0.71, 0.31, false, 2},
        {8, 1, 2, 0.71, 0.31, false, 2},   {8, 2, 1, 1.3, 0.0, false, 1},
        {8, 1, 1, 1.3, 0.0, false, 1}};
    for (const Cand& v : cands) {
      if (m < v.min_m) continue;
      if (!pick_kernel(q, v.rpw, v.mc, c.gq, off, v.w, 0, false, v.pr)) continue;
      const int64_t rows = (int64_t)v.w * v.rpw;            // row tiles per item
      const int64_t n_rb = (G.RT + rows - 1) / rows;
      const int64_t n_bg = (m + v.mc - 1) / v.mc;
      const int64_t smax = G.KT < 64 ? G.KT : 64;
      for (int64_t s = 1; s <= smax; ++s) {
        const int64_t items = n_rb * n_bg * s;
        const int64_t per_cu = (items + kCUs - 1) / kCUs;
        const int64_t tiles = (G.KT + s - 1) / s;
        const double unit = v.eff * (double)rows * v.mc / 16.0;
        const double step = unit + v.bar * v.mc;
        // per item: filling and draining the pipeline, about one tile step for
        // several batch rows (measured: short batched items lose to long ones)
        const double fix = v.mc > 1 ? step : 0.3 * unit;
        const double cost = (double)per_cu * (tiles * step + fix) + (s > 1 ? 2.0 : 0.0);
        if (cost < best - 1e-9) {
          best = cost;
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
    c.xl = !c.pr && xl_ok && pick_kernel(q, c.RPW, c.MC, c.gq, off, c.W, 0, true) != nullptr;
  }
  TileOverride o;
  if (tile_override(&o)) {
    const int w = o.w ? o.w : c.W;
    const int mc = o.mc ? o.mc : c.MC;
    const bool pr = o.pr > 0;
    const bool xl = pr ? false
                    : o.xl < 0 ? xl_ok && pick_kernel(q, o.rpw, mc, c.gq, off, w, o.ring, true)
                               : (o.xl > 0 && xl_ok);
    const bool ei = o.ei > 0 && xl && o.ring < 3 &&
                    pick_kernel(q, o.rpw, mc, c.gq, off, w, o.ring, xl, pr, true) != nullptr;
    if (pick_kernel(q, o.rpw, mc, c.gq, off, w, o.ring, xl, pr)) {
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
  if (c.S < 1) c.S = 1;
  if (c.n_rb * c.n_bg > kMaxCounters) c.S = 1;   // counters live in a fixed region
  // batch 1 without x in LDS: each sign byte is still read once per product
  // (where a read-once instance exists for the choice, it differs from the
  // ordinary one)
  c.once = m == 1 && !c.xl && !c.pr && c.MC == 1 &&
           pick_kernel(q, c.RPW, c.MC, c.gq, off, c.W, c.ring, false, false, false, true) !=
               pick_kernel(q, c.RPW, c.MC, c.gq, off, c.W, c.ring, false, false, false, false);
  c.ws_bytes = c.S > 1 ? kCounterBytes + (size_t)c.S * (size_t)m * (size_t)G.Npad * sizeof(float) : 0;
  return c;
}

std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LUTGEMM_ERR_HIP;
  int known = (dev >= 0 && dev < 64) ? g_arch_ok[dev].load(std::memory_order_relaxed) : 0;
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LUTGEMM_ERR_HIP;
    known = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (dev >= 0 && dev < 64) g_arch_ok[dev].store(known, std::memory_order_relaxed);
  }
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
  const Config c = choose_config(G, m);
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
    int st = check_shape(s);
    if (st) return st;
    if (m < 0 || m > kMaxBatch) return LUTGEMM_ERR_SHAPE;
    Geometry G = geometry(s);
    if (!buffers_fit(G, m)) return LUTGEMM_ERR_SHAPE;
    if (m == 0 || G.N == 0) return LUTGEMM_OK;
    if (!d_y) return LUTGEMM_ERR_NULL;
    if (!aligned(d_y, 2)) return LUTGEMM_ERR_ALIGN;
    Config c{};
    if (G.K > 0) {
      if (!d_bits || !d_alpha || !d_x || (G.has_offset && !d_offset)) return LUTGEMM_ERR_NULL;
      if (!aligned(d_bits, 16) || !aligned(d_x, 16) || !aligned(d_alpha, 4) ||
          (G.has_offset && !aligned(d_offset, 4)))
        return LUTGEMM_ERR_ALIGN;
      c = choose_config(G, m);
      if (c.W == 0) return LUTGEMM_ERR_INTERNAL;
      if (c.ws_bytes) {
        if (!d_workspace) return LUTGEMM_ERR_NULL;
        if (workspace_bytes < c.ws_bytes) return LUTGEMM_ERR_BUFFER;
        if (!aligned(d_workspace, 16)) return LUTGEMM_ERR_ALIGN;
      }
    }
    st = check_device();
    if (st) return st;
    hipStream_t strm = (hipStream_t)stream;

    if (G.K == 0) {  // empty reduction: y = 0
      const size_t n = (size_t)m * G.N;
      const size_t want = (n + 255) / 256;
      const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
      hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, strm, (uint16_t*)d_y, n);
      return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
    }

    KernelFn fn = pick_kernel((int)G.q, c.RPW, c.MC, c.gq, G.has_offset, c.W, c.ring, c.xl, c.pr,
                              c.ei, c.once);
    if (!fn) return LUTGEMM_ERR_INTERNAL;
    Params p{};
    p.bits = (const uint8_t*)d_bits;
    p.alpha = (const uint32_t*)d_alpha;
    p.offset = G.has_offset ? (const uint32_t*)d_offset : nullptr;
    p.x = (const uint16_t*)d_x;
    p.y = (uint16_t*)d_y;
    p.counters = c.S > 1 ? (uint32_t*)d_workspace : nullptr;
    p.partial = c.S > 1 ? (float*)((char*)d_workspace + kCounterBytes) : nullptr;
    p.N = (int)G.N;
    p.K = (int)G.K;
    p.g = (int)G.g;
    p.m = m;
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
    p.xcd_bg = (!c.pr && c.n_bg > 1 && c.n_bg <= 3 && (c.n_rb * c.S) % 8 == 0) ? 1 : 0;
    const int64_t items = c.n_rb * c.n_bg * c.S;
    if (items > 0x7FFFFFFF - kCUs) return LUTGEMM_ERR_SHAPE;
    p.n_items = (int)items;
    dim3 grid((unsigned)(items < kCUs ? items : kCUs));
    void* args[] = {&p};
    if (hipLaunchKernel((const void*)fn, grid, dim3(64 * c.W), args, 0, strm) != hipSuccess)
      return LUTGEMM_ERR_HIP;
    return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

}  // extern "C"
