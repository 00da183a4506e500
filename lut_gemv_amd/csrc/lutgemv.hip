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

int g_ring_override = 0;   // tuning: 3 selects the deeper ring where it exists

KernelFn pick_kernel(int q, int rpw, int mc, bool gq, bool off, int w) {
  const int ring = g_ring_override;
  switch (q) {
    case 1: return kernels_of_q<1>(rpw, mc, gq, off, w, ring);
    case 2: return kernels_of_q<2>(rpw, mc, gq, off, w, ring);
    case 3: return kernels_of_q<3>(rpw, mc, gq, off, w, ring);
    case 4: return kernels_of_q<4>(rpw, mc, gq, off, w, ring);
    case 5: return kernels_of_q<5>(rpw, mc, gq, off, w, ring);
    case 6: return kernels_of_q<6>(rpw, mc, gq, off, w, ring);
    case 7: return kernels_of_q<7>(rpw, mc, gq, off, w, ring);
    case 8: return kernels_of_q<8>(rpw, mc, gq, off, w, ring);
    default: return nullptr;
  }
}

struct Config {
  int RPW, MC, S, W;
  int RI;                // row tiles per row block (<= W * RPW)
  int64_t n_rb, n_bg;
  bool gq;
  size_t ws_bytes;
};

// Optional tuning override "RPW,S[,W[,MC[,ring[,RI]]]]" (LUTGEMM_TILE); never
// needed for correctness.
bool tile_override(int* rpw, int* s, int* w, int* mc, int* ri) {
  const char* e = getenv("LUTGEMM_TILE");
  g_ring_override = 0;
  if (!e || !*e) return false;
  int a = 0, b = 0, c = 0, d = 0, r = 0, t = 0;
  const int n = sscanf(e, "%d,%d,%d,%d,%d,%d", &a, &b, &c, &d, &r, &t);
  if (n < 2) return false;
  *rpw = a;
  *s = b;
  *w = n >= 3 ? c : 0;
  *mc = n >= 4 ? d : 0;
  g_ring_override = n >= 5 ? r : 0;
  *ri = n >= 6 ? t : 0;
  return true;
}

// Pick waves, rows per wave, batch rows per item and the split of the input
// tiles. The kernel is persistent (one workgroup per CU, LDS-bound), so each
// CU works through ceil(items / kCUs) items. The estimate charges each item
// its tiles, weighted by the row tiles it covers and its batch rows (a tile
// step of 16 row tiles is one unit; 8-wave instances pay for their lower
// latency hiding), plus a small cost per item and one for the extra
// reduction kernel a split needs.
Config choose_config(const Geometry& G, int64_t m) {
  Config c{};
  c.gq = (G.g % 32) == 0;
  c.W = 0;   // stays 0 if no instance fits (reported as an internal error)
  double best = 1e300;
  struct Cand { int w, rpw, mc; double eff; };
  const Cand cands[] = {{16, 2, 1, 1.0}, {16, 1, 1, 1.0}, {8, 2, 4, 1.3}, {8, 1, 4, 1.3},
                        {8, 2, 2, 1.3}, {8, 1, 2, 1.3}, {8, 2, 1, 1.3}, {8, 1, 1, 1.3}};
  for (const Cand& v : cands) {
    if (v.mc > 1 && m < v.mc) continue;
    if (!pick_kernel((int)G.q, v.rpw, v.mc, c.gq, G.has_offset, v.w)) continue;
    const int64_t rows = (int64_t)v.w * v.rpw;            // row tiles per item
    const int64_t n_rb = (G.RT + rows - 1) / rows;
    const int64_t n_bg = (m + v.mc - 1) / v.mc;
    const int64_t smax = G.KT < 64 ? G.KT : 64;
    for (int64_t s = 1; s <= smax; ++s) {
      const int64_t items = n_rb * n_bg * s;
      const int64_t per_cu = (items + kCUs - 1) / kCUs;
      const int64_t tiles = (G.KT + s - 1) / s;
      const double unit = v.eff * (double)rows * v.mc / 16.0;
      const double cost = (double)per_cu * (tiles * unit + 0.3 * unit) + (s > 1 ? 2.0 : 0.0);
      if (cost < best - 1e-9) {
        best = cost;
        c.W = v.w;
        c.RPW = v.rpw;
        c.MC = v.mc;
        c.RI = (int)rows;
        c.n_rb = n_rb;
        c.n_bg = n_bg;
        c.S = (int)s;
      }
    }
  }
  int orpw = 0, os = 0, ow = 0, omc = 0, ori = 0;
  if (tile_override(&orpw, &os, &ow, &omc, &ori)) {
    const int w = ow ? ow : c.W;
    const int mc = omc ? omc : c.MC;
    if (pick_kernel((int)G.q, orpw, mc, c.gq, G.has_offset, w)) {
      c.W = w;
      c.RPW = orpw;
      c.MC = mc;
      c.RI = (ori >= 1 && ori <= c.W * c.RPW) ? ori : c.W * c.RPW;
      c.n_rb = (G.RT + c.RI - 1) / c.RI;
      c.n_bg = (m + c.MC - 1) / c.MC;
    }
    if (os >= 1) c.S = (int)(os < G.KT ? os : (G.KT > 0 ? G.KT : 1));
  }
  if (c.S < 1) c.S = 1;
  if (c.n_rb * c.n_bg > kMaxCounters) c.S = 1;   // counters live in a fixed region
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

    KernelFn fn = pick_kernel((int)G.q, c.RPW, c.MC, c.gq, G.has_offset, c.W);
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
    p.n_bg = (int)c.n_bg;
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
