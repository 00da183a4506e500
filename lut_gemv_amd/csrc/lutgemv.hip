// BCQ LUT-GEMV for gfx950 (MI355X): y = W_hat x with W_hat held as q sign
// planes plus group-wise fp16 scales (and an optional offset).
//
// The method (LUT-GEMM, Park et al.; Elamur card "LUT-GEMM -- paper by Park et
// al. (2022)", sections "Summary" and "Interesting ideas: Lookup tables instead
// of multiplications"): for every 8-input chunk of x, all 256 signed sums are
// computed once into a table; each weight byte then selects its sum, which is
// scaled by the plane's group scale and accumulated, so the weights are never
// expanded to fp16.
//
// Mapping onto CDNA4 (our design, not the pages'):
//  * one workgroup = W wave64s sharing one 64 KiB table tile in LDS: 64 chunks
//    (512 inputs) x 256 fp32 entries, entry p of chunk t at word p*64 + t. Lane
//    l of every wave always looks up chunk l, so the 64 lanes of a lookup hit 64
//    consecutive words modulo 256 B: no bank conflicts whatever the bytes are;
//  * a lane streams, per (row tile, plane), the 16 bytes of its chunk for 16
//    rows with one 128-bit load; a wave reads 1 KiB contiguously;
//  * per lookup: one byte-to-address op, one ds_read_b32, one v_fma_mix_f32
//    (fp16 scale times fp32 table entry into an fp32 accumulator);
//  * group scales are fetched once per quad of lanes and broadcast inside the
//    quad with DPP (a quad covers 32 inputs, inside one group when g % 32 == 0);
//  * the reduction dimension is split over blockIdx.y when needed to fill 256
//    CUs; the last workgroup to finish a row block sums the fp32 partials in a
//    fixed order, so results are bitwise reproducible;
//  * no MFMA: this is a lookup-accumulate, not a dense contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "layout.h"
#include "lutgemm.h"

namespace lutgemm {
namespace {

constexpr int kLutWords = 256 * kChunkTile;   // 64 KiB of fp32 table entries
constexpr size_t kCounterBytes = 64 * 1024;   // arrival counters, start of workspace
constexpr int64_t kMaxCounters = kCounterBytes / sizeof(uint32_t);
constexpr int kWaves = 4;                     // waves per workgroup
constexpr int kThreads = kWaves * 64;

struct Params {
  const uint8_t* bits;      // packed sign bytes
  const uint32_t* alpha;    // packed fp16 scales, two per dword
  const uint32_t* offset;   // packed fp16 offsets, two per dword (or null)
  const uint16_t* x;        // fp16 [m][K]
  uint16_t* y;              // fp16 [m][N]
  float* partial;           // fp32 [S][m][Npad] (split reduction only)
  uint32_t* counters;       // [n_bg][n_rb]     (split reduction only)
  int N, K, g, m;
  int C, KT, RT, G, S, Npad;
  int n_rb;
  int has_offset;
};

__device__ __forceinline__ float h2f(uint32_t word, int hi) {
  const uint16_t bitsv = hi ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
  return (float)__builtin_bit_cast(_Float16, bitsv);
}

// Broadcast the value of lane u of each quad to the whole quad (DPP quad_perm).
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int u) {
  switch (u) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
  }
}

// Sum 16 per-lane values across the 64 lanes of a wave. Each step halves the
// set a lane keeps and trades the other half with its partner, so the cost is
// 8+4+2+1 exchanges instead of 16*6. On return lane l holds the total of row
// l >> 2 (each row replicated in one quad). The summation order is fixed.
__device__ __forceinline__ float reduce16(float (&v)[16], int lane) {
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int dist = 32 >> st;
    const int half = 8 >> st;
    const bool up = (lane & dist) != 0;
#pragma unroll
    for (int k = 0; k < half; ++k) {
      const float vlo = v[k], vhi = v[k + half];   // select values, not addresses
      const float send = up ? vlo : vhi;
      const float keep = up ? vhi : vlo;
      v[k] = keep + __shfl_xor(send, dist, 64);
    }
  }
  float t = v[0];
  t += __shfl_xor(t, 2, 64);
  t += __shfl_xor(t, 1, 64);
  return t;
}

// One workgroup: row block blockIdx.x (kWaves*RPW row tiles), split
// blockIdx.y of the input tiles, batch rows [MC*blockIdx.z, +MC).
// Q: sign planes; QUAD: scales shared by the 4 lanes of a quad (g % 32 == 0),
// else every lane fetches the scales of its own group.
template <int Q, int RPW, int MC, bool QUAD>
__global__ void __launch_bounds__(kThreads, 2) lutgemv_kernel(Params p) {
  __shared__ float lut[kLutWords];
  __shared__ int s_last;

  constexpr int AW = QUAD ? 2 * Q : 8 * Q;   // scale dwords held per lane and row tile
  constexpr int OW = QUAD ? 2 : 8;           // offset dwords held per lane and row tile

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rb = blockIdx.x;
  const int split = blockIdx.y;
  const int r0 = blockIdx.z * MC;
  const int rows_here = min(MC, p.m - r0);
  const int kt0 = (int)((int64_t)split * p.KT / p.S);
  const int kt1 = (int)((int64_t)(split + 1) * p.KT / p.S);
  const int rt_first = (rb * kWaves + wave) * RPW;
  const uint32_t lane_off = (uint32_t)lane << 2;
  const int quad_lane = lane & 3;

  float acc[MC][RPW][16];
#pragma unroll
  for (int r = 0; r < MC; ++r)
#pragma unroll
    for (int t = 0; t < RPW; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[r][t][j] = 0.f;

  for (int kt = kt0; kt < kt1; ++kt) {
    const int chunk = kt * kChunkTile + lane;
    // ---- activations for this tile (issued first: the table build waits only for these)
    uint4 xv[MC];
#pragma unroll
    for (int r = 0; r < MC; ++r) {
      xv[r] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows_here && chunk < p.C)
        xv[r] = *reinterpret_cast<const uint4*>(p.x + (size_t)(r0 + r) * p.K + (size_t)chunk * 8);
    }
    // ---- sign bytes, scales and offsets of this tile for the wave's row tiles
    int grp = (kt * kChunkTile * 8 + lane * 8) / p.g;
    grp = grp < p.G - 1 ? grp : p.G - 1;
    uint4 bw[RPW][Q];
    uint32_t aw[RPW][AW];
    uint32_t ow[RPW][OW];
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int rt = rt_first + t;
      if (rt < p.RT) {
        const uint8_t* bp = p.bits + (((size_t)rt * p.KT + kt) * Q) * (kChunkTile * kRowTile) + lane * 16;
#pragma unroll
        for (int i = 0; i < Q; ++i)
          bw[t][i] = *reinterpret_cast<const uint4*>(bp + i * (kChunkTile * kRowTile));
        const uint32_t* ap = p.alpha + ((size_t)rt * p.G + grp) * (8 * Q) + (QUAD ? quad_lane * 2 * Q : 0);
#pragma unroll
        for (int d = 0; d < AW; ++d) aw[t][d] = ap[d];
        if (p.has_offset) {
          const uint32_t* op = p.offset + ((size_t)rt * p.G + grp) * 8 + (QUAD ? quad_lane * 2 : 0);
#pragma unroll
          for (int d = 0; d < OW; ++d) ow[t][d] = op[d];
        } else {
#pragma unroll
          for (int d = 0; d < OW; ++d) ow[t][d] = 0u;
        }
      } else {
#pragma unroll
        for (int i = 0; i < Q; ++i) bw[t][i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int d = 0; d < AW; ++d) aw[t][d] = 0u;
#pragma unroll
        for (int d = 0; d < OW; ++d) ow[t][d] = 0u;
      }
    }

#pragma unroll
    for (int r = 0; r < MC; ++r) {
      if (r < rows_here) {  // uniform over the workgroup
      __syncthreads();  // every wave is done reading the previous table
      // ---- build: lane l fills chunk l's entries whose high nibble is this wave's
      const uint4 xr = xv[r];
      const float x0 = h2f(xr.x, 0), x1 = h2f(xr.x, 1), x2 = h2f(xr.y, 0), x3 = h2f(xr.y, 1);
      const float x4 = h2f(xr.z, 0), x5 = h2f(xr.z, 1), x6 = h2f(xr.w, 0), x7 = h2f(xr.w, 1);
      // low nibble (inputs 0..3): lo[l] = (+-x0 +-x1) + (+-x2 +-x3), sign + where bit set
      const float a[4] = {-x0 - x1, x0 - x1, x1 - x0, x0 + x1};
      const float b[4] = {-x2 - x3, x2 - x3, x3 - x2, x2 + x3};
      float lo[16];
#pragma unroll
      for (int l = 0; l < 16; ++l) lo[l] = a[l & 3] + b[l >> 2];
      constexpr int HPW = 16 / kWaves;   // high nibbles per wave
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int h = wave * HPW + hh;
        const float c = ((h & 1) ? x4 : -x4) + ((h & 2) ? x5 : -x5);
        const float d = ((h & 4) ? x6 : -x6) + ((h & 8) ? x7 : -x7);
        const float hi = c + d;
        float* dst = lut + (h * 16) * kChunkTile + lane;
#pragma unroll
        for (int l = 0; l < 16; ++l) dst[l * kChunkTile] = lo[l] + hi;
      }
      // sum of the chunk's 8 inputs (table entry 0xFF), for the offset term
      const float csum = lo[15] + ((x4 + x5) + (x6 + x7));
      __syncthreads();  // table complete

      // ---- lookups: acc[row] += alpha(plane, row) * T[byte(plane, row)]
#pragma unroll
      for (int t = 0; t < RPW; ++t) {
        if (rt_first + t < p.RT) {  // uniform over the wave
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          const uint32_t words[4] = {bw[t][i].x, bw[t][i].y, bw[t][i].z, bw[t][i].w};
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            // table byte address = byte(j) * 256 + lane * 4 in one v_perm_b32:
            // result byte 1 <- byte (j & 3) of the word, byte 0 <- lane_off, bytes 2-3 <- 0
            const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)(j & 3)) << 8);
            const uint32_t addr = __builtin_amdgcn_perm(words[j >> 2], lane_off, sel);
            const float e = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut) + addr);
            const int D = i * 8 + (j >> 1);     // scale dword index within the group block
            uint32_t aword;
            if constexpr (QUAD) {
              aword = quad_bcast(aw[t][D % (2 * Q)], D / (2 * Q));
            } else {
              aword = aw[t][D];
            }
            acc[r][t][j] = __builtin_fmaf(h2f(aword, j & 1), e, acc[r][t][j]);
          }
        }
        if (p.has_offset) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int D = j >> 1;
            uint32_t oword;
            if constexpr (QUAD) {
              oword = quad_bcast(ow[t][D % 2], D / 2);
            } else {
              oword = ow[t][D];
            }
            acc[r][t][j] = __builtin_fmaf(h2f(oword, j & 1), csum, acc[r][t][j]);
          }
        }
        }
      }
      }
    }
  }

  // ---- cross-lane reduction and output
  const bool split_mode = p.S > 1;
#pragma unroll
  for (int r = 0; r < MC; ++r) {
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      const int rt = rt_first + t;
      if (r < rows_here && rt < p.RT) {
        const float tot = reduce16(acc[r][t], lane);
        const int row = rt * kRowTile + (lane >> 2);
        if (quad_lane == 0) {
          if (split_mode) {
            p.partial[((size_t)split * p.m + (r0 + r)) * p.Npad + row] = tot;
          } else if (row < p.N) {
            p.y[(size_t)(r0 + r) * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)tot);
          }
        }
      }
    }
  }
  if (!split_mode) return;

  // ---- split reduction: the last workgroup of this (row block, batch group) sums
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* ctr = p.counters + (size_t)blockIdx.z * p.n_rb + rb;
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (uint32_t)(p.S - 1);
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  constexpr int kRowsPerBlock = kWaves * RPW * kRowTile;
  const int row0 = rb * kRowsPerBlock;
  for (int idx = threadIdx.x; idx < rows_here * kRowsPerBlock; idx += kThreads) {
    const int r = idx / kRowsPerBlock;
    const int row = row0 + (idx - r * kRowsPerBlock);
    if (row >= p.N) continue;
    float sum = 0.f;
    for (int s = 0; s < p.S; ++s)
      sum += p.partial[((size_t)s * p.m + (r0 + r)) * p.Npad + row];
    p.y[(size_t)(r0 + r) * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

__global__ void zero_fill_kernel(uint16_t* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

// ------------------------------------------------------------------ dispatch

using KernelFn = void (*)(Params);

// Instances the dispatcher may choose; each keeps accumulators, sign bytes and
// scales of one tile within the 256-VGPR budget of two waves per SIMD.
template <int Q, int RPW, int MC, bool QUAD>
constexpr bool kInstantiated =
    RPW == 1 ||
    (MC == 1 && RPW == 2 && Q <= 6) ||
    (MC == 1 && RPW == 4 && Q <= (QUAD ? 3 : 2)) ||
    (MC == 2 && RPW == 2 && QUAD && Q <= 5) ||
    (MC == 4 && RPW == 2 && QUAD && Q <= 4);

template <int Q, int RPW, int MC, bool QUAD>
KernelFn kernel_or_null() {
  if constexpr (kInstantiated<Q, RPW, MC, QUAD>) {
    return lutgemv_kernel<Q, RPW, MC, QUAD>;
  } else {
    return nullptr;
  }
}

template <int Q, int RPW, int MC>
KernelFn pick_quad(bool quad) {
  return quad ? kernel_or_null<Q, RPW, MC, true>() : kernel_or_null<Q, RPW, MC, false>();
}

template <int RPW, int MC>
KernelFn pick_q(int q, bool quad) {
  switch (q) {
    case 1: return pick_quad<1, RPW, MC>(quad);
    case 2: return pick_quad<2, RPW, MC>(quad);
    case 3: return pick_quad<3, RPW, MC>(quad);
    case 4: return pick_quad<4, RPW, MC>(quad);
    case 5: return pick_quad<5, RPW, MC>(quad);
    case 6: return pick_quad<6, RPW, MC>(quad);
    case 7: return pick_quad<7, RPW, MC>(quad);
    case 8: return pick_quad<8, RPW, MC>(quad);
    default: return nullptr;
  }
}

KernelFn pick_kernel(int q, int rpw, int mc, bool quad) {
  if (mc == 1) {
    if (rpw == 4) return pick_q<4, 1>(q, quad);
    if (rpw == 2) return pick_q<2, 1>(q, quad);
    if (rpw == 1) return pick_q<1, 1>(q, quad);
  } else if (mc == 2) {
    if (rpw == 2) return pick_q<2, 2>(q, quad);
    if (rpw == 1) return pick_q<1, 2>(q, quad);
  } else if (mc == 4) {
    if (rpw == 2) return pick_q<2, 4>(q, quad);
    if (rpw == 1) return pick_q<1, 4>(q, quad);
  }
  return nullptr;
}

struct Config {
  int RPW, MC, S;
  int64_t n_rb, n_bg;
  bool quad;
  size_t ws_bytes;
};

// Optional tuning override "RPW,S" (LUTGEMM_TILE); never needed for correctness.
bool tile_override(int* rpw, int* s) {
  const char* e = getenv("LUTGEMM_TILE");
  if (!e || !*e) return false;
  int a = 0, b = 0;
  if (sscanf(e, "%d,%d", &a, &b) != 2) return false;
  *rpw = a;
  *s = b;
  return true;
}

Config choose_config(const Geometry& G, int64_t m) {
  Config c{};
  c.quad = (G.g % 32) == 0;
  c.MC = m >= 4 ? 4 : (m >= 2 ? 2 : 1);
  // register budget: accumulators MC*RPW*16, sign bytes RPW*Q*4, scales RPW*AW;
  // take the largest row-tile count per wave that has an instance
  c.RPW = 1;
  for (int rpw : {4, 2}) {
    if (pick_kernel((int)G.q, rpw, c.MC, c.quad)) {
      c.RPW = rpw;
      break;
    }
  }
  // enough workgroups before splitting the reduction
  const int64_t rt_per_wave_min = 1;
  while (c.RPW > rt_per_wave_min &&
         ((G.RT + kWaves * c.RPW - 1) / (kWaves * c.RPW)) * ((m + c.MC - 1) / c.MC) < 256)
    c.RPW /= 2;
  c.n_rb = (G.RT + kWaves * c.RPW - 1) / (kWaves * c.RPW);
  c.n_bg = (m + c.MC - 1) / c.MC;
  const int64_t base = c.n_rb * c.n_bg;
  int64_t S = 1;
  const int64_t target = 1024;
  if (base < target && G.KT > 1) {
    S = (target + base - 1) / base;
    if (S > G.KT) S = G.KT;
  }
  int orpw = 0, os = 0;
  if (tile_override(&orpw, &os)) {
    if (orpw == 1 || orpw == 2 || orpw == 4) {
      if (pick_kernel(G.q, orpw, c.MC, c.quad)) {
        c.RPW = orpw;
        c.n_rb = (G.RT + kWaves * c.RPW - 1) / (kWaves * c.RPW);
      }
    }
    if (os >= 1) S = os < G.KT ? os : (G.KT > 0 ? G.KT : 1);
  }
  if (c.n_rb * c.n_bg > kMaxCounters) S = 1;
  c.S = (int)(S < 1 ? 1 : S);
  c.ws_bytes = c.S > 1 ? kCounterBytes + (size_t)c.S * (size_t)m * (size_t)G.Npad * sizeof(float) : 0;
  return c;
}

std::atomic<int> g_arch_ok[64];   // 0 unknown, 1 gfx950, 2 other

int check_device(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LUTGEMM_ERR_HIP;
  *dev_out = dev;
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
  *bytes = choose_config(G, m).ws_bytes;
  return LUTGEMM_OK;
}

int lutgemm_workspace_init(void* d_workspace, size_t bytes, void* stream) {
  if (bytes == 0) return LUTGEMM_OK;
  if (!d_workspace) return LUTGEMM_ERR_NULL;
  if (hipMemsetAsync(d_workspace, 0, bytes, (hipStream_t)stream) != hipSuccess) return LUTGEMM_ERR_HIP;
  return LUTGEMM_OK;
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
      if (c.ws_bytes) {
        if (!d_workspace) return LUTGEMM_ERR_NULL;
        if (workspace_bytes < c.ws_bytes) return LUTGEMM_ERR_BUFFER;
        if (!aligned(d_workspace, 16)) return LUTGEMM_ERR_ALIGN;
      }
    }
    int dev = 0;
    st = check_device(&dev);
    if (st) return st;
    hipStream_t strm = (hipStream_t)stream;

    if (G.K == 0) {  // empty reduction: y = 0
      const size_t n = (size_t)m * G.N;
      const size_t want = (n + 255) / 256;
      const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
      hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, strm, (uint16_t*)d_y, n);
      return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
    }

    KernelFn fn = pick_kernel((int)G.q, c.RPW, c.MC, c.quad);
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
    p.has_offset = G.has_offset ? 1 : 0;
    if (c.n_rb > 0x7FFFFFFF || c.n_bg > 65535) return LUTGEMM_ERR_SHAPE;
    dim3 grid((unsigned)c.n_rb, (unsigned)c.S, (unsigned)c.n_bg);
    void* args[] = {&p};
    if (hipLaunchKernel((const void*)fn, grid, dim3(kThreads), args, 0, strm) != hipSuccess)
      return LUTGEMM_ERR_HIP;
    return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

}  // extern "C"
