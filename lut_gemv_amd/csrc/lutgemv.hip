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
//  * one workgroup of 8 wave64s per CU. Tables for one input tile (64 chunks =
//    512 inputs) take 64 KiB of LDS: entry p of chunk t at word p*64 + t. Two
//    such tables are kept (128 KiB) so the next step's table is built while the
//    current one is read, with one barrier per step;
//  * lane l of every wave always looks up chunk l, so the 64 lanes of a lookup
//    hit 64 consecutive words modulo 256 B: no bank conflicts whatever the bytes;
//  * a lane streams, per (row tile, plane), the 16 bytes of its chunk for 16 rows
//    with one 128-bit buffer load; a wave reads 1 KiB contiguously. Each wave
//    keeps the loads of the next two input tiles in flight (a ring of three
//    register sets);
//  * per lookup: one v_perm_b32 forms the LDS address from the weight byte, one
//    ds_read_b32, one v_fma_mix_f32 (fp16 scale times fp32 entry into fp32);
//  * group scales are fetched once per quad of lanes and broadcast inside the
//    quad with DPP (a quad covers 32 inputs, inside one group when g % 32 == 0);
//  * when the input dimension is split over workgroups to fill the CUs, each
//    writes fp32 partial sums and a second kernel adds them in a fixed order:
//    results are bitwise reproducible, and no cross-workgroup synchronisation
//    (whose cache maintenance is costly across XCDs) is needed;
//  * no MFMA: this is a lookup-accumulate, not a dense contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "layout.h"
#include "lutgemm.h"

namespace lutgemm {
namespace {

constexpr int kLutWords = 256 * kChunkTile;   // one table tile: 64 KiB of fp32 entries
constexpr int kWaves = 8;                     // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kHiPerWave = 16 / kWaves;       // high nibbles of the pattern each wave builds
constexpr int kCUs = 256;                     // MI355X compute units (dispatch heuristic)

struct Params {
  const uint8_t* bits;      // packed sign bytes
  const uint32_t* alpha;    // packed fp16 scales, two per dword
  const uint32_t* offset;   // packed fp16 offsets, two per dword (or null)
  const uint16_t* x;        // fp16 [m][K]
  uint16_t* y;              // fp16 [m][N]
  float* partial;           // fp32 [S][m][Npad] (split reduction only)
  int N, K, g, m;
  int C, KT, RT, G, S, Npad;
  int n_rb, n_bg, n_items;  // row blocks, batch groups, work items
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

// Raw buffer loads: an offset at or past num_records returns zero without a
// memory access, so row tiles past the end of the matrix and prefetches past a
// workgroup's last tile need no branches around the loads (branches there make
// the compiler wait for every outstanding load before the table build).
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a gfx9 raw buffer descriptor

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           kBufferFlags);
}

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Where one work item's tiles are: item = (row block, split, batch group), with
// the row block varying fastest. All fields are uniform over the workgroup.
struct TileCtx {
  int item, kt, kt1;      // input tile kt of the item's range [.., kt1)
  int rt_first;           // first row tile of this wave in the item's row block
  int valid_rpw;          // row tiles of this wave inside the matrix
  int r0, rows_here;      // batch rows of the item
  int split;
  bool live;              // item exists (false: loads touch no memory)
};

__device__ __forceinline__ void item_range(const Params& p, int item, int* kt0, int* kt1) {
  const int per = p.n_rb * p.S;
  const int s = (item % per) / p.n_rb;
  *kt0 = (int)((int64_t)s * p.KT / p.S);
  *kt1 = (int)((int64_t)(s + 1) * p.KT / p.S);
}

template <int RPW, int MC>
__device__ __forceinline__ TileCtx tile_ctx(const Params& p, int wave, int item, int kt, int kt1) {
  TileCtx c;
  c.item = item;
  c.kt = kt;
  c.kt1 = kt1;
  c.live = item < p.n_items;
  const int per = p.n_rb * p.S;
  const int bg = item / per;
  const int rem = item - bg * per;
  c.split = rem / p.n_rb;
  const int rb = rem - c.split * p.n_rb;
  c.rt_first = (rb * kWaves + wave) * RPW;
  c.valid_rpw = min(RPW, p.RT - c.rt_first);
  c.r0 = bg * MC;
  c.rows_here = c.live ? min(MC, p.m - c.r0) : 0;
  return c;
}

// The tile after c in this workgroup's sequence: the next tile of the item, or
// the first tile of the workgroup's next item (items advance by gridDim.x).
template <int RPW, int MC>
__device__ __forceinline__ TileCtx next_ctx(const Params& p, int wave, const TileCtx& c) {
  if (c.kt + 1 < c.kt1) return tile_ctx<RPW, MC>(p, wave, c.item, c.kt + 1, c.kt1);
  const int item = c.item + (int)gridDim.x;
  int kt0, kt1;
  item_range(p, item, &kt0, &kt1);
  return tile_ctx<RPW, MC>(p, wave, item, kt0, kt1);
}

// Everything one wave needs from memory for one input tile.
template <int Q, int RPW, int MC, bool QUAD, bool OFF>
struct TileRegs {
  static constexpr int AW = QUAD ? 2 * Q : 8 * Q;   // scale dwords per lane and row tile
  static constexpr int OW = OFF ? (QUAD ? 2 : 8) : 0;
  TileCtx c;
  uint4 bw[RPW][Q];          // sign bytes: 16 rows of this lane's chunk, per plane
  uint32_t aw[RPW][AW];      // fp16 scale pairs
  uint32_t ow[RPW][OW > 0 ? OW : 1];
  uint4 xv[MC];              // this lane's 8 activations, per batch row
};

struct LaneCtx {
  int lane, wave, quad_lane;
};

// Issue the loads of the tile described by T.c (all of them unconditional). A
// dead item gives zero-length ranges: the instructions issue but touch no memory.
template <int Q, int RPW, int MC, bool QUAD, bool OFF>
__device__ __forceinline__ void load_tile(const Params& p, const LaneCtx& l,
                                          TileRegs<Q, RPW, MC, QUAD, OFF>& T) {
  using TR = TileRegs<Q, RPW, MC, QUAD, OFF>;
  constexpr uint32_t kTileBytes = Q * kChunkTile * kRowTile;
  const TileCtx& c = T.c;
  const int kt = c.kt;
  // activations first: the table build waits only for these
  const int64_t k0 = (int64_t)kt * kChunkTile * 8;
  const int64_t kin = c.live ? min((int64_t)kChunkTile * 8, (int64_t)p.K - k0) : 0;
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    const uint32_t nb = (r < c.rows_here) ? (uint32_t)(kin * 2) : 0u;
    const auto xr = make_rsrc(p.x + (size_t)(c.r0 + r) * p.K + k0, nb);
    T.xv[r] = load16(xr, (uint32_t)l.lane * 16u);
  }
  // group of this lane's chunk, relative to the tile's first group
  const int g_first = (int)(k0 / p.g);
  int grp = (int)((k0 + l.lane * 8) / p.g);
  grp = grp < p.G - 1 ? grp : p.G - 1;
  const int g_rel = grp - g_first;
  const int g_span = min(p.G - g_first, (kChunkTile * 8 + p.g - 1) / p.g + 1);
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    const bool on = c.live && t < c.valid_rpw;
    const size_t rt = (size_t)(c.rt_first + t);
    const auto br = make_rsrc(p.bits + (rt * p.KT + kt) * kTileBytes, on ? kTileBytes : 0u);
#pragma unroll
    for (int i = 0; i < Q; ++i)
      T.bw[t][i] = load16(br, (uint32_t)(i * kChunkTile * kRowTile + l.lane * 16));
    // scale block of (row tile, group): Q planes x 16 rows of fp16 = 8Q dwords
    const auto ar = make_rsrc(p.alpha + (rt * p.G + g_first) * (8 * Q),
                              on ? (uint32_t)(g_span * 32 * Q) : 0u);
    const uint32_t abase =
        (uint32_t)(g_rel * 32 * Q) + (QUAD ? (uint32_t)(l.quad_lane * 8 * Q) : 0u);
#pragma unroll
    for (int d = 0; d < TR::AW; d += 2) {
      const uint2 v = load8(ar, abase + (uint32_t)d * 4u);
      T.aw[t][d] = v.x;
      T.aw[t][d + 1] = v.y;
    }
    if constexpr (OFF) {
      const auto orr = make_rsrc(p.offset + (rt * p.G + g_first) * 8,
                                 on ? (uint32_t)(g_span * 32) : 0u);
      const uint32_t obase = (uint32_t)(g_rel * 32) + (QUAD ? (uint32_t)(l.quad_lane * 8) : 0u);
#pragma unroll
      for (int d = 0; d < TR::OW; d += 2) {
        const uint2 v = load8(orr, obase + (uint32_t)d * 4u);
        T.ow[t][d] = v.x;
        T.ow[t][d + 1] = v.y;
      }
    }
  }
}

__device__ __forceinline__ void unpack8(const uint4 xr, float (&x)[8]) {
  x[0] = h2f(xr.x, 0); x[1] = h2f(xr.x, 1); x[2] = h2f(xr.y, 0); x[3] = h2f(xr.y, 1);
  x[4] = h2f(xr.z, 0); x[5] = h2f(xr.z, 1); x[6] = h2f(xr.w, 0); x[7] = h2f(xr.w, 1);
}

// Table of lane l's chunk into buffer `buf`: the 256/kWaves entries whose high
// nibble belongs to this wave. Entry p = sum_t (bit t of p ? +x_t : -x_t), as
// ((+-x0 +-x1) + (+-x2 +-x3)) + ((+-x4 +-x5) + (+-x6 +-x7)) in fp32.
__device__ __forceinline__ void build_table(float* lut, int buf, const LaneCtx& l, const uint4 xr) {
  float x[8];
  unpack8(xr, x);
  const float a[4] = {-x[0] - x[1], x[0] - x[1], x[1] - x[0], x[0] + x[1]};
  const float b[4] = {-x[2] - x[3], x[2] - x[3], x[3] - x[2], x[2] + x[3]};
  float lo[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) lo[k] = a[k & 3] + b[k >> 2];
#pragma unroll
  for (int hh = 0; hh < kHiPerWave; ++hh) {
    const int h = l.wave * kHiPerWave + hh;
    const float c = ((h & 1) ? x[4] : -x[4]) + ((h & 2) ? x[5] : -x[5]);
    const float d = ((h & 4) ? x[6] : -x[6]) + ((h & 8) ? x[7] : -x[7]);
    const float hi = c + d;
    float* dst = lut + buf * kLutWords + (h * 16) * kChunkTile + l.lane;
#pragma unroll
    for (int k = 0; k < 16; ++k) dst[k * kChunkTile] = lo[k] + hi;
  }
}

// Look up every row tile of batch row r in table buffer `buf`.
template <int Q, int RPW, int MC, bool QUAD, bool OFF>
__device__ __forceinline__ void lookups(const LaneCtx& l, int r, int buf, const float* lut,
                                        const TileRegs<Q, RPW, MC, QUAD, OFF>& T,
                                        float (&acc)[MC][RPW][16]) {
  // S1 operand of the address permute: byte 0 = lane * 4, byte 2 = table buffer
  const uint32_t lane_sel = ((uint32_t)l.lane << 2) | ((uint32_t)buf << 16);
  float csum = 0.f;
  if constexpr (OFF) {   // sum of the chunk's 8 inputs (table entry 0xFF)
    float x[8];
    unpack8(T.xv[r], x);
    csum = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
  }
#pragma unroll
  for (int t = 0; t < RPW; ++t) {
    if (t < T.c.valid_rpw) {  // uniform over the wave
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const uint32_t words[4] = {T.bw[t][i].x, T.bw[t][i].y, T.bw[t][i].z, T.bw[t][i].w};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          // byte address = buf * 64 KiB + byte(j) * 256 + lane * 4, one v_perm_b32:
          // result byte 1 <- byte (j & 3) of the word; bytes 0, 2 <- lane_sel; byte 3 <- 0
          const uint32_t sel = 0x0C020000u | ((4u + (uint32_t)(j & 3)) << 8);
          const uint32_t addr = __builtin_amdgcn_perm(words[j >> 2], lane_sel, sel);
          const float e = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut) + addr);
          const int D = i * 8 + (j >> 1);     // scale dword index within the group block
          uint32_t aword;
          if constexpr (QUAD) {
            aword = quad_bcast(T.aw[t][D % (2 * Q)], D / (2 * Q));
          } else {
            aword = T.aw[t][D];
          }
          acc[r][t][j] = __builtin_fmaf(h2f(aword, j & 1), e, acc[r][t][j]);
        }
      }
      if constexpr (OFF) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int D = j >> 1;
          uint32_t oword;
          if constexpr (QUAD) {
            oword = quad_bcast(T.ow[t][D % 2], D / 2);
          } else {
            oword = T.ow[t][D];
          }
          acc[r][t][j] = __builtin_fmaf(h2f(oword, j & 1), csum, acc[r][t][j]);
        }
      }
    }
  }
}

// Reduce the accumulators of a finished item across lanes, store them (fp16 y,
// or this split's fp32 partials) and clear them for the next item.
template <int RPW, int MC>
__device__ __forceinline__ void finish_item(const Params& p, const LaneCtx& l, const TileCtx& c,
                                            float (&acc)[MC][RPW][16]) {
  const bool split_mode = p.S > 1;
#pragma unroll
  for (int r = 0; r < MC; ++r) {
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
      if (r < c.rows_here && t < c.valid_rpw) {
        const float tot = reduce16(acc[r][t], l.lane);
        const int row = (c.rt_first + t) * kRowTile + (l.lane >> 2);
        if (l.quad_lane == 0) {
          if (split_mode) {
            p.partial[((size_t)c.split * p.m + (c.r0 + r)) * p.Npad + row] = tot;
          } else if (row < p.N) {
            p.y[(size_t)(c.r0 + r) * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)tot);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[r][t][j] = 0.f;
    }
  }
}

// All steps (one per batch row) of the tile in `cur`; `nxt` holds the next
// tile (in flight) and `pre` receives the one after. Each step builds the next
// step's table in the other buffer, reads its own, then waits at the step's
// one barrier. A finished item is reduced and stored.
template <int Q, int RPW, int MC, bool QUAD, bool OFF>
__device__ __forceinline__ void tile_steps(const Params& p, const LaneCtx& l, float* lut, int& buf,
                                           const TileRegs<Q, RPW, MC, QUAD, OFF>& cur,
                                           const TileRegs<Q, RPW, MC, QUAD, OFF>& nxt,
                                           TileRegs<Q, RPW, MC, QUAD, OFF>& pre,
                                           float (&acc)[MC][RPW][16]) {
  pre.c = next_ctx<RPW, MC>(p, l.wave, nxt.c);
  load_tile(p, l, pre);
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    if (r < cur.c.rows_here) {  // uniform over the workgroup
      if (r + 1 < cur.c.rows_here) {
        build_table(lut, buf ^ 1, l, cur.xv[r + 1]);
      } else if (nxt.c.live) {
        build_table(lut, buf ^ 1, l, nxt.xv[0]);
      }
      lookups(l, r, buf, lut, cur, acc);
      __syncthreads();
      buf ^= 1;
    }
  }
  if (cur.c.kt + 1 == cur.c.kt1) finish_item<RPW, MC>(p, l, cur.c, acc);
}

// Persistent kernel: workgroup b processes items b, b + gridDim.x, ... where an
// item is (row block of kWaves*RPW row tiles, split of the input tiles, batch
// group of MC rows). The three-tile load pipeline runs across item boundaries.
// Q: sign planes; QUAD: scales shared by the 4 lanes of a quad (g % 32 == 0),
// else every lane fetches the scales of its own group; OFF: offset term.
template <int Q, int RPW, int MC, bool QUAD, bool OFF>
__global__ void __launch_bounds__(kThreads, 2) lutgemv_kernel(Params p) {
  __shared__ float lut[2 * kLutWords];

  LaneCtx l;
  l.lane = threadIdx.x & 63;
  // wave index as a scalar: buffer descriptors built from it stay in SGPRs
  l.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  l.quad_lane = l.lane & 3;

  float acc[MC][RPW][16];
#pragma unroll
  for (int r = 0; r < MC; ++r)
#pragma unroll
    for (int t = 0; t < RPW; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[r][t][j] = 0.f;

  TileRegs<Q, RPW, MC, QUAD, OFF> A, B, C;
  {
    int kt0, kt1;
    item_range(p, blockIdx.x, &kt0, &kt1);
    A.c = tile_ctx<RPW, MC>(p, l.wave, blockIdx.x, kt0, kt1);
  }
  if (!A.c.live) return;
  load_tile(p, l, A);
  B.c = next_ctx<RPW, MC>(p, l.wave, A.c);
  load_tile(p, l, B);
  int buf = 0;
  build_table(lut, 0, l, A.xv[0]);
  __syncthreads();
  for (;;) {
    tile_steps(p, l, lut, buf, A, B, C, acc);
    if (!B.c.live) break;
    tile_steps(p, l, lut, buf, B, C, A, acc);
    if (!C.c.live) break;
    tile_steps(p, l, lut, buf, C, A, B, acc);
    if (!A.c.live) break;
  }
}

// y[r][n] = fp16(sum over splits s = 0..S-1 of partial[s][r][n]), in that order.
__global__ void __launch_bounds__(256) finalize_kernel(const float* __restrict__ partial,
                                                       uint16_t* __restrict__ y, int S, int m,
                                                       int N, int Npad) {
  const size_t total = (size_t)m * N;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / N, n = i - r * N;
    const float* src = partial + r * Npad + n;
    float sum = 0.f;
    for (int s = 0; s < S; ++s) sum += src[(size_t)s * m * Npad];
    y[i] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

__global__ void zero_fill_kernel(uint16_t* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

// ------------------------------------------------------------------ dispatch

using KernelFn = void (*)(Params);

// Instances the dispatcher may choose; each keeps three tiles of sign bytes and
// scales plus the accumulators within 256 VGPRs (two waves per SIMD).
// (Scales fetched per lane, g % 32 != 0, run one batch row per workgroup.)
template <int Q, int RPW, int MC, bool QUAD, bool OFF>
constexpr bool kInstantiated =
    (RPW == 1 && (MC == 1 || QUAD)) || (MC == 1 && RPW == 2 && (QUAD ? Q <= 4 : Q <= 2));

template <int Q, int RPW, int MC, bool QUAD, bool OFF>
KernelFn kernel_or_null() {
  if constexpr (kInstantiated<Q, RPW, MC, QUAD, OFF>) {
    return lutgemv_kernel<Q, RPW, MC, QUAD, OFF>;
  } else {
    return nullptr;
  }
}

template <int Q, int RPW, int MC>
KernelFn pick_flags(bool quad, bool off) {
  if (quad) return off ? kernel_or_null<Q, RPW, MC, true, true>() : kernel_or_null<Q, RPW, MC, true, false>();
  return off ? kernel_or_null<Q, RPW, MC, false, true>() : kernel_or_null<Q, RPW, MC, false, false>();
}

template <int RPW, int MC>
KernelFn pick_q(int q, bool quad, bool off) {
  switch (q) {
    case 1: return pick_flags<1, RPW, MC>(quad, off);
    case 2: return pick_flags<2, RPW, MC>(quad, off);
    case 3: return pick_flags<3, RPW, MC>(quad, off);
    case 4: return pick_flags<4, RPW, MC>(quad, off);
    case 5: return pick_flags<5, RPW, MC>(quad, off);
    case 6: return pick_flags<6, RPW, MC>(quad, off);
    case 7: return pick_flags<7, RPW, MC>(quad, off);
    case 8: return pick_flags<8, RPW, MC>(quad, off);
    default: return nullptr;
  }
}

KernelFn pick_kernel(int q, int rpw, int mc, bool quad, bool off) {
  if (mc == 1) {
    if (rpw == 2) return pick_q<2, 1>(q, quad, off);
    if (rpw == 1) return pick_q<1, 1>(q, quad, off);
  } else if (mc == 2) {
    if (rpw == 1) return pick_q<1, 2>(q, quad, off);
  } else if (mc == 4) {
    if (rpw == 1) return pick_q<1, 4>(q, quad, off);
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

// Pick rows per wave and the split of the input tiles. The kernel is
// persistent (one workgroup per CU, LDS-bound), so each CU works through
// ceil(items / kCUs) items; the estimate charges that many items the tiles
// they stream (weighted by row tiles per wave and batch rows) plus a reduction
// cost per item, and a small cost for the extra reduction kernel.
Config choose_config(const Geometry& G, int64_t m) {
  Config c{};
  c.quad = (G.g % 32) == 0;
  c.MC = !c.quad ? 1 : (m >= 4 ? 4 : (m >= 2 ? 2 : 1));
  c.n_bg = (m + c.MC - 1) / c.MC;
  double best = 1e300;
  for (int rpw : {2, 1}) {
    if (!pick_kernel((int)G.q, rpw, c.MC, c.quad, G.has_offset)) continue;
    const int64_t n_rb = (G.RT + kWaves * rpw - 1) / (kWaves * rpw);
    const int64_t smax = G.KT < 64 ? G.KT : 64;
    for (int64_t s = 1; s <= smax; ++s) {
      const int64_t items = n_rb * c.n_bg * s;
      const int64_t per_cu = (items + kCUs - 1) / kCUs;
      const int64_t tiles = (G.KT + s - 1) / s;
      const double cost = (double)per_cu * ((double)rpw * tiles * c.MC + 0.5 * rpw * c.MC) +
                          (s > 1 ? 1.0 : 0.0) - 0.01 * rpw;
      if (cost < best) {
        best = cost;
        c.RPW = rpw;
        c.n_rb = n_rb;
        c.S = (int)s;
      }
    }
  }
  int orpw = 0, os = 0;
  if (tile_override(&orpw, &os)) {
    if ((orpw == 1 || orpw == 2) && pick_kernel((int)G.q, orpw, c.MC, c.quad, G.has_offset)) {
      c.RPW = orpw;
      c.n_rb = (G.RT + kWaves * c.RPW - 1) / (kWaves * c.RPW);
    }
    if (os >= 1) c.S = (int)(os < G.KT ? os : (G.KT > 0 ? G.KT : 1));
  }
  if (c.S < 1) c.S = 1;
  c.ws_bytes = c.S > 1 ? (size_t)c.S * (size_t)m * (size_t)G.Npad * sizeof(float) : 0;
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
  *bytes = choose_config(G, m).ws_bytes;
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

    KernelFn fn = pick_kernel((int)G.q, c.RPW, c.MC, c.quad, G.has_offset);
    if (!fn) return LUTGEMM_ERR_INTERNAL;
    Params p{};
    p.bits = (const uint8_t*)d_bits;
    p.alpha = (const uint32_t*)d_alpha;
    p.offset = G.has_offset ? (const uint32_t*)d_offset : nullptr;
    p.x = (const uint16_t*)d_x;
    p.y = (uint16_t*)d_y;
    p.partial = c.S > 1 ? (float*)d_workspace : nullptr;
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
    p.n_bg = (int)c.n_bg;
    const int64_t items = c.n_rb * c.n_bg * c.S;
    if (items > 0x7FFFFFFF - kCUs) return LUTGEMM_ERR_SHAPE;
    p.n_items = (int)items;
    dim3 grid((unsigned)(items < kCUs ? items : kCUs));
    void* args[] = {&p};
    if (hipLaunchKernel((const void*)fn, grid, dim3(kThreads), args, 0, strm) != hipSuccess)
      return LUTGEMM_ERR_HIP;
    if (c.S > 1) {
      const size_t n = (size_t)m * G.N;
      const size_t want = (n + 255) / 256;
      const unsigned blocks = (unsigned)(want < 2048 ? want : 2048);
      hipLaunchKernelGGL(finalize_kernel, dim3(blocks), dim3(256), 0, strm,
                         (const float*)d_workspace, (uint16_t*)d_y, c.S, (int)m, (int)G.N,
                         (int)G.Npad);
    }
    return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
  } catch (...) {
    return LUTGEMM_ERR_INTERNAL;
  }
}

}  // extern "C"
