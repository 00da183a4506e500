// lutgemv_kernel.h -- the BCQ LUT-GEMV kernel for gfx950 (MI355X): y = W_hat x
// with W_hat held as q sign planes plus group-wise fp16 scales (and an optional offset).
//
// The method (LUT-GEMM, Park et al.; Elamur card "LUT-GEMM -- paper by Park et
// al. (2022)", sections "Summary" and "Interesting ideas: Lookup tables instead
// of multiplications"): for every 8-input chunk of x, all 256 signed sums are
// computed once into a table; each weight byte then selects its sum, which is
// scaled by the plane's group scale and accumulated, so the weights are never
// expanded to fp16.
//
// Mapping onto CDNA4 (our design, not the pages'):
//  * one persistent workgroup per CU (8 or 16 wave64s) walks a list of work
//    items (row block, split of the input dimension, batch group). Tables for
//    one input tile (64 chunks = 512 inputs) take 64 KiB of LDS: entry p of
//    chunk t at word p*64 + t. Two such tables are kept (128 KiB), so the next
//    step's table is built while the current one is read, with one barrier per
//    step; the build walks each lane's entries in Gray-code order (one add per
//    entry);
//  * for the lookups a lane owns a 4-row x 4-chunk block of sign bytes (16
//    bytes per plane, one 128-bit buffer load; a wave reads 1 KiB contiguously)
//    and visits its chunks in a lane-rotated order, so the 64 lanes of every
//    lookup read 64 different tables: no LDS bank conflicts whatever the bytes;
//  * per lookup: one v_perm_b32 forms the LDS address from the weight byte, one
//    ds_read_b32 and one add; when the block's four chunks share a scale group
//    (g % 32 == 0) the four entries of a row are summed and scaled once with a
//    v_fma_mix_f32 (fp16 scale times fp32 sum into an fp32 accumulator);
//  * each wave keeps the loads of the next one or two input tiles in flight (a
//    ring of register sets filled by unconditional buffer loads); on the
//    batch-1 launch that streams one row block per CU, a set is refilled as
//    soon as its lookups are done, so two tiles are in flight from the start;
//    at batch 1 the sign planes, read once per product, are loaded with the
//    non-temporal cache hint so that they do not evict what is read again;
//  * at batch 1 the whole of x is staged in LDS once per workgroup (up to
//    15360 inputs); from two batch rows on, the tables of two rows can be
//    interleaved entry by entry so that one 64-bit read serves both rows;
//  * when the input dimension is split over workgroups to fill the CUs, each
//    writes fp32 partial sums with device-scope (write-through) stores; after
//    its last item a workgroup waits for those stores to complete and counts
//    its items in per-row-block arrival counters with device-scope atomics, and
//    the last arrival of a row block adds its partials in split order (so
//    results are bitwise reproducible). This avoids the L2-wide writeback and
//    invalidate that release/acquire fences cost across the XCDs;
//  * the lookup is a gather, not a dense product, and stays on the vector
//    ALUs and LDS; the paired tables of two batch rows can be built on the
//    matrix cores (the 256 x 8 sign matrix times the tile's activations), and
//    from 4 batch rows on the launcher uses the sign-plane MFMA kernel
//    (sign_mfma_kernel.h) instead of the tables.
//
// Device code only. Each plane count q is instantiated in its own translation
// unit (lutgemv_q.hip compiled with -DLUTGEMM_Q=q) so that the instances build
// in parallel; the host launcher (lutgemv.hip) reaches them through
// kernels_of_q<q>.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace lutgemm {

constexpr int kLutWords = 256 * kChunkTile;   // one table tile: 64 KiB of fp32 entries
// At batch 1 the whole of x can be staged in LDS next to the two tables (128 KiB):
// up to 1920 chunks of 8 inputs (30 KiB), i.e. K <= 15360.
constexpr int kXChunks = 1920;
// Compute units of a full MI355X. The workspace size query (host only) sizes the
// split reduction for this count; launches use the device's own count.
constexpr int kNominalCUs = 256;
// Split reductions keep their arrival counters in a fixed region at the start
// of the workspace, so any later call finds its counters zero whatever its shape.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxCounters = kCounterBytes / sizeof(uint32_t);

struct Params {
  const uint8_t* bits;      // packed sign bytes
  const uint32_t* alpha;    // packed fp16 scales, two per dword
  const uint32_t* offset;   // packed fp16 offsets, two per dword (or null)
  const uint16_t* x;        // fp16 [m][K]
  uint16_t* y;              // fp16 [m][N]
  float* partial;           // fp32 [S][m][Npad] (split reduction only)
  uint32_t* counters;       // [n_bg][n_rb] arrivals per row block (split reduction only)
  int N, K, g, m;
  int C, KT, RT, G, S, Npad;
  int n_rb, n_bg, n_items;  // row blocks, batch groups, work items
  int ri;                   // row tiles per row block (at most waves * RPW)
  int g_shift;              // log2(g) when g is a power of two, else -1
  int g_span;               // most scale groups one input tile touches
  int g_tile;               // 1 if g divides 512: every input tile starts a group
  int xcd_bg;               // 1: the batch groups of one weight block are 8 items apart
  unsigned long long* trace;   // phase stamps [workgroup][kTracePoints] (traced builds only)
  int trace_wgs;               // workgroups the trace buffer holds
};

// Phase tracing (a tracing aid, compiled in only with LUTGEMM_PHASE_TRACE):
// thread 0 of each workgroup stamps the GPU's constant 100 MHz clock at the
// phase boundaries of a launch: 0 start, 1 x staged in LDS, 2 first table
// built, 3 first step done, 4 last lookups done, 5 end. In the regular build
// the macros are empty and the two fields above stay null.
constexpr int kTracePoints = 8;
#ifdef LUTGEMM_PHASE_TRACE
#define LUTGEMM_PHASE(k)                                                                   \
  do {                                                                                     \
    if (p.trace && threadIdx.x == 0 && (int)blockIdx.x < p.trace_wgs)                       \
      p.trace[(size_t)blockIdx.x * kTracePoints + (k)] = __builtin_amdgcn_s_memrealtime();  \
  } while (0)
#define LUTGEMM_PHASE_FLAG(f) bool f = false
#define LUTGEMM_PHASE_ONCE(k, f) \
  do {                           \
    if (!(f)) {                  \
      (f) = true;                \
      LUTGEMM_PHASE(k);          \
    }                            \
  } while (0)
#else
#define LUTGEMM_PHASE(k) \
  do {                   \
  } while (0)
#define LUTGEMM_PHASE_FLAG(f) \
  do {                        \
  } while (0)
#define LUTGEMM_PHASE_ONCE(k, f) \
  do {                           \
  } while (0)
#endif

__device__ __forceinline__ float h2f(uint32_t word, int hi) {
  const uint16_t bitsv = hi ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
  return (float)__builtin_bit_cast(_Float16, bitsv);
}

// Raw buffer loads: an offset at or past num_records returns zero without a
// memory access, so row tiles past the end of the matrix and prefetches past a
// workgroup's last tile need no branches around the loads (branches there make
// the compiler wait for every outstanding load before the table build).
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a gfx9 raw buffer descriptor

// Buffer descriptors and scalar offsets must live in scalar registers; the
// values put there are uniform over the wave, and readfirstlane says so (it
// is free for a value already in a scalar register, and otherwise replaces a
// loop over distinct lane values by one instruction).
__device__ __forceinline__ uint32_t uni(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)uni(nbytes),
                                           kBufferFlags);
}

// The range check covers voff (per lane) plus soff (scalar): a descriptor
// whose num_records is soff + n admits exactly voff < n.
// NT sets the non-temporal cache policy bit (for data read once per product,
// so that it does not evict what is read again, such as x).
template <bool NT = false>
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, uni(soff), NT ? 2 : 0));
}

template <bool NT = false>
__device__ __forceinline__ uint2 load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, uni(soff), NT ? 2 : 0));
}

// ------------------------------------------------------------------ work items
// An item is (row block, split of the input tiles, batch group), row block
// varying fastest. Its fields are uniform over the workgroup and are computed
// once per item (the only integer divisions of the kernel).
struct ItemCtx {
  int item;               // item index (>= n_items: none)
  int kt1;                // end of the item's input tiles
  int rt_first;           // first row tile of this wave
  int valid_rpw;          // row tiles of this wave inside the matrix (may be <= 0)
  int nrt;                // row tiles this wave reads: 0 .. RPW, 0 when there is no item
  int r0, rows_here;      // batch rows of the item
  int split;
};

// Position of one input tile in a workgroup's sequence of tiles.
struct TilePos {
  ItemCtx c;
  int kt;
  bool live;              // false past the workgroup's last item: loads touch no memory
};

// Work item -> (batch group, split, weight block = row block + n_rb * split).
// Normally the row block varies fastest, then the split, then the batch group.
// With xcd_bg (several batch groups, items per batch group a multiple of 8) the
// batch groups of one weight block are 8 items apart instead: workgroups b and
// b + 8 run on the same XCD (dispatch goes round-robin over the 8 XCDs), so the
// batch groups that re-read one block's weights run at the same time and share
// that XCD's L2.
__device__ __forceinline__ void decode_item(const Params& p, int item, int& bg, int& split,
                                            int& rb) {
  const int per = p.n_rb * p.S;
  int w;
  if (p.xcd_bg) {
    const int j = item >> 3;
    const int y = j / p.n_bg;
    bg = j - y * p.n_bg;
    w = (item & 7) + 8 * y;
  } else {
    bg = item / per;
    w = item - bg * per;
  }
  split = w / p.n_rb;
  rb = w - split * p.n_rb;
}

template <int RPW, int MC, int W>
__device__ __forceinline__ TilePos first_tile(const Params& p, int wave, int item) {
  TilePos t;
  t.c.item = item;
  t.live = item < p.n_items;
  int bg, rb;
  decode_item(p, item, bg, t.c.split, rb);
  t.kt = t.c.split * p.KT / p.S;
  t.c.kt1 = (t.c.split + 1) * p.KT / p.S;
  t.c.rt_first = rb * p.ri + wave * RPW;
  t.c.valid_rpw = min(min(RPW, p.ri - wave * RPW), p.RT - t.c.rt_first);
  // uniform over the wave: keep it (and the descriptors sized by it) scalar
  t.c.nrt = __builtin_amdgcn_readfirstlane(t.live ? max(t.c.valid_rpw, 0) : 0);
  t.c.r0 = bg * MC;
  t.c.rows_here = t.live ? min(MC, p.m - t.c.r0) : 0;
  return t;
}

// The tile after t: the next tile of the item, or the first tile of the
// workgroup's next item (items advance by gridDim.x).
template <int RPW, int MC, int W>
__device__ __forceinline__ TilePos next_tile(const Params& p, int wave, const TilePos& t) {
  if (t.kt + 1 < t.c.kt1) {
    TilePos n = t;
    n.kt = t.kt + 1;
    return n;
  }
  return first_tile<RPW, MC, W>(p, wave, t.c.item + (int)gridDim.x);
}

// Lane roles. For the table build and the activations, lane l owns chunk l of
// the input tile. For the lookups, lane l owns the lane block (r4, c4) of rows
// 4*r4 .. +3 and chunks 4*c4 .. +3 (16 sign bytes per plane), with
// r4 = bits 3-4 of l and c4 = bits 0-2 of l plus bit 5 of l as bit 3; it visits
// its four chunks in the order b_k = (k + r4) & 3. At each of the four lookup
// steps the 32 lanes of each half-wave then read 32 consecutive tables, one per
// LDS bank, whatever the bytes are.
struct LaneCtx {
  int lane, wave, r4, c4;
  uint32_t block;     // byte offset of this lane's block in a 1 KiB plane block
  uint32_t tsel[4];   // (table index 4*c4 + b_k) * 4: byte 0 of the address
  uint32_t psel[4];   // v_perm selector taking byte b_k of a sign word into byte 1
  uint32_t ptsel[4];  // paired tables: bytes 0 and 2 of the address of chunk 4*c4 + b_k
  uint32_t hsel[4];   // half tables and split paired tables: byte 0 of the address of
                      // chunk 4*c4 + b_k, i.e. 8 * ((4*c4 + b_k) % 32)
  uint32_t hmask;     // half tables: 0x80808080 for the lanes of chunks 32..63, else 0
  uint32_t rot8;      // 8 * r4: rotating a sign word right by this puts byte b_k in byte k
  uint32_t aoff, ooff;  // g % 32 == 0 and g divides 512: byte offset of this lane's
                        // scales (and offsets) in a tile's scale block
};

__device__ __forceinline__ LaneCtx lane_ctx() {
  LaneCtx l;
  l.lane = threadIdx.x & 63;
  // wave index as a scalar: buffer descriptors built from it stay in SGPRs
  l.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  l.r4 = (l.lane >> 3) & 3;
  l.c4 = (l.lane & 7) | ((l.lane >> 5) << 3);
  l.block = (uint32_t)(16 * l.r4 + l.c4) * 16u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t b = (uint32_t)((k + l.r4) & 3);
    l.tsel[k] = (4u * (uint32_t)l.c4 + b) << 2;
    // byte 0 <- S1 byte 0 (table index), byte 1 <- S0 byte b (sign byte),
    // byte 2 <- S1 byte 2 (table buffer), byte 3 <- 0
    l.psel[k] = 0x0C020000u | ((4u + b) << 8);
    const uint32_t t = 4u * (uint32_t)l.c4 + b;
    l.ptsel[k] = ((t & 31u) << 3) | ((t >> 5) << 16);
    l.hsel[k] = (t & 31u) << 3;
  }
  l.hmask = (l.lane >> 5) ? 0x80808080u : 0u;
  l.rot8 = 8u * (uint32_t)l.r4;
  return l;
}

// Everything one wave needs from memory for one input tile.
// GQ: the four chunks of a lane block share one scale group (g % 32 == 0), so
// scales (and offsets) are held per row; otherwise per row and visited chunk.
template <int Q, int RPW, int MC, bool GQ, bool OFF>
struct TileRegs {
  static constexpr int AW = GQ ? 2 * Q : 8 * Q;   // scale dwords (fp16 pairs) per row tile
  static constexpr int OW = OFF ? (GQ ? 2 : 8) : 0;
  TilePos pos;
  uint4 xv[MC];              // activations of chunk `lane`, per batch row
  uint4 bw[RPW][Q];          // lane block per plane: word a = row 4*r4+a, byte b = chunk 4*c4+b
  uint32_t aw[RPW][AW];      // GQ: [plane][row pair]; else [visit k][plane][row pair]
  uint32_t ow[RPW][OW > 0 ? OW : 1];
};

__device__ __forceinline__ int group_of(const Params& p, int k) {
  return p.g_shift >= 0 ? (k >> p.g_shift) : (k / p.g);
}

// When g divides 512 every input tile starts a group, so the group of a lane's
// chunks (one group when g % 32 == 0), relative to the tile's first group, is
// the same for every tile: the lane's scale offsets are computed once.
template <int Q>
__device__ __forceinline__ void tile_group_offsets(const Params& p, LaneCtx& l) {
  const uint32_t g_rel = p.g_tile ? (uint32_t)((32 * l.c4) >> p.g_shift) : 0u;
  l.aoff = g_rel * 32u * Q + 8u * (uint32_t)l.r4;
  l.ooff = g_rel * 32u + 8u * (uint32_t)l.r4;
}

// Issue the loads of the tile at T.pos (all of them unconditional; activations
// first, so the table build waits only for those). A dead position gives
// zero-length ranges: the instructions issue but touch no memory. NT: every
// sign byte is read once per product (batch 1), each load consuming whole
// lines, and those loads are non-temporal. Scale and offset loads stay ordinary:
// the loads of the planes share their lines, and a non-temporal line can be
// gone before the next plane's load. With several batch groups the groups
// re-read the same weights, which the caches then serve.
// MB: the tables are built by MFMA (build_pair_mfma); xv[h] then holds the B
// operands of batch rows (2h, 2h+1) for this wave's two n-blocks instead of
// chunk `lane` of each row.
template <int Q, int RPW, int MC, bool GQ, bool OFF, bool XL, bool NT, bool MB = false>
__device__ __forceinline__ void load_tile(const Params& p, const LaneCtx& l,
                                          TileRegs<Q, RPW, MC, GQ, OFF>& T) {
  constexpr uint32_t kTileBytes = Q * kChunkTile * kRowTile;
  constexpr int NV = GQ ? 1 : 4;
  const TilePos& t = T.pos;
  const int k0 = t.kt * kChunkTile * 8;
  // Every descriptor starts at its buffer's base and ends after this tile's
  // bytes for this wave; the tile's position goes in the scalar offset (each
  // buffer is under 4 GiB). A dead position is an empty range.
  const uint32_t kin = t.live ? (uint32_t)min(kChunkTile * 8, p.K - k0) : 0u;
  if constexpr (MB) {
    // lane l: column l % 32 of n-blocks nb0 and nb0 + 1, i.e. chunk
    // 16 * nb + (l % 32) / 2 of row 2h + (l & 1), inputs 4 * (l / 32) .. + 3 of
    // that chunk (8 bytes). One descriptor spans the pair's rows that exist;
    // lanes past the input dimension or the batch read at its end (zero).
    const uint32_t col = (uint32_t)(l.lane & 31), kh = (uint32_t)(l.lane >> 5);
    const uint32_t rl = (uint32_t)(l.lane & 1);
    const uint32_t nb0 = 2u * (uint32_t)(l.wave >> 3);
    const uint32_t rowb = (uint32_t)p.K * 2u;
#pragma unroll
    for (int h = 0; h < MC / 2; ++h) {
      const int rows = t.live ? min(2, t.c.rows_here - 2 * h) : 0;
      const uint32_t span = rows > 0 ? (uint32_t)rows * rowb : 0u;
      const uint32_t xs = ((uint32_t)(t.c.r0 + 2 * h) * (uint32_t)p.K + (uint32_t)k0) * 2u;
      const auto rs = make_rsrc(p.x, span ? xs + span : 0u);
      uint2 v[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t kk = 8u * (16u * (nb0 + (uint32_t)j) + col / 2u) + 4u * kh;
        const bool ok = kk < kin && (int)rl < rows;
        v[j] = load8(rs, ok ? rl * rowb + kk * 2u : span, xs);
      }
      T.xv[h] = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
    }
  } else if constexpr (!XL) {   // (with XL the activations are in LDS)
#pragma unroll
    for (int r = 0; r < MC; ++r) {
      const uint32_t nb = (r < t.c.rows_here) ? kin * 2u : 0u;
      const uint32_t xs = ((uint32_t)(t.c.r0 + r) * (uint32_t)p.K + (uint32_t)k0) * 2u;
      T.xv[r] = load16(make_rsrc(p.x, nb ? xs + nb : 0u), (uint32_t)l.lane * 16u, xs);
    }
  }
  // sign blocks of this wave's row tiles (adjacent in the input-tile-first order)
  const int nrt = t.live ? t.c.nrt : 0;
  const uint32_t bs = ((uint32_t)t.kt * (uint32_t)p.RT + (uint32_t)t.c.rt_first) * kTileBytes;
  const auto br = make_rsrc(p.bits, nrt ? bs + (uint32_t)nrt * kTileBytes : 0u);
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int q = 0; q < Q; ++q)
      T.bw[i][q] = load16<NT>(br, (uint32_t)(i * kTileBytes + q * kChunkTile * kRowTile) + l.block, bs);
  const int g_first = group_of(p, k0);
  const uint32_t g_span = (uint32_t)min(p.G - g_first, p.g_span);
  // byte offset of the scales (offsets) of each chunk this lane visits
  uint32_t aoff[NV], ooff[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (GQ && p.g_tile) {
      aoff[k] = l.aoff;
      ooff[k] = l.ooff;
    } else {
      const int chunk = 4 * l.c4 + (GQ ? 0 : ((k + l.r4) & 3));
      int grp = group_of(p, k0 + 8 * chunk);
      grp = grp < p.G - 1 ? grp : p.G - 1;
      const uint32_t g_rel = (uint32_t)(grp - g_first);
      aoff[k] = g_rel * 32u * Q + 8u * (uint32_t)l.r4;
      ooff[k] = g_rel * 32u + 8u * (uint32_t)l.r4;
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const bool on = i < nrt;
    // scale block of (row tile, group): [plane][16 rows] fp16; this lane's four
    // rows of plane q are 8 bytes at q*32 + 8*r4
    const uint32_t blk = (uint32_t)(t.c.rt_first + i) * (uint32_t)p.G + (uint32_t)g_first;
    const auto ar = make_rsrc(p.alpha, on ? (blk + g_span) * (32u * Q) : 0u);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint2 v = load8(ar, aoff[k] + (uint32_t)(q * 32), blk * (32u * Q));
        T.aw[i][(k * Q + q) * 2] = v.x;
        T.aw[i][(k * Q + q) * 2 + 1] = v.y;
      }
    }
    if constexpr (OFF) {
      const auto orr = make_rsrc(p.offset, on ? (blk + g_span) * 32u : 0u);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const uint2 v = load8(orr, ooff[k], blk * 32u);
        T.ow[i][2 * k] = v.x;
        T.ow[i][2 * k + 1] = v.y;
      }
    }
  }
}

__device__ __forceinline__ void unpack8(const uint4 xr, float (&x)[8]) {
  x[0] = h2f(xr.x, 0); x[1] = h2f(xr.x, 1); x[2] = h2f(xr.y, 0); x[3] = h2f(xr.y, 1);
  x[4] = h2f(xr.z, 0); x[5] = h2f(xr.z, 1); x[6] = h2f(xr.w, 0); x[7] = h2f(xr.w, 1);
}

// Table of lane l's chunk into buffer `buf`: the entries whose high nibble
// belongs to this wave (one high nibble with 16 waves, two with 8). Entry
// p = sum_t (bit t of p ? +x_t : -x_t).
// The entries are visited in Gray-code order of their varying bits, so each is
// the previous one plus or minus 2 x_t (one add, sign known at compile time);
// the first is summed directly.
template <int W>
__device__ __forceinline__ void build_table(float* lut, int buf, const LaneCtx& l, const uint4 xr) {
  constexpr int HPW = W == 16 ? 1 : 2;        // high nibbles per building wave
  constexpr int NB = HPW == 2 ? 5 : 4;        // pattern bits that vary within the wave
  static_assert(W == 8 || W == 16, "8 or 16 waves per workgroup");
  float x[8];
  unpack8(xr, x);
  const int h0 = l.wave * HPW;                // first high nibble (even when HPW == 2)
  const float c = ((h0 & 1) ? x[4] : -x[4]) + ((h0 & 2) ? x[5] : -x[5]);
  const float d = ((h0 & 4) ? x[6] : -x[6]) + ((h0 & 8) ? x[7] : -x[7]);
  float T = (-(x[0] + x[1]) - (x[2] + x[3])) + (c + d);   // pattern h0*16: low bits clear
  float two[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) two[t] = x[t] + x[t];       // bit 4 of the local pattern is x4
  float* base = lut + buf * kLutWords + (h0 * 16) * kChunkTile + l.lane;
  base[0] = T;
#pragma unroll
  for (int n = 1; n < (1 << NB); ++n) {
    const int t = __builtin_ctz(n);           // the bit that flips from gray(n-1) to gray(n)
    const int pat = n ^ (n >> 1);
    T += ((pat >> t) & 1) ? two[t] : -two[t];
    base[pat * kChunkTile] = T;
  }
}

__device__ __forceinline__ float lut_at(const float* lut, uint32_t byte_addr) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut) + byte_addr);
}

// ------------------------------------------------------------------ paired tables
// With two or more batch rows per item the tables of two rows can share one
// 128 KiB buffer, entry by entry: the pair (row 2h, row 2h+1) of entry p of
// chunk t sits at byte p*256 + (t % 32)*8 + (t / 32)*64 KiB. One 64-bit read
// then serves both rows: half the LDS instructions of two single-row lookups
// (the LDS takes about as long per instruction for 64-bit as for 32-bit reads).
// The bank of an entry depends only on t % 32 and each half-wave reads 32
// different chunks, so the reads are free of bank conflicts whatever the bytes.
// The price is one buffer instead of two: the build waits for the previous
// lookups to finish.
__device__ __forceinline__ float2 lut_at2(const float* lut, uint32_t byte_addr) {
  return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(lut) + byte_addr);
}

// Paired table of lane l's chunk: the same Gray-code walk as build_table, for
// two batch rows at once (xa: row 2h, xb: row 2h+1), one 64-bit store per entry.
template <int W>
__device__ __forceinline__ void build_table_pair(float* lut, const LaneCtx& l, const uint4 xa,
                                                 const uint4 xb) {
  constexpr int HPW = W == 16 ? 1 : 2;
  constexpr int NB = HPW == 2 ? 5 : 4;
  static_assert(W == 8 || W == 16, "8 or 16 waves per workgroup");
  float x[8], y[8];
  unpack8(xa, x);
  unpack8(xb, y);
  const int h0 = l.wave * HPW;
  const float cx = ((h0 & 1) ? x[4] : -x[4]) + ((h0 & 2) ? x[5] : -x[5]);
  const float dx = ((h0 & 4) ? x[6] : -x[6]) + ((h0 & 8) ? x[7] : -x[7]);
  const float cy = ((h0 & 1) ? y[4] : -y[4]) + ((h0 & 2) ? y[5] : -y[5]);
  const float dy = ((h0 & 4) ? y[6] : -y[6]) + ((h0 & 8) ? y[7] : -y[7]);
  float T = (-(x[0] + x[1]) - (x[2] + x[3])) + (cx + dx);
  float U = (-(y[0] + y[1]) - (y[2] + y[3])) + (cy + dy);
  float twx[NB], twy[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    twx[t] = x[t] + x[t];
    twy[t] = y[t] + y[t];
  }
  char* base = reinterpret_cast<char*>(lut) + (h0 * 16) * 256 + (l.lane & 31) * 8 +
               (l.lane >> 5) * (kLutWords * 4);
  *reinterpret_cast<float2*>(base) = make_float2(T, U);
#pragma unroll
  for (int n = 1; n < (1 << NB); ++n) {
    const int t = __builtin_ctz(n);
    const int pat = n ^ (n >> 1);
    T += ((pat >> t) & 1) ? twx[t] : -twx[t];
    U += ((pat >> t) & 1) ? twy[t] : -twy[t];
    *reinterpret_cast<float2*>(base + pat * 256) = make_float2(T, U);
  }
}

// ------------------------------------------------------------------ MFMA-built paired tables
// The paired table of two batch rows is a dense product: entry p of column
// (chunk t, row r) is sum_k S[p][k] x_r[8t + k] with S[p][k] = +1 if bit k of p
// is set, else -1, a 256 x 8 sign matrix times the 8 x 128 matrix of the tile's
// activations. v_mfma_f32_32x32x8f16 computes one 32 x 32 block of it from fp16
// x (exact products, fp32 sums): wave w takes patterns 32 * (w % 8) .. + 31 and
// n-blocks 2 * (w / 8) and + 1 (column n = 2 * (chunk % 16) + row, chunk
// = 16 * nb + n / 2), two MFMAs per table and no vector-ALU arithmetic.
// Operand layouts (32x32x8): A[i][k] in lane i + 32 * (k / 4), element k % 4;
// B[k][j] in lane j + 32 * (k / 4), element k % 4; D[i][j] in lane
// j + 32 * ((i / 4) % 2), register (i % 4) + 4 * (i / 8).
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));

// The A operand of this wave: signs of pattern 32 * (w % 8) + l % 32, inputs
// 4 * (l / 32) .. + 3.
__device__ __forceinline__ half4v mfma_signs(const LaneCtx& l) {
  const int pt = 32 * (l.wave & 7) + (l.lane & 31);
  const int k0 = 4 * (l.lane >> 5);
  half4v a;
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = ((pt >> (k0 + e)) & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
  return a;
}

// This wave's part of the paired table of one pair of batch rows (xb: its B
// operands, from load_tile with MB), written in the paired layout.
__device__ __forceinline__ void build_pair_mfma(float* lut, const LaneCtx& l, const half4v a,
                                                const uint4 xb) {
  const int nb0 = 2 * (l.wave >> 3);
  const int col = l.lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const half4v b = __builtin_bit_cast(half4v, j ? make_uint2(xb.z, xb.w) : make_uint2(xb.x, xb.y));
    float16v c = {};
    c = __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, c, 0, 0, 0);
    const int t = 16 * (nb0 + j) + col / 2;
    char* base = reinterpret_cast<char*>(lut) + (32 * (l.wave & 7) + 4 * (l.lane >> 5)) * 256 +
                 (t & 31) * 8 + (t >> 5) * (kLutWords * 4) + (col & 1) * 4;
#pragma unroll
    for (int v = 0; v < 16; ++v)
      *reinterpret_cast<float*>(base + (8 * (v / 4) + (v % 4)) * 256) = c[v];
  }
}

// Look up every row tile of batch row r in table buffer `buf`. Per plane and
// row, a lane reads the entries its four sign bytes select; with GQ they are
// summed and scaled once, else each is scaled by its chunk's group scale.
template <int Q, int RPW, int MC, bool GQ, bool OFF>
__device__ __forceinline__ void lookups(const LaneCtx& l, int r, int buf, const float* lut,
                                        const TileRegs<Q, RPW, MC, GQ, OFF>& T,
                                        float (&acc)[MC][RPW][4]) {
  const uint32_t bufbits = (uint32_t)buf << 16;
  uint32_t tsel[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) tsel[k] = l.tsel[k] | bufbits;
  // offset term: entry 0xFF of a chunk's table is the sum of its 8 inputs
  float csum[GQ ? 1 : 4];
  if constexpr (OFF) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e = lut_at(lut, (0xFFu << 8) | tsel[k]);
      if constexpr (GQ) {
        csum[0] = k == 0 ? e : csum[0] + e;
      } else {
        csum[k] = e;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    if (i < T.pos.c.valid_rpw) {  // uniform over the wave
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint32_t words[4] = {T.bw[i][q].x, T.bw[i][q].y, T.bw[i][q].z, T.bw[i][q].w};
        if constexpr (GQ) {
          // All 16 reads of the plane are issued before any is used, so that
          // they are in flight together whatever order the scheduler keeps.
          float e[4][4];
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              e[a][k] = lut_at(lut, __builtin_amdgcn_perm(words[a], tsel[k], l.psel[k]));
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const float s = (e[a][0] + e[a][1]) + (e[a][2] + e[a][3]);
            const uint32_t aword = T.aw[i][q * 2 + (a >> 1)];
            acc[r][i][a] = __builtin_fmaf(h2f(aword, a & 1), s, acc[r][i][a]);
          }
        } else {
          // each entry has its own scale: four reads (one row) at a time
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            float e[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              e[k] = lut_at(lut, __builtin_amdgcn_perm(words[a], tsel[k], l.psel[k]));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t aword = T.aw[i][(k * Q + q) * 2 + (a >> 1)];
              acc[r][i][a] = __builtin_fmaf(h2f(aword, a & 1), e[k], acc[r][i][a]);
            }
          }
        }
      }
      if constexpr (OFF) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
          for (int k = 0; k < (GQ ? 1 : 4); ++k) {
            const uint32_t oword = T.ow[i][2 * k + (a >> 1)];
            acc[r][i][a] = __builtin_fmaf(h2f(oword, a & 1), csum[k], acc[r][i][a]);
          }
        }
      }
    }
  }
}

// Lookups of batch rows 2h and 2h+1 from the paired table (scale groups of 32
// or more inputs: the four chunks of a lane block share one scale).
template <int Q, int RPW, int MC, bool OFF>
__device__ __forceinline__ void lookups_pair(const LaneCtx& l, int h, const float* lut,
                                             const TileRegs<Q, RPW, MC, true, OFF>& T,
                                             float (&acc)[MC][RPW][4]) {
  const int r0 = 2 * h, r1 = 2 * h + 1;
  float cs0 = 0.f, cs1 = 0.f;
  if constexpr (OFF) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 e = lut_at2(lut, (0xFFu << 8) | l.ptsel[k]);
      cs0 = k == 0 ? e.x : cs0 + e.x;
      cs1 = k == 0 ? e.y : cs1 + e.y;
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    if (i < T.pos.c.valid_rpw) {  // uniform over the wave
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint32_t words[4] = {T.bw[i][q].x, T.bw[i][q].y, T.bw[i][q].z, T.bw[i][q].w};
        float2 e[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            e[a][k] = lut_at2(lut, __builtin_amdgcn_perm(words[a], l.ptsel[k], l.psel[k]));
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float s0 = (e[a][0].x + e[a][1].x) + (e[a][2].x + e[a][3].x);
          const float s1 = (e[a][0].y + e[a][1].y) + (e[a][2].y + e[a][3].y);
          const float al = h2f(T.aw[i][q * 2 + (a >> 1)], a & 1);
          acc[r0][i][a] = __builtin_fmaf(al, s0, acc[r0][i][a]);
          acc[r1][i][a] = __builtin_fmaf(al, s1, acc[r1][i][a]);
        }
      }
      if constexpr (OFF) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float o = h2f(T.ow[i][a >> 1], a & 1);
          acc[r0][i][a] = __builtin_fmaf(o, cs0, acc[r0][i][a]);
          acc[r1][i][a] = __builtin_fmaf(o, cs1, acc[r1][i][a]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ half tables
// Complementing all eight signs negates an entry: entry (b ^ 0xFF) = -entry b.
// A half table keeps only the 128 entries whose bit 7 is clear; a byte b with
// bit 7 set reads entry b ^ 0xFF and takes it negated. A half-size paired table
// (64 KiB for the 64 chunks of an input tile, two batch rows per entry) leaves
// room for two buffers, so the next pair's table is built while the current
// one is read, with one barrier per step instead of the paired tables' two.
// The price is paid per lookup: folding the byte and applying its sign.
// Layout: the pair of entry c < 128 of chunk t in buffer `buf` is at byte
//   c*256 + (t / 32)*32 KiB + (t % 32)*8 + buf*64 KiB,
// so bits 8-14 of an address are c and bit 15 is t / 32. Any byte in bits 8-15
// gives an address inside the 128 KiB. As with the paired tables, the bank of
// an entry depends only on t % 32: the reads are free of bank conflicts.

// Half paired table of lane l's chunk into buffer `buf`: the entries whose bits
// NB..6 equal the wave index (NB = 3 with 16 waves, 4 with 8), walked in
// Gray-code order of bits 0..NB-1 as in build_table. Entry c (bit 7 clear) is
// sum_{t<7} (bit t of c ? +x_t : -x_t) - x_7.
template <int W>
__device__ __forceinline__ void build_half_pair(float* lut, int buf, const LaneCtx& l,
                                                const uint4 xa, const uint4 xb) {
  constexpr int NB = W == 16 ? 3 : 4;
  static_assert(W == 8 || W == 16, "8 or 16 waves per workgroup");
  float x[8], y[8];
  unpack8(xa, x);
  unpack8(xb, y);
  const int h0 = l.wave << NB;
  float T = -x[7], U = -y[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    if (j < NB) {
      T -= x[j];
      U -= y[j];
    } else {
      const bool on = ((h0 >> j) & 1) != 0;
      T += on ? x[j] : -x[j];
      U += on ? y[j] : -y[j];
    }
  }
  float twx[NB], twy[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    twx[t] = x[t] + x[t];
    twy[t] = y[t] + y[t];
  }
  char* base = reinterpret_cast<char*>(lut) + buf * (kLutWords * 4) + h0 * 256 +
               (l.lane >> 5) * 32768 + (l.lane & 31) * 8;
  *reinterpret_cast<float2*>(base) = make_float2(T, U);
#pragma unroll
  for (int n = 1; n < (1 << NB); ++n) {
    const int t = __builtin_ctz(n);
    const int pat = n ^ (n >> 1);
    T += ((pat >> t) & 1) ? twx[t] : -twx[t];
    U += ((pat >> t) & 1) ? twy[t] : -twy[t];
    *reinterpret_cast<float2*>(base + pat * 256) = make_float2(T, U);
  }
}

// Lookups of batch rows 2h and 2h+1 from the half paired table in buffer `buf`
// (grouped scales). Per sign word (four chunk bytes of one row): rotate it so
// that byte k is the byte of visit k; a v_perm with sign-extending selectors
// gives 0xFF in each byte whose bit 7 is set, and xor with that folds every
// byte below 128 (the chunk half goes into bit 7). The sign of a byte is put on
// the row's fp16 scale (bit 15 or 31 of its scale word), so that each entry is
// accumulated with one fma per batch row.
template <int Q, int RPW, int MC, bool OFF>
__device__ __forceinline__ void lookups_half(const LaneCtx& l, int h, int buf, const float* lut,
                                             const TileRegs<Q, RPW, MC, true, OFF>& T,
                                             float (&acc)[MC][RPW][4]) {
  const int r0 = 2 * h, r1 = 2 * h + 1;
  const uint32_t bb = (uint32_t)buf << 16;
  uint32_t hs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) hs[k] = l.hsel[k] | bb;
  float cs0 = 0.f, cs1 = 0.f;
  if constexpr (OFF) {
    // entry 0xFF (the sum of a chunk's 8 inputs) is minus half-table entry 0
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 e = lut_at2(lut, hs[k] | (l.hmask & 0x8000u));
      cs0 -= e.x;
      cs1 -= e.y;
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    if (i < T.pos.c.valid_rpw) {  // uniform over the wave
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const uint32_t words[4] = {T.bw[i][q].x, T.bw[i][q].y, T.bw[i][q].z, T.bw[i][q].w};
        uint32_t wr[4];
        float2 e[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          wr[a] = __builtin_amdgcn_alignbit(words[a], words[a], l.rot8);
          const uint32_t neg = __builtin_amdgcn_perm(wr[a] << 8, wr[a], 0x090B080Au);
          const uint32_t wf = (wr[a] ^ neg) | l.hmask;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            e[a][k] = lut_at2(lut, __builtin_amdgcn_perm(wf, hs[k], 0x0C020000u | ((4u + k) << 8)));
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t aword = T.aw[i][q * 2 + (a >> 1)];
          // the row's scale is bits 16-31 (a odd) or 0-15 (a even) of aword
          constexpr int kPos[2] = {15, 31};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int pos = kPos[a & 1], src = 8 * k + 7;
            const uint32_t sgn = pos >= src ? wr[a] << (pos - src) : wr[a] >> (src - pos);
            const float al = h2f(aword ^ (sgn & (1u << pos)), a & 1);
            acc[r0][i][a] = __builtin_fmaf(al, e[a][k].x, acc[r0][i][a]);
            acc[r1][i][a] = __builtin_fmaf(al, e[a][k].y, acc[r1][i][a]);
          }
        }
      }
      if constexpr (OFF) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float o = h2f(T.ow[i][a >> 1], a & 1);
          acc[r0][i][a] = __builtin_fmaf(o, cs0, acc[r0][i][a]);
          acc[r1][i][a] = __builtin_fmaf(o, cs1, acc[r1][i][a]);
        }
      }
    }
  }
}

// Sum each of a lane's four row accumulators (rows 4*r4 + a) over the 16
// lanes that share its row quad (lanes differing in bits 0-2 and 5), with
// cross-lane moves that do not go through LDS: v_permlane32_swap exchanges the
// two halves of the wave (rows 0 and 1 stay in lanes 0-31, rows 2 and 3 go to
// lanes 32-63), then three DPP moves within rows of 16 lanes: a quad swap that
// leaves row 2*bit5 + bit0 in each lane, a quad swap over bit 1 and a shift by
// 4 over bit 2. The result is the sum of row reduced_row(lane) in the lanes with
// (lane & 6) == 4 (partial sums elsewhere). The order of the additions is fixed.
__device__ __forceinline__ float row_sum16(const float (&v)[4], int lane) {
  float w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v[k]),
                                                    __builtin_bit_cast(unsigned, v[k + 2]), false,
                                                    false);
    w[k] = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  }
  const bool odd = (lane & 1) != 0;
  const float keep = odd ? w[1] : w[0];
  const float send = odd ? w[0] : w[1];
  // quad_perm [1,0,3,2] (0xB1), quad_perm [2,3,0,1] (0x4E), row_shr:4 (0x114)
  float t = keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                 __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
  t += __builtin_bit_cast(float,
                          __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x4E, 0xF, 0xF, false));
  t += __builtin_bit_cast(float,
                          __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x114, 0xF, 0xF, false));
  return t;
}

// The row (within its row tile) whose sum row_sum16 leaves in `lane`, and
// whether that lane holds it.
__device__ __forceinline__ int reduced_row(int lane) {
  return 4 * ((lane >> 3) & 3) + ((lane & 32) ? 2 : 0) + (lane & 1);
}
__device__ __forceinline__ bool holds_row_sum(int lane) { return (lane & 6) == 4; }

// ------------------------------------------------------------------ split paired tables
// Paired tables (two batch rows per entry) of half an input tile: 32 chunks,
// 64 KiB, so two buffers fit and each step builds the next table while it
// reads the current one, with one barrier per step and no change to the
// lookup itself. A tile is looked up in two steps, chunks 0-31 from buffer 0
// and chunks 32-63 from buffer 1. The pair of entry p of chunk t of the half
// is at byte p*256 + t*8 + buffer*64 KiB (row 2h in the low word). The bank of
// an entry depends only on t, and the lanes of each half-wave read 32
// different chunks: no bank conflicts.
//
// Lanes. The loads are those of the other kernels (lane l holds the lane block
// of rows 4*r4..+3 and chunks 4*c4..+3, c4 = (l & 7) + 8*(l >> 5), and its
// scales). In each step every lane looks up two rows of four chunks of the
// current half: lane l takes rows 4*r4 + 2*rh + {0, 1} (rh = l >> 5) of
// chunks 4*(l & 7)..+3 of the half. One v_permlane32_swap per register pair
// moves the data there: after swapping the lower lanes of (words 2, 3) with
// the upper lanes of (words 0, 1), words 0 and 1 hold the two rows of the
// first half and words 2 and 3 those of the second. The same swap arranges
// the scales (and offsets) of each plane.
template <int Q, int MC, bool OFF>
__device__ __forceinline__ void split_arrange(TileRegs<Q, 1, MC, true, OFF>& T) {
  auto swap = [](uint32_t& lo, uint32_t& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
    lo = (uint32_t)r[0];
    hi = (uint32_t)r[1];
  };
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    swap(T.bw[0][q].x, T.bw[0][q].z);
    swap(T.bw[0][q].y, T.bw[0][q].w);
    swap(T.aw[0][2 * q], T.aw[0][2 * q + 1]);
  }
  if constexpr (OFF) swap(T.ow[0][0], T.ow[0][1]);
}

// Activations of the table of half H for batch rows (a, b): lane l gets chunk
// (l & 31) + 32*H of row a (lanes 0-31) or of row b (lanes 32-63). The tile's
// chunk l of each row is in lane l, so one swap per register gives both
// halves.
template <int H>
__device__ __forceinline__ uint4 split_x(const uint4 a, const uint4 b) {
  const auto sx = __builtin_amdgcn_permlane32_swap(a.x, b.x, false, false);
  const auto sy = __builtin_amdgcn_permlane32_swap(a.y, b.y, false, false);
  const auto sz = __builtin_amdgcn_permlane32_swap(a.z, b.z, false, false);
  const auto sw = __builtin_amdgcn_permlane32_swap(a.w, b.w, false, false);
  return make_uint4((uint32_t)sx[H], (uint32_t)sy[H], (uint32_t)sz[H], (uint32_t)sw[H]);
}

// Table of one half for one batch row into buffer `buf`: lane l builds chunk
// l & 31 for the row of its half-wave (the low word of each pair for lanes
// 0-31, the high word for 32-63), the 16 entries whose high nibble is the
// wave index, in Gray-code order as in build_table.
__device__ __forceinline__ void build_split(float* lut, int buf, const LaneCtx& l, const uint4 xr) {
  float x[8];
  unpack8(xr, x);
  const int h0 = l.wave;
  const float c = ((h0 & 1) ? x[4] : -x[4]) + ((h0 & 2) ? x[5] : -x[5]);
  const float d = ((h0 & 4) ? x[6] : -x[6]) + ((h0 & 8) ? x[7] : -x[7]);
  float T = (-(x[0] + x[1]) - (x[2] + x[3])) + (c + d);
  float two[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) two[t] = x[t] + x[t];
  float* base = reinterpret_cast<float*>(reinterpret_cast<char*>(lut) + buf * (kLutWords * 4) +
                                         h0 * 16 * 256 + (l.lane & 31) * 8 + (l.lane >> 5) * 4);
  base[0] = T;
#pragma unroll
  for (int n = 1; n < 16; ++n) {
    const int t = __builtin_ctz(n);
    const int pat = n ^ (n >> 1);
    T += ((pat >> t) & 1) ? two[t] : -two[t];
    base[pat * 64] = T;
  }
}

// Lookups of half H of batch rows 2h and 2h+1 (T arranged by split_arrange;
// the table of half H is in buffer H). acc[r][j]: batch row r, row
// 4*r4 + 2*rh + j of the lane's row tile.
template <int Q, int MC, bool OFF, int H>
__device__ __forceinline__ void lookups_split(const LaneCtx& l, int h, const float* lut,
                                              const TileRegs<Q, 1, MC, true, OFF>& T,
                                              float (&acc)[MC][2]) {
  const int r0 = 2 * h, r1 = 2 * h + 1;
  uint32_t hs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) hs[k] = l.hsel[k] | ((uint32_t)H << 16);
  float cs0 = 0.f, cs1 = 0.f;
  if constexpr (OFF) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 e = lut_at2(lut, (0xFFu << 8) | hs[k]);
      cs0 = k == 0 ? e.x : cs0 + e.x;
      cs1 = k == 0 ? e.y : cs1 + e.y;
    }
  }
  if (T.pos.c.valid_rpw > 0) {  // uniform over the wave
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const uint32_t words[2] = {H ? T.bw[0][q].z : T.bw[0][q].x,
                                 H ? T.bw[0][q].w : T.bw[0][q].y};
      float2 e[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          e[j][k] = lut_at2(lut, __builtin_amdgcn_perm(words[j], hs[k], l.psel[k]));
      const uint32_t aword = T.aw[0][2 * q + H];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float s0 = (e[j][0].x + e[j][1].x) + (e[j][2].x + e[j][3].x);
        const float s1 = (e[j][0].y + e[j][1].y) + (e[j][2].y + e[j][3].y);
        const float al = h2f(aword, j);
        acc[r0][j] = __builtin_fmaf(al, s0, acc[r0][j]);
        acc[r1][j] = __builtin_fmaf(al, s1, acc[r1][j]);
      }
    }
    if constexpr (OFF) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float o = h2f(T.ow[0][H], j);
        acc[r0][j] = __builtin_fmaf(o, cs0, acc[r0][j]);
        acc[r1][j] = __builtin_fmaf(o, cs1, acc[r1][j]);
      }
    }
  }
}

// Sum a lane's two row accumulators over the 8 lanes of its row pair (bits
// 0-2 of the lane) with DPP moves, as the last three steps of row_sum16: the
// sum of row j = lane & 1 ends in the lanes with (lane & 6) == 4.
__device__ __forceinline__ float row_sum8(const float (&v)[2], int lane) {
  const bool odd = (lane & 1) != 0;
  const float keep = odd ? v[1] : v[0];
  const float send = odd ? v[0] : v[1];
  float t = keep + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                                 __builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
  t += __builtin_bit_cast(float,
                          __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x4E, 0xF, 0xF, false));
  t += __builtin_bit_cast(float,
                          __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x114, 0xF, 0xF, false));
  return t;
}

// finish_item for the split paired tables: reduce, store, clear.
template <int MC>
__device__ __forceinline__ void finish_split(const Params& p, const LaneCtx& l, const ItemCtx& c,
                                             float (&acc)[MC][2]) {
  const bool split_mode = p.S > 1;
#pragma unroll
  for (int r = 0; r < MC; ++r) {
    if (r < c.rows_here && c.valid_rpw > 0) {
      const float v[2] = {acc[r][0], acc[r][1]};
      const float t = row_sum8(v, l.lane);
      const int row = c.rt_first * kRowTile + 4 * l.r4 + 2 * (l.lane >> 5) + (l.lane & 1);
      if (holds_row_sum(l.lane)) {
        if (split_mode) {
          __hip_atomic_store(&p.partial[((size_t)c.split * p.m + (c.r0 + r)) * p.Npad + row], t,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (row < p.N) {
          p.y[(size_t)(c.r0 + r) * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)t);
        }
      }
    }
    acc[r][0] = 0.f;
    acc[r][1] = 0.f;
  }
}

// Reduce the accumulators of a finished item over the 16 lanes that share a
// row quad (row_sum16), store them (fp16 y, or this split's fp32 partials)
// and clear them.
template <int RPW, int MC>
__device__ __forceinline__ void finish_item(const Params& p, const LaneCtx& l, const ItemCtx& c,
                                            float (&acc)[MC][RPW][4]) {
  const bool split_mode = p.S > 1;
#pragma unroll
  for (int r = 0; r < MC; ++r) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      if (r < c.rows_here && i < c.valid_rpw) {
        const float v[4] = {acc[r][i][0], acc[r][i][1], acc[r][i][2], acc[r][i][3]};
        const float t = row_sum16(v, l.lane);
        const int row = (c.rt_first + i) * kRowTile + reduced_row(l.lane);
        if (holds_row_sum(l.lane)) {
          if (split_mode) {
            // device-scope store: written through to where every XCD reads it
            __hip_atomic_store(&p.partial[((size_t)c.split * p.m + (c.r0 + r)) * p.Npad + row], t,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else if (row < p.N) {
            p.y[(size_t)(c.r0 + r) * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)t);
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[r][i][a] = 0.f;
    }
  }
}

// Split reduction, run once after a workgroup's last item (its loads have all
// returned, so waiting costs nothing). Every wave waits until its partial-sum
// stores are complete at device scope; then one thread per item of this
// workgroup counts the item's arrival in its row-block counter (device-scope
// atomics, all in flight together). An arrival that completes a row block (S
// of them) makes this workgroup add the S partials of each of the block's rows
// in split order, round to fp16 and store y; it also resets the counter to zero
// for the next call. The sums of all such blocks are done in one pass.
template <int RPW, int MC, int W>
__device__ __forceinline__ void split_epilogue(const Params& p, int* s_last) {
  constexpr int kThreads = W * 64;
  const int kRows = p.ri * kRowTile;   // rows per row block
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt = expcnt = lgkmcnt = 0: own stores complete
  __syncthreads();
  const int n_mine = (p.n_items - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  for (int j0 = 0; j0 < n_mine; j0 += kThreads) {
    const int nj = min(kThreads, n_mine - j0);
    if ((int)threadIdx.x < nj) {
      const int item = (int)blockIdx.x + (j0 + (int)threadIdx.x) * (int)gridDim.x;
      int bg, split, rb;
      decode_item(p, item, bg, split, rb);
      uint32_t* ctr = p.counters + (size_t)bg * p.n_rb + rb;
      const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = prev == (uint32_t)(p.S - 1);
      if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last[threadIdx.x] = last ? item : -1;
    }
    __syncthreads();
    // every (completed block, batch row, row) of this chunk, one output per thread
    const int per_item = MC * kRows;
    for (int idx = threadIdx.x; idx < nj * per_item; idx += kThreads) {
      const int j = idx / per_item;
      const int item = s_last[j];
      if (item < 0) continue;
      const int rem = idx - j * per_item;
      const int r = rem / kRows;
      int bg, split, rb;
      decode_item(p, item, bg, split, rb);
      const int row = rb * kRows + (rem - r * kRows);
      const int rr = bg * MC + r;
      if (row >= p.N || rr >= p.m) continue;
      // the partials are read eight at a time, all eight in flight together
      // (one memory round trip per eight splits), and added in split order
      const float* part = p.partial + (size_t)rr * p.Npad + row;
      const size_t sstride = (size_t)p.m * p.Npad;
      float sum = 0.f;
      for (int s0 = 0; s0 < p.S; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int s = min(s0 + u, p.S - 1);   // past the last split: a valid slot, unused
          v[u] = __hip_atomic_load(part + (size_t)s * sstride, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < p.S) sum += v[u];
      }
      p.y[(size_t)rr * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)sum);
    }
    __syncthreads();
  }
}

// Persistent kernel: workgroup b processes items b, b + gridDim.x, ... A ring
// of NR register sets holds the tiles in flight: at the start of each tile the
// loads of the tile NR-1 ahead are issued into the set the previous tile used.
// Each step (one batch row of one tile) looks up its table, builds the next
// step's table in the other LDS buffer, and ends at the step's one barrier.
// Q: sign planes; RPW: row tiles per wave; MC: batch rows per item; GQ: see
// TileRegs; OFF: offset term; W: waves per workgroup (8 or 16).
// XL (batch 1 only): x is staged whole in LDS at the start, and the tables are
// built from there, instead of every wave loading each x tile from L2 (all
// waves of all CUs reading the same lines).
// PR (two or more batch rows, grouped scales): paired tables in one buffer; each
// tile takes, per pair of batch rows, a barrier, the pair's table build, a
// barrier and the pair's lookups.
// EI (with XL and two register sets): a set is refilled with the tile two
// ahead as soon as its lookups are done, instead of at the start of the next
// step, so two tiles are in flight from the start (the first table build
// overlaps both, the staging of x the first). That loop leaves only after its second
// step and issues its loads unconditionally: every path into the loop head
// then has the same loads outstanding, and the compiler's wait counts before
// the lookups stay exact (they would otherwise also wait for the tile ahead).
// ONCE (batch 1 without x in LDS): each sign byte is read once per product, and
// its loads are non-temporal as they are with XL.
// HT (with PR): half paired tables in two buffers; each step (one pair of
// batch rows of one tile) looks up one buffer, builds the next step's table in
// the other and ends at the step's one barrier.
// SP (with PR, 16 waves, one row tile per wave): split paired tables; each
// tile takes two steps per pair of batch rows, one per half of its chunks,
// each looking up one buffer, building the next step's table in the other and
// ending at its one barrier.
// MB (with PR, 16 waves): the paired tables are built by MFMA (build_pair_mfma).
template <int Q, int RPW, int MC, bool GQ, bool OFF, int W, int NR, bool XL, bool PR = false,
          bool EI = false, bool ONCE = false, bool HT = false, bool SP = false, bool MB = false>
// The 128 KiB of LDS allows one workgroup per CU, so W/4 waves per SIMD is
// also the most that can ever run; saying so lets the scheduler use the
// whole register budget to keep table lookups in flight.
__global__ void __launch_bounds__(W * 64, W / 4)
    __attribute__((amdgpu_waves_per_eu(W / 4, W / 4))) lutgemv_kernel(Params p) {
  static_assert(!XL || MC == 1, "x in LDS is for batch 1");
  static_assert(!PR || (GQ && !XL && MC % 2 == 0), "paired tables: grouped scales, even MC");
  static_assert(!EI || (XL && NR == 2 && !PR), "early issue: x in LDS, two register sets");
  static_assert(!ONCE || (!XL && !PR && MC == 1), "read-once loads: batch 1 without x in LDS");
  static_assert(!HT || PR, "half tables are paired");
  static_assert(!SP || (PR && !HT && RPW == 1 && W == 16), "split paired tables: 16 waves x 1 row tile");
  static_assert(!MB || (PR && !HT && !SP && W == 16), "MFMA-built tables: paired, 16 waves");
  LUTGEMM_PHASE(0);
  LUTGEMM_PHASE_FLAG(traced_table);
  LUTGEMM_PHASE_FLAG(traced_step);
  __shared__ float lut[2 * kLutWords];
  __shared__ uint4 xs[XL ? kXChunks : 1];
  using TR = TileRegs<Q, RPW, MC, GQ, OFF>;

  LaneCtx l = lane_ctx();
  if constexpr (GQ) tile_group_offsets<Q>(p, l);

  float acc[MC][RPW][4];
#pragma unroll
  for (int r = 0; r < MC; ++r)
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[r][i][a] = 0.f;

  // XL: the loads of x are issued first, all at once (NX per thread, reads past
  // the end of x return zero), then those of the first tiles; the stores into
  // LDS wait only for x. The first table build waits for these loads, so their
  // latency is paid once, not once per loop trip.
  constexpr int NX = XL ? (kXChunks + W * 64 - 1) / (W * 64) : 1;
  uint4 xr[NX];
  if constexpr (XL) {
    const auto xrs = make_rsrc(p.x, (uint32_t)p.K * 2u);
#pragma unroll
    for (int j = 0; j < NX; ++j) xr[j] = load16(xrs, ((uint32_t)threadIdx.x + (uint32_t)(j * W * 64)) * 16u);
    // A compiler-only barrier: without it the loads of x are sunk below the
    // exit and the item arithmetic that follow (two integer divisions and a
    // second round of argument loads), and the fetch of x, the first thing
    // every workgroup waits for, starts that much later.
    asm volatile("" ::: "memory");
  }
  TR R[NR];
  R[0].pos = first_tile<RPW, MC, W>(p, l.wave, blockIdx.x);
  if constexpr (XL) {
    if (!R[0].pos.live) return;
    load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, R[0]);
  } else {
    // The first tile's loads go ahead of the exit (a dead position touches no
    // memory), and the barrier keeps them there, so the buffer addresses they
    // need are fetched with the other kernel arguments in one round instead of
    // a third round after the exit.
    load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, R[0]);
    asm volatile("" ::: "memory");
    if (!R[0].pos.live) return;
  }
#pragma unroll
  for (int s = 1; s + 1 < NR; ++s) {
    R[s].pos = next_tile<RPW, MC, W>(p, l.wave, R[s - 1].pos);
    load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, R[s]);
  }
  if constexpr (XL) {   // chunk c of x at xs[c], for the KT input tiles (zero past K)
    const int nchunks = p.KT * kChunkTile;
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int c = (int)threadIdx.x + j * W * 64;
      if (c < nchunks) xs[c] = xr[j];
    }
    __syncthreads();
    LUTGEMM_PHASE(1);
  }
  // EI: the second tile's loads go out once x is staged, not with the first
  // tile's: a wave held at issuing them (the CU's memory queue is full at the
  // start) then no longer delays the barrier above (x staged at 1.9 instead of
  // 3.6 us on 49152 x 12288; 0.3-1% faster on 32768-65536 rows).
  if constexpr (EI) {
    R[1].pos = next_tile<RPW, MC, W>(p, l.wave, R[0].pos);
    load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, R[1]);
  }
  // activations of chunk `lane` of a tile, for the table build
  auto xtile = [&](const TR& T, int r) -> uint4 {
    if constexpr (XL) {
      return xs[T.pos.kt * kChunkTile + l.lane];
    } else {
      return T.xv[r];
    }
  };
  if constexpr (SP) {
    float sacc[MC][2];
#pragma unroll
    for (int r = 0; r < MC; ++r) sacc[r][0] = sacc[r][1] = 0.f;
    build_split(lut, 0, l, split_x<0>(R[0].xv[0], R[0].xv[1]));
    __syncthreads();
    LUTGEMM_PHASE(2);
    bool done = false;
    while (!done) {
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        if (!done) {
          TR& cur = R[s];
          TR& nxt = R[(s + 1) % NR];
          TR& pre = R[(s + NR - 1) % NR];
          pre.pos = next_tile<RPW, MC, W>(p, l.wave, R[(s + NR - 2) % NR].pos);
          load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, pre);
          split_arrange<Q, MC, OFF>(cur);
#pragma unroll
          for (int h = 0; h < MC / 2; ++h) {
            if (2 * h < cur.pos.c.rows_here) {  // uniform over the workgroup
              lookups_split<Q, MC, OFF, 0>(l, h, lut, cur, sacc);
              build_split(lut, 1, l, split_x<1>(cur.xv[2 * h], cur.xv[2 * h + 1]));
              __syncthreads();
              lookups_split<Q, MC, OFF, 1>(l, h, lut, cur, sacc);
              const int hn = 2 * h + 2 < MC ? 2 * h + 2 : 0;   // a constant once unrolled
              if (2 * h + 2 < cur.pos.c.rows_here) {
                build_split(lut, 0, l, split_x<0>(cur.xv[hn], cur.xv[hn + 1]));
              } else if (nxt.pos.live) {
                build_split(lut, 0, l, split_x<0>(nxt.xv[0], nxt.xv[1]));
              }
              __syncthreads();
              LUTGEMM_PHASE_ONCE(3, traced_step);
            }
          }
          if (cur.pos.kt + 1 == cur.pos.c.kt1) finish_split<MC>(p, l, cur.pos.c, sacc);
          done = !nxt.pos.live;
        }
      }
    }
    LUTGEMM_PHASE(4);
    if (p.S > 1) split_epilogue<RPW, MC, W>(p, reinterpret_cast<int*>(lut));
    LUTGEMM_PHASE(5);
    return;
  } else if constexpr (HT) {
    int buf = 0;
    build_half_pair<W>(lut, 0, l, R[0].xv[0], R[0].xv[1]);
    __syncthreads();
    LUTGEMM_PHASE(2);
    bool done = false;
    while (!done) {
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        if (!done) {
          TR& cur = R[s];
          TR& nxt = R[(s + 1) % NR];
          TR& pre = R[(s + NR - 1) % NR];
          pre.pos = next_tile<RPW, MC, W>(p, l.wave, R[(s + NR - 2) % NR].pos);
          load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, pre);
#pragma unroll
          for (int h = 0; h < MC / 2; ++h) {
            if (2 * h < cur.pos.c.rows_here) {  // uniform over the workgroup
              lookups_half<Q, RPW, MC, OFF>(l, h, buf, lut, cur, acc);
              const int hn = 2 * h + 2 < MC ? 2 * h + 2 : 0;   // a constant once unrolled
              if (2 * h + 2 < cur.pos.c.rows_here) {
                build_half_pair<W>(lut, buf ^ 1, l, cur.xv[hn], cur.xv[hn + 1]);
              } else if (nxt.pos.live) {
                build_half_pair<W>(lut, buf ^ 1, l, nxt.xv[0], nxt.xv[1]);
              }
              __syncthreads();
              LUTGEMM_PHASE_ONCE(3, traced_step);
              buf ^= 1;
            }
          }
          if (cur.pos.kt + 1 == cur.pos.c.kt1) finish_item<RPW, MC>(p, l, cur.pos.c, acc);
          done = !nxt.pos.live;
        }
      }
    }
    LUTGEMM_PHASE(4);
    if (p.S > 1) split_epilogue<RPW, MC, W>(p, reinterpret_cast<int*>(lut));
    LUTGEMM_PHASE(5);
    return;
  } else if constexpr (PR) {
    half4v sgn = {};
    if constexpr (MB) sgn = mfma_signs(l);
    bool done = false;
    while (!done) {
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        if (!done) {
          TR& cur = R[s];
          TR& nxt = R[(s + 1) % NR];
          TR& pre = R[(s + NR - 1) % NR];
          pre.pos = next_tile<RPW, MC, W>(p, l.wave, R[(s + NR - 2) % NR].pos);
          load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, pre);
#pragma unroll
          for (int h = 0; h < MC / 2; ++h) {
            if (2 * h < cur.pos.c.rows_here) {  // uniform over the workgroup
              __syncthreads();                  // the previous lookups are done
              if constexpr (MB) {
                build_pair_mfma(lut, l, sgn, cur.xv[h]);
              } else {
                build_table_pair<W>(lut, l, cur.xv[2 * h], cur.xv[2 * h + 1]);
              }
              __syncthreads();
              LUTGEMM_PHASE_ONCE(2, traced_table);
              lookups_pair<Q, RPW, MC, OFF>(l, h, lut, cur, acc);
            }
          }
          LUTGEMM_PHASE_ONCE(3, traced_step);
          if (cur.pos.kt + 1 == cur.pos.c.kt1) finish_item<RPW, MC>(p, l, cur.pos.c, acc);
          done = !nxt.pos.live;
        }
      }
    }
    LUTGEMM_PHASE(4);
    if (p.S > 1) split_epilogue<RPW, MC, W>(p, reinterpret_cast<int*>(lut));
    LUTGEMM_PHASE(5);
    return;
  }
  int buf = 0;
  build_table<W>(lut, 0, l, xtile(R[0], 0));
  __syncthreads();
  LUTGEMM_PHASE(2);
  if constexpr (EI) {
    for (;;) {
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        TR& cur = R[s];
        TR& nxt = R[(s + 1) % NR];
        const TilePos was = cur.pos;
        if (was.live) lookups(l, 0, buf, lut, cur, acc);   // uniform over the workgroup
        cur.pos = next_tile<RPW, MC, W>(p, l.wave, nxt.pos);
        load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, cur);
        if (was.live) {
          if (nxt.pos.live) build_table<W>(lut, buf ^ 1, l, xtile(nxt, 0));
          __syncthreads();
          LUTGEMM_PHASE_ONCE(3, traced_step);
          buf ^= 1;
          if (was.kt + 1 == was.c.kt1) finish_item<RPW, MC>(p, l, was.c, acc);
        }
      }
      if (!R[0].pos.live) break;
    }
    LUTGEMM_PHASE(4);
    if (p.S > 1) split_epilogue<RPW, MC, W>(p, reinterpret_cast<int*>(lut));
    LUTGEMM_PHASE(5);
    return;
  }
  bool done = false;
  while (!done) {
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      if (!done) {
        TR& cur = R[s];
        TR& nxt = R[(s + 1) % NR];
        TR& pre = R[(s + NR - 1) % NR];
        pre.pos = next_tile<RPW, MC, W>(p, l.wave, R[(s + NR - 2) % NR].pos);
        load_tile<Q, RPW, MC, GQ, OFF, XL, XL || ONCE, MB>(p, l, pre);
#pragma unroll
        for (int r = 0; r < MC; ++r) {
          if (r < cur.pos.c.rows_here) {  // uniform over the workgroup
            lookups(l, r, buf, lut, cur, acc);
            if (r + 1 < cur.pos.c.rows_here) {
              build_table<W>(lut, buf ^ 1, l, xtile(cur, r + 1 < MC ? r + 1 : r));
            } else if (nxt.pos.live) {
              build_table<W>(lut, buf ^ 1, l, xtile(nxt, 0));
            }
            __syncthreads();
            LUTGEMM_PHASE_ONCE(3, traced_step);
            buf ^= 1;
          }
        }
        if (cur.pos.kt + 1 == cur.pos.c.kt1) finish_item<RPW, MC>(p, l, cur.pos.c, acc);
        done = !nxt.pos.live;
      }
    }
  }
  LUTGEMM_PHASE(4);
  if (p.S > 1) split_epilogue<RPW, MC, W>(p, reinterpret_cast<int*>(lut));
  LUTGEMM_PHASE(5);
}

// ------------------------------------------------------------------ unit kernel
// Batch 1 with few row tiles per compute unit (the nibble-table kernel below).
// A workgroup takes ri row tiles over the whole input dimension, and the work
// is spread over its 16 waves in units of one (row tile, plane): unit u = row
// tile u / Q, plane u % Q of the workgroup, held by wave u % 16 (UPW units per
// wave at most). Each wave keeps the loads of its units for the next NR input
// tiles in flight. At the end each unit's 16 row sums are written to LDS and
// added over the planes in plane order. No split of the input dimension: no
// partial sums in memory.
template <int UPW>
struct UnitRegs {
  uint4 bw[UPW];          // lane block of the unit's plane block
  uint32_t aw[UPW][2];    // scales of the lane's four rows (fp16 pairs)
  uint32_t ow[UPW][2];    // offsets of the lane's four rows (plane-0 units only)
};

// Where this wave's units are, computed once per workgroup (all uniform over the
// wave but the lane offsets of the scales). The unit kernels take group sizes
// that divide 512 (every input tile starts a group; a lane's group within the
// tile is fixed) or are multiples of 512 (an input tile lies in one group).
template <int Q, int UPW>
struct UnitPlan {
  bool on[UPW];            // unit exists in this workgroup
  bool q0[UPW];            // unit holds plane 0 (adds the offset term)
  uint32_t bits0[UPW];     // byte offset of the unit's block in input tile 0
  uint32_t arow[UPW];      // the unit's row tile times the groups per row
  uint32_t avoff[UPW];     // lane's byte offset in a scale block (per lane)
  uint32_t ovoff;          // lane's byte offset in an offset block (per lane)
  uint32_t tile_stride;    // bytes of packed sign planes per input tile
  uint32_t ginc, gper;     // groups per input tile (g divides 512) / input tiles per group
};

template <int Q, int UPW>
__device__ __forceinline__ UnitPlan<Q, UPW> unit_plan(const Params& p, const LaneCtx& l, int rt0,
                                                    int nunits) {
  UnitPlan<Q, UPW> P;
  const bool tile_groups = (512 % p.g) == 0;
  P.ginc = tile_groups ? (uint32_t)(512 / p.g) : 0u;
  P.gper = tile_groups ? 0x7FFFFFFFu : (uint32_t)(p.g / 512);
  const uint32_t g_rel = tile_groups ? (uint32_t)((32 * l.c4) >> p.g_shift) : 0u;
  P.tile_stride = (uint32_t)p.RT * (uint32_t)(Q * 1024);
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = l.wave + 16 * j;
    const int rtl = u / Q, q = u - (u / Q) * Q;
    P.on[j] = u < nunits;
    P.q0[j] = q == 0;
    // blocks of consecutive row tiles are consecutive, plane by plane
    P.bits0[j] = ((uint32_t)rt0 * Q + (uint32_t)u) * 1024u;
    P.arow[j] = (uint32_t)(rt0 + rtl) * (uint32_t)p.G;
    P.avoff[j] = g_rel * 32u * Q + (uint32_t)q * 32u + 8u * (uint32_t)l.r4;
  }
  P.ovoff = g_rel * 32u + 8u * (uint32_t)l.r4;
  return P;
}

// The input tile whose loads are issued next: its index, its sign-plane offset
// and its first scale group, advanced by a few scalar adds per tile.
struct UnitCursor {
  int kt;
  uint32_t bts;            // kt * tile_stride
  uint32_t grp, cnt;       // first group of the tile; tiles into that group
};

template <int Q, int UPW>
__device__ __forceinline__ void advance(const UnitPlan<Q, UPW>& P, UnitCursor& c) {
  c.kt += 1;
  c.bts += P.tile_stride;
  c.grp += P.ginc;
  c.cnt += 1;
  if (c.cnt == P.gper) {
    c.cnt = 0;
    c.grp += 1;
  }
}

// Issue the loads of the cursor's tile for this wave's units (unconditional; a
// unit past the workgroup's units or a tile past the end gets empty ranges),
// then advance the cursor.
template <int Q, bool OFF, int UPW>
__device__ __forceinline__ void load_units(const Params& p, const LaneCtx& l,
                                           const UnitPlan<Q, UPW>& P, UnitCursor& c,
                                           UnitRegs<UPW>& R) {
  const bool live = c.kt < p.KT;
  // groups this tile's loads may touch (g_span, fewer at the end of a row)
  const uint32_t span = (uint32_t)min(p.G - (int)c.grp, p.g_span);
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const bool on = live && P.on[j];
    const uint32_t bs = P.bits0[j] + c.bts;
    R.bw[j] = load16<true>(make_rsrc(p.bits, on ? bs + 1024u : 0u), l.block, bs);
    const uint32_t blk = P.arow[j] + c.grp;
    const uint32_t ab = blk * (32u * Q);
    const uint2 a = load8(make_rsrc(p.alpha, on ? ab + span * (32u * Q) : 0u), P.avoff[j], ab);
    R.aw[j][0] = a.x;
    R.aw[j][1] = a.y;
    if constexpr (OFF) {
      const bool ono = on && P.q0[j];
      const uint2 o = load8(make_rsrc(p.offset, ono ? (blk + span) * 32u : 0u), P.ovoff,
                            blk * 32u);
      R.ow[j][0] = o.x;
      R.ow[j][1] = o.y;
    }
  }
  advance(P, c);
}

// ------------------------------------------------------------------ nibble tables
// The unit kernel with 4-input tables. Chunk t (8 inputs) is split into two
// halves j (inputs 8t + 4j .. +3); the table of a half holds its 16 signed sums,
// entry e = sum_s (bit s of e ? +x : -x). A weight byte b then selects
// T[0][b & 15] + T[1][b >> 4], which is the 8-input table's entry b, so the
// packed format is unchanged. The tables of 1024 chunks (8192 inputs, one
// phase) take 128 KiB: entry e of half j of chunk t at word (2 e + j) * 1024 + t,
// so the lanes of a lookup read consecutive chunks (no bank conflicts), and a
// lane's base address and the tile's offset stay below 16 KiB (the tile's
// offset goes in the read's immediate offset). They
// are built once per phase (two phases at most, as x is staged whole), so the
// loop over the input tiles has no table builds and no barriers: each wave
// streams its units freely. A lookup costs two VALU operations for its address
// (a rotate that brings the nibble to bits 13-16 and a mask-or with the
// table's base) where the 8-input table needs one, and two reads per weight
// byte instead of one; for workgroups with few row tiles the build it saves
// costs more than that.
constexpr int kPhaseChunks = 1024;                         // 8192 inputs per phase
constexpr int kPhaseTiles = kPhaseChunks / kChunkTile;     // 16 input tiles

// Tables of the phase that starts at chunk c0 (chunk c0 + t at column t): thread
// t builds both halves of its chunk, 16 entries each, in Gray-code order.
__device__ __forceinline__ void build_nibbles(float* lut, const uint4* xs, int c0, int nchunks) {
  const int t = threadIdx.x;                    // 1024 threads = kPhaseChunks
  if (c0 + t >= nchunks) return;
  float x[8];
  unpack8(xs[c0 + t], x);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float* h = x + 4 * j;
    float T = -((h[0] + h[1]) + (h[2] + h[3]));  // entry 0: every sign negative
    float two[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) two[b] = h[b] + h[b];
    float* base = lut + j * kPhaseChunks + t;
    base[0] = T;
#pragma unroll
    for (int n = 1; n < 16; ++n) {
      const int b = __builtin_ctz(n);
      const int e = n ^ (n >> 1);
      T += ((e >> b) & 1) ? two[b] : -two[b];
      base[2 * e * kPhaseChunks] = T;
    }
  }
}

template <int Q, bool OFF, int UPW, int NR>
__global__ void __launch_bounds__(1024, 4) __attribute__((amdgpu_waves_per_eu(4, 4)))
    lutgemv_nibble_kernel(Params p) {
  static_assert(kPhaseTiles % NR == 0, "the ring depth divides the tiles of a phase");
  LUTGEMM_PHASE(0);
  LUTGEMM_PHASE_FLAG(traced_step);
  __shared__ float lut[2 * 16 * kPhaseChunks];
  __shared__ uint4 xs[kXChunks];
  LaneCtx l = lane_ctx();
  const int item = blockIdx.x;
  const int rt0 = item * p.ri;
  const int ri = min(p.ri, p.RT - rt0);
  const int nunits = ri * Q;
  const int nchunks = p.KT * kChunkTile;

  constexpr int NX = (kXChunks + 1023) / 1024;
  uint4 xr[NX];
  {
    const auto xrs = make_rsrc(p.x, (uint32_t)p.K * 2u);
#pragma unroll
    for (int j = 0; j < NX; ++j)
      xr[j] = load16(xrs, ((uint32_t)threadIdx.x + (uint32_t)(j * 1024)) * 16u);
    // x reaches LDS before the weight loads are issued: issued behind the
    // first NR tiles of every workgroup, its loads would wait in the memory
    // queues behind all of them (measured 5-6% faster on 28672 x 8192 and
    // 512 x 512)
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int c = (int)threadIdx.x + j * 1024;
      if (c < nchunks) xs[c] = xr[j];
    }
    asm volatile("" ::: "memory");
  }
  const UnitPlan<Q, UPW> P = unit_plan<Q, UPW>(p, l, rt0, nunits);
  const bool has_units = P.on[0];               // uniform over the wave
  UnitCursor ic{0, 0u, 0u, 0u};                 // the tile whose loads go out next
  UnitRegs<UPW> R[NR];
  if (has_units) {
#pragma unroll
    for (int s = 0; s < NR; ++s) load_units<Q, OFF, UPW>(p, l, P, ic, R[s]);
  }
  __syncthreads();
  LUTGEMM_PHASE(1);
  build_nibbles(lut, xs, 0, nchunks);
  __syncthreads();
  LUTGEMM_PHASE(2);

  // per visit k and half j: the rotation that brings the half's nibble of byte
  // b_k to bits 13-16, and the table base (half, chunk 4*c4 + b_k of the tile)
  uint32_t rot[4][2], nbase[4][2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t b = (uint32_t)((k + l.r4) & 3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      rot[k][j] = (8u * b + 4u * (uint32_t)j + 19u) & 31u;     // right by 8b + 4j - 13
      nbase[k][j] = ((uint32_t)j << 12) | ((4u * (uint32_t)l.c4 + b) << 2);
    }
  }

  float acc[UPW][4];
#pragma unroll
  for (int j = 0; j < UPW; ++j)
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[j][a] = 0.f;

  // Steps leave the loop only after a whole phase, and every step issues its
  // loads (empty past the end): the wait counts are the same on every path.
  // Waves without units only take part in the builds.
  for (int kt0 = 0; kt0 < p.KT; kt0 += kPhaseTiles) {
    if (kt0 > 0) {                              // uniform: the next phase's tables
      __syncthreads();
      build_nibbles(lut, xs, kt0 * kChunkTile, nchunks);
      __syncthreads();
    }
    if (!has_units) continue;
#pragma unroll
    for (int s = 0; s < kPhaseTiles; ++s) {
      const int kt = kt0 + s;
      UnitRegs<UPW>& cur = R[s % NR];
      if (kt < p.KT) {                          // uniform over the workgroup
        const uint32_t toff = (uint32_t)s * (kChunkTile * 4);   // the tile's chunks in the phase
        float csum = 0.f;
        if constexpr (OFF) {
          bool has0 = false;
#pragma unroll
          for (int j = 0; j < UPW; ++j) has0 = has0 || (P.on[j] && P.q0[j]);
          if (has0) {                            // entry 15 of both halves: the chunk's sum
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
              for (int j = 0; j < 2; ++j) csum += lut_at(lut, (nbase[k][j] | (15u << 13)) + toff);
          }
        }
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
          if (P.on[j]) {                        // uniform over the wave
            const uint32_t words[4] = {cur.bw[j].x, cur.bw[j].y, cur.bw[j].z, cur.bw[j].w};
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              float e[4][2];
#pragma unroll
              for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const uint32_t r = __builtin_amdgcn_alignbit(words[a], words[a], rot[k][h]);
                  e[k][h] = lut_at(lut, ((r & 0x1E000u) | nbase[k][h]) + toff);
                }
              const float sm = ((e[0][0] + e[0][1]) + (e[1][0] + e[1][1])) +
                               ((e[2][0] + e[2][1]) + (e[3][0] + e[3][1]));
              acc[j][a] = __builtin_fmaf(h2f(cur.aw[j][a >> 1], a & 1), sm, acc[j][a]);
            }
            if constexpr (OFF) {
              if (P.q0[j]) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
                  acc[j][a] = __builtin_fmaf(h2f(cur.ow[j][a >> 1], a & 1), csum, acc[j][a]);
              }
            }
          }
        }
      }
      load_units<Q, OFF, UPW>(p, l, P, ic, cur);
      LUTGEMM_PHASE_ONCE(3, traced_step);       // wave 0's first tile
    }
  }
  LUTGEMM_PHASE(4);
  __syncthreads();                              // every lookup done: the tables are free
  float* red = lut;
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = l.wave + 16 * j;
    if (P.on[j]) {
      const float v[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      const float t = row_sum16(v, l.lane);
      if (holds_row_sum(l.lane)) red[u * kRowTile + reduced_row(l.lane)] = t;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < ri * kRowTile; idx += 1024) {
    const int rtl = idx / kRowTile, row = idx - rtl * kRowTile;
    float sum = red[(rtl * Q) * kRowTile + row];
#pragma unroll
    for (int q = 1; q < Q; ++q) sum += red[(rtl * Q + q) * kRowTile + row];
    const int n = (rt0 + rtl) * kRowTile + row;
    if (n < p.N) p.y[n] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
  LUTGEMM_PHASE(5);
}

// ------------------------------------------------------------------ instances

using KernelFn = void (*)(Params);

// Register budget per wave: 256 VGPRs with 8 waves (two per SIMD), 128 with 16
// (four per SIMD). An instance keeps a ring of NR tiles in flight, the
// accumulators and some temporaries in that budget: three tiles when they fit,
// else two (16 waves use two, plus a deeper ring where it fits).
template <int Q, int RPW, int MC, bool GQ, bool OFF, int NR, bool XL = false, bool PR = false>
constexpr int kVgprEstimate =
    NR * (RPW * Q * 4 + RPW * (GQ ? 2 * Q : 8 * Q) + (XL ? 0 : MC * 4) +
          (OFF ? RPW * (GQ ? 2 : 8) : 0)) +
    4 * RPW * MC + (GQ ? 16 + 2 : 4) + 32 +  // + the table entries of one lookup group in
    (PR ? 16 + 4 : 0);                       // flight (+ lane scale offsets); paired: entry
                                             // pairs and address selectors

template <int W>
constexpr int kBudget = W == 16 ? 128 : 256;

template <int Q, int RPW, int MC, bool GQ, bool OFF, int W>
constexpr int kRing =
    (W == 8 && kVgprEstimate<Q, RPW, MC, GQ, OFF, 3> + 8 <= kBudget<W>) ? 3 : 2;

template <int Q, int RPW, int MC, bool GQ, bool OFF, int W>
constexpr bool kInstantiated =
    (W == 16 ? (MC == 1 && GQ) : (W == 8)) &&
    kVgprEstimate<Q, RPW, MC, GQ, OFF, kRing<Q, RPW, MC, GQ, OFF, W>> <= kBudget<W>;

// Whether a 16-wave instance with an NR-deep ring fits the register budget.
template <int Q, int RPW, int MC, bool GQ, bool OFF, int W, bool XL, int NR>
constexpr bool kFits16 =
    W == 16 && MC == 1 && GQ && kVgprEstimate<Q, RPW, MC, GQ, OFF, NR, XL> <= kBudget<W>;

// Ring depth of a paired-table instance: three tiles where they fit (8 waves),
// else two; 0 when not even two fit. At 16 waves the estimate is allowed 8
// registers over the budget: it counts every entry pair of a lookup group as
// live at once, and the compiler fits those instances (q <= 3, one row tile,
// two batch rows) in 105-113 registers without spilling.
template <int Q, int RPW, int MC, bool OFF, int W>
constexpr int kRingPair =
    (MC % 2 != 0) ? 0
    : (W == 8 && kVgprEstimate<Q, RPW, MC, true, OFF, 3, false, true> + 8 <= kBudget<W>) ? 3
    : (kVgprEstimate<Q, RPW, MC, true, OFF, 2, false, true> <= kBudget<W> + (W == 16 ? 8 : 0)) ? 2
    : 0;

// ring 3 or 4 selects a deeper ring where an instance has one (16 waves); xl
// the x-in-LDS variant (16 waves, batch 1, grouped scales); pr the paired
// tables (grouped scales, even MC); ei the early-issue ring of the x-in-LDS
// variant (default ring only); once the read-once (non-temporal) sign-plane
// loads of the 16-wave batch-1 instances without x in LDS.
// pr: 1 paired tables, 2 half paired tables (one row tile per wave only), 3
// split paired tables (16 waves, one row tile per wave, two batch rows), 4
// paired tables built by MFMA (16 waves).
template <int Q, int RPW, int MC, bool GQ, bool OFF, int W>
KernelFn kernel_or_null(int ring, bool xl, int pr, bool ei, bool once) {
  if (pr) {
    if constexpr (GQ && kRingPair<Q, RPW, MC, OFF, W> > 0) {
      if (xl) return nullptr;
      if (pr == 4) {
        if constexpr (W == 16) {
          return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, kRingPair<Q, RPW, MC, OFF, W>, false, true,
                                false, false, false, false, true>;
        } else {
          return nullptr;
        }
      }
      if (pr == 3) {
        if constexpr (RPW == 1 && W == 16 && MC == 2) {
          return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, kRingPair<Q, RPW, MC, OFF, W>, false, true,
                                false, false, false, true>;
        } else {
          return nullptr;
        }
      }
      if (pr == 2) {
        if constexpr (RPW == 1) {
          return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, kRingPair<Q, RPW, MC, OFF, W>, false, true,
                                false, false, true>;
        } else {
          return nullptr;
        }
      }
      return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, kRingPair<Q, RPW, MC, OFF, W>, false, true>;
    } else {
      return nullptr;
    }
  }
  if constexpr (kInstantiated<Q, RPW, MC, GQ, OFF, W>) {
    if constexpr (W == 16 && MC == 1 && GQ) {
      if (xl) {
        if (ei && ring < 3) return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, 2, true, false, true>;
        if constexpr (kFits16<Q, RPW, MC, GQ, OFF, W, true, 4>) {
          if (ring == 4) return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, 4, true>;
        }
        if constexpr (kFits16<Q, RPW, MC, GQ, OFF, W, true, 3>) {
          if (ring >= 3) return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, 3, true>;
        }
        return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, 2, true>;
      }
      if constexpr (kFits16<Q, RPW, MC, GQ, OFF, W, false, 3>) {
        if (ring >= 3) {
          return once ? lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, 3, false, false, false, true>
                      : lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, 3, false>;
        }
      }
      if (once && !xl)
        return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, kRing<Q, RPW, MC, GQ, OFF, W>, false, false,
                              false, true>;
    }
    if (xl) return nullptr;
    return lutgemv_kernel<Q, RPW, MC, GQ, OFF, W, kRing<Q, RPW, MC, GQ, OFF, W>, false>;
  } else {
    (void)ring;
    (void)xl;
    (void)ei;
    (void)once;
    return nullptr;
  }
}

template <int Q, int RPW, int MC, int W>
KernelFn pick_flags(bool gq, bool off, int ring, bool xl, int pr, bool ei, bool once) {
  if (gq)
    return off ? kernel_or_null<Q, RPW, MC, true, true, W>(ring, xl, pr, ei, once)
               : kernel_or_null<Q, RPW, MC, true, false, W>(ring, xl, pr, ei, once);
  return off ? kernel_or_null<Q, RPW, MC, false, true, W>(ring, xl, pr, ei, once)
             : kernel_or_null<Q, RPW, MC, false, false, W>(ring, xl, pr, ei, once);
}

template <int Q, int W>
KernelFn pick_rpw_mc(int rpw, int mc, bool gq, bool off, int ring, bool xl, int pr, bool ei,
                     bool once) {
  if (mc == 1) {
    if (rpw == 2) return pick_flags<Q, 2, 1, W>(gq, off, ring, xl, pr, ei, once);
    if (rpw == 1) return pick_flags<Q, 1, 1, W>(gq, off, ring, xl, pr, ei, once);
  } else if (mc == 2) {
    if (rpw == 2) return pick_flags<Q, 2, 2, W>(gq, off, ring, xl, pr, ei, once);
    if (rpw == 1) return pick_flags<Q, 1, 2, W>(gq, off, ring, xl, pr, ei, once);
  } else if (mc == 4) {
    if (rpw == 2) return pick_flags<Q, 2, 4, W>(gq, off, ring, xl, pr, ei, once);
    if (rpw == 1) return pick_flags<Q, 1, 4, W>(gq, off, ring, xl, pr, ei, once);
  }
  return nullptr;
}

// The instance for q = Q planes, rpw row tiles per wave, mc batch rows per
// item, scale groups aligned to 32 inputs (gq), an offset term (off), w waves
// per workgroup, ring depth (0 default, >= 3 deeper), x in LDS (xl), paired
// tables (pr: 1 paired, 2 half paired, 3 split paired, 4 MFMA-built paired), the
// early-issue ring (ei) and read-once
// sign-plane loads (once), or nullptr if none is built.
template <int Q>
KernelFn kernels_of_q(int rpw, int mc, bool gq, bool off, int w, int ring, bool xl, int pr,
                      bool ei, bool once) {
  if (w == 16) return pick_rpw_mc<Q, 16>(rpw, mc, gq, off, ring, xl, pr, ei, once);
  if (w == 8) return pick_rpw_mc<Q, 8>(rpw, mc, gq, off, ring, xl, pr, ei, once);
  return nullptr;
}

// Nibble-table instances: (units per wave, ring depth) with the ring dividing
// the 16 tiles of a phase: (1, 8), (2, 4), (3, 2), (4, 2), plus (1, 4) and
// (2, 2) for tuning; nr = 0 picks the deepest for upw.
template <int Q>
KernelFn nibble_kernel_of_q(bool off, int upw, int nr) {
  if (upw == 1) {
    if (nr == 4) return off ? lutgemv_nibble_kernel<Q, true, 1, 4> : lutgemv_nibble_kernel<Q, false, 1, 4>;
    if (nr == 0 || nr == 8)
      return off ? lutgemv_nibble_kernel<Q, true, 1, 8> : lutgemv_nibble_kernel<Q, false, 1, 8>;
  } else if (upw == 2) {
    if (nr == 2) return off ? lutgemv_nibble_kernel<Q, true, 2, 2> : lutgemv_nibble_kernel<Q, false, 2, 2>;
    if (nr == 0 || nr == 4)
      return off ? lutgemv_nibble_kernel<Q, true, 2, 4> : lutgemv_nibble_kernel<Q, false, 2, 4>;
  } else if (upw == 3) {
    if (nr == 0 || nr == 2)
      return off ? lutgemv_nibble_kernel<Q, true, 3, 2> : lutgemv_nibble_kernel<Q, false, 3, 2>;
  } else if (upw == 4) {
    if (nr == 0 || nr == 2)
      return off ? lutgemv_nibble_kernel<Q, true, 4, 2> : lutgemv_nibble_kernel<Q, false, 4, 2>;
  }
  return nullptr;
}

extern template KernelFn nibble_kernel_of_q<1>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<2>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<3>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<4>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<5>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<6>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<7>(bool, int, int);
extern template KernelFn nibble_kernel_of_q<8>(bool, int, int);

extern template KernelFn kernels_of_q<1>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<2>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<3>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<4>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<5>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<6>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<7>(int, int, bool, bool, int, int, bool, int, bool, bool);
extern template KernelFn kernels_of_q<8>(int, int, bool, bool, int, int, bool, int, bool, bool);

}  // namespace lutgemm
