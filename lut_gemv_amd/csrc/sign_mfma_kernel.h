// sign_mfma_kernel.h -- y = W_hat x for batches of several rows on the matrix
// cores of gfx950, on the same packed BCQ format as the LUT kernels.
//
// The product the method computes (Elamur card "LUT-GEMM -- paper by Park et
// al. (2022)", sections "Summary" and "Interesting ideas: Lookup tables instead
// of multiplications"): y = sum_i alpha_i * (b_i x) per scale group, b_i in
// {-1,+1}. The LUT kernels get b_i x from tables of signed sums of x, built
// once per 8-input chunk and read once per weight byte and batch row. With
// many batch rows the reads grow with the batch while the weights do not, and
// the vector ALUs and LDS become the bound. Here the same signed sums are a
// dense product instead: for one plane, one 16-row tile and 32 inputs,
// D[row][col] = sum_k b[row][k] x[col][k] is one v_mfma_f32_16x16x32_f16 with
// the signs (+-1.0, exact in fp16) as the A operand and 16 batch rows of x as
// B. The products are exact and the sums fp32, as in the tables; each 128-input
// group's sums are then scaled by the plane's fp16 scale and added into fp32
// accumulators, as the LUT kernels do per group.
//
// Mapping onto CDNA4 (our design):
//  * a workgroup of W wave64s takes a row block of W row tiles (one per wave)
//    over a range of input tiles (512 inputs) for up to 16 * CG batch rows;
//    items (row block, input split, batch group) are walked persistently; a
//    split input dimension is reduced by a fused epilogue like the table
//    kernels', with 128-bit write-through partial stores and loads;
//  * operand layout of the 16x16x32 f16 MFMA: lane l holds row l % 16 of A
//    and column l % 16 of B, each with 8 consecutive k of k-group l / 16; the
//    result D[i][j] is in lane j + 16 * (i / 4), register i % 4. Only the
//    pairing of A's and B's k slots matters, so k-group j of step s = 4u + b
//    of an input tile is chunk 16u + 4j + b: every step's 32 inputs lie in one
//    128-input scale group (u), and lane l needs its row's sign bytes for the
//    four steps of group u, dword (l % 16) % 4 of lane block
//    16 * ((l % 16) / 4) + 4u + l / 16 of the packed format. Each lane loads
//    one whole lane block per plane (a 128-bit load, 1 KiB per wave) and a 4 x 4
//    dword transpose among the four lanes of a row quad (DPP quad
//    permutations) hands every lane its dwords;
//  * a sign byte becomes its 8 fp16 signs by one 128-bit LDS read from a
//    table of the 256 byte values (16 copies, 64 KiB; the copy of lane l is
//    (l % 16) ^ (8 if l >= 32), so 16 consecutive lanes, and lanes l and l + 32,
//    hit different banks); its address is one
//    v_perm_b32 (the sign byte into bits 8-15, the copy into bits 4-7);
//  * x of the current input tile is staged in LDS by the whole workgroup
//    (double-buffered, rows padded to 1040 bytes so that the 16 batch columns
//    of a B read fall in different banks); each wave stages its own row tile's
//    scales (and offsets), so the group scaling reads them with 64-bit LDS
//    broadcasts;
//  * the offset term o * sum(x over the group) takes one more MFMA per step
//    with an all-ones A operand;
//  * one barrier per input tile: the next tile's x is written to the other
//    buffer while this one is read; the sign, scale and x loads of the next
//    tile are in flight during the current tile's MFMAs.
// Scale groups must be multiples of 128 inputs (so a group never starts
// inside a step group); the launcher uses the LUT kernels otherwise.
#pragma once
#include "lutgemv_kernel.h"

namespace lutgemm {

constexpr int kSignCopies = 16;
constexpr int kSignTableBytes = 256 * kSignCopies * 16;   // 64 KiB
constexpr int kXRowBytes = kChunkTile * 16 + 16;           // one batch row of an input tile, padded
constexpr int kStepGroups = 4;                             // 128-input step groups per input tile

template <int CG>
constexpr int kXBufBytes = 16 * CG * kXRowBytes;
// per wave and buffer: the scales of its row tile for the (up to) four scale
// groups an input tile touches, [group][plane][16 rows] fp16, then the offsets
// [group][16 rows] fp16
template <int Q, bool OFF>
constexpr int kSBufBytes = kStepGroups * Q * 32 + (OFF ? kStepGroups * 32 : 0);
// x of a whole item (XI): the 16 batch rows of up to kXITiles input tiles,
// rows padded to kXIRowBytes so that the 16 columns of a B read still fall in
// different banks (row stride = 4 banks mod 64)
constexpr int kXITiles = 5;
constexpr int kXIRowBytes = kXITiles * kChunkTile * 16 + 16;
template <int CG, bool XI>
constexpr int kXRegion = XI ? 16 * CG * kXIRowBytes : 2 * kXBufBytes<CG>;
template <int Q, int CG, bool OFF, int W, bool XI = false>
constexpr int kSignMfmaLds = kSignTableBytes + kXRegion<CG, XI> + 2 * W * kSBufBytes<Q, OFF>;

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Everything one wave needs from memory for one input tile.
template <int Q, int CG, bool OFF, int W, bool XI = false>
struct MfmaTile {
  static constexpr int NXP = XI ? 0 : 16 * CG / W;   // x pieces (16 B) this thread stages per tile
  TilePos pos;
  uint32_t sw[Q][kStepGroups];   // sign bytes of this lane's row: [plane][u], byte b = step 4u + b
  uint4 xv[NXP > 0 ? NXP : 1];   // x pieces for the workgroup's staging (none with XI)
  uint4 sv;                      // this lane's piece of the wave's scale block
  uint4 ov;                      // ... and of its offset block (lanes 0..7)
};

// The scale group of input k (g a multiple of 128).
__device__ __forceinline__ int mfma_group(const Params& p, int k) { return group_of(p, k); }

// Issue the loads of the tile at T.pos. Sign dwords: see the header; x: piece
// j of thread t is batch row (t + j * 64 W) / 64 of the group, chunk t % 64;
// scales: lanes 0 .. 8Q-1 load 16 bytes each of the row tile's block from the
// tile's first group on (the range check zeroes reads past the buffer).
template <int Q, int CG, bool OFF, int W, bool NT, bool XI = false>
__device__ __forceinline__ void mfma_load(const Params& p, int lane, int wave,
                                          MfmaTile<Q, CG, OFF, W, XI>& T) {
  using MT = MfmaTile<Q, CG, OFF, W, XI>;
  const TilePos& t = T.pos;
  const int k0 = t.kt * kChunkTile * 8;
  const bool rows = t.live && t.c.nrt > 0;   // uniform over the wave
  const uint32_t rt = (uint32_t)max(t.c.rt_first, 0);
  {
    // lane i + 16 j (row quad i / 4, a = i % 4) loads lane block 16 (i / 4) + 4a + j
    // of each plane: rows 4 (i / 4) .. + 3 of step group u = a (mfma_transpose
    // then gives each lane its own row of every step group)
    const uint32_t base = ((uint32_t)t.kt * (uint32_t)p.RT + rt) * (uint32_t)Q * 1024u;
    const auto rs = make_rsrc(p.bits, rows ? base + (uint32_t)Q * 1024u : 0u);
    const uint32_t ir = (uint32_t)(lane & 15), jg = (uint32_t)(lane >> 4);
    const uint32_t voff = 256u * (ir >> 2) + 64u * (ir & 3u) + 16u * jg;
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const uint4 v = load16<NT>(rs, voff + (uint32_t)(i * 1024), base);
      T.sw[i][0] = v.x;
      T.sw[i][1] = v.y;
      T.sw[i][2] = v.z;
      T.sw[i][3] = v.w;
    }
  }
  if constexpr (!XI) {
    const uint32_t nx = (uint32_t)p.m * (uint32_t)p.K * 2u;
    const auto rs = make_rsrc(p.x, t.live ? nx : 0u);
#pragma unroll
    for (int j = 0; j < MT::NXP; ++j) {
      const int piece = wave * 64 + lane + j * W * 64;
      const int col = piece >> 6, chunk = piece & 63;
      const int kk = k0 + 8 * chunk;
      const bool ok = col < t.c.rows_here && kk < p.K;
      const uint32_t off = ((uint32_t)(t.c.r0 + col) * (uint32_t)p.K + (uint32_t)kk) * 2u;
      T.xv[j] = load16(rs, ok ? off : 0xFFFFFFF0u);
    }
  }
  {
    const int grp0 = mfma_group(p, k0);
    const uint32_t sbase = ((uint32_t)rt * (uint32_t)p.G + (uint32_t)grp0) * (uint32_t)Q * 32u;
    const uint32_t nbytes = (uint32_t)Q * (uint32_t)p.Npad * (uint32_t)p.G * 2u;
    const auto rs = make_rsrc(p.alpha, rows ? nbytes : 0u);
    T.sv = load16(rs, lane < 8 * Q ? sbase + 16u * (uint32_t)lane : 0xFFFFFFF0u);
    if constexpr (OFF) {
      const uint32_t obase = ((uint32_t)rt * (uint32_t)p.G + (uint32_t)grp0) * 32u;
      const uint32_t onbytes = (uint32_t)p.Npad * (uint32_t)p.G * 2u;
      const auto ro = make_rsrc(p.offset, rows ? onbytes : 0u);
      T.ov = load16(ro, lane < 8 ? obase + 16u * (uint32_t)lane : 0xFFFFFFF0u);
    }
  }
}

// The four lanes 4r .. 4r + 3 (same j) of a row quad hold, as loaded, the
// 4 x 4 dword matrix M[a][a'] = dword a' (row 4r + a') of step group a; lane a
// needs M[u][a] for u = 0..3. Two exchange rounds in the quad (lane bit 0 with
// dword bit 0, then bit 1 with bit 1), each a DPP quad permutation and selects.
__device__ __forceinline__ void mfma_transpose(uint32_t (&v)[4], bool a0, bool a1) {
#pragma unroll
  for (int p = 0; p < 4; p += 2) {
    const uint32_t send = a0 ? v[p] : v[p + 1];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    v[p] = a0 ? recv : v[p];
    v[p + 1] = a0 ? v[p + 1] : recv;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t send = a1 ? v[p] : v[p + 2];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);
    v[p] = a1 ? recv : v[p];
    v[p + 2] = a1 ? v[p + 2] : recv;
  }
}

// Write a loaded tile's x pieces and this wave's scales (offsets) into LDS buffer `buf`.
template <int Q, int CG, bool OFF, int W, bool XI = false>
__device__ __forceinline__ void mfma_stage(uint8_t* smem, int buf, int lane, int wave,
                                           const MfmaTile<Q, CG, OFF, W, XI>& T) {
  using MT = MfmaTile<Q, CG, OFF, W, XI>;
  if constexpr (!XI) {
    uint8_t* xb = smem + kSignTableBytes + buf * kXBufBytes<CG>;
#pragma unroll
    for (int j = 0; j < MT::NXP; ++j) {
      const int piece = wave * 64 + lane + j * W * 64;
      *reinterpret_cast<uint4*>(xb + (piece >> 6) * kXRowBytes + (piece & 63) * 16) = T.xv[j];
    }
  }
  uint8_t* sb = smem + kSignTableBytes + kXRegion<CG, XI> + (wave * 2 + buf) * kSBufBytes<Q, OFF>;
  if (lane < 8 * Q) *reinterpret_cast<uint4*>(sb + 16 * lane) = T.sv;
  if constexpr (OFF) {
    if (lane < 8) *reinterpret_cast<uint4*>(sb + kStepGroups * Q * 32 + 16 * lane) = T.ov;
  }
}

// The MFMAs and group scaling of one input tile for this wave's row tile.
// acc[cg][r]: row 4 * (lane / 16) + r of the row tile, batch row lane % 16 + 16 cg.
// XI: x of the whole item is staged, the tile at input tile xt of it.
template <int Q, int CG, bool OFF, int W, bool XI = false>
__device__ __forceinline__ void mfma_tile(const Params& p, const uint8_t* smem, int buf,
                                          int lane, int wave, const MfmaTile<Q, CG, OFF, W, XI>& T,
                                          float (&acc)[CG][4], int xt = 0) {
  const int k0 = T.pos.kt * kChunkTile * 8;
  const int nu = min(kStepGroups, (p.K - k0) >> 7);   // step groups inside K (K % 128 == 0)
  const int jg = lane >> 4;
  // table copy of this lane: all 16 differ within any 16 consecutive lanes and
  // within lanes l, l + 32 (however the LDS groups the lanes of a 128-bit read)
  const uint32_t cb = (uint32_t)((lane & 15) ^ ((lane >> 2) & 8)) << 4;
  constexpr int kRow = XI ? kXIRowBytes : kXRowBytes;   // bytes per batch row of staged x
  const uint8_t* xb = XI ? smem + kSignTableBytes + (lane & 15) * kXIRowBytes + xt * (kChunkTile * 16) + 64 * jg
                         : smem + kSignTableBytes + buf * kXBufBytes<CG> + (lane & 15) * kXRowBytes + 64 * jg;
  const uint8_t* sb = smem + kSignTableBytes + kXRegion<CG, XI> +
                      (wave * 2 + buf) * kSBufBytes<Q, OFF> + 8 * jg;
  const int grp0 = mfma_group(p, k0);
  const half8v ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
  for (int u = 0; u < kStepGroups; ++u) {
    if (u < nu) {
      const int gu = mfma_group(p, k0 + 128 * u) - grp0;
      const float4v zero = {0.f, 0.f, 0.f, 0.f};
      float4v D[Q][CG];
      float4v D1[CG];
      uint2 a2[Q], o2;   // the group's scales (and offsets)
      auto read_scales = [&]() {
#pragma unroll
        for (int i = 0; i < Q; ++i) a2[i] = *reinterpret_cast<const uint2*>(sb + (gu * Q + i) * 32);
        if constexpr (OFF) o2 = *reinterpret_cast<const uint2*>(sb + kStepGroups * Q * 32 + gu * 32);
      };
      // Where the registers allow a second operand set (at most 3 planes per
      // group of 16 batch rows at 16 waves, 6 at 8 waves, the offset counted
      // as a plane), the four steps are software-pipelined: the operand reads
      // of step b + 1 (its B pieces of x, its A sign vectors; the scales in
      // the last step's place) are issued before the MFMAs of step b, and
      // scheduling barriers keep that order, so an MFMA waits only for reads
      // issued a step earlier. Left to itself the compiler issues each read
      // just before the MFMA that takes it, and every MFMA waits for a full
      // LDS round trip; that is still the order where the set does not fit.
      constexpr bool kPipe = (Q + (OFF ? 1 : 0)) * CG <= (W == 16 ? 3 : 6);
      if constexpr (kPipe) {
        half8v A[2][Q], B[2][CG];
        auto read_step = [&](int b, int slot) {
#pragma unroll
          for (int c = 0; c < CG; ++c)
            B[slot][c] = *reinterpret_cast<const half8v*>(xb + c * 16 * kRow + 256 * u + 16 * b);
          const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)b) << 8);
#pragma unroll
          for (int i = 0; i < Q; ++i)
            A[slot][i] = *reinterpret_cast<const half8v*>(smem + __builtin_amdgcn_perm(T.sw[i][u], cb, sel));
        };
        read_step(0, 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < 3) {
            read_step(b + 1, (b + 1) & 1);
          } else {
            read_scales();
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < Q; ++i)
#pragma unroll
            for (int c = 0; c < CG; ++c)
              D[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[b & 1][i], B[b & 1][c], b ? D[i][c] : zero, 0, 0, 0);
          if constexpr (OFF) {
#pragma unroll
            for (int c = 0; c < CG; ++c)
              D1[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, B[b & 1][c], b ? D1[c] : zero, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          half8v B[CG];
#pragma unroll
          for (int c = 0; c < CG; ++c)
            B[c] = *reinterpret_cast<const half8v*>(xb + c * 16 * kRow + 256 * u + 16 * b);
          const uint32_t sel = 0x0C0C0000u | ((4u + (uint32_t)b) << 8);
#pragma unroll
          for (int i = 0; i < Q; ++i) {
            const uint32_t addr = __builtin_amdgcn_perm(T.sw[i][u], cb, sel);
            const half8v A = *reinterpret_cast<const half8v*>(smem + addr);
#pragma unroll
            for (int c = 0; c < CG; ++c)
              D[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B[c], b ? D[i][c] : zero, 0, 0, 0);
          }
          if constexpr (OFF) {
#pragma unroll
            for (int c = 0; c < CG; ++c)
              D1[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, B[c], b ? D1[c] : zero, 0, 0, 0);
          }
        }
        read_scales();
      }
#pragma unroll
      for (int i = 0; i < Q; ++i) {
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[c][r] = fmaf(h2f(r < 2 ? a2[i].x : a2[i].y, r & 1), D[i][c][r], acc[c][r]);
      }
      if constexpr (OFF) {
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[c][r] = fmaf(h2f(r < 2 ? o2.x : o2.y, r & 1), D1[c][r], acc[c][r]);
      }
    }
  }
}

// Cache policy of the split partials' loads and stores: sc1, device scope (a
// store is written through to the coherence point every XCD reads, a load
// reads there rather than a possibly stale L2 line).
constexpr int kDeviceScope = 16;

// Store a finished item's accumulators (fp16 y, or this split's fp32
// partials, four rows of one batch row in one 128-bit write-through store)
// and clear them. The partials [S][m][Npad] are under 4 GiB (the launcher
// checks), so one descriptor covers them.
template <int CG>
__device__ __forceinline__ void mfma_finish(const Params& p, int lane, const ItemCtx& c,
                                            float (&acc)[CG][4]) {
  const int jg = lane >> 4;
  const int row0 = c.rt_first * kRowTile + 4 * jg;
  const auto pr = make_rsrc(p.partial, p.S > 1 ? (uint32_t)p.S * (uint32_t)p.m * (uint32_t)p.Npad * 4u : 0u);
#pragma unroll
  for (int cg = 0; cg < CG; ++cg) {
    const int col = (lane & 15) + 16 * cg;
    if (c.nrt > 0 && col < c.rows_here) {
      if (p.S > 1) {
        const uint32_t off =
            (((uint32_t)c.split * (uint32_t)p.m + (uint32_t)(c.r0 + col)) * (uint32_t)p.Npad + (uint32_t)row0) * 4u;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4v, float4v{acc[cg][0], acc[cg][1], acc[cg][2], acc[cg][3]}), pr, off, 0,
            kDeviceScope);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (row0 + r < p.N)
            p.y[(size_t)(c.r0 + col) * p.N + row0 + r] = __builtin_bit_cast(uint16_t, (_Float16)acc[cg][r]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[cg][r] = 0.f;
  }
}

// The split reduction of this kernel, run once after a workgroup's last item:
// the arrival counting of split_epilogue (the same order argument: the
// partial stores above are write-through, every wave waits for them before
// the barrier and the counting), then the last arrival of an item's row block
// adds its S partials in split order, four rows of one batch row per thread
// with 128-bit loads (eight splits in flight), rounds to fp16 and stores y.
template <int MC, int W>
__device__ __forceinline__ void mfma_split_epilogue(const Params& p, int* s_last) {
  constexpr int kThreads = W * 64;
  const int kRows = p.ri * kRowTile;
  const int kQuads = kRows / 4;
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt = expcnt = lgkmcnt = 0: own stores complete
  __syncthreads();
  const auto pr = make_rsrc(p.partial, (uint32_t)p.S * (uint32_t)p.m * (uint32_t)p.Npad * 4u);
  const uint32_t sstride = (uint32_t)p.m * (uint32_t)p.Npad * 4u;
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
    const int per_item = MC * kQuads;
    for (int idx = threadIdx.x; idx < nj * per_item; idx += kThreads) {
      const int j = idx / per_item;
      const int item = s_last[j];
      if (item < 0) continue;
      const int rem = idx - j * per_item;
      const int col = rem / kQuads;
      int bg, split, rb;
      decode_item(p, item, bg, split, rb);
      const int row = rb * kRows + 4 * (rem - col * kQuads);
      const int rr = bg * MC + col;
      if (row >= p.N || rr >= p.m) continue;
      const uint32_t off = ((uint32_t)rr * (uint32_t)p.Npad + (uint32_t)row) * 4u;
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < p.S; s0 += 8) {
        float4v v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sp = min(s0 + u, p.S - 1);   // past the last split: a valid slot, unused
          v[u] = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                 pr, off + (uint32_t)sp * sstride, 0, kDeviceScope));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < p.S)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[e] += v[u][e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (row + e < p.N) p.y[(size_t)rr * p.N + row + e] = __builtin_bit_cast(uint16_t, (_Float16)sum[e]);
    }
    __syncthreads();
  }
}

// XI: 16-byte pieces of an item's x per thread
template <int W>
constexpr int kXIPieces = 16 * kXITiles * 64 / (W * 64);

// XI: the tile after t within the workgroup's one item, dead past its end.
// Every register set then holds the same item state (the same values, kept
// once), instead of what a move to another item would need.
__device__ __forceinline__ TilePos xi_next_tile(const TilePos& t) {
  TilePos n = t;
  n.kt = t.kt + 1;
  n.live = t.live && n.kt < t.c.kt1;
  return n;
}

// XI: x of a workgroup's item, batch rows r0 .. r0 + 15 over its input tiles
// kt .. kt1 - 1 (at most kXITiles), loaded by every thread (piece j of thread
// t: index t + 64 W j = (row, tile, chunk) in that order; zero past the batch,
// the item's tiles and K) and written once into the x region.
template <int W>
__device__ __forceinline__ void mfma_item_x_load(const Params& p, const TilePos& t, uint4 (&xr)[kXIPieces<W>]) {
  const uint32_t nx = (uint32_t)p.m * (uint32_t)p.K * 2u;
  const auto rs = make_rsrc(p.x, t.live ? nx : 0u);
  const int nt = t.c.kt1 - t.kt;
#pragma unroll
  for (int j = 0; j < kXIPieces<W>; ++j) {
    const int idx = (int)threadIdx.x + j * W * 64;
    const int row = idx / (kXITiles * 64);
    const int rem = idx - row * (kXITiles * 64);
    const int tt = rem >> 6, chunk = rem & 63;
    const int k = (t.kt + tt) * kChunkTile * 8 + 8 * chunk;
    const bool ok = row < t.c.rows_here && tt < nt && k < p.K;
    const uint32_t off = ((uint32_t)(t.c.r0 + row) * (uint32_t)p.K + (uint32_t)k) * 2u;
    xr[j] = load16(rs, ok ? off : 0xFFFFFFF0u);
  }
}

template <int W>
__device__ __forceinline__ void mfma_item_x_store(uint8_t* smem, const uint4 (&xr)[kXIPieces<W>]) {
#pragma unroll
  for (int j = 0; j < kXIPieces<W>; ++j) {
    const int idx = (int)threadIdx.x + j * W * 64;
    const int row = idx / (kXITiles * 64);
    const int rem = idx - row * (kXITiles * 64);
    *reinterpret_cast<uint4*>(smem + kSignTableBytes + row * kXIRowBytes + (rem >> 6) * (kChunkTile * 16) +
                              (rem & 63) * 16) = xr[j];
  }
}

// Persistent kernel: workgroup b processes items b, b + gridDim.x, ...; an
// item is (row block of W row tiles, split of the input tiles, group of 16 CG
// batch rows). While one tile's MFMAs run, the next two tiles' loads are in
// flight. NT: every sign byte is read once per product (one batch group), and
// those loads are non-temporal. XI (one group of 16 batch rows, one item per
// workgroup, at most kXITiles input tiles per item): x of the whole item is
// staged in LDS once, at the start, and the tile loop has no barrier (no LDS
// written by one wave is read by another after the start).
template <int Q, int CG, bool OFF, int W, bool NT, bool XI = false>
__global__ void __launch_bounds__(W * 64, W / 4)
    __attribute__((amdgpu_waves_per_eu(W / 4, W / 4))) sign_mfma_kernel(Params p) {
  static_assert(16 * CG % W == 0, "x pieces per thread");
  static_assert(!XI || CG == 1, "x per item: one group of 16 batch rows");
  constexpr int MC = 16 * CG;
  using MT = MfmaTile<Q, CG, OFF, W, XI>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSignMfmaLds<Q, CG, OFF, W, XI>];
  LUTGEMM_PHASE(0);
  LUTGEMM_PHASE_FLAG(traced_staged);
  LUTGEMM_PHASE_FLAG(traced_step);
  const int lane = (int)(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  // Three register sets: while one tile's MFMAs run, the loads of the next
  // two tiles are in flight (a tile's loads have two tiles' MFMAs to arrive).
  MT S[3];
  S[0].pos = first_tile<1, MC, W>(p, wave, blockIdx.x);
  // XI: the item's x first, so that staging it waits for nothing else
  uint4 xr[XI ? kXIPieces<W> : 1];
  if constexpr (XI) mfma_item_x_load<W>(p, S[0].pos, xr);
  mfma_load<Q, CG, OFF, W, NT, XI>(p, lane, wave, S[0]);
  asm volatile("" ::: "memory");
  if (!S[0].pos.live) return;
  const int kt0 = S[0].pos.kt;   // XI: the staged item's first input tile
  S[1].pos = XI ? xi_next_tile(S[0].pos) : next_tile<1, MC, W>(p, wave, S[0].pos);
  mfma_load<Q, CG, OFF, W, NT, XI>(p, lane, wave, S[1]);

  // The sign table: entry v (a sign byte) copy c at byte 256 v + 16 c, its 8
  // fp16 values +1.0 where bit e of v is set and -1.0 elsewhere (bit e is
  // input 8 * chunk + e).
  for (int e = (int)threadIdx.x; e < 256 * kSignCopies; e += W * 64) {
    const uint32_t v = (uint32_t)e >> 4;
    uint32_t w4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t lo = ((v >> (2 * t)) & 1u) ? 0x3C00u : 0xBC00u;
      const uint32_t hi = ((v >> (2 * t + 1)) & 1u) ? 0x3C00u : 0xBC00u;
      w4[t] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(smem + 16 * e) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  LUTGEMM_PHASE(2);
  if constexpr (XI) {
    mfma_item_x_store<W>(smem, xr);
    __syncthreads();   // the table and the item's x, for every wave
  }

  float acc[CG][4];
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] = 0.f;

  // One input tile per trip: stage the oldest loaded tile into buffer `buf`
  // (once it is staged its loads are complete: x and the scales are its last
  // loads), issue the loads of the tile two ahead into the set just staged,
  // wait at the barrier (none with XI: only the wave's own scales are staged),
  // then the staged tile's MFMAs and, at its item's end, the store. The buffer written here was last read two trips ago, before
  // the previous barrier. Tiles past the workgroup's last are dead: their
  // loads touch no memory, zeros are staged and nothing is computed, so the
  // loop runs whole rounds of three trips and its one exit is at its head;
  // with the staged tile's sign words passing through an empty asm, no path
  // into the MFMAs has their loads in flight, and the compiler's wait counts
  // keep the newer tiles' loads outstanding there.
  MT cur;
  int buf = 0;
  int ntrip = 0;
  auto trip = [&](MT& st, MT& ld, const TilePos& after) {
    // XI: with no barrier the four waves of a SIMD drift apart (its issue
    // favours the oldest), and the last tiles then run with fewer waves to
    // hide latency; the waves' priorities rotate from tile to tile instead
    // (12288 x 12288, m = 4 / 8 / 16: 2% faster)
    if constexpr (XI) {
      switch (((wave >> 2) + ntrip) & 3) {
        case 0: __builtin_amdgcn_s_setprio(0); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        default: __builtin_amdgcn_s_setprio(3); break;
      }
      ++ntrip;
    }
    mfma_stage<Q, CG, OFF, W, XI>(smem, buf, lane, wave, st);
#pragma unroll
    for (int i = 0; i < Q; ++i) {
#pragma unroll
      for (int u = 0; u < kStepGroups; ++u) {
        asm volatile("" : "+v"(st.sw[i][u]));
        cur.sw[i][u] = st.sw[i][u];
      }
      mfma_transpose(cur.sw[i], lane & 1, lane & 2);
    }
    cur.pos = st.pos;
    // XI: a workgroup's one item (the launch has no more items than workgroups)
    ld.pos = XI ? xi_next_tile(after) : next_tile<1, MC, W>(p, wave, after);
    mfma_load<Q, CG, OFF, W, NT, XI>(p, lane, wave, ld);
    if constexpr (!XI) __syncthreads();
    LUTGEMM_PHASE_ONCE(1, traced_staged);
    if (cur.pos.live) {
      if (cur.pos.c.nrt > 0)
        mfma_tile<Q, CG, OFF, W, XI>(p, smem, buf, lane, wave, cur, acc, cur.pos.kt - kt0);
      if (cur.pos.kt + 1 == cur.pos.c.kt1) mfma_finish<CG>(p, lane, cur.pos.c, acc);
    }
    LUTGEMM_PHASE_ONCE(3, traced_step);
    buf ^= 1;
  };
  while (S[0].pos.live) {
    trip(S[0], S[2], S[1].pos);
    trip(S[1], S[0], S[2].pos);
    trip(S[2], S[1], S[0].pos);
  }
  LUTGEMM_PHASE(4);
  if (p.S > 1) mfma_split_epilogue<MC, W>(p, reinterpret_cast<int*>(smem));
  LUTGEMM_PHASE(5);
}

// Instances are built where the compiler keeps everything in registers
// (128 per lane at 16 waves, 256 at 8): the three register sets of loads in
// flight and the accumulators grow with the planes (and the offset) times the
// groups of 16 batch rows.
template <int Q, int CG, bool OFF, int W>
constexpr bool kMfmaFits =
    W == 16 ? (CG == 1 ? Q + OFF <= 4 : Q + OFF <= 2) : (CG == 1 || Q + OFF <= 7);

// The instance for q planes, cg groups of 16 batch rows, an offset term, w
// waves, non-temporal sign loads (nt) and x staged once per item (xi), or
// nullptr where none is built (see kMfmaFits; xi needs cg = 1 and the LDS for
// kXITiles input tiles of x).
template <int Q>
KernelFn sign_mfma_kernel_of_q(int cg, bool off, int w, bool nt, bool xi) {
#define LUTGEMM_SM(CG, OFF, W)                                                           \
  if constexpr (kSignMfmaLds<Q, CG, OFF, W> <= 160 * 1024 &&                               \
                kMfmaFits<Q, CG, OFF, W>) {                                                \
    if (xi) {                                                                             \
      if constexpr (CG == 1 && kSignMfmaLds<Q, CG, OFF, W, true> <= 160 * 1024) {          \
        return nt ? sign_mfma_kernel<Q, CG, OFF, W, true, true>                           \
                  : sign_mfma_kernel<Q, CG, OFF, W, false, true>;                         \
      } else {                                                                            \
        return nullptr;                                                                   \
      }                                                                                   \
    }                                                                                     \
    return nt ? sign_mfma_kernel<Q, CG, OFF, W, true> : sign_mfma_kernel<Q, CG, OFF, W, false>; \
  } else {                                                                                \
    return nullptr;                                                                       \
  }
  if (w == 16) {
    if (cg == 1) {
      if (off) { LUTGEMM_SM(1, true, 16); } else { LUTGEMM_SM(1, false, 16); }
    } else if (cg == 2) {
      if (off) { LUTGEMM_SM(2, true, 16); } else { LUTGEMM_SM(2, false, 16); }
    }
  } else if (w == 8) {
    if (cg == 1) {
      if (off) { LUTGEMM_SM(1, true, 8); } else { LUTGEMM_SM(1, false, 8); }
    } else if (cg == 2) {
      if (off) { LUTGEMM_SM(2, true, 8); } else { LUTGEMM_SM(2, false, 8); }
    }
  }
#undef LUTGEMM_SM
  return nullptr;
}

extern template KernelFn sign_mfma_kernel_of_q<1>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<2>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<3>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<4>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<5>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<6>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<7>(int, bool, int, bool, bool);
extern template KernelFn sign_mfma_kernel_of_q<8>(int, bool, int, bool, bool);

}  // namespace lutgemm
