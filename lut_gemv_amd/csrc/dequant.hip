// dequant.hip -- the comparison point for the LUT-GEMV: y = W_hat x computed by
// expanding every weight to fp16 and taking dot products, the way dequantizing
// weight-only kernels work (the approach LUT-GEMM is measured against: Elamur
// card "LUT-GEMM -- paper by Park et al. (2022)", section "Summary"; pith.science
// page of the same title, original abstract). It reads the same packed format
// as lutgemm_run and computes the same product, so the two can be timed on the
// same data.
//
// Mapping onto CDNA4:
//  * a workgroup of four waves; each wave owns one row tile (16 rows) over the
//    whole input dimension, lane l holding lane block l of every 1 KiB plane
//    block (rows 4*(l/16) + a, chunks 4*(l%16) + b);
//  * for each of its rows and chunks a lane rebuilds the 8 weights as four fp16
//    pairs: per plane, the complemented sign byte is spread to the two fp16
//    sign bits of each pair and XORed into the (alpha, alpha) pair (one shift
//    and one three-input bit operation per pair), and the planes are summed with
//    packed fp16 adds;
//  * v_dot2_f32_f16 multiplies a weight pair by an activation pair and adds into
//    an fp32 accumulator; the expanded weights are reused for every batch row of
//    the launch (up to 8; more rows run as further batch groups);
//  * latency is hidden by occupancy (small register footprint, many waves per
//    SIMD) rather than by an explicit prefetch ring.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "layout.h"
#include "lutgemm.h"

namespace lutgemm {
namespace {

constexpr int kDqWaves = 4;      // waves (row tiles) per workgroup
constexpr int kDqMaxBatch = 8;   // batch rows per launch of a group

struct DqParams {
  const uint8_t* bits;
  const uint32_t* alpha;     // fp16 pairs
  const uint32_t* offset;    // fp16 pairs, or null
  const uint16_t* x;
  uint16_t* y;
  int N, K, g, m, RT, KT, G, g_shift;
};

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

std::atomic<int> g_dq_arch[64];   // 0 unknown, 1 gfx950, 2 other

// The current device must be gfx950 (LUTGEMM_FAKE_ARCH, a debugging aid,
// replaces the reported name and bypasses the per-device cache).
int dq_check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LUTGEMM_ERR_HIP;
  const char* fake = getenv("LUTGEMM_FAKE_ARCH");
  const bool use_cache = dev >= 0 && dev < 64 && !(fake && *fake);
  int known = use_cache ? g_dq_arch[dev].load(std::memory_order_relaxed) : 0;
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LUTGEMM_ERR_HIP;
    known = strncmp((fake && *fake) ? fake : prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (use_cache) g_dq_arch[dev].store(known, std::memory_order_relaxed);
  }
  return known == 1 ? LUTGEMM_OK : LUTGEMM_ERR_UNSUPPORTED;
}

__device__ __forceinline__ uint32_t bcast_half(uint32_t word, int hi) {
  // (h, h) from half `hi` of word
  return __builtin_amdgcn_perm(word, word, hi ? 0x07060706u : 0x05040504u);
}

__device__ __forceinline__ int dq_group(const DqParams& p, int k) {
  return p.g_shift >= 0 ? (k >> p.g_shift) : (k / p.g);
}

// Q planes; OFF: offset term; MB: batch rows per launch (1 or 8); GQ: the 32
// inputs of a lane's block share one scale group (g % 32 == 0), so the lane's
// scales are loaded and broadcast once per input tile; otherwise each chunk
// finds its own group, so any group size works.
template <int Q, bool OFF, int MB, bool GQ>
__global__ void __launch_bounds__(kDqWaves * 64) dequant_gemv_kernel(DqParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = blockIdx.x * kDqWaves + wave;
  if (rt >= p.RT) return;                       // uniform over the wave
  const int r0 = blockIdx.y * MB;
  const int rows = min(MB, p.m - r0);
  const int r4 = lane >> 4, c4 = lane & 15;
  const uint32_t tile_bytes = Q * 1024u;

  float acc[MB][4];
#pragma unroll
  for (int r = 0; r < MB; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[r][a] = 0.f;

  for (int kt = 0; kt < p.KT; ++kt) {
    const int k0 = kt * 512 + 32 * c4;          // first input of this lane's block
    // sign bytes: plane i, byte 4a + b = row 4*r4 + a, chunk 4*c4 + b
    uint4 bw[Q];
    const uint8_t* blk = p.bits + ((size_t)kt * p.RT + rt) * tile_bytes + (size_t)lane * 16;
#pragma unroll
    for (int i = 0; i < Q; ++i) bw[i] = *reinterpret_cast<const uint4*>(blk + i * 1024);
    // activations of the lane's 32 inputs, per batch row (zero past K)
    uint4 xv[MB][4];
#pragma unroll
    for (int r = 0; r < MB; ++r)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool in = r < rows && k0 + 8 * b < p.K;
        xv[r][b] = in ? *reinterpret_cast<const uint4*>(p.x + (size_t)(r0 + r) * p.K + k0 + 8 * b)
                      : uint4{0u, 0u, 0u, 0u};
      }
    // GQ: the (alpha, alpha) pairs of the lane's four rows, per plane, for the
    // group of its 32 inputs (and the offsets), loaded once per input tile
    uint32_t alq[GQ ? Q : 1][4], ofq[4];
    if constexpr (GQ) {
      const int grp = k0 < p.K ? dq_group(p, k0) : 0;
      const uint32_t* ab = p.alpha + ((size_t)rt * p.G + grp) * (8 * Q) + 2 * r4;
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const uint2 v = *reinterpret_cast<const uint2*>(ab + i * 8);
#pragma unroll
        for (int a = 0; a < 4; ++a) alq[i][a] = bcast_half(a < 2 ? v.x : v.y, a & 1);
      }
      if constexpr (OFF) {
        const uint2 v = *reinterpret_cast<const uint2*>(p.offset + ((size_t)rt * p.G + grp) * 8 + 2 * r4);
#pragma unroll
        for (int a = 0; a < 4; ++a) ofq[a] = bcast_half(a < 2 ? v.x : v.y, a & 1);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int kc = k0 + 8 * b;
      if (kc >= p.K) continue;                  // padded chunk: nothing to add
      const int grp = GQ ? 0 : dq_group(p, kc);
      const uint32_t* ab = p.alpha + ((size_t)rt * p.G + grp) * (8 * Q);   // [plane][16 rows]
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int row = 4 * r4 + a;
        h2 w[4];
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          const uint32_t words[4] = {bw[i].x, bw[i].y, bw[i].z, bw[i].w};
          // complemented sign byte of (row a, chunk b), spread so that bit 2u
          // lands on bit 15 and bit 2u+1 on bit 31 after a left shift by 15-2u
          const uint32_t nb = __builtin_amdgcn_ubfe(~words[a], 8 * b, 8);
          const uint32_t xs = nb | (nb << 15);
          const uint32_t al = GQ ? alq[i][a] : bcast_half(ab[i * 8 + (row >> 1)], row & 1);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            // (alpha, alpha) with each half negated where its sign bit is 0
            const uint32_t sw = __builtin_amdgcn_bitop3_b32(xs << (15 - 2 * u), 0x80008000u, al, 0x6A);
            const h2 v = __builtin_bit_cast(h2, sw);
            w[u] = i == 0 ? v : w[u] + v;
          }
        }
        if constexpr (OFF) {
          const uint32_t* ob = p.offset + ((size_t)rt * p.G + grp) * 8;
          const h2 o = __builtin_bit_cast(h2, GQ ? ofq[a] : bcast_half(ob[row >> 1], row & 1));
#pragma unroll
          for (int u = 0; u < 4; ++u) w[u] = w[u] + o;
        }
#pragma unroll
        for (int r = 0; r < MB; ++r) {
          const uint32_t xw[4] = {xv[r][b].x, xv[r][b].y, xv[r][b].z, xv[r][b].w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc[r][a] = __builtin_amdgcn_fdot2(w[u], __builtin_bit_cast(h2, xw[u]), acc[r][a], false);
        }
      }
    }
  }
  // sum the 16 lanes of a row quad (lanes differing in bits 0-3) and store
#pragma unroll
  for (int r = 0; r < MB; ++r) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float v = acc[r][a];
      v += __shfl_xor(v, 8, 64);
      v += __shfl_xor(v, 4, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 1, 64);
      const int row = rt * 16 + 4 * r4 + a;
      if (c4 == 0 && r < rows && row < p.N)
        p.y[(size_t)(r0 + r) * p.N + row] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
  }
}

using DqFn = void (*)(DqParams);

template <int Q, bool GQ>
DqFn dq_pick(bool off, int mb) {
  if (mb == 1)
    return off ? dequant_gemv_kernel<Q, true, 1, GQ> : dequant_gemv_kernel<Q, false, 1, GQ>;
  return off ? dequant_gemv_kernel<Q, true, kDqMaxBatch, GQ>
             : dequant_gemv_kernel<Q, false, kDqMaxBatch, GQ>;
}

template <int Q>
DqFn dq_pick(bool off, int mb, bool gq) {
  return gq ? dq_pick<Q, true>(off, mb) : dq_pick<Q, false>(off, mb);
}

DqFn dq_kernel(int q, bool off, int mb, bool gq) {
  switch (q) {
    case 1: return dq_pick<1>(off, mb, gq);
    case 2: return dq_pick<2>(off, mb, gq);
    case 3: return dq_pick<3>(off, mb, gq);
    case 4: return dq_pick<4>(off, mb, gq);
    case 5: return dq_pick<5>(off, mb, gq);
    case 6: return dq_pick<6>(off, mb, gq);
    case 7: return dq_pick<7>(off, mb, gq);
    case 8: return dq_pick<8>(off, mb, gq);
    default: return nullptr;
  }
}

__global__ void dq_zero_kernel(uint16_t* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

inline bool dq_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace
}  // namespace lutgemm

using namespace lutgemm;

extern "C" int bcq_dequant_gemv(const lutgemm_shape* s, int32_t m, const void* d_bits,
                                const void* d_alpha, const void* d_offset, const void* d_x,
                                void* d_y, void* stream) {
  int st = check_shape(s);
  if (st) return st;
  if (m < 0 || m > kMaxBatch) return LUTGEMM_ERR_SHAPE;
  const Geometry G = geometry(s);
  if (m == 0 || G.N == 0) return LUTGEMM_OK;
  if (!d_y) return LUTGEMM_ERR_NULL;
  if (!dq_aligned(d_y, 2)) return LUTGEMM_ERR_ALIGN;
  hipStream_t strm = (hipStream_t)stream;
  if (G.K > 0) {
    if (!d_bits || !d_alpha || !d_x || (G.has_offset && !d_offset)) return LUTGEMM_ERR_NULL;
    if (!dq_aligned(d_bits, 16) || !dq_aligned(d_x, 16) || !dq_aligned(d_alpha, 4) ||
        (G.has_offset && !dq_aligned(d_offset, 4)))
      return LUTGEMM_ERR_ALIGN;
  }
  st = dq_check_device();
  if (st) return st;
  if (G.K == 0) {
    const size_t n = (size_t)m * G.N;
    const size_t want = (n + 255) / 256;
    hipLaunchKernelGGL(dq_zero_kernel, dim3((unsigned)(want < 4096 ? want : 4096)), dim3(256), 0,
                       strm, (uint16_t*)d_y, n);
    return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
  }
  const int mb = m == 1 ? 1 : kDqMaxBatch;
  DqFn fn = dq_kernel((int)G.q, G.has_offset, mb, G.g % 32 == 0);
  if (!fn) return LUTGEMM_ERR_INTERNAL;
  DqParams p{};
  p.bits = (const uint8_t*)d_bits;
  p.alpha = (const uint32_t*)d_alpha;
  p.offset = G.has_offset ? (const uint32_t*)d_offset : nullptr;
  p.x = (const uint16_t*)d_x;
  p.y = (uint16_t*)d_y;
  p.N = (int)G.N;
  p.K = (int)G.K;
  p.g = (int)G.g;
  p.m = m;
  p.RT = (int)G.RT;
  p.KT = (int)G.KT;
  p.G = (int)G.G;
  p.g_shift = -1;
  for (int b = 3; b < 31; ++b)
    if (((int64_t)1 << b) == G.g) p.g_shift = b;
  const int64_t groups = (m + mb - 1) / mb;
  if (groups > 65535) return LUTGEMM_ERR_SHAPE;
  dim3 grid((unsigned)((G.RT + kDqWaves - 1) / kDqWaves), (unsigned)groups);
  void* args[] = {&p};
  if (hipLaunchKernel((const void*)fn, grid, dim3(kDqWaves * 64), args, 0, strm) != hipSuccess)
    return LUTGEMM_ERR_HIP;
  return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
}
