// probe.hip -- a plain streaming-read kernel: the achievable HBM read rate of
// this part, measured with the same kind of loads the GEMV streams its weights
// with (128-bit raw buffer loads, optionally non-temporal). It is the measured
// ceiling the GEMV's bandwidth is compared against, not part of the product.
//
// One workgroup of 16 wave64s per compute unit walks 64 KiB blocks of the
// source, block b + k * grid on its k-th trip, so all workgroups read one
// window of memory together (as the GEMV's input-tile-first layout does). A
// thread keeps four 16-byte loads in flight and folds them into one word; the
// fold is stored only if it equals a value no input makes likely, so the loads
// cannot be removed and the kernel writes (almost) nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "lutgemm.h"

namespace lutgemm {
namespace {

constexpr int kProbeThreads = 1024;
constexpr uint32_t kProbeBlock = kProbeThreads * 4 * 16;   // bytes per workgroup trip
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

__device__ __forceinline__ uint32_t uni_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

template <bool NT>
__global__ void __launch_bounds__(kProbeThreads, 4) stream_read_kernel(const uint8_t* src,
                                                                     uint32_t bytes,
                                                                     uint32_t* sink) {
  // one descriptor over the whole source: reads at or past `bytes` return zero
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(src), (short)0, (int)uni_u32(bytes), 0x00020000);
  const uint32_t nblocks = (bytes + kProbeBlock - 1) / kProbeBlock;
  const uint32_t t16 = (uint32_t)threadIdx.x * 16u;
  uint32_t acc = 0;
  for (uint32_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
    const uint32_t base = uni_u32(b * kProbeBlock);
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, t16 + (uint32_t)u * (kProbeThreads * 16u), base,
                                           NT ? 2 : 0));
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kSinkMagic) sink[blockIdx.x] = acc;
}

std::atomic<int> g_probe_cus[64];

int probe_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int n = (dev >= 0 && dev < 64) ? g_probe_cus[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    if (dev >= 0 && dev < 64) g_probe_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace
}  // namespace lutgemm

extern "C" int lutgemm_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink,
                                   size_t sink_count, int nontemporal, void* stream) {
  using namespace lutgemm;
  if (bytes == 0) return LUTGEMM_OK;
  if (!d_src || !d_sink) return LUTGEMM_ERR_NULL;
  if (bytes > 0xFFFFFFFFull - kProbeBlock) return LUTGEMM_ERR_SHAPE;
  if (((uintptr_t)d_src & 15) || ((uintptr_t)d_sink & 3)) return LUTGEMM_ERR_ALIGN;
  if (nontemporal != 0 && nontemporal != 1) return LUTGEMM_ERR_VALUE;
  if (sink_count == 0) return LUTGEMM_ERR_BUFFER;
  const int cus = probe_cus();
  if (cus <= 0) return LUTGEMM_ERR_HIP;
  const uint32_t nblocks = (uint32_t)((bytes + kProbeBlock - 1) / kProbeBlock);
  const uint32_t grid = nblocks < (uint32_t)cus ? nblocks : (uint32_t)cus;
  if (sink_count < grid) return LUTGEMM_ERR_BUFFER;
  auto fn = nontemporal ? stream_read_kernel<true> : stream_read_kernel<false>;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                     (const uint8_t*)d_src, (uint32_t)bytes, d_sink);
  return hipGetLastError() == hipSuccess ? LUTGEMM_OK : LUTGEMM_ERR_HIP;
}
