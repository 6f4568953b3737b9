// Streaming-read probe: the HBM read rate this GPU actually reaches with a plain
// coalesced stream, the practical ceiling next to the 8 TB/s peak for judging the
// attention kernel's bandwidth. Work-group g reads the g-th of kProbeBlocks contiguous
// chunks of the buffer, 16-byte nontemporal loads with four in flight per thread, so
// each group streams through consecutive DRAM pages. Every 16-byte word is read once;
// each work-group writes the XOR of the 32-bit words it read, so the loads cannot be
// dropped and the host can check the result bit for bit.
#include <hip/hip_runtime.h>

#include "mlra_internal.h"

namespace mlra {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                    uint32_t* __restrict__ out) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  constexpr int T = kProbeThreads;
  int64_t i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * T < b1; i += 4 * T) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + T);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * T);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * T);
    const u32x4 x = a ^ b ^ c ^ d;
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  for (; i < b1; i += T) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace mlra
