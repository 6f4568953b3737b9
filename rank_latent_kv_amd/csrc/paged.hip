// Paged cache maintenance: append one row per sequence, and gather a
// sequence's logical rows out of the pool. Both are bit-exact byte copies.
// Logical token s of sequence beta lives in physical row
//   page_table[beta][s / page_size] * page_size + s % page_size.
#include <hip/hip_runtime.h>

#include "mlra_internal.h"

namespace mlra {
namespace {

__device__ __forceinline__ void copy_bytes(char* dst, const char* src, int64_t n, int lane, int lanes) {
  const bool a16 = (((uintptr_t)dst | (uintptr_t)src | (uintptr_t)n) & 15) == 0;
  const bool a4 = (((uintptr_t)dst | (uintptr_t)src | (uintptr_t)n) & 3) == 0;
  if (a16) {
    for (int64_t i = lane; i < n / 16; i += lanes)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else if (a4) {
    for (int64_t i = lane; i < n / 4; i += lanes)
      reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
  } else {
    for (int64_t i = lane; i < n / 2; i += lanes)
      reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[i];
  }
}

__global__ __launch_bounds__(256) void append_kernel(char* pool, int64_t row_stride_b, int64_t row_bytes, int page_shift,
                                                      int num_pages, const int32_t* page_table, int max_pages,
                                                      const int32_t* positions, const char* rows, uint32_t* flags) {
  const int beta = blockIdx.x;
  const int pos = positions[beta];
  const int lp = pos >> page_shift;
  int pg = -1;
  if (pos >= 0 && lp < max_pages) pg = page_table[(int64_t)beta * max_pages + lp];
  if (pg < 0 || pg >= num_pages) {
    if (threadIdx.x == 0 && flags) atomicOr(flags, 2u);
    return;
  }
  const int64_t row = ((int64_t)pg << page_shift) | (pos & ((1 << page_shift) - 1));
  copy_bytes(pool + row * row_stride_b, rows + beta * row_bytes, row_bytes, threadIdx.x, blockDim.x);
}

constexpr int kGatherRows = 64;

__global__ __launch_bounds__(256) void gather_kernel(const char* pool, int64_t row_stride_b, int64_t row_bytes,
                                                      int page_shift, int num_pages, const int32_t* page_table,
                                                      int max_pages, const int32_t* seq_lens, int max_seq_len,
                                                      char* out, uint32_t* flags) {
  const int beta = blockIdx.y;
  int L = seq_lens[beta];
  L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
  const int s0 = blockIdx.x * kGatherRows;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = wave; r < kGatherRows; r += 4) {
    const int s = s0 + r;
    if (s >= L) break;
    const int lp = s >> page_shift;
    int pg = lp < max_pages ? page_table[(int64_t)beta * max_pages + lp] : -1;
    if (pg < 0 || pg >= num_pages) {
      if (lane == 0 && flags) atomicOr(flags, 2u);
      continue;
    }
    const int64_t row = ((int64_t)pg << page_shift) | (s & ((1 << page_shift) - 1));
    copy_bytes(out + ((int64_t)beta * max_seq_len + s) * row_bytes, pool + row * row_stride_b, row_bytes, lane, 64);
  }
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

hipError_t launch_paged_append(void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size, int32_t num_pages,
                               const int32_t* page_table, int32_t max_pages, const int32_t* positions, const void* rows,
                               int32_t batch, int32_t elem_bytes, uint32_t* error_flags, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(batch), dim3(256), 0, stream, static_cast<char*>(pool), row_stride * elem_bytes,
                     (int64_t)row_elems * elem_bytes, log2_exact(page_size), num_pages, page_table, max_pages, positions,
                     static_cast<const char*>(rows), error_flags);
  return hipGetLastError();
}

hipError_t launch_paged_gather(const void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size,
                               int32_t num_pages, const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                               int32_t max_seq_len, int32_t batch, int32_t elem_bytes, void* out, uint32_t* error_flags,
                               hipStream_t stream) {
  dim3 grid((max_seq_len + kGatherRows - 1) / kGatherRows, batch);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, stream, static_cast<const char*>(pool), row_stride * elem_bytes,
                     (int64_t)row_elems * elem_bytes, log2_exact(page_size), num_pages, page_table, max_pages, seq_lens,
                     max_seq_len, static_cast<char*>(out), error_flags);
  return hipGetLastError();
}

}  // namespace mlra
