// Generic split attention for MLRA / MLA decode: fp32 or bf16 inputs, any
// branch count and widths within the limits below. It serves the fp32 path and
// shapes without an MFMA build; it writes the same partial state as the MFMA
// kernel (o, m, l in log2 units), so the same merge kernel finishes the call.
//
// One work-group per (split, sequence, head). Tokens go in chunks of 256: each
// thread scores one token for every branch (branch latent block plus the shared
// RoPE key, MLRA page "原生支持张量并行的多分支低秩注意力MLRA", §3.1), the block
// updates each branch's running max and sum, then each thread accumulates its
// share of the o[b][f] entries over the chunk.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <cmath>

#include "mlra_internal.h"

namespace mlra {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxNB = 16;
constexpr int kMaxDC = 4096;
constexpr int kMaxDR = 512;
constexpr int kMaxE = kMaxDC / kThreads;

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<__hip_bfloat16>(const __hip_bfloat16* p, int64_t i) {
  return __bfloat162float(p[i]);
}

__device__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < kThreads / 64; ++w) r += red[w];
  return r;
}

template <typename T, bool PAGED>
__global__ __launch_bounds__(kThreads) void attn_generic_kernel(AttnParams p) {
  __shared__ float qs[kMaxDC + kMaxDR];
  __shared__ float zs[kMaxNB][kThreads];
  __shared__ float red[kThreads / 64];
  __shared__ float mst[kMaxNB], lst[kMaxNB], scl[kMaxNB];

  const int split = blockIdx.x, beta = blockIdx.y, head = blockIdx.z;
  const int tid = threadIdx.x;
  const int NB = p.NB, DB = p.DB, DR = p.DR, DC = NB * DB;
  int L = p.seq_lens[beta];
  if (L < 1 || L > p.max_seq_len) {
    if (tid == 0 && split == 0 && head == 0 && p.error_flags) atomicOr(p.error_flags, 1u);
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  }
  const int t0 = split * p.split_tokens;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + p.split_tokens);

  const T* ql = reinterpret_cast<const T*>(p.q_lat) + ((int64_t)beta * p.H + head) * DC;
  const T* qr = reinterpret_cast<const T*>(p.q_rope) + ((int64_t)beta * p.H + head) * DR;
  for (int i = tid; i < DC; i += kThreads) qs[i] = ld(ql, i) * p.q_scale;
  for (int i = tid; i < DR; i += kThreads) qs[DC + i] = ld(qr, i) * p.q_scale;
  if (tid < NB) {
    mst[tid] = -INFINITY;
    lst[tid] = 0.f;
  }
  float o[kMaxE];
#pragma unroll
  for (int k = 0; k < kMaxE; ++k) o[k] = 0.f;
  __syncthreads();

  auto row_of = [&](int tok) -> int64_t {
    if constexpr (PAGED) {
      int pg = p.page_table[(int64_t)beta * p.max_pages + (tok >> p.page_shift)];
      if (pg < 0 || pg >= p.num_pages) {
        if (p.error_flags) atomicOr(p.error_flags, 2u);
        pg = 0;
      }
      return ((int64_t)pg << p.page_shift) | (tok & ((1 << p.page_shift) - 1));
    } else {
      return tok;
    }
  };
  const char* lat = p.kv_lat + (PAGED ? 0 : (int64_t)beta * p.seq_stride_b);
  const char* rop = p.kv_rope + (PAGED ? 0 : (int64_t)beta * p.seq_stride_b);

  for (int c0 = t0; c0 < t1; c0 += kThreads) {
    const int n = min(kThreads, t1 - c0);
    if (tid < n) {
      const int64_t row = row_of(c0 + tid);
      const T* cl = reinterpret_cast<const T*>(lat + row * p.row_stride_b);
      const T* cr = reinterpret_cast<const T*>(rop + row * p.row_stride_b);
      float zr = 0.f;
      for (int r = 0; r < DR; ++r) zr += qs[DC + r] * ld(cr, r);
      for (int b = 0; b < NB; ++b) {
        float z = zr;
        for (int j = 0; j < DB; ++j) z += qs[b * DB + j] * ld(cl, b * DB + j);
        zs[b][tid] = z;
      }
    } else {
      for (int b = 0; b < NB; ++b) zs[b][tid] = -INFINITY;
    }
    __syncthreads();
    for (int b = 0; b < NB; ++b) {
      const float z = zs[b][tid];
      const float cm = block_max(z, red);
      const float mold = mst[b];
      const float mnew = fmaxf(mold, cm);
      const float e = exp2f(z - mnew);
      const float s = block_sum(tid < n ? e : 0.f, red);
      zs[b][tid] = tid < n ? e : 0.f;
      __syncthreads();
      if (tid == 0) {
        const float f = (mold == -INFINITY) ? 0.f : exp2f(mold - mnew);
        scl[b] = f;
        lst[b] = lst[b] * f + s;
        mst[b] = mnew;
      }
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < kMaxE; ++k) {
      const int e = tid + k * kThreads;
      if (e >= DC) break;
      const int b = e / DB;
      float acc = o[k] * scl[b];
      for (int t = 0; t < n; ++t) {
        const int64_t row = row_of(c0 + t);
        acc += zs[b][t] * ld(reinterpret_cast<const T*>(lat + row * p.row_stride_b), e);
      }
      o[k] = acc;
    }
    __syncthreads();
  }

  const int64_t rec0 = (((int64_t)beta * p.num_splits + split) * p.H + head) * NB;
#pragma unroll
  for (int k = 0; k < kMaxE; ++k) {
    const int e = tid + k * kThreads;
    if (e >= DC) break;
    static_cast<float*>(p.ws_o)[rec0 * DB + e] = o[k];
  }
  if (tid < NB) {
    p.ws_ml[(rec0 + tid) * 2] = mst[tid];
    p.ws_ml[(rec0 + tid) * 2 + 1] = lst[tid];
  }
}

}  // namespace

bool generic_supported(int nb, int db, int dr) {
  return nb >= 1 && nb <= kMaxNB && db >= 1 && nb * db <= kMaxDC && dr >= 0 && dr <= kMaxDR;
}

hipError_t launch_attn_generic(const AttnParams& p, bool paged, int dtype, int grid_splits, hipStream_t stream) {
  dim3 grid(grid_splits, p.B, p.H);
  if (dtype == 0) {
    if (paged) hipLaunchKernelGGL((attn_generic_kernel<__hip_bfloat16, true>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_generic_kernel<__hip_bfloat16, false>), grid, dim3(kThreads), 0, stream, p);
  } else {
    if (paged) hipLaunchKernelGGL((attn_generic_kernel<float, true>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_generic_kernel<float, false>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mlra
