// Cross-split merge and branch-sum epilogue.
//
// For sequence beta, head i, branch b the attention kernels left one partial
// state (o_s, m_s, l_s) per context split s (log2 units). The exact merge is
//   m* = max_s m_s,  w_s = 2^(m_s - m*),  u_{i,b} = sum_s w_s o_s / sum_s w_s l_s,
// and the output applies W^V per branch and sums the branches with the scale
// alpha (MLRA page "原生支持张量并行的多分支低秩注意力MLRA", §三 block outputs
// summed after attention, §3.3 scaled sum; §1.3 step 3 for MLA):
//   y[beta, i, :] = alpha * sum_b W^V_{i,b} u_{i,b} = alpha * W^V_i [u_{i,0}; ...; u_{i,nb-1}].
//
// One work-group per (head, block of kSeqBlock sequences): W^V_i is read once per
// block and reused for its sequences.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <cmath>

#include "mlra_internal.h"

namespace mlra {
namespace {

constexpr int kMergeThreads = 256;
constexpr int kSeqBlock = 4;

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == 0) return __bfloat162float(reinterpret_cast<const __hip_bfloat16*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  extern __shared__ float sm[];
  const int S = p.num_splits;
  const int DC = p.NB * p.DB;
  float* wts = sm;                                   // [kSeqBlock][NB][S]: m, then weights
  float* lsv = wts + kSeqBlock * p.NB * S;           // [kSeqBlock][NB][S]: l
  float* u = lsv + kSeqBlock * p.NB * S;             // [kSeqBlock][DC]
  __shared__ int nsplit[kSeqBlock];

  const int head = blockIdx.x;
  const int beta0 = blockIdx.y * kSeqBlock;
  const int tid = threadIdx.x;

  if (tid < kSeqBlock) {
    const int beta = beta0 + tid;
    int ns = 0;
    if (beta < p.B) {
      int L = p.seq_lens[beta];
      L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
      ns = (L + p.split_tokens - 1) / p.split_tokens;
    }
    nsplit[tid] = ns;
  }
  __syncthreads();

  // 1. gather (m, l) of every split
  for (int idx = tid; idx < kSeqBlock * p.NB * S; idx += kMergeThreads) {
    const int s = idx % S;
    const int b = (idx / S) % p.NB;
    const int bl = idx / (S * p.NB);
    const int beta = beta0 + bl;
    float m = -INFINITY, l = 0.f;
    if (beta < p.B && s < nsplit[bl]) {
      const int64_t rec = (((int64_t)beta * S + s) * p.H + head) * p.NB + b;
      m = p.ws_ml[rec * 2];
      l = p.ws_ml[rec * 2 + 1];
    }
    wts[idx] = m;
    lsv[idx] = l;
  }
  __syncthreads();
  // 2. per (sequence, branch): m*, normaliser, weights w_s / sum_s w_s l_s
  for (int pr = tid; pr < kSeqBlock * p.NB; pr += kMergeThreads) {
    float* w = wts + pr * S;
    const float* l = lsv + pr * S;
    float mstar = -INFINITY;
    for (int s = 0; s < S; ++s) mstar = fmaxf(mstar, w[s]);
    float den = 0.f;
    for (int s = 0; s < S; ++s) {
      const float e = (w[s] == -INFINITY) ? 0.f : exp2f(w[s] - mstar);
      w[s] = e;
      den += e * l[s];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int s = 0; s < S; ++s) w[s] *= inv;
  }
  __syncthreads();
  // 3. u = sum_s w_s o_s
  for (int idx = tid; idx < kSeqBlock * DC; idx += kMergeThreads) {
    const int e = idx % DC;
    const int bl = idx / DC;
    const int b = e / p.DB;
    const int f = e - b * p.DB;
    const int beta = beta0 + bl;
    float acc = 0.f;
    if (beta < p.B) {
      const float* w = wts + (bl * p.NB + b) * S;
      for (int s = 0; s < nsplit[bl]; ++s) {
        const int64_t rec = (((int64_t)beta * S + s) * p.H + head) * p.NB + b;
        acc += w[s] * p.ws_o[rec * p.DB + f];
      }
    }
    u[idx] = acc;
  }
  __syncthreads();
  // 4. y = alpha * W^V_i u   (row n of W^V_i is the d_c-long input vector of output n)
  for (int idx = tid; idx < kSeqBlock * p.DH; idx += kMergeThreads) {
    const int n = idx % p.DH;
    const int bl = idx / p.DH;
    const int beta = beta0 + bl;
    if (beta >= p.B) continue;
    const int64_t wrow = ((int64_t)head * p.DH + n) * DC;
    const float* uu = u + bl * DC;
    float acc = 0.f;
    for (int k = 0; k < DC; ++k) acc += uu[k] * load_elem(p.w_v, wrow + k, p.w_dtype);
    acc *= p.alpha;
    const int64_t o = ((int64_t)beta * p.H + head) * p.DH + n;
    if (p.out_dtype == 0) reinterpret_cast<__hip_bfloat16*>(p.out)[o] = __float2bfloat16(acc);
    else reinterpret_cast<float*>(p.out)[o] = acc;
  }
}

}  // namespace

bool merge_supported(int nb, int db, int dh) {
  (void)dh;
  return nb >= 1 && db >= 1 && nb * db <= 4096;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const size_t smem = sizeof(float) * ((size_t)kSeqBlock * p.NB * p.num_splits * 2 + (size_t)kSeqBlock * p.NB * p.DB);
  if (smem > 60 * 1024) return hipErrorInvalidValue;
  dim3 grid(p.H, (p.B + kSeqBlock - 1) / kSeqBlock);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), smem, stream, p);
  return hipGetLastError();
}

}  // namespace mlra
