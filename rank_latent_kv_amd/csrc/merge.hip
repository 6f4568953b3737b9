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
// One work-group per (head, block of sequences): W^V_i is read once per block and
// reused for its sequences (the MFMA kernel takes 1, 2 or 4 sequences per block, fewer
// when there are many splits to merge). The general kernel below handles fp32 W^V and
// odd widths on the vector ALUs, with blocks of kSeqBlock sequences.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <cmath>
#include <type_traits>

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
        acc += w[s] * (p.ws_o_f16 ? (float)static_cast<const _Float16*>(p.ws_o)[rec * p.DB + f]
                                  : static_cast<const float*>(p.ws_o)[rec * p.DB + f]);
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

// MFMA variant for bf16 W^V: one work-group per (head, SEQB sequences).
//  - The W^V_i operands of this wave's output tiles, seq_lens and every split's
//    partial state are requested up front, so the kernel pays about one memory
//    latency. Partials of splits past a sequence's end are read (they lie inside
//    the workspace) and discarded with selects.
//  - Each thread merges a slice of the splits for four features of one
//    (sequence, branch); the slices combine through LDS into u.
//  - u is split into bf16 hi + lo parts (|u - hi - lo| <= 2^-16 |u|) and
//      Y[seq x d_h] = U[seq x d_c] . W^V_i^T[d_c x d_h]
//    runs on 16x16x32 MFMAs (rows past the block's sequences are zero).
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kChunk = 8;   // splits whose loads are issued together per thread

// F16: the output records are scaled fp16 (the scale is already in m and l). A compile-time
// choice, so that every split's loads still go out together before the first is used.
template <int DC, int DH, int SEQB, bool F16>
__global__ __launch_bounds__(kMergeThreads) void merge_mfma_kernel(MergeParams p) {
  constexpr int KC = DC / 32;                      // K-chunks of the epilogue
  constexpr int NT = DH / 16;                      // 16-wide output tiles
  constexpr int NTW = (NT + 3) / 4;                // tiles per wave
  constexpr int ITEMS = SEQB * (DC / 4);      // (sequence, 4 features)
  constexpr int PAR = kMergeThreads / ITEMS >= 1 ? kMergeThreads / ITEMS : 1;   // threads per item
  constexpr int UROW = DC + 8;
  static_assert(ITEMS * PAR <= kMergeThreads || PAR == 1, "item mapping");
  __shared__ float red_m[PAR][ITEMS], red_l[PAR][ITEMS];
  __shared__ float4 red_o[PAR][ITEMS];
  __shared__ __attribute__((aligned(16))) __bf16 uhi[16][UROW];
  __shared__ __attribute__((aligned(16))) __bf16 ulo[16][UROW];

  const int head = blockIdx.x;
  const int beta0 = blockIdx.y * SEQB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = p.NB, DB = p.DB, S = p.num_splits;
  const int r16 = lane & 15, kg = lane >> 4;

  // this thread's (sequence, 4 features) item and its slice of the splits
  const int item = tid % ITEMS, part = tid / ITEMS;
  const int bl = item / (DC / 4);
  const int k = (item % (DC / 4)) * 4;
  const int b = k / DB;
  const int beta = beta0 + bl;
  const bool active = part < PAR && beta < p.B;
  const int beta_c = beta < p.B ? beta : p.B - 1;

  // The W^V_i operands of this wave's output tiles go out first: every output tile is some
  // wave's (d_h / 16 tiles over 4 waves), so the loads are unconditional and nothing waits
  // between them. Then the sequence length and the first round of split records, kept raw
  // (fp16 records are converted where the merge uses them), so that no conversion makes the
  // wave wait for one load before it issues the next: one memory latency covers them all.
  static_assert(NT % 4 == 0, "the 4 waves own every output tile");
  const __bf16* wv = reinterpret_cast<const __bf16*>(p.w_v) + (int64_t)head * DH * DC;
  bf16x8 wreg[NTW][KC];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int nt = wave + 4 * t;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      wreg[t][kc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                        wv + (int64_t)(nt * 16 + r16) * DC + 32 * kc + 8 * kg));
  }
  // loads of one round of kChunk splits (clamped to the last split; unused ones are discarded)
  float2 mlv[kChunk];
  typedef typename std::conditional<F16, uint2, float4>::type Raw;
  Raw ov[kChunk];
  auto load_round = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int sp = s0 + j * PAR;
      const int spc = sp < S ? sp : S - 1;
      const int64_t rec = (((int64_t)beta_c * S + spc) * p.H + head) * NB + b;
      mlv[j] = *reinterpret_cast<const float2*>(p.ws_ml + rec * 2);
      const int64_t oi = rec * DB + (k - b * DB);
      if constexpr (F16) ov[j] = *reinterpret_cast<const uint2*>(static_cast<const _Float16*>(p.ws_o) + oi);
      else ov[j] = *reinterpret_cast<const float4*>(static_cast<const float*>(p.ws_o) + oi);
    }
  };
  auto value = [&](int j) __attribute__((always_inline)) -> float4 {
    if constexpr (F16) {
      const uint2 w = ov[j];
      return make_float4((float)__builtin_bit_cast(_Float16, (unsigned short)(w.x & 0xffffu)),
                         (float)__builtin_bit_cast(_Float16, (unsigned short)(w.x >> 16)),
                         (float)__builtin_bit_cast(_Float16, (unsigned short)(w.y & 0xffffu)),
                         (float)__builtin_bit_cast(_Float16, (unsigned short)(w.y >> 16)));
    } else {
      return ov[j];
    }
  };
  int ns = 0;
  if (active) {
    int L = p.seq_lens[beta];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    ns = (L + p.split_tokens - 1) / p.split_tokens;
    load_round(part);
  }
  for (int i = tid; i < 16 * UROW; i += kMergeThreads) {
    (&uhi[0][0])[i] = (__bf16)0.f;
    (&ulo[0][0])[i] = (__bf16)0.f;
  }

  // 1. partial merges over this thread's splits
  if (part < PAR) {
    float m_loc = -INFINITY, l_loc = 0.f;
    float4 o_loc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active) {
      for (int s0 = part; s0 < S; s0 += PAR * kChunk) {
        if (s0 != part) load_round(s0);
        float mc = m_loc;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          const bool ok = s0 + j * PAR < ns;
          mc = ok ? fmaxf(mc, mlv[j].x) : mc;
        }
        const float fold = (m_loc == -INFINITY) ? 0.f : exp2f(m_loc - mc);
        l_loc *= fold;
        o_loc.x *= fold; o_loc.y *= fold; o_loc.z *= fold; o_loc.w *= fold;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          const bool ok = s0 + j * PAR < ns;
          const float wj = ok ? exp2f(mlv[j].x - mc) : 0.f;
          const float4 v = value(j);
          l_loc += ok ? wj * mlv[j].y : 0.f;
          o_loc.x += ok ? wj * v.x : 0.f;
          o_loc.y += ok ? wj * v.y : 0.f;
          o_loc.z += ok ? wj * v.z : 0.f;
          o_loc.w += ok ? wj * v.w : 0.f;
        }
        m_loc = mc;
      }
    }
    red_m[part][item] = m_loc;
    red_l[part][item] = l_loc;
    red_o[part][item] = o_loc;
  }
  __syncthreads();
  // 2. combine the slices: u = sum_q 2^(m_q - m*) o_q / sum_q 2^(m_q - m*) l_q
  if (tid < ITEMS) {
    float ms = -INFINITY;
#pragma unroll
    for (int q = 0; q < PAR; ++q) ms = fmaxf(ms, red_m[q][tid]);
    float den = 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < PAR; ++q) {
      const float f = (red_m[q][tid] == -INFINITY) ? 0.f : exp2f(red_m[q][tid] - ms);
      den += f * red_l[q][tid];
      num.x += f * red_o[q][tid].x; num.y += f * red_o[q][tid].y;
      num.z += f * red_o[q][tid].z; num.w += f * red_o[q][tid].w;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const float v[4] = {num.x * inv, num.y * inv, num.z * inv, num.w * inv};
    const int ib = tid / (DC / 4), ik = (tid % (DC / 4)) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const __bf16 hi = (__bf16)v[q];
      uhi[ib][ik + q] = hi;
      ulo[ib][ik + q] = (__bf16)(v[q] - (float)hi);
    }
  }
  __syncthreads();

  // 3. Y = U . W^T on 16x16x32 MFMAs; each wave owns every 4th 16-column tile of d_h. The
  //    tiles' chains run interleaved (each still in K order, hi before lo), over U operands
  //    read from LDS once per K-chunk.
  f32x4 acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&uhi[r16][32 * kc + 8 * kg]);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&ulo[r16][32 * kc + 8 * kg]);
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wreg[t][kc], acc[t], 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wreg[t][kc], acc[t], 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int nt = wave + 4 * t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bo = 4 * kg + j;
      const int bt = beta0 + bo;
      if (bo >= SEQB || bt >= p.B) continue;
      const int64_t o = ((int64_t)bt * p.H + head) * DH + nt * 16 + r16;
      const float yv = acc[t][j] * p.alpha;
      if (p.out_dtype == 0) reinterpret_cast<__hip_bfloat16*>(p.out)[o] = __float2bfloat16(yv);
      else reinterpret_cast<float*>(p.out)[o] = yv;
    }
  }
}

}  // namespace

bool merge_supported(int nb, int db, int dh) {
  (void)dh;
  return nb >= 1 && db >= 1 && nb * db <= 4096;
}

namespace {
bool mfma_merge_shape(int dc, int dh) {
  return (dh == 128 && (dc == 32 || dc == 64 || dc == 128 || dc == 256)) || (dc == 128 && (dh == 64 || dh == 256));
}
}  // namespace

bool merge_uses_mfma(int nb, int db, int dh, int w_dtype, const void* w_v) {
  return w_dtype == 0 && (reinterpret_cast<uintptr_t>(w_v) & 15) == 0 && db % 4 == 0 && mfma_merge_shape(nb * db, dh);
}

size_t merge_lds_bytes(int nb, int db, int num_splits) {
  return sizeof(float) * ((size_t)kSeqBlock * nb * num_splits * 2 + (size_t)kSeqBlock * nb * db);
}

// Sequences per work-group of the MFMA merge: W^V_i is read once per block, but a block
// of SB sequences leaves 256 / (SB * d_c / 4) threads for each (sequence, 4 features),
// each loading kChunk splits per round. Take the largest block whose split loads fit one
// round; with more splits, one sequence per group (most threads per item, most groups).
static int merge_seq_block(int dc, int num_splits) {
  for (int sb = 4; sb > 1; sb /= 2) {
    const int items = sb * (dc / 4);
    const int par = kMergeThreads / items >= 1 ? kMergeThreads / items : 1;
    if (num_splits <= par * kChunk) return sb;
  }
  return 1;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  dim3 grid(p.H, (p.B + kSeqBlock - 1) / kSeqBlock);
  const int DC = p.NB * p.DB;
  if (merge_uses_mfma(p.NB, p.DB, p.DH, p.w_dtype, p.w_v)) {
    const int sb = merge_seq_block(DC, p.num_splits);
    const dim3 mgrid(p.H, (p.B + sb - 1) / sb);
#define MLRA_MERGE_CASE(xDC, xDH)                                                                       \
    if (DC == xDC && p.DH == xDH) {                                                                     \
      if (p.ws_o_f16) {                                                                                 \
        if (sb == 4) hipLaunchKernelGGL((merge_mfma_kernel<xDC, xDH, 4, true>), mgrid, dim3(kMergeThreads), 0, stream, p); \
        else if (sb == 2) hipLaunchKernelGGL((merge_mfma_kernel<xDC, xDH, 2, true>), mgrid, dim3(kMergeThreads), 0, stream, p); \
        else hipLaunchKernelGGL((merge_mfma_kernel<xDC, xDH, 1, true>), mgrid, dim3(kMergeThreads), 0, stream, p); \
      } else {                                                                                          \
        if (sb == 4) hipLaunchKernelGGL((merge_mfma_kernel<xDC, xDH, 4, false>), mgrid, dim3(kMergeThreads), 0, stream, p); \
        else if (sb == 2) hipLaunchKernelGGL((merge_mfma_kernel<xDC, xDH, 2, false>), mgrid, dim3(kMergeThreads), 0, stream, p); \
        else hipLaunchKernelGGL((merge_mfma_kernel<xDC, xDH, 1, false>), mgrid, dim3(kMergeThreads), 0, stream, p); \
      }                                                                                                 \
      return hipGetLastError();                                                                         \
    }
    MLRA_MERGE_CASE(32, 128)
    MLRA_MERGE_CASE(64, 128)
    MLRA_MERGE_CASE(128, 128)
    MLRA_MERGE_CASE(256, 128)
    MLRA_MERGE_CASE(128, 64)
    MLRA_MERGE_CASE(128, 256)
#undef MLRA_MERGE_CASE
    return hipErrorInvalidValue;   // mfma_merge_shape and the cases above disagree
  }
  const size_t smem = merge_lds_bytes(p.NB, p.DB, p.num_splits);
  if (smem > kMergeLdsLimit) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeThreads), smem, stream, p);
  return hipGetLastError();
}

}  // namespace mlra
