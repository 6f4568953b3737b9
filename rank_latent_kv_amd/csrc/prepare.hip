// The step before a decode call, for one new token per sequence at position m:
//  - query absorption ([MLRA] page "原生支持张量并行的多分支低秩注意力MLRA", §1.3
//    step 1; §二 for the branch split): q~_i = W^UK_i^T q^N_i, written as the
//    branches' absorbed queries q_lat[beta][i][b][:] = q~_i[b*d_b:(b+1)*d_b];
//  - the RoPE query rotated to position m (decoupled RoPE: per-head RoPE queries
//    and one shared RoPE key);
//  - the new token's cache row: its latent and its RoPE key rotated to m.
// Rotation of a RoPE vector at position m: pair (x_2j, x_2j+1) turns by
// m * base^(-2j/d_R). The angle and its sine and cosine are computed in fp64 so
// that long positions keep their accuracy; the rotation itself runs in fp32.
//
// On the MFMA path each wave of the absorption work-groups computes one 16-column tile of
// one head's absorbed queries for every sequence (a head's tiles spread over
// ceil(d_c / 64) groups), issuing all of its loads before its first MFMA; one work-group
// per sequence computes the sequence's rotation angles once (fp64, into LDS), rotates the
// RoPE query of every head and writes the cache row, with its first query loads issued
// before the angles are computed. For
// bf16 with d_h % 32 == 0 (at most 256) and d_c % 16 == 0 the absorption runs on
// 16x16x32 MFMAs, each wave loading all its operands before its first MFMA:
//   Q~[seq x d_c] = Q^N[seq x d_h] . W^UK_i[d_h x d_c],
// with W^UK_i stored transposed ([d_c][d_h]) so that every MFMA operand is one
// 16-byte load; otherwise on the vector ALUs.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <cmath>

#include "mlra_internal.h"

namespace mlra {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kMaxKc = 8;   // K-chunks of 32 in the MFMA absorption: d_h <= 256

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float ld(const void* base, int64_t idx, int dtype) {
  if (dtype == 0) return __bfloat162float(reinterpret_cast<const __hip_bfloat16*>(base)[idx]);
  return reinterpret_cast<const float*>(base)[idx];
}
__device__ __forceinline__ void st(void* base, int64_t idx, float v, int dtype) {
  if (dtype == 0) reinterpret_cast<__hip_bfloat16*>(base)[idx] = __float2bfloat16(v);
  else reinterpret_cast<float*>(base)[idx] = v;
}

constexpr int kMaxHalf = 128;   // RoPE pairs: d_R <= 256

// cos and sin of m * base^(-2j/d_R), in fp64
__device__ __forceinline__ void rope_cs(int m, int j, int dr, double base, float* c, float* s) {
  const double theta = exp2(-2.0 * (double)j / (double)dr * log2(base));
  double sd, cd;
  sincos((double)m * theta, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// Absorption work-groups per head: on the MFMA path one 16-column output tile per wave, so
// that every wave issues all of its loads at once; otherwise one group per head.
__host__ __device__ inline int absorb_groups(const PrepareParams& p) {
  constexpr int kWaves = kPrepThreads / 64;
  return p.mfma ? (p.NB * p.DB / 16 + kWaves - 1) / kWaves : 1;
}

constexpr int kQPre = 4;   // RoPE-query pairs per thread loaded before the angles are known

__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(PrepareParams p) {
  const int tid = threadIdx.x;
  const int DC = p.NB * p.DB;
  const int ag = absorb_groups(p);
  if (blockIdx.x < (unsigned)(p.H * ag)) {
    const int head = blockIdx.x / ag;
    // ---- absorption ----------------------------------------------------------------------
    if (p.mfma) {
      const int lane = tid & 63, wave = tid >> 6;
      const int r16 = lane & 15, kg = lane >> 4;
      const int nt = (blockIdx.x - head * ag) * (kPrepThreads / 64) + wave;   // this wave's output tile
      if (nt >= DC / 16) return;
      const int kchunks = p.DH / 32;
      const __bf16* qn = reinterpret_cast<const __bf16*>(p.q_nope);
      const __bf16* wrow = reinterpret_cast<const __bf16*>(p.w_uk) + ((int64_t)head * DC + 16 * nt + r16) * p.DH;
      // B operands (W^UK_i rows of this tile), used for every block of 16 sequences
      bf16x8 b[kMaxKc];
#pragma unroll
      for (int kc = 0; kc < kMaxKc; ++kc)
        if (kc < kchunks) b[kc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(wrow + 32 * kc + 8 * kg));
      for (int m0 = 0; m0 < p.B; m0 += 16) {
        const int beta_a = m0 + r16;                 // A row of this lane
        bf16x8 a[kMaxKc];
#pragma unroll
        for (int kc = 0; kc < kMaxKc; ++kc)
          if (kc < kchunks)
            a[kc] = beta_a < p.B ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                       qn + ((int64_t)beta_a * p.H + head) * p.DH + 32 * kc + 8 * kg))
                                 : bf16x8{};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < kMaxKc; ++kc)
          if (kc < kchunks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kc], b[kc], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int beta = m0 + 4 * kg + r;
          if (beta < p.B) st(p.q_lat, ((int64_t)beta * p.H + head) * DC + 16 * nt + r16, acc[r], p.dtype);
        }
      }
    } else {
      for (int idx = tid; idx < p.B * DC; idx += kPrepThreads) {
        const int beta = idx / DC, n = idx - beta * DC;
        float acc = 0.f;
        for (int k = 0; k < p.DH; ++k)
          acc += ld(p.q_nope, ((int64_t)beta * p.H + head) * p.DH + k, p.dtype) *
                 ld(p.w_uk, ((int64_t)head * DC + n) * p.DH + k, p.dtype);
        st(p.q_lat, ((int64_t)beta * p.H + head) * DC + n, acc, p.dtype);
      }
    }
    return;
  }
  // ---- sequence: rotation angles, RoPE queries of every head, cache row -------------------------
  __shared__ float cs_c[kMaxHalf], cs_s[kMaxHalf];
  const int eb = p.dtype == 0 ? 2 : 4;
  const int half = p.DR / 2;
  const int beta = blockIdx.x - p.H * ag;
  const int m = p.positions[beta];
  const int nq = p.H * half;                 // RoPE-query pairs of this sequence
  // The first kQPre query pairs of this thread are loaded before the angles, so that the
  // loads are in flight while the fp64 angles are computed.
  float qx0[kQPre], qx1[kQPre];
#pragma unroll
  for (int it = 0; it < kQPre; ++it) {
    const int idx = tid + it * kPrepThreads;
    const int head = idx / half, j = idx - head * half;
    const int64_t o = ((int64_t)beta * p.H + head) * p.DR + 2 * j;
    qx0[it] = idx < nq ? ld(p.q_pe, o, p.dtype) : 0.f;
    qx1[it] = idx < nq ? ld(p.q_pe, o + 1, p.dtype) : 0.f;
  }
  if (tid < half) rope_cs(m, tid, p.DR, (double)p.rope_base, &cs_c[tid], &cs_s[tid]);
  __syncthreads();
  auto rotate_query = [&](int idx, float x0, float x1) {
    const int head = idx / half, j = idx - head * half;
    const int64_t o = ((int64_t)beta * p.H + head) * p.DR + 2 * j;
    st(p.q_rope, o, x0 * cs_c[j] - x1 * cs_s[j], p.dtype);
    st(p.q_rope, o + 1, x0 * cs_s[j] + x1 * cs_c[j], p.dtype);
  };
#pragma unroll
  for (int it = 0; it < kQPre; ++it)
    if (tid + it * kPrepThreads < nq) rotate_query(tid + it * kPrepThreads, qx0[it], qx1[it]);
  for (int idx = tid + kQPre * kPrepThreads; idx < nq; idx += kPrepThreads) {
    const int head = idx / half, j = idx - head * half;
    const int64_t o = ((int64_t)beta * p.H + head) * p.DR + 2 * j;
    rotate_query(idx, ld(p.q_pe, o, p.dtype), ld(p.q_pe, o + 1, p.dtype));
  }
  const int per = DC + half;                 // latent elements + RoPE pairs of one row
  for (int e = tid; e < per; e += kPrepThreads) {
    int64_t row;
    if (p.page_table) {
      const int lp = m >> p.page_shift;
      if (m < 0 || lp >= p.max_pages) {
        if (e == 0 && p.error_flags) atomicOr(p.error_flags, 1u);
        continue;
      }
      const int pg = p.page_table[(int64_t)beta * p.max_pages + lp];
      if (pg < 0 || pg >= p.num_pages) {
        if (e == 0 && p.error_flags) atomicOr(p.error_flags, 2u);
        continue;
      }
      row = ((int64_t)pg << p.page_shift) | (m & ((1 << p.page_shift) - 1));
    } else {
      if (m < 0 || m >= p.max_seq_len) {
        if (e == 0 && p.error_flags) atomicOr(p.error_flags, 1u);
        continue;
      }
      row = m;
    }
    const int64_t off = (p.page_table ? 0 : (int64_t)beta * p.seq_stride_b) + row * p.row_stride_b;
    char* lat = static_cast<char*>(p.kv_lat) + off;
    char* rope = static_cast<char*>(p.kv_rope) + off;
    if (e < DC) {
      // bit-exact copy of the latent
      if (eb == 2)
        reinterpret_cast<uint16_t*>(lat)[e] = reinterpret_cast<const uint16_t*>(p.c_new)[(int64_t)beta * DC + e];
      else
        reinterpret_cast<uint32_t*>(lat)[e] = reinterpret_cast<const uint32_t*>(p.c_new)[(int64_t)beta * DC + e];
    } else {
      const int j = e - DC;
      const int64_t o = (int64_t)beta * p.DR + 2 * j;
      const float x0 = ld(p.k_pe_new, o, p.dtype), x1 = ld(p.k_pe_new, o + 1, p.dtype);
      st(rope, 2 * j, x0 * cs_c[j] - x1 * cs_s[j], p.dtype);
      st(rope, 2 * j + 1, x0 * cs_s[j] + x1 * cs_c[j], p.dtype);
    }
  }
}

}  // namespace

bool prepare_mfma_supported(int dh, int dc) { return dh % 32 == 0 && dh <= 32 * kMaxKc && dc % 16 == 0; }

hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(prepare_kernel, dim3(p.H * absorb_groups(p) + p.B), dim3(kPrepThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mlra
