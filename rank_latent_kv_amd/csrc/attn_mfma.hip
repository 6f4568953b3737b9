// Split-context flash-decode attention for MLRA / MLA on gfx950 (bf16 inputs,
// fp32 accumulation, MFMA 32x32x16).
//
// One work-group of W waves (8 for MLRA-4 and most single-latent shapes, 4 for the 16-head
// MLA shard) owns one (sequence, context split). The split's cache rows stream
// HBM -> LDS once, through a ring of as many stages as fit in LDS (at most eight) filled by
// asynchronous LDS-DMA loads, and every query head
// reads them from LDS: all heads share one cached latent (MLRA page
// "原生支持张量并行的多分支低秩注意力MLRA", §1.3 step 2, MQA-style attention over the
// latent; §3.1, each branch attends over its own latent block plus the RoPE key shared
// by all branches).
//
// Work split inside the group. A "unit" is (branch b, group of 32 heads). Each wave owns
// BPW branches (a branch group) and some head groups, and possibly only every P-th 32-token
// sub-tile (a "phase"); phases are merged in LDS at the end.
//
// Per 32-token sub-tile and unit:
//   scores  S^T[tok x head] = C_ext[tok x (d_R+d_b)] . Q_ext^T, MFMA with the exact bf16
//           query and fp32 accumulation. The RoPE part q^R . k^R does not depend on the
//           branch: with two branches per wave it is computed once and seeds both
//           branches' latent chains. The logit in log2 units is x = S * tau*log2(e) minus
//           the reference max, one fma;
//   softmax lazy running max: the reference m is the exact max of the split's first
//           sub-tile and only moves (with a rescale of O and l) when a sub-tile's
//           weights sum past 2^16; p = 2^(x-m) is packed to bf16 and l accumulates the
//           packed values (4x4x4 bf16 MFMAs with an all-ones operand add four of a lane's
//           weights at a time), so the normaliser sums exactly the weights the P.C
//           product uses;
//   values  O^T[feat x head] += C_b^T[feat x tok] . P^T[tok x head], MFMA, with the
//           transposed latent read by ds_read_b64_tr_b16.
// The loop is software-pipelined: the score MFMAs of the next sub-tile go out before the
// softmax of the current one (with several branches per wave, together with the P.C MFMAs of
// the previous sub-tile, interleaved with the softmax's vector instructions).
// Each split writes its unnormalised (o, m, l): with several branches o in fp16, scaled by a
// power of two folded into m, else in fp32 through L2 to memory where a store fills whole
// 32-byte pieces; the merge kernel combines the splits (log-sum-exp) and applies W^V per
// branch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "mlra_internal.h"

namespace mlra {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) const int lds_cint;

constexpr int kMaxStages = 8;
constexpr int kMfmaGap = 6;                // vector instructions between two matrix instructions of a pipelined block
constexpr int kSubPerStage = 4;            // 32-token sub-tiles per stage (more when there are more phases)
constexpr int kLdsBytes = 160 * 1024;
constexpr int kPageCache = 256;            // page ids of one split kept in LDS (paged mode)
constexpr int kPageLanes = 64;             // or in one register, one page id per lane
constexpr int kRotateStages = 64;          // splits of at least this many full stages rotate their start
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p = 2^x stays <= 256
constexpr float kStageSumMax = 65536.0f;   // a lane's sub-tile weights summing past this trigger the exact max

template <int NB, int DB, int DR, int HEADS, int W, bool PAGED, int BPW>
struct Cfg {
  static constexpr int WAVES = W;                        // waves per work-group
  static constexpr int THREADS = W * 64;
  static constexpr int NHG = (HEADS + 31) / 32;          // head groups (MFMA N = 32)
  static constexpr int NBG = NB / BPW;                   // branch groups (BPW branches per wave)
  static constexpr int WPB = W / NBG;                    // waves per branch group
  static constexpr int HGSPLIT = WPB < NHG ? WPB : NHG;  // head-group slots per branch group
  static constexpr int HPW = NHG / HGSPLIT;              // head groups per wave
  static constexpr int P = WPB / HGSPLIT;                // token phases
  static constexpr int SUB = P > kSubPerStage ? P : kSubPerStage;     // 32-token sub-tiles per stage
  static constexpr int NSW = SUB / P;                    // sub-tiles of one wave per stage
  // one branch per wave: the next sub-tile's scores are issued before the current softmax
  static constexpr bool PIPE = BPW == 1;
  // several branches per wave with two waves per SIMD (PIPE2, below): the registers hold two
  // sub-tiles' scores, so the scores of sub-tile k + 1 and the P.C of sub-tile k - 1 are
  // issued in the same block as the softmax of sub-tile k. The delayed P.C keeps a stage's
  // ring slot in use until two barriers later, which needs a ring of four stages; with more
  // waves (fewer registers each) or a shallower ring the same work split runs unpipelined.
  static constexpr int ST = 32 * SUB;                    // tokens per stage
  static constexpr int NCL = NB * DB / 8;                // latent 16-byte chunks per row
  static constexpr int NCR = DR / 8;                     // RoPE 16-byte chunks per row
  static constexpr int NCH = NCL + NCR;
  // Latent chunks never wrap around their LDS row (largest latent chunk + largest rotation
  // < NCH): their per-lane offsets are then one base plus compile-time constants.
  static constexpr int MAXROT = NCH % 8 == 0 ? 7 : 3;
  static constexpr bool LAT_FLAT = NCL - 1 + MAXROT < NCH;
  static constexpr int SUB_BYTES = 32 * NCH * 16;
  static constexpr int STAGE_BYTES = ST * NCH * 16;
  static constexpr int DMA_PER_STAGE = ST * NCH / 64;    // wave-wide 1 KiB DMA instructions
  static constexpr int DW = W;                                         // DMA-issuing waves
  static constexpr int DMA_HI = (DMA_PER_STAGE + DW - 1) / DW;         // instructions of waves < DMA_SPLIT
  static constexpr int DMA_LO = DMA_PER_STAGE / DW;                    // instructions of waves DMA_SPLIT..DW-1
  static constexpr int DMA_SPLIT = DMA_PER_STAGE - DMA_LO * DW;
  static constexpr int MT = DB / 32;                     // value M-tiles (32 features)
  static constexpr int KR = DR / 16;                     // RoPE K-chunks of the score
  static constexpr int KL = DB / 16;                     // latent K-chunks of the score
  static constexpr int QL_BYTES = HEADS * NB * DB * 2;  // one sequence's absorbed queries
  static constexpr int QR_BYTES = HEADS * DR * 2;       // and RoPE queries
  static constexpr int QL_DMA = (QL_BYTES + 1023) / 1024;
  static constexpr int QR_DMA = (QR_BYTES + 1023) / 1024;
  static constexpr int MERGE_WAVES = P > 1 ? W : 0;     // every wave publishes a merge record
  static constexpr int MERGE_FLOATS = HPW * BPW * (16 * MT + 2) * 64;   // per wave record
  // Paged instances with several branches per wave keep the split's page ids in registers and
  // give each wave a block of TPW consecutive tokens per stage (one page when pages hold at
  // least TPW tokens), so the ring keeps all of LDS; the others cache the page ids in LDS.
  static constexpr bool PAGE_REGS = PAGED && BPW > 1;
  static constexpr int TPW = DMA_HI * 64 / NCH;          // tokens per wave per stage (blocked plan)
  static constexpr int PTAB_BYTES = (PAGED && !PAGE_REGS) ? kPageCache * 4 : 0;
  static constexpr int NS_FIT = (kLdsBytes - PTAB_BYTES) / STAGE_BYTES;
  static constexpr int NS = NS_FIT < kMaxStages ? NS_FIT : kMaxStages;   // ring depth
  static constexpr int RING_BYTES = NS * STAGE_BYTES;
  static constexpr bool PIPE2 = BPW > 1 && W <= 8 && NS >= 4;
  // fp16 split records where the phase merge leaves each wave whole 4-row groups (two phases
  // with several branches, four with one); with eight phases a wave writes 2-row pieces, which
  // as fp16 would be 4-byte stores, and keeps fp32 records
  static constexpr bool F16REC = P == 2 || P == 4;
  static constexpr int MERGE_BYTES = MERGE_WAVES * MERGE_FLOATS * 4;
  static constexpr int LDS_BYTES = (RING_BYTES > MERGE_BYTES ? RING_BYTES : MERGE_BYTES) + PTAB_BYTES;
  static_assert(NB % BPW == 0, "branches per wave must divide the branches");
  static_assert(W % NBG == 0, "branch groups must divide the waves");
  static_assert(NHG % HGSPLIT == 0, "head groups must split evenly");
  static_assert(SUB % P == 0, "phases must divide the sub-tiles");
  static_assert(DB % 32 == 0 && DR % 16 == 0, "MFMA tiling");
  static_assert((NCH % 8 == 0 && NCH >= 8) || NCH % 16 == 4, "chunk rotation assumes NCH = 0 mod 8 or 4 mod 16");
  static_assert(NS >= 3, "the ring needs three stages");
  static_assert(DMA_HI * (NS - 2) < 64, "vmcnt range of the DMA waits");
  static_assert(!PAGE_REGS || (DMA_PER_STAGE == W * DMA_HI && (DMA_HI * 64) % NCH == 0 && ST == W * TPW),
                "the blocked DMA plan gives every wave the same whole tokens");
  static_assert(LDS_BYTES <= kLdsBytes, "LDS budget");
  static_assert((QL_DMA + QR_DMA) * 1024 <= STAGE_BYTES, "the queries fit one ring slot");
  static_assert(QL_BYTES % 16 == 0 && QR_BYTES % 16 == 0, "16-byte query chunks");
};

// Rotation of the 16-byte chunk positions of token t inside its LDS row. The LDS
// serves 16 lanes of 16 bytes per cycle (64 banks of 4 bytes), so
//  - 16 consecutive tokens reading the same chunk (score operand) and
//  - 4 consecutive tokens (first one a multiple of 4) reading 4 consecutive
//    chunks (transposed value operand)
// must land in 16 different 16-byte bank groups. Row widths of 20 chunks
// (= 4 mod 16) and 8 chunks each get a rotation with that property.
template <int NCH>
__device__ __forceinline__ int chunk_rot(int t) {
  if constexpr (NCH % 8 == 0) return ((t >> 2) & 3) + 4 * ((t >> 1) & 1);
  else return (t & 15) >> 2;
}

template <int NCH>
__device__ __forceinline__ int lds_chunk_offset(int t, int c) {
  int pos = c + chunk_rot<NCH>(t);
  if (pos >= NCH) pos -= NCH;
  return (t * NCH + pos) * 16;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16*lane.
// Issued through asm so that the compiler does not add a conservative wait for
// the whole queue before LDS reads; the kernel waits on vmcnt itself. Every cache
// row is read once per call, so the loads carry the non-temporal hint (nt): the
// streaming-bound shapes run 7-12% faster with it, the others unchanged.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off nt"
      :
      : "v"(gaddr), "s"(lds_addr)
      : "memory", "m0");
}

// A split's partial state is written once and read once, by the merge kernel. Its stores carry
// the system-scope bits (sc0 sc1), which write through L2 to memory instead of leaving dirty lines
// for the end-of-kernel write-back: the attention kernel runs 0.3-2.5% faster with them. The
// same bits on compiler-visible buffer stores measured 1% slower on MLRA-4, so they are asm.
// Two hazards that the compiler's hazard recognizer handles for its own stores are then ours:
// - a VALU write of the data registers of a store wider than 8 bytes needs one wait state after
//   the store; the block holds it (s_nop 0);
// - a memory instruction that reads an MFMA result needs several wait states after the MFMA.
//   These helpers therefore store only values written by VALU instructions (the phase merge's
//   arithmetic); MFMA accumulators go out through ordinary stores.
// vmcnt only ever over-counts for asm stores (see dma16).
__device__ __forceinline__ void store_through4(float* dst, float a, float b, float c, float d) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v v = {a, b, c, d};
  asm volatile(
      "global_store_dwordx4 %0, %1, off sc0 sc1\n\t"
      "s_nop 0"
      :
      : "v"(dst), "v"(v)
      : "memory");
}

__device__ __forceinline__ void store_through2(float* dst, float a, float b) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v v = {a, b};
  asm volatile("global_store_dwordx2 %0, %1, off sc0 sc1" : : "v"(dst), "v"(v) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait until at most `ahead` (<= MAXA) stages of `PER` DMA instructions each are outstanding.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_dma(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) {
      wait_vmcnt<PER * MAXA>();
      return;
    }
    wait_dma<PER, MAXA - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" : : : "memory"); }

// f(std::integral_constant<int, v>) for the runtime value v in [0, N): a wave-uniform branch
// to code in which v is a compile-time constant (so register arrays are indexed statically).
template <int N, class F>
__device__ __forceinline__ void static_phase(int v, F&& f) {
  if constexpr (N > 0) {
    if (v == N - 1) f(std::integral_constant<int, N - 1>{});
    else static_phase<N - 1>(v, f);
  }
}

// Max and sum of the values held by lanes l and l ^ 32 (the two lanes holding the two
// 16-token halves of one head's column). v_permlane32_swap with the same register as both
// operands leaves x[l] in one result and x[l ^ 32] in the other, in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


template <int NB, int DB, int DR, int HEADS, int W, bool PAGED, int BPW>
__global__ __launch_bounds__(W * 64, 1) void attn_mfma_kernel(AttnParams p) {
  using C = Cfg<NB, DB, DR, HEADS, W, PAGED, BPW>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  int* ptab = reinterpret_cast<int*>(smem + C::LDS_BYTES - C::PTAB_BYTES);

  const int beta = blockIdx.y;
  const int split = blockIdx.x;
  int L = p.seq_lens[beta];
  if (L < 1 || L > p.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && p.error_flags) atomicOr(p.error_flags, 1u);
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  }
  const int t0 = split * p.split_tokens;
  if (t0 >= L) return;
  const int t1 = min(L, t0 + p.split_tokens);
  const int nst = (t1 - t0 + C::ST - 1) / C::ST;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bg = wave / C::WPB;     // branch group: branches bg * BPW ... bg * BPW + BPW - 1
  const int wr = wave % C::WPB;
  const int hgslot = wr % C::HGSPLIT;
  const int phase = wr / C::HGSPLIT;
  const int g = lane >> 5;          // lane half
  const int n32 = lane & 31;        // head within a group / token within a sub-tile

  // ---- paged: this split's page ids, in LDS or in registers (lane l of register k holds
  // page first_page + 64 k + l) ---------------------------------------------------------------
  int first_page = 0;
  int preg = 0;
  if constexpr (PAGED) {
    first_page = t0 >> p.page_shift;
    const int npages = ((t1 - 1) >> p.page_shift) - first_page + 1;
    auto checked = [&](int pg) __attribute__((always_inline)) {
      if (pg < 0 || pg >= p.num_pages) {
        if (p.error_flags) atomicOr(p.error_flags, 2u);
        pg = 0;
      }
      return pg;
    };
    if constexpr (C::PAGE_REGS) {
      // a split spans at most kPageLanes pages (the host sizes splits so)
      if (lane < npages) preg = checked(p.page_table[(int64_t)beta * p.max_pages + first_page + lane]);
    } else {
      for (int i = tid; i < npages; i += C::THREADS) ptab[i] = checked(p.page_table[(int64_t)beta * p.max_pages + first_page + i]);
      __syncthreads();
    }
  }
  // the page id of the split's page pi (< kPageLanes): the same pi in every lane (one register
  // read) or one pi per lane (a cross-lane permute)
  auto page_uniform = [&](int pi) __attribute__((always_inline)) -> int { return __builtin_amdgcn_readlane(preg, pi); };
  auto page_lane = [&](int pi) __attribute__((always_inline)) -> int {
    return __builtin_amdgcn_ds_bpermute(pi << 2, preg);
  };

  // ---- DMA lane plan (stage-invariant) --------------------------------------------------
  // wave w < DW issues the stage's DMA instructions w, w + DW, w + 2 DW, ...; the first
  // DMA_SPLIT waves have one more than the others. Instruction i of this wave moves
  // 16-byte LDS slot f = (w + DW i) * 64 + lane: token f / NCH of the stage, chunk
  // position f % NCH, i.e. cache chunk (position - rotation) mod NCH.
  const int ndma = wave >= C::DW ? 0 : (wave < C::DMA_SPLIT ? C::DMA_HI : C::DMA_LO);
  struct DmaLane {
    int tok;
    int chunk;
  };
  // the stage's DMA instruction that this wave's i-th one is: interleaved over the waves, or
  // (page ids in registers) blocked, wave w moving tokens [w TPW, (w + 1) TPW) of the stage
  auto dma_index = [&](int i) __attribute__((always_inline)) -> int {
    return C::PAGE_REGS ? wave * C::DMA_HI + i : min(wave + C::DW * i, C::DMA_PER_STAGE - 1);
  };
  auto dma_lane = [&](int i, int ln) __attribute__((always_inline)) -> DmaLane {
    const int f = dma_index(i) * 64 + ln;
    const int t = f / C::NCH;
    int c = f - t * C::NCH - chunk_rot<C::NCH>(t);
    if (c < 0) c += C::NCH;
    return {t, c};
  };
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char*)(smem);
  const char* seq_lat = p.kv_lat + (PAGED ? 0 : (int64_t)beta * p.seq_stride_b);
  const char* seq_rope = p.kv_rope + (PAGED ? 0 : (int64_t)beta * p.seq_stride_b);
  // Per-lane source pointers of full stages. Contiguous: the lane's row of stage 0
  // of this split (later stages add s * ST rows). Paged: the lane's row inside its
  // page (the page base is added per stage).
  const int pmask = PAGED ? (1 << p.page_shift) - 1 : 0;
  const bool big_pages = PAGED && (1 << p.page_shift) > C::ST;
  auto chunk_src = [&](int c) __attribute__((always_inline)) -> const char* {
    return c >= C::NCL ? seq_rope + (c - C::NCL) * 16 : seq_lat + c * 16;
  };
  // Paged, pages of at most one stage: `pid_addr` = LDS byte address of the lane's page-id
  // slot for the split's first stage (a stage adds a uniform offset). The page size in bytes
  // is below 2^32 (checked on the host), so a page's offset is one 32 x 32 -> 64-bit product.
  const char* dptr[C::DMA_HI];
  uint32_t pid_addr[C::DMA_HI];
  const uint32_t ptab_lds = (uint32_t)(uintptr_t)(lds_char*)(smem + C::LDS_BYTES - C::PTAB_BYTES);
#pragma unroll
  for (int i = 0; i < C::DMA_HI; ++i) {
    const DmaLane d = dma_lane(i, lane);
    const char* sel = chunk_src(d.chunk);
    if constexpr (C::PAGE_REGS) {
      dptr[i] = sel + (int64_t)(d.tok - wave * C::TPW) * p.row_stride_b;   // row inside the wave's block
      pid_addr[i] = 0;
    } else if constexpr (PAGED) {
      const int rin = big_pages ? d.tok : (d.tok & pmask);
      dptr[i] = sel + (int64_t)rin * p.row_stride_b;
      pid_addr[i] = ptab_lds + 4u * (uint32_t)(big_pages ? 0 : (d.tok >> p.page_shift));
    } else {
      dptr[i] = sel + (int64_t)(t0 + d.tok) * p.row_stride_b;
      pid_addr[i] = 0;
    }
  }
  const int64_t page_bytes = PAGED ? ((int64_t)1 << p.page_shift) * p.row_stride_b : 0;
  const uint32_t page_bytes32 = (uint32_t)page_bytes;
  const int64_t stage_bytes_g = (int64_t)C::ST * p.row_stride_b;

  // Full stage s of the split holds cache stage (s + rot) mod nrot (set below for long splits;
  // the identity otherwise); a ragged last stage stays last.
  int rot = 0, nrot = 1;
  auto issue_stage = [&](int s) __attribute__((always_inline)) {
    const int ps = s < nrot ? (s + rot) % nrot : s;
    const int tok0 = t0 + ps * C::ST;
    const uint32_t ring = smem_lds + (uint32_t)((s % C::NS) * C::STAGE_BYTES);
    if (tok0 + C::ST <= t1) {
      // full stage: one pointer add (and for small pages one LDS page-id read) per DMA
      const uint32_t slot0 = ring + (uint32_t)(wave * 1024);
      if constexpr (C::PAGE_REGS) {
        // this wave's TPW tokens lie in one page (pages hold at least TPW tokens, checked on the
        // host): one uniform page id and one uniform offset for all its DMAs
        const int tw = tok0 + wave * C::TPW;
        const int pg = page_uniform((tw >> p.page_shift) - first_page);
        const int64_t off = (int64_t)((uint64_t)(uint32_t)pg * page_bytes32) + (int64_t)(tw & pmask) * p.row_stride_b;
#pragma unroll
        for (int i = 0; i < C::DMA_HI; ++i)
          dma16(dptr[i] + off, __builtin_amdgcn_readfirstlane(ring + (uint32_t)(dma_index(i) * 1024)));
      } else if constexpr (PAGED) {
        if (big_pages) {
          // one page holds the whole stage: a uniform offset
          const int pg = __builtin_amdgcn_readfirstlane(ptab[(tok0 >> p.page_shift) - first_page]);
          const int64_t off = (int64_t)((uint64_t)(uint32_t)pg * page_bytes32) + (int64_t)(tok0 & pmask) * p.row_stride_b;
#pragma unroll
          for (int i = 0; i < C::DMA_HI; ++i) {
            if (i >= ndma) break;
            dma16(dptr[i] + off, __builtin_amdgcn_readfirstlane(slot0 + (uint32_t)(C::DW * i * 1024)));
          }
        } else {
          // all page ids first (the DMA asm is a compiler barrier for LDS reads), then the DMAs
          const uint32_t pid_off = 4u * (uint32_t)((tok0 - t0) >> p.page_shift);
          int pg[C::DMA_HI];
#pragma unroll
          for (int i = 0; i < C::DMA_HI; ++i) pg[i] = *(const lds_cint*)(uintptr_t)(pid_addr[i] + pid_off);
#pragma unroll
          for (int i = 0; i < C::DMA_HI; ++i) {
            if (i >= ndma) break;
            dma16(dptr[i] + (uint64_t)(uint32_t)pg[i] * page_bytes32,
                  __builtin_amdgcn_readfirstlane(slot0 + (uint32_t)(C::DW * i * 1024)));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::DMA_HI; ++i) {
          if (i >= ndma) break;
          dma16(dptr[i] + (int64_t)ps * stage_bytes_g, __builtin_amdgcn_readfirstlane(slot0 + (uint32_t)(C::DW * i * 1024)));
        }
      }
    } else {
      // ragged last stage: rows past the end repeat the last row (finite data, masked later).
      // The source is the lane's full-stage pointer moved to the wanted row, and the lane's
      // token is recomputed here from an opaque copy of the lane index, so that nothing of
      // this once-per-split path stays live (or spills) through the main loop.
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int i = 0; i < C::DMA_HI; ++i) {
        if (i >= ndma) break;
        const DmaLane d = dma_lane(i, ln);
        const int tok = min(tok0 + d.tok, t1 - 1);
        int64_t row, row_of_dptr;
        if constexpr (C::PAGE_REGS) {
          const int pg = page_lane((tok >> p.page_shift) - first_page);
          row = ((int64_t)pg << p.page_shift) | (tok & pmask);
          row_of_dptr = d.tok - wave * C::TPW;
        } else if constexpr (PAGED) {
          const int pg = ptab[(tok >> p.page_shift) - first_page];
          row = ((int64_t)pg << p.page_shift) | (tok & pmask);
          row_of_dptr = big_pages ? d.tok : (d.tok & pmask);
        } else {
          row = tok;
          row_of_dptr = t0 + d.tok;
        }
        const char* src = dptr[i] + (row - row_of_dptr) * p.row_stride_b;
        dma16(src, __builtin_amdgcn_readfirstlane(ring + (uint32_t)(dma_index(i) * 1024)));
      }
    }
  };

  // ---- queries: B operands (exact bf16 values) ---------------------------------------------
  // The sequence's queries (q_lat then q_rope, HEADS x (d_c + d_R) bf16) are copied into the
  // last ring slot by LDS-DMA together with stage 0, and every wave reads its operands from
  // there right after the first barrier. Through the DMA their arrival is covered by the
  // kernel's own vmcnt accounting; loaded into registers directly, the compiler would wait for
  // every outstanding load (the stages in flight included) before the first score MFMA.
  bf16x8 qr[C::HPW][C::KR];
  bf16x8 ql[C::HPW][BPW][C::KL];
  const uint32_t q_lds = smem_lds + (uint32_t)((C::NS - 1) * C::STAGE_BYTES);
  auto issue_queries = [&]() __attribute__((always_inline)) {
    const char* ql_src = reinterpret_cast<const char*>(p.q_lat) + (int64_t)beta * C::QL_BYTES;
    const char* qr_src = reinterpret_cast<const char*>(p.q_rope) + (int64_t)beta * C::QR_BYTES;
    for (int i = wave; i < C::QL_DMA; i += C::WAVES)
      if (i * 64 + lane < C::QL_BYTES / 16)
        dma16(ql_src + (i * 64 + lane) * 16, __builtin_amdgcn_readfirstlane(q_lds + (uint32_t)(i * 1024)));
    for (int i = wave; i < C::QR_DMA; i += C::WAVES)
      if (i * 64 + lane < C::QR_BYTES / 16)
        dma16(qr_src + (i * 64 + lane) * 16,
              __builtin_amdgcn_readfirstlane(q_lds + (uint32_t)(C::QL_DMA * 1024 + i * 1024)));
  };
  auto read_queries = [&]() __attribute__((always_inline)) {
    const lds_char* qb = (const lds_char*)smem + (C::NS - 1) * C::STAGE_BYTES;
#pragma unroll
    for (int h = 0; h < C::HPW; ++h) {
      const int head = (hgslot * C::HPW + h) * 32 + n32;
      const bool live = head < HEADS;
#pragma unroll
      for (int k = 0; k < C::KR; ++k)
        qr[h][k] = live ? *(const lds_bf16x8*)(qb + C::QL_DMA * 1024 + (head * DR + 16 * k + 8 * g) * 2) : bf16x8{};
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb)
#pragma unroll
        for (int k = 0; k < C::KL; ++k)
          ql[h][bb][k] = live ? *(const lds_bf16x8*)(qb + ((head * NB + bg * BPW + bb) * DB + 16 * k + 8 * g) * 2)
                              : bf16x8{};
    }
  };

  // ---- per-lane LDS offsets inside a sub-tile -------------------------------------------
  int off_r[C::KR], off_l[BPW][C::KL], off_v[BPW][C::MT][2];
#pragma unroll
  for (int k = 0; k < C::KR; ++k) off_r[k] = lds_chunk_offset<C::NCH>(n32, C::NCL + 2 * k + g);
  {
    const int q4 = lane >> 4, jj = lane & 15;
    const int tt = 4 * (q4 >> 1) + (jj >> 2);                        // token within an 8-token half
    // score operand: chunk 2k + g of branch br for token n32; value operand: the 8-byte word
    // of feature f for tokens tt and tt + 8 (whose rotation is 2 larger)
    const int lat0 = lds_chunk_offset<C::NCH>(n32, bg * BPW * (DB / 8) + g);
    const int f0 = bg * BPW * DB + 16 * (q4 & 1) + 4 * (jj & 3);
    const int val0 = lds_chunk_offset<C::NCH>(tt, f0 >> 3) + (f0 & 7) * 2;
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
      const int br = bg * BPW + bb;
#pragma unroll
      for (int k = 0; k < C::KL; ++k)
        off_l[bb][k] = C::LAT_FLAT ? lat0 + (bb * (DB / 8) + 2 * k) * 16
                                   : lds_chunk_offset<C::NCH>(n32, br * (DB / 8) + 2 * k + g);
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const int f = br * DB + 32 * mt + 16 * (q4 & 1) + 4 * (jj & 3); // feature of this lane's 8-byte word
#pragma unroll
        for (int r = 0; r < 2; ++r)
          off_v[bb][mt][r] = C::LAT_FLAT ? val0 + (bb * (DB / 8) + 4 * mt) * 16 + r * (8 * C::NCH * 16 + 2 * 16)
                                         : lds_chunk_offset<C::NCH>(tt + 8 * r, f >> 3) + (f & 7) * 2;
      }
    }
  }

  // ---- running state ---------------------------------------------------------------------
  f32x16 acc[C::HPW][BPW][C::MT];
  float mref[C::HPW][BPW], lsum[C::HPW][BPW];
  bool started[C::HPW][BPW];
  const float qs = p.q_scale;       // tau * log2(e) > 0
#pragma unroll
  for (int h = 0; h < C::HPW; ++h)
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) acc[h][bb][mt] = f32x16{};
      mref[h][bb] = -INFINITY;
      lsum[h][bb] = 0.f;
      started[h][bb] = false;
    }
  const s16x4 ones4 = {0x3f80, 0x3f80, 0x3f80, 0x3f80};

  // ---- per-sub-tile building blocks ------------------------------------------------------
  // Scores of one 32-token sub-tile for every head group and branch of this wave (raw
  // units). The RoPE part is the same for every branch: it is accumulated once into the
  // first branch's tile, whose value then seeds (as the C operand) the latent chains of
  // the other branches before the first branch continues its own.
  auto scores = [&](const lds_char* sub, f32x16 (&sc)[C::HPW][BPW]) __attribute__((always_inline)) {
    bf16x8 ar[C::KR], al[BPW][C::KL];
#pragma unroll
    for (int k = 0; k < C::KR; ++k) ar[k] = *(const lds_bf16x8*)(sub + off_r[k]);
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb)
#pragma unroll
      for (int k = 0; k < C::KL; ++k) al[bb][k] = *(const lds_bf16x8*)(sub + off_l[bb][k]);
#pragma unroll
    for (int h = 0; h < C::HPW; ++h) {
      sc[h][0] = f32x16{};
#pragma unroll
      for (int k = 0; k < C::KR; ++k)
        sc[h][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[k], qr[h][k], sc[h][0], 0, 0, 0);
#pragma unroll
      for (int bb = 1; bb < BPW; ++bb) {
        sc[h][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[bb][0], ql[h][bb][0], sc[h][0], 0, 0, 0);
#pragma unroll
        for (int k = 1; k < C::KL; ++k)
          sc[h][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[bb][k], ql[h][bb][k], sc[h][bb], 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < C::KL; ++k)
        sc[h][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[0][k], ql[h][0][k], sc[h][0], 0, 0, 0);
    }
  };
  // transposed latent block [feature x token] of one sub-tile and branch: two 4-token
  // halves per K-chunk
  auto values_a = [&](const lds_char* sub, int bb, bf16x8 (&av)[2][C::MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) {
        const lds_char* a0 = sub + off_v[bb][mt][0] + (16 * kc) * C::NCH * 16;
        const lds_char* a1 = sub + off_v[bb][mt][1] + (16 * kc) * C::NCH * 16;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
        bf16x4 blo = __builtin_bit_cast(bf16x4, lo), bhi = __builtin_bit_cast(bf16x4, hi);
        av[kc][mt] = bf16x8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
      }
    }
  };
  // lazy running max: move the reference only when a logit exceeds it by more than the threshold
  auto maybe_rescale = [&](int h, int bb, float mx) __attribute__((always_inline)) {
    const float xm = fmaf(mx, qs, -mref[h][bb]);
    if (__builtin_amdgcn_ballot_w64(xm > kRescaleThreshold) != 0) {
      const float d = fmaxf(halves_max(xm), 0.f);
      const float f = __builtin_amdgcn_exp2f(-d);
      mref[h][bb] += d;
      lsum[h][bb] *= f;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) acc[h][bb][mt] *= f;
    }
  };
  // p = 2^(x - m) packed to bf16; returns ls + the sum of the packed weights
  // p = 2^(x - m) packed to bf16; returns ls + the sum of the packed weights. The sum runs on
  // the matrix pipe, which has room to spare, instead of the vector ALUs, which bound the loop:
  // a 4x4x4 MFMA whose A operand is all ones leaves in each lane the sum of the four bf16
  // weights that lane holds in its B operand, so the normaliser sums exactly the weights the
  // P.C product uses.
  auto weights = [&](int h, int bb, const f32x16& x, bf16x2 (&pk)[8], float ls) __attribute__((always_inline)) -> float {
    const float negm = -mref[h][bb];
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      f32x2 e = {__builtin_amdgcn_exp2f(fmaf(x[2 * k], qs, negm)), __builtin_amdgcn_exp2f(fmaf(x[2 * k + 1], qs, negm))};
      pk[k] = __builtin_convertvector(e, bf16x2);
      if (k & 1) {
        const s16x4 b = __builtin_bit_cast(s16x4, bf16x4{pk[k - 1][0], pk[k - 1][1], pk[k][0], pk[k][1]});
        d = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones4, b, d, 0, 0, 0);
      }
    }
    return ls + d[0];
  };
  // O += P.C for one sub-tile and branch, reading the transposed latent one 32-feature tile at a time
  auto pv_lds = [&](int h, int bb, const bf16x2 (&pk)[8], const lds_char* sub) __attribute__((always_inline)) {
    bf16x8 pb[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
      pb[kc] = bf16x8{pk[4 * kc][0], pk[4 * kc][1], pk[4 * kc + 1][0], pk[4 * kc + 1][1],
                      pk[4 * kc + 2][0], pk[4 * kc + 2][1], pk[4 * kc + 3][0], pk[4 * kc + 3][1]};
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const lds_char* a0 = sub + off_v[bb][mt][0] + (16 * kc) * C::NCH * 16;
        const lds_char* a1 = sub + off_v[bb][mt][1] + (16 * kc) * C::NCH * 16;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
        bf16x4 blo = __builtin_bit_cast(bf16x4, lo), bhi = __builtin_bit_cast(bf16x4, hi);
        const bf16x8 a = bf16x8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
        acc[h][bb][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], acc[h][bb][mt], 0, 0, 0);
      }
    }
  };
  // O += P.C for one sub-tile and branch
  auto pv = [&](int h, int bb, const bf16x2 (&pk)[8], const bf16x8 (&av)[2][C::MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 pb = {pk[4 * kc][0], pk[4 * kc][1], pk[4 * kc + 1][0], pk[4 * kc + 1][1],
                   pk[4 * kc + 2][0], pk[4 * kc + 2][1], pk[4 * kc + 3][0], pk[4 * kc + 3][1]};
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        acc[h][bb][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kc][mt], pb, acc[h][bb][mt], 0, 0, 0);
    }
  };
  auto accumulate = [&](int h, int bb, const f32x16& x, const bf16x8 (&av)[2][C::MT]) __attribute__((always_inline)) {
    bf16x2 pk[8];
    lsum[h][bb] = weights(h, bb, x, pk, lsum[h][bb]);
    pv(h, bb, pk, av);
  };

  // ---- stages ------------------------------------------------------------------------------
  auto stage_ptr = [&](int s) __attribute__((always_inline)) { return (const lds_char*)smem + (s % C::NS) * C::STAGE_BYTES; };
  // ragged last stage (possibly also the first): one sub-tile at a time, masking tokens past the end
  auto slow_stage = [&](int s) __attribute__((always_inline)) {
    const int stage_tok0 = t0 + s * C::ST;
    const lds_char* stage = stage_ptr(s);
#pragma unroll
    for (int u = 0; u < C::SUB; ++u) {
      if (u % C::P != phase) continue;
      const int valid = t1 - (stage_tok0 + 32 * u);
      if (valid <= 0) continue;
      const lds_char* sub = stage + u * C::SUB_BYTES;
      f32x16 sc[C::HPW][BPW];
      scores(sub, sc);
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb) {
        bf16x8 av[2][C::MT];
        values_a(sub, bb, av);
#pragma unroll
        for (int h = 0; h < C::HPW; ++h) {
          f32x16& x = sc[h][bb];
          if (valid < 32) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int tok = 8 * (r >> 2) + 4 * g + (r & 3);
              if (tok >= valid) x[r] = -INFINITY;
            }
          }
          float mx = x[0];            // raw units (scale > 0 keeps the order)
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
          if (!started[h][bb]) {
            mref[h][bb] = halves_max(mx) * qs;
            started[h][bb] = true;
          } else {
            maybe_rescale(h, bb, mx);
          }
          accumulate(h, bb, x, av);
        }
      }
    }
  };

  // ---- main loop: full stages (the first seeds the running max), ragged last stage ----------
  const int nfull = (t1 - t0) / C::ST;       // stages with ST valid tokens
  // Long splits stream their full stages from a per-sequence starting stage (37 beta mod n).
  // Sequences whose caches lie a large power-of-two multiple apart otherwise read in lockstep
  // and collide in the same HBM channels: the 16-head MLA shard (64 sequences of 20 MiB, four
  // 5 MiB splits each) ran 229 -> 197 us. On 16-stage splits the rotation cost 2-3%, so only
  // long splits rotate. The sum over a split's tokens is order-dependent only in rounding.
  if (nfull >= kRotateStages) {
    nrot = nfull;
    rot = (int)(((unsigned)beta * 37u) % (unsigned)nfull);
  }
  // With one branch per wave the loop is software-pipelined over this wave's sub-tiles
  // k = 0, 1, ... of the full stages: the score MFMAs of sub-tile k + 1 are issued before
  // the softmax of sub-tile k, so the matrix cores work while the vector ALUs
  // exponentiate. A ring slot is still read by the lagging P.C of its last sub-tile after
  // the next stage's barrier, so the refill at stage s's barrier targets the slot of stage
  // s - 2: LOOK = NS - 2 stages ahead. Without the pipelining every wave is done with stage
  // s - 1 when it passes stage s's barrier, so any slot but stage s's may be refilled; two
  // stages ahead measured best there (three ahead was slower on a 4-stage ring, one ahead
  // much slower on a 3-stage ring).
  constexpr int LOOK = (C::PIPE || C::PIPE2) ? C::NS - 2 : 2;
  // stage 0 first, then the queries (into the last ring slot, which the prologue's stages do
  // not use: LOOK <= NS - 1), then the rest of the prologue's stages
  static_assert(LOOK <= C::NS - 1, "the prologue leaves the query slot free");
  issue_stage(0);
  issue_queries();
  // The rest of the prologue goes out once all but three fifths of a stage's worth of this
  // wave's DMAs have landed: stage 0 has the memory to itself for a while and lands sooner,
  // and stage 1 is still in flight well before it is needed (attention kernel -1.7% headline,
  // -1.4% paged, -0.9% MLA; issued only after stage 0's barrier, stage 1 arrived late).
  constexpr int kHeadStart = (3 * C::DMA_HI) / 5 >= 1 ? (3 * C::DMA_HI) / 5 : 1;
  if (1 < LOOK && 1 < nst) wait_vmcnt<kHeadStart>();
  for (int s = 1; s < LOOK && s < nst; ++s) issue_stage(s);
  // Wait for stage s (the queries with stage 0: they went out before stage 1), barrier, refill
  // LOOK stages ahead. At s = 0 the waves first read their query operands from the last ring
  // slot and wait for those reads, since the refill may target that slot.
  auto begin_piped = [&](int s) __attribute__((always_inline)) {
    const int ahead = min(nst - 1 - s, LOOK - 1);
    if (ndma == C::DMA_HI) wait_dma<C::DMA_HI, LOOK - 1>(ahead);
    else wait_dma<C::DMA_LO, LOOK - 1>(ahead);
    block_barrier();
    if (s == 0) {
      read_queries();
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    }
    if (s + LOOK < nst) issue_stage(s + LOOK);
  };
  auto sub_of = [&](int k) __attribute__((always_inline)) {
    return stage_ptr(k / C::NSW) + ((k % C::NSW) * C::P + phase) * C::SUB_BYTES;
  };
  const int K = nfull * C::NSW;
  // softmax and P.C of sub-tile k from its scores
  auto consume = [&](int k, f32x16 (&cur)[C::HPW][BPW]) __attribute__((always_inline)) {
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb)
#pragma unroll
      for (int h = 0; h < C::HPW; ++h) {
        bf16x2 pk[8];
        float ls = weights(h, bb, cur[h][bb], pk, 0.f);
        if (__builtin_amdgcn_ballot_w64(!(ls <= kStageSumMax)) != 0) {
          float mx = cur[h][bb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, cur[h][bb][r]);
          maybe_rescale(h, bb, mx);
          ls = weights(h, bb, cur[h][bb], pk, 0.f);
        }
        lsum[h][bb] += ls;
        pv_lds(h, bb, pk, sub_of(k));
      }
  };
  // the reference starts at the exact max of the first sub-tile
  auto seed = [&](f32x16 (&sc)[C::HPW][BPW]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < C::HPW; ++h)
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb) {
        float mx = sc[h][bb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[h][bb][r]);
        mref[h][bb] = halves_max(mx) * qs;
        started[h][bb] = true;
      }
  };
  if (K > 0) {
    if constexpr (C::PIPE2) {
      // softmax of every (head group, branch) of sub-tile k; one vote decides whether any
      // lane's weights summed past the threshold (then the reference moves and the weights
      // of that unit are recomputed)
      // weights of every (head group, branch) of sub-tile k; true if any lane's weights
      // summed past the threshold
      auto soft_weights = [&](f32x16 (&cur)[C::HPW][BPW], bf16x2 (&pk)[C::HPW][BPW][8],
                              float (&ls)[C::HPW][BPW]) __attribute__((always_inline)) -> bool {
        bool over = false;
#pragma unroll
        for (int h = 0; h < C::HPW; ++h)
#pragma unroll
          for (int bb = 0; bb < BPW; ++bb) {
            ls[h][bb] = weights(h, bb, cur[h][bb], pk[h][bb], 0.f);
            over |= !(ls[h][bb] <= kStageSumMax);
          }
        return over;
      };
      // one vote decides whether any unit needs the rare path: its reference moves to the
      // exact max and its weights are recomputed
      auto soft_finish = [&](bool over, f32x16 (&cur)[C::HPW][BPW], bf16x2 (&pk)[C::HPW][BPW][8],
                             float (&ls)[C::HPW][BPW]) __attribute__((always_inline)) {
        if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
          for (int h = 0; h < C::HPW; ++h)
#pragma unroll
            for (int bb = 0; bb < BPW; ++bb) {
              if (__builtin_amdgcn_ballot_w64(!(ls[h][bb] <= kStageSumMax)) != 0) {
                float mx = cur[h][bb][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, cur[h][bb][r]);
                maybe_rescale(h, bb, mx);
                ls[h][bb] = weights(h, bb, cur[h][bb], pk[h][bb], 0.f);
              }
            }
        }
#pragma unroll
        for (int h = 0; h < C::HPW; ++h)
#pragma unroll
          for (int bb = 0; bb < BPW; ++bb) lsum[h][bb] += ls[h][bb];
      };
      auto soft = [&](f32x16 (&cur)[C::HPW][BPW], bf16x2 (&pk)[C::HPW][BPW][8]) __attribute__((always_inline)) {
        float ls[C::HPW][BPW];
        soft_finish(soft_weights(cur, pk, ls), cur, pk, ls);
      };
      auto pv_all = [&](int k, const bf16x2 (&pk)[C::HPW][BPW][8]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < C::HPW; ++h)
#pragma unroll
          for (int bb = 0; bb < BPW; ++bb) pv_lds(h, bb, pk[h][bb], sub_of(k));
      };
      // Sub-tile k: the scores of k + 1 (NXT) and the P.C of k - 1 (PREV, weights in pkp) go
      // out with the softmax of k, in one block that the scheduler interleaves, so the
      // matrix cores work while the vector ALUs do. The P.C of k - 1 precedes any rescale
      // made by the softmax of k, which therefore scales it with the rest of the
      // accumulator. BOUNDARY: sub-tile k + 1 opens a stage (wait, barrier, refill first).
      auto step2 = [&](auto nxt_c, auto prev_c, auto boundary_c, int k, f32x16 (&cur)[C::HPW][BPW],
                       f32x16 (&nxt)[C::HPW][BPW], bf16x2 (&pkc)[C::HPW][BPW][8],
                       bf16x2 (&pkp)[C::HPW][BPW][8]) __attribute__((always_inline)) {
        constexpr bool NXT = decltype(nxt_c)::value, PREV = decltype(prev_c)::value;
        // The two waves of a SIMD (branch groups 0 and 1) meet at every stage barrier. The
        // sequencer issues the older wave first, so the younger one used to finish its stage
        // alone; raising its priority for the stage's first step and levelling it for the
        // second lets both end together (1.6% per headline call, 0.7% paged).
        if constexpr (decltype(boundary_c)::value) {
          if (bg == 1) __builtin_amdgcn_s_setprio(1);
          else __builtin_amdgcn_s_setprio(0);
        } else {
          __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (NXT && decltype(boundary_c)::value) begin_piped((k + 1) / C::NSW);
        if constexpr (NXT) scores(sub_of(k + 1), nxt);
        if constexpr (PREV) pv_all(k - 1, pkp);
        float ls[C::HPW][BPW];
        const bool over = soft_weights(cur, pkc, ls);
        if constexpr (NXT || PREV) {
          // operand reads first, then one matrix instruction per MFMA_GAP vector instructions
          constexpr int NM = (NXT ? C::HPW * (C::KR + BPW * C::KL) : 0) + (PREV ? C::HPW * BPW * 2 * C::MT : 0);
          constexpr int ND = (NXT ? C::KR + BPW * C::KL : 0) + (PREV ? C::HPW * BPW * 2 * C::MT * 2 : 0);
          __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
#pragma unroll
          for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kMfmaGap, 0);
          }
        }
        soft_finish(over, cur, pkc, ls);
      };
      using T_ = std::true_type;
      using F_ = std::false_type;
      static_assert(C::NSW == 2, "the unrolled loop puts a stage boundary after every odd sub-tile");
      begin_piped(0);
      f32x16 sa[C::HPW][BPW], sb[C::HPW][BPW];
      bf16x2 pa[C::HPW][BPW][8], pb[C::HPW][BPW][8];
      scores(sub_of(0), sa);
      seed(sa);
      if (K == 1) {
        soft(sa, pa);
        pv_all(0, pa);
      } else {
        step2(T_{}, F_{}, F_{}, 0, sa, sb, pa, pb);          // k = 0: scores of 1, softmax of 0
        int k = 1;
        for (; k + 2 < K; k += 2) {                          // k odd: sub-tile k + 1 opens a stage
          step2(T_{}, T_{}, T_{}, k, sb, sa, pb, pa);
          step2(T_{}, T_{}, F_{}, k + 1, sa, sb, pa, pb);
        }
        if (K - k == 2) {
          step2(T_{}, T_{}, T_{}, k, sb, sa, pb, pa);
          step2(F_{}, T_{}, F_{}, k + 1, sa, sb, pa, pb);
          pv_all(k + 1, pa);
        } else {
          step2(F_{}, T_{}, F_{}, k, sb, sa, pb, pa);
          pv_all(k, pb);
        }
      }
    } else if constexpr (C::PIPE) {
      // consume the scores `cur` of sub-tile k; first issue the scores of sub-tile k + 1 into `nxt`
      auto step = [&](int k, f32x16 (&cur)[C::HPW][BPW], f32x16 (&nxt)[C::HPW][BPW]) __attribute__((always_inline)) {
        if (k + 1 < K) {
          if ((k + 1) % C::NSW == 0) begin_piped((k + 1) / C::NSW);
          scores(sub_of(k + 1), nxt);
        }
        consume(k, cur);
      };
      begin_piped(0);
      f32x16 sa[C::HPW][BPW], sb[C::HPW][BPW];
      scores(sub_of(0), sa);
      seed(sa);
      for (int k = 0; k < K; k += 2) {
        step(k, sa, sb);
        if (k + 1 < K) step(k + 1, sb, sa);
      }
    } else {
      for (int k = 0; k < K; ++k) {
        if (k % C::NSW == 0) begin_piped(k / C::NSW);
        f32x16 sc[C::HPW][BPW];
        // the score MFMAs stay one block, apart from the DMA issue before and the softmax
        // after (measured about 1% faster than the scheduler's interleaving)
        __builtin_amdgcn_sched_barrier(0);
        scores(sub_of(k), sc);
        __builtin_amdgcn_sched_barrier(0);
        if (k == 0) seed(sc);
        consume(k, sc);
      }
    }
  }
  if (nfull < nst) {
    begin_piped(nst - 1);
    slow_stage(nst - 1);
  }

  // ---- combine halves, merge phases, write this split's partial state -----------------------
#pragma unroll
  for (int h = 0; h < C::HPW; ++h)
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) lsum[h][bb] = halves_sum(lsum[h][bb]);

  // Rows [r0, r0 + nr) of every output tile of this wave, and (with ml) its (m, l), into the
  // split's record. A lane's rows 4j..4j+3 are 4 consecutive features. With `through`, the values
  // were written by VALU instructions and may go out through the write-through asm stores. Only
  // stores that fill whole 32-byte pieces do: a lane pair's 4-row stores, and the (m, l) pairs
  // when there is one branch (then 32 heads' pairs are contiguous). Narrower pieces (2-row
  // stores, (m, l) pairs interleaved by branch) stay in L2, which merges them into lines:
  // written through, each became a partial write of its own (1.5 MB more at the MLRA-4
  // headline; the 16-head MLRA-4 shard +0.4% per call, MLA +1.0% with its pairs held back).
  auto store_rows = [&](int r0, int nr, bool ml, auto through_c) __attribute__((always_inline)) {
    constexpr bool through = decltype(through_c)::value;
    auto put4 = [&](float* dst, float a, float b, float c, float d) __attribute__((always_inline)) {
      if constexpr (through) store_through4(dst, a, b, c, d);
      else *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
    };
    auto put_ml = [&](float* dst, float a, float b) __attribute__((always_inline)) {
      if constexpr (through && NB == 1) store_through2(dst, a, b);
      else *reinterpret_cast<float2*>(dst) = make_float2(a, b);
    };
    if constexpr (NB > 1) {
      // fp16 records, scaled per record by 2^-e with l = f 2^e, f in [0.5, 1); e folds into m
      // (exact: a power of two, and an integer added to m). |o| <= l max|c| keeps them in
      // range. Half the bytes of fp32 records: the attention kernel 2.5-4% and the call about
      // 3% faster (MLRA-4, MLRA-2, paged); the error against the oracle 4.19e-3 -> 4.42e-3 at
      // the headline. The phase owns 4-row groups qa and qa + 1; the lanes l and l + 32 of a
      // head exchange halves (v_permlane32_swap) so that each writes 8 consecutive features
      // (16 bytes, 32 for the lane pair). Ordinary stores: fed from the swap's results, the
      // write-through asm store left corrupt records on MLRA-2, and compiler-made stores, plain
      // or buffer stores with the same bits, measured alike.
      static_assert(C::P == 2, "multi-branch shapes merge two phases");
      typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
      auto pk = [&](float a, float b) __attribute__((always_inline)) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
      };
      const int qa = r0 / 4;
#pragma unroll
      for (int h = 0; h < C::HPW; ++h) {
        const int head = (hgslot * C::HPW + h) * 32 + n32;
        if (head >= p.H) continue;
#pragma unroll
        for (int bb = 0; bb < BPW; ++bb) {
          const int64_t rec = (((int64_t)beta * p.num_splits + split) * p.H + head) * NB + bg * BPW + bb;
          const float l = lsum[h][bb];
          const int e = (int)((__float_as_uint(l) >> 23) & 0xff) - 126;
          const float sc = __uint_as_float((uint32_t)(127 - e) << 23);
          _Float16* o16 = static_cast<_Float16*>(p.ws_o) + rec * DB;
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) {
            const f32x16& v = acc[h][bb][mt];
            const int q = 4 * qa;
            const uint32_t a0 = pk(v[q] * sc, v[q + 1] * sc), a1 = pk(v[q + 2] * sc, v[q + 3] * sc);
            const uint32_t b0 = pk(v[q + 4] * sc, v[q + 5] * sc), b1 = pk(v[q + 6] * sc, v[q + 7] * sc);
            const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
            *reinterpret_cast<uint4*>(o16 + 32 * mt + 8 * qa + 8 * g) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
          }
          if (ml && g == 0)
            *reinterpret_cast<float2*>(p.ws_ml + rec * 2) = make_float2(mref[h][bb] + (float)e, l * sc);
        }
      }
      return;
    } else if constexpr (C::F16REC) {
      // One branch over four phases: the phase owns the 4-row group qa = r0 / 4 of every
      // output tile, 4 consecutive features per lane (8 bytes of fp16; lanes l and l + 32 of a
      // head cover 16 contiguous bytes), scaled per record as above. Ordinary stores.
      static_assert(C::P == 4, "one-branch fp16 records: each phase owns one 4-row group");
      typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
      auto pk = [&](float a, float b) __attribute__((always_inline)) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
      };
      const int qa = r0 / 4;
#pragma unroll
      for (int h = 0; h < C::HPW; ++h) {
        const int head = (hgslot * C::HPW + h) * 32 + n32;
        if (head >= p.H) continue;
#pragma unroll
        for (int bb = 0; bb < BPW; ++bb) {
          const int64_t rec = (((int64_t)beta * p.num_splits + split) * p.H + head) * NB + bg * BPW + bb;
          const float l = lsum[h][bb];
          const int e = (int)((__float_as_uint(l) >> 23) & 0xff) - 126;
          const float sc = __uint_as_float((uint32_t)(127 - e) << 23);
          _Float16* o16 = static_cast<_Float16*>(p.ws_o) + rec * DB;
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt) {
            const f32x16& v = acc[h][bb][mt];
            const int q = 4 * qa;
            *reinterpret_cast<uint2*>(o16 + 32 * mt + 8 * qa + 4 * g) =
                make_uint2(pk(v[q] * sc, v[q + 1] * sc), pk(v[q + 2] * sc, v[q + 3] * sc));
          }
          if (ml && g == 0)
            *reinterpret_cast<float2*>(p.ws_ml + rec * 2) = make_float2(mref[h][bb] + (float)e, l * sc);
        }
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < C::HPW; ++h) {
      const int head = (hgslot * C::HPW + h) * 32 + n32;
      if (head >= p.H) continue;
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb) {
        const int64_t rec = (((int64_t)beta * p.num_splits + split) * p.H + head) * NB + bg * BPW + bb;
        float* o = static_cast<float*>(p.ws_o) + rec * DB;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
          if (nr >= 4) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              if (q4 < r0 / 4 || q4 >= (r0 + nr) / 4) continue;
              put4(o + 32 * mt + 8 * q4 + 4 * g, acc[h][bb][mt][4 * q4], acc[h][bb][mt][4 * q4 + 1],
                   acc[h][bb][mt][4 * q4 + 2], acc[h][bb][mt][4 * q4 + 3]);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              if (r != r0) continue;
              *reinterpret_cast<float2*>(o + 32 * mt + 8 * (r / 4) + 4 * g + (r % 4)) =
                  make_float2(acc[h][bb][mt][r], acc[h][bb][mt][r + 1]);
            }
          }
        }
        if (ml && g == 0) put_ml(p.ws_ml + rec * 2, mref[h][bb], lsum[h][bb]);
      }
    }
  };

  if constexpr (C::P > 1) {
    // The P phase waves of a (branch group, head group) merge their states through LDS, each
    // finalising 16 / P of the 16 rows a lane holds per output tile, and write those rows.
    constexpr int RP = 16 / C::P;
    static_assert(16 % C::P == 0 && RP >= 2, "phases split a lane's 16 output rows");
    block_barrier();   // every wave is done with the ring; reuse it for the merge records
    float* rec = reinterpret_cast<float*>(smem);
    constexpr int RECF = (16 * C::MT + 2) * 64;     // floats of one (head group, branch) record
    auto slot_of = [&](int q) __attribute__((always_inline)) { return bg * C::WPB + q * C::HGSPLIT + hgslot; };
    // 1. publish the rows the other phases finalise, and (m, l)
    auto publish = [&](auto pc) __attribute__((always_inline)) {
      constexpr int R0 = decltype(pc)::value * RP;
      float* mine = rec + wave * C::MERGE_FLOATS;
#pragma unroll
      for (int h = 0; h < C::HPW; ++h)
#pragma unroll
        for (int bb = 0; bb < BPW; ++bb) {
          float* d = mine + (h * BPW + bb) * RECF;
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (r < R0 || r >= R0 + RP) d[(16 * mt + r) * 64 + lane] = acc[h][bb][mt][r];
          d[(16 * C::MT) * 64 + lane] = mref[h][bb];
          d[(16 * C::MT + 1) * 64 + lane] = lsum[h][bb];
        }
    };
    // 2. merge this wave's rows over the phases and write them
    auto finish = [&](auto pc) __attribute__((always_inline)) {
      constexpr int PH = decltype(pc)::value;
      constexpr int R0 = PH * RP;
#pragma unroll
      for (int h = 0; h < C::HPW; ++h)
#pragma unroll
        for (int bb = 0; bb < BPW; ++bb) {
          float mq[C::P];
          float mstar = mref[h][bb];
#pragma unroll
          for (int q = 0; q < C::P; ++q) {
            if (q == PH) continue;
            mq[q] = rec[slot_of(q) * C::MERGE_FLOATS + (h * BPW + bb) * RECF + (16 * C::MT) * 64 + lane];
            mstar = fmaxf(mstar, mq[q]);
          }
          // the phases in order 0 .. P-1, whichever wave finalises the rows
          float l = 0.f;
          float o[C::MT][RP];
#pragma unroll
          for (int q = 0; q < C::P; ++q) {
            const float* d = rec + slot_of(q) * C::MERGE_FLOATS + (h * BPW + bb) * RECF;
            const float fq = __builtin_amdgcn_exp2f((q == PH ? mref[h][bb] : mq[q]) - mstar);
            const float lq = q == PH ? lsum[h][bb] : d[(16 * C::MT + 1) * 64 + lane];
            l = q == 0 ? lq * fq : l + lq * fq;
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
              for (int r = 0; r < RP; ++r) {
                const float v = q == PH ? acc[h][bb][mt][R0 + r] : d[(16 * mt + R0 + r) * 64 + lane];
                o[mt][r] = q == 0 ? v * fq : o[mt][r] + v * fq;
              }
          }
#pragma unroll
          for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int r = 0; r < RP; ++r) acc[h][bb][mt][R0 + r] = o[mt][r];
          mref[h][bb] = mstar;
          lsum[h][bb] = l;
        }
      store_rows(R0, RP, PH == 0, std::true_type{});   // merged values: VALU results
    };
    static_phase<C::P>(phase, publish);
    __syncthreads();
    static_phase<C::P>(phase, finish);
  } else {
    store_rows(0, 16, true, std::false_type{});       // the accumulators as the MFMAs left them
  }
}

template <int NB, int DB, int DR, int HEADS, int W, int BPW>
hipError_t launch_shape(const AttnParams& p, bool paged, int grid_splits, hipStream_t stream) {
  dim3 grid(grid_splits, p.B);
  if (paged)
    hipLaunchKernelGGL((attn_mfma_kernel<NB, DB, DR, HEADS, W, true, BPW>), grid, dim3(W * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<NB, DB, DR, HEADS, W, false, BPW>), grid, dim3(W * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Shapes built with the MFMA path: (branches, branch width, RoPE width, heads, waves,
// branches per wave). Two branches per wave share the RoPE score. The contiguous and paged
// instances of a shape split the work identically, so they sum every split's tokens in the
// same order and agree bit for bit.
#define MLRA_MFMA_SHAPES(X)     \
  X(4, 32, 32, 64, 8, 2)        \
  X(1, 128, 32, 64, 8, 1)       \
  X(1, 128, 32, 16, 4, 1)       \
  X(1, 32, 32, 16, 8, 1)        \
  X(1, 32, 32, 64, 8, 1)        \
  X(2, 64, 32, 64, 8, 1)

int mfma_page_cache(int nb, int db, int dr, int heads) {
#define X(xNB, xDB, xDR, xH, xW, xBPW)                                                 \
  if (nb == xNB && db == xDB && dr == xDR && heads == xH)                             \
    return Cfg<xNB, xDB, xDR, xH, xW, true, xBPW>::PAGE_REGS ? kPageLanes : kPageCache;
  MLRA_MFMA_SHAPES(X)
#undef X
  return kPageCache;
}

int mfma_min_page_size(int nb, int db, int dr, int heads) {
#define X(xNB, xDB, xDR, xH, xW, xBPW)                                                 \
  if (nb == xNB && db == xDB && dr == xDR && heads == xH) {                           \
    using CP = Cfg<xNB, xDB, xDR, xH, xW, true, xBPW>;                                \
    return CP::PAGE_REGS ? CP::TPW : 1;                                               \
  }
  MLRA_MFMA_SHAPES(X)
#undef X
  return 1;
}

bool mfma_f16_records(int nb, int db, int dr, int heads) {
#define X(xNB, xDB, xDR, xH, xW, xBPW) \
  if (nb == xNB && db == xDB && dr == xDR && heads == xH) return Cfg<xNB, xDB, xDR, xH, xW, false, xBPW>::F16REC;
  MLRA_MFMA_SHAPES(X)
#undef X
  return false;
}

int mfma_stage_tokens(int nb, int db, int dr, int heads) {
#define X(xNB, xDB, xDR, xH, xW, xBPW) \
  if (nb == xNB && db == xDB && dr == xDR && heads == xH) return Cfg<xNB, xDB, xDR, xH, xW, false, xBPW>::ST;
  MLRA_MFMA_SHAPES(X)
#undef X
  return 0;
}

hipError_t launch_attn_mfma(const AttnParams& p, bool paged, int grid_splits, hipStream_t stream) {
#define X(xNB, xDB, xDR, xH, xW, xBPW) \
  if (p.NB == xNB && p.DB == xDB && p.DR == xDR && p.H == xH) \
    return launch_shape<xNB, xDB, xDR, xH, xW, xBPW>(p, paged, grid_splits, stream);
  MLRA_MFMA_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace mlra
