// Internal interface between the host API (mlra_api.cpp) and the HIP kernels.
// Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace mlra {

// Partial softmax state written by the attention kernels, one record per
// (sequence, split, head, branch):
//   o  [B][S][H][NB][DB] unnormalised sum_s 2^(x_s - m) c_s: fp32, or (ws_o_f16: the MFMA
//                        shapes of mfma_f16_records) fp16 scaled by 2^-e, where l = f 2^e
//                        with f in [0.5, 1), and e added to m, so that (o, m, l) describe the
//                        same softmax state and the records stay in fp16's range
//   ml [B][S][H][NB][2]  fp32  (m, l): reference max in log2 units and sum 2^(x_s - m)
// where x_s = z_s * log2(e) is the logit in log2 units.
struct AttnParams {
  const void* q_lat;       // [B][H][NB][DB]
  const void* q_rope;      // [B][H][DR]
  const char* kv_lat;      // byte pointers
  const char* kv_rope;
  int64_t row_stride_b;    // bytes between consecutive rows
  int64_t seq_stride_b;    // bytes between sequences (contiguous mode)
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t max_seq_len;
  int32_t page_shift;      // log2(page_size)
  int32_t max_pages;
  int32_t num_pages;
  int32_t B, H, NB, DB, DR;
  float q_scale;           // sm_scale * log2(e)
  int32_t split_tokens;    // tokens per split (multiple of the kernel's stage)
  int32_t num_splits;      // splits of the longest sequence (record stride S)
  void* ws_o;              // fp32, or fp16 scaled records (ws_o_f16)
  float* ws_ml;
  uint32_t* error_flags;
  int32_t ws_o_f16;
};

struct MergeParams {
  const void* ws_o;
  const float* ws_ml;
  const int32_t* seq_lens;
  const void* w_v;         // [H][DH][NB*DB]
  void* out;               // [B][H][DH]
  int32_t max_seq_len;
  int32_t B, H, NB, DB, DH;
  int32_t split_tokens;
  int32_t num_splits;
  float alpha;
  int32_t w_dtype;         // mlra_dtype
  int32_t out_dtype;
  int32_t ws_o_f16;
};

// MFMA (bf16) attention: kernel shapes compiled into the library.
struct MfmaShape {
  int nb, db, dr, heads;
};
// Stage size in tokens of the MFMA kernel for this shape (0 if not built).
int mfma_stage_tokens(int nb, int db, int dr, int heads);
// Whether the MFMA kernel of this shape writes fp16 split records (else fp32).
bool mfma_f16_records(int nb, int db, int dr, int heads);
// Pages one split of the paged MFMA kernel of this shape may span.
int mfma_page_cache(int nb, int db, int dr, int heads);
// Smallest page size (tokens) the paged MFMA kernel of this shape takes.
int mfma_min_page_size(int nb, int db, int dr, int heads);
// Launch the MFMA attention kernel; returns hipSuccess or the launch error.
hipError_t launch_attn_mfma(const AttnParams& p, bool paged, int grid_splits, hipStream_t stream);

// Generic attention kernel (fp32 or bf16 inputs, any supported dims).
constexpr int kGenericStage = 256;
bool generic_supported(int nb, int db, int dr);
hipError_t launch_attn_generic(const AttnParams& p, bool paged, int dtype, int grid_splits, hipStream_t stream);

// Split merge + W^V epilogue.
bool merge_supported(int nb, int db, int dh);
// true when the MFMA merge (no per-split LDS) runs for this shape and W^V
bool merge_uses_mfma(int nb, int db, int dh, int w_dtype, const void* w_v);
// LDS the vector-ALU merge needs: (m, l) of every split of a block of sequences, and their u
size_t merge_lds_bytes(int nb, int db, int num_splits);
constexpr size_t kMergeLdsLimit = 60 * 1024;
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

// Streaming-read probe (measurement support): kProbeBlocks work-groups of kProbeThreads
// threads; out[g] = XOR of the 32-bit words work-group g read.
constexpr int kProbeBlocks = 2048;
constexpr int kProbeThreads = 256;
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, hipStream_t stream);

// The step before a decode call: query absorption, RoPE rotation, new cache rows.
struct PrepareParams {
  int B, H, NB, DB, DR, DH;
  int dtype;                 // 0 bf16, 1 f32
  bool mfma;                 // bf16 with d_h % 32 == 0, d_c % 16 == 0 and 16-byte aligned operands
  float rope_base;
  const void* q_nope;
  const void* q_pe;
  const void* w_uk;
  const void* c_new;
  const void* k_pe_new;
  const int32_t* positions;
  void* q_lat;
  void* q_rope;
  void* kv_lat;
  void* kv_rope;
  int64_t row_stride_b;
  int64_t seq_stride_b;
  int max_seq_len;
  int page_shift;
  const int32_t* page_table;
  int max_pages;
  int num_pages;
  uint32_t* error_flags;
};
bool prepare_mfma_supported(int dh, int dc);
hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream);

// Paged cache copies.
hipError_t launch_paged_append(void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size,
                               int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                               const int32_t* positions, const void* rows, int32_t batch, int32_t elem_bytes,
                               uint32_t* error_flags, hipStream_t stream);
hipError_t launch_paged_gather(const void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size,
                               int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                               const int32_t* seq_lens, int32_t max_seq_len, int32_t batch, int32_t elem_bytes,
                               void* out, uint32_t* error_flags, hipStream_t stream);

}  // namespace mlra
