/*
 * mlra.h — C ABI of libmlra.so: decode-step attention of Multi-Head Low-Rank
 * Attention (MLRA) and of single-latent Multi-Head Latent Attention (MLA) on
 * MI355X (gfx950), plus a paged-cache page-table API.
 *
 * Pages cited (by title and section):
 *   [MLRA]   "原生支持张量并行的多分支低秩注意力MLRA：优化KV缓存，实现2.8倍解码加速"
 *            (yunpan.plus): §1.3 MLA's three-step decode, §二 block decomposition,
 *            §三 / §3.1 MLRA-4, §3.2 per-device load, §3.3 output scaling.
 *   [DS-MLA] DeepSeek MLA analysis (dlbhg.com), section on MLA: decoupled RoPE
 *            with per-head RoPE queries and one shared RoPE key.
 *
 * What one decode call computes. Step 1 of [MLRA] §1.3 (absorbing the key
 * up-projection into the query) happens before the call, so the call receives the
 * absorbed query q~ and the RoPE query q^R. Inside the call, for every sequence
 * beta, head i and branch b, over the seq_lens[beta] cached tokens s:
 *     z_s     = sm_scale * (q~[beta,i,b,:] . c[beta,s,b*d_b:(b+1)*d_b]
 *                           + q^R[beta,i,:] . k^R[beta,s,:])
 *     p       = softmax over s of z          (independent per (i, b), [MLRA] §3.1)
 *     u_{i,b} = sum_s p_s c[beta,s,b*d_b:(b+1)*d_b]
 *     y[beta,i,:] = alpha * sum_b W^V_{i,b} u_{i,b}       ([MLRA] §三, §3.3)
 * MLA is the case num_branches == 1 (one latent of width d_c, [MLRA] §1.3).
 * The RoPE key is shared by every head and branch ([DS-MLA]; [MLRA] §3.1).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory on the current device; "host" marks
 *     host memory. The caller owns every buffer; the library keeps no pointer
 *     past the call and allocates no device memory. Its one device buffer is the
 *     array of mlra_decode_noalloc, which comes with the library's code.
 *   - Work is enqueued on the given stream (NULL = the default stream) and the
 *     call returns without waiting. Calls that overlap on one workspace race.
 *   - Nothing throws across the ABI. Every failure returns a status and sets a
 *     thread-local message readable with mlra_last_error(). Argument checks run
 *     on the host before any HIP call; when they fail nothing is enqueued and no
 *     output is touched.
 *   - Element types: MLRA_BF16 (bfloat16) or MLRA_F32. Accumulation is fp32.
 */
#ifndef MLRA_H_
#define MLRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mlra_status {
  MLRA_OK = 0,
  MLRA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, stride, alignment or table entry */
  MLRA_ERR_UNSUPPORTED = 2,   /* valid but not built (shape / dtype combination) */
  MLRA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than mlra_decode_workspace_size() */
  MLRA_ERR_NO_PAGES = 4,      /* page pool exhausted */
  MLRA_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} mlra_status;

typedef enum mlra_dtype { MLRA_BF16 = 0, MLRA_F32 = 1 } mlra_dtype;

/* Context-side error bits a kernel may set in *error_flags (see mlra_decode_args). */
#define MLRA_FLAG_SEQ_LEN_CLAMPED 1u   /* a seq_lens entry was < 1 or > max_seq_len */
#define MLRA_FLAG_BAD_PAGE        2u   /* a page-table entry was outside [0, num_pages) */

/*
 * Arguments of one decode call. Element strides count elements, not bytes.
 *
 * Shapes (B = batch, h = num_heads, n_b = num_branches, d_b = branch_dim,
 * d_c = n_b * d_b, d_R = rope_dim, d_h = head_dim):
 *   q_lat   [B][h][n_b][d_b]  absorbed queries, contiguous, type dtype
 *   q_rope  [B][h][d_R]       RoPE queries (already rotated), contiguous
 *   kv_lat / kv_rope: latent row and RoPE-key row of a cached token.
 *     Contiguous mode (page_table == NULL): token s of sequence beta is at
 *       kv_lat  + beta*seq_stride + s*row_stride  (d_c elements)
 *       kv_rope + beta*seq_stride + s*row_stride  (d_R elements)
 *     Paged mode: token s of sequence beta lives in physical row
 *       r = page_table[beta*max_pages + s/page_size]*page_size + s%page_size
 *       at kv_lat + r*row_stride and kv_rope + r*row_stride (seq_stride unused).
 *     The usual layout stores both in one row: kv_rope = kv_lat + d_c and
 *     row_stride = d_c + d_R ([MLRA] §3.1: each branch reads its latent block
 *     plus the shared RoPE key).
 *   w_v     [h][d_h][d_c]     W^V_{i,b} = rows of head i, columns [b*d_b,(b+1)*d_b)
 *   out     [B][h][d_h]       type out_dtype
 *   seq_lens  device int32 [B]; the query attends to exactly seq_lens[beta] rows
 *             (1 <= seq_lens[beta] <= max_seq_len). Values outside that range are
 *             clamped on the device and reported in *error_flags.
 *   seq_lens_host optional host copy of seq_lens; when given it is validated
 *             (an empty context is rejected, the softmax of no tokens is undefined)
 *             and the automatic split is sized from the real lengths, so that every
 *             shader engine holds at most one working group per CU (one pass).
 *   max_seq_len host upper bound on every seq_lens entry; sizes the launch.
 *   page_table device int32 [B][max_pages] or NULL; page_size must be a power of
 *             two; num_pages = rows of the pool / page_size (entries outside
 *             [0, num_pages) are replaced by page 0 and flagged).
 *   workspace device scratch of at least mlra_decode_workspace_size(args) bytes,
 *             256-byte aligned. Holds per-split partial softmax state; no
 *             initialisation needed.
 *   num_splits 0 = automatic; else the number of context splits of the longest
 *             sequence (each split covers ceil(max_seq_len/num_splits) tokens,
 *             rounded up to the kernel's tile).
 *   error_flags optional device uint32; MLRA_FLAG_* bits are OR-ed in. The caller
 *             zeroes it when it wants a fresh reading.
 *   event_attn_begin / event_attn_end optional hipEvent_t recorded on the stream
 *             around the attention kernel (the epilogue kernel runs after the end
 *             event), for timing the dominant kernel alone.
 * Alignment for the bf16 MFMA path: kv_lat, kv_rope, q_lat, q_rope, w_v 16-byte
 * aligned, row_stride and seq_stride multiples of 8 elements. Other inputs go
 * through the generic kernel.
 */
typedef struct mlra_decode_args {
  int32_t batch;
  int32_t num_heads;
  int32_t num_branches;
  int32_t branch_dim;
  int32_t rope_dim;
  int32_t head_dim;
  int32_t dtype;          /* mlra_dtype of q_lat, q_rope, kv_*, w_v */
  int32_t out_dtype;      /* mlra_dtype of out */
  float sm_scale;         /* softmax scale tau applied to the logits; must be > 0 */
  float alpha;            /* scale of the branch sum ([MLRA] §3.3) */
  const void* q_lat;
  const void* q_rope;
  const void* kv_lat;
  const void* kv_rope;
  int64_t row_stride;
  int64_t seq_stride;
  const int32_t* seq_lens;
  const int32_t* seq_lens_host;
  int32_t max_seq_len;
  int32_t page_size;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t num_pages;
  int32_t num_splits;
  const void* w_v;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  uint32_t* error_flags;
  void* event_attn_begin;
  void* event_attn_end;
} mlra_decode_args;

/* Thread-local message of the last failure on this thread ("" after success). */
const char* mlra_last_error(void);

/* Library version string. */
const char* mlra_version(void);

/*
 * Bytes of workspace a decode call with these arguments needs on the current
 * device. Host function: it launches nothing; the first call on a device reads
 * that device's compute-unit and XCD counts (hipDeviceGetAttribute) and keeps
 * them, exactly as mlra_decode does, so both plan the same splits; without a
 * usable device it plans for the largest gfx950 part (256 compute units).
 * Returns 0 and sets the error message when the arguments are invalid.
 */
size_t mlra_decode_workspace_size(const mlra_decode_args* args);

/*
 * Validate the arguments without launching anything (host function; plans for
 * the current device as mlra_decode_workspace_size does). Returns MLRA_OK or the
 * error mlra_decode would return before enqueuing.
 */
mlra_status mlra_decode_validate(const mlra_decode_args* args);

/*
 * How a decode call with these arguments would run (pointers are checked only
 * for alignment, since alignment picks the kernel).
 *   cu_count > 0: plan for a device with that many compute units (a what-if
 *     query; pure host function, no HIP call);
 *   cu_count == 0: plan for the current device, whose CU and XCD counts are read
 *     once with hipDeviceGetAttribute and cached (mlra_decode plans the same way).
 * kernel tells which attention kernel runs. MLRA_KERNEL_GENERIC (the scalar
 * kernel: fp32 inputs, shapes without a matrix-core build, misaligned operands,
 * see generic_reason) runs one work-group per (split, sequence, head) and so
 * reads the cache once per head, about num_heads times the bytes of the MFMA
 * path.
 */
enum { MLRA_KERNEL_MFMA = 0, MLRA_KERNEL_GENERIC = 1 };
#define MLRA_PLAN_GENERIC_DTYPE     1u   /* dtype is MLRA_F32 */
#define MLRA_PLAN_GENERIC_SHAPE     2u   /* no matrix-core build for (n_b, d_b, d_R, h) */
#define MLRA_PLAN_GENERIC_ALIGNMENT 4u   /* an operand or stride breaks the 16-byte alignment */
#define MLRA_PLAN_GENERIC_PAGE_SIZE 8u   /* pages smaller than the matrix-core kernel takes (16 tokens for MLRA-4) */
typedef struct mlra_plan_info {
  int32_t kernel;          /* MLRA_KERNEL_MFMA or MLRA_KERNEL_GENERIC */
  int32_t generic_reason;  /* MLRA_PLAN_GENERIC_* bits, 0 on the MFMA path */
  int32_t num_splits;      /* context splits of the longest sequence */
  int32_t split_tokens;    /* tokens per split */
  int32_t work_groups;     /* attention work-groups that hold tokens */
  int32_t cu_count;        /* compute units planned for */
  size_t workspace_bytes;  /* workspace this plan uses (with cu_count == 0: mlra_decode_workspace_size) */
} mlra_plan_info;
mlra_status mlra_decode_plan(const mlra_decode_args* args, int32_t cu_count, mlra_plan_info* info);

/*
 * MLRA decode ([MLRA] §三 and §3.1): per (head, branch) attention over that
 * branch's latent block plus the shared RoPE key with an independent softmax,
 * W^V per branch, scaled sum. Any num_branches >= 1. Enqueues two kernels on
 * `stream` (attention over context splits, then the split merge with the W^V
 * epilogue). `stream` is a hipStream_t.
 */
mlra_status mlra_decode(const mlra_decode_args* args, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): mlra_decode with the
 * split-partials workspace taken from a device array inside the library instead of
 * args->workspace (which is ignored). The array is MLRA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) per GPU, allocated when the library's code is loaded on that GPU and
 * held until the process ends; the call itself allocates nothing. Its device
 * address is looked up once per device on the first call there. Every call on one
 * GPU uses the same array: calls that overlap on one GPU (other streams, other
 * threads) race, so the caller serialises them. Nothing in it needs clearing
 * between calls (each call writes every record it reads). Errors: as mlra_decode,
 * plus MLRA_ERR_WORKSPACE (nothing enqueued) when the call's split state exceeds the
 * array.
 */
#define MLRA_NOALLOC_SCRATCH_BYTES (16u << 20)
mlra_status mlra_decode_noalloc(const mlra_decode_args* args, void* stream);

/*
 * MLA decode ([MLRA] §1.3): the single-latent comparison path. Same arguments;
 * requires num_branches == 1 (branch_dim is then the latent width d_c).
 */
mlra_status mla_decode(const mlra_decode_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * The step before a decode call, for one new token per sequence:
 *  - query absorption, [MLRA] §1.3 step 1 (and §二 for the branch split):
 *      q~_i = W^UK_i^T q^N_i,  q_lat[beta][i][b][:] = q~_i[b*d_b:(b+1)*d_b];
 *  - the RoPE query rotated to the new token's position m;
 *  - the new token's cache row: its latent, and its RoPE key rotated to m.
 * Rotation at position m ([DS-MLA] decoupled RoPE; the pages print no formula,
 * the original rotary form is taken): consecutive pairs (x_2j, x_2j+1) become
 *   (x_2j cos a - x_2j+1 sin a, x_2j sin a + x_2j+1 cos a),  a = m * rope_base^(-2j/d_R).
 * The angle and its sine and cosine are computed in fp64, the rotation in fp32.
 *
 * Shapes (all contiguous, type dtype):
 *   q_nope   [B][h][d_h]    NoPE query of each head, before absorption
 *   q_pe     [B][h][d_R]    RoPE query, before rotation (d_R even, at most 256)
 *   w_uk     [h][d_c][d_h]  W^UK_i transposed: row n of head i is the d_h-vector
 *                           whose dot with q^N_i gives q~_i[n] (W^UK_i maps a
 *                           latent to the head's NoPE key)
 *   c_new    [B][d_c]       latent of the new token
 *   k_pe_new [B][d_R]       RoPE key of the new token, before rotation
 *   positions device int32 [B]: the new token's position m, which is also its row
 *            in the cache; the decode that follows uses seq_lens = positions + 1.
 *   positions_host optional host copy, validated (0 <= m, m < max_seq_len when
 *            contiguous, m < max_pages*page_size when paged).
 *   q_lat, q_rope  outputs in the layout mlra_decode takes.
 *   kv_lat, kv_rope, row_stride, seq_stride, max_seq_len, page_size, page_table,
 *   max_pages, num_pages: the cache, addressed exactly as in mlra_decode_args.
 *   The latent is copied bit-exactly; the rotated RoPE key is rounded once to dtype.
 * Errors: host validation as for mlra_decode. On the device, a position outside
 * the cache sets MLRA_FLAG_SEQ_LEN_CLAMPED and a page-table entry outside
 * [0, num_pages) sets MLRA_FLAG_BAD_PAGE in *error_flags; that sequence's row is
 * then not written (its queries still are).
 * The bf16 path uses MFMAs for the absorption when d_h % 32 == 0, d_h <= 256,
 * d_c % 16 == 0 and q_nope, w_uk are 16-byte aligned; other shapes and fp32 use
 * the vector ALUs.
 * ------------------------------------------------------------------------- */
typedef struct mlra_prepare_args {
  int32_t batch;
  int32_t num_heads;
  int32_t num_branches;
  int32_t branch_dim;
  int32_t rope_dim;
  int32_t head_dim;
  int32_t dtype;
  float rope_base;
  const void* q_nope;
  const void* q_pe;
  const void* w_uk;
  const void* c_new;
  const void* k_pe_new;
  const int32_t* positions;
  const int32_t* positions_host;
  void* q_lat;
  void* q_rope;
  void* kv_lat;
  void* kv_rope;
  int64_t row_stride;
  int64_t seq_stride;
  int32_t max_seq_len;
  int32_t page_size;
  const int32_t* page_table;
  int32_t max_pages;
  int32_t num_pages;
  uint32_t* error_flags;
} mlra_prepare_args;

/* Enqueue the step above (one kernel) on `stream`. */
mlra_status mlra_decode_prepare(const mlra_prepare_args* args, void* stream);

/* ---------------------------------------------------------------------------
 * Paged cache. A pool is `num_pages` pages of `page_size` rows of `row_stride`
 * elements; a page table maps a sequence's logical page j to a physical page.
 * ------------------------------------------------------------------------- */

/*
 * Write one new row per sequence into its slot: for each beta < batch,
 * pos = positions[beta] and
 *   pool[(page_table[beta*max_pages + pos/page_size]*page_size + pos%page_size)*row_stride + e]
 *     = rows[beta*row_elems + e]   for e < row_elems.
 * Bit-exact copy. Device pointers: pool, page_table, positions, rows. A
 * negative position or an entry outside [0, num_pages) skips that sequence's
 * write and sets MLRA_FLAG_BAD_PAGE in *error_flags (if not NULL).
 */
mlra_status mlra_paged_append(void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size,
                              int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* positions, const void* rows, int32_t batch, int32_t dtype,
                              uint32_t* error_flags, void* stream);

/*
 * Copy each sequence's logical rows out of the pool:
 *   out[(beta*max_seq_len + s)*row_elems + e] = pool[(row of (beta, s))*row_stride + e]
 * for s < min(seq_lens[beta], max_seq_len), e < row_elems; other rows of `out`
 * are left untouched. Bit-exact. Device pointers: pool, page_table, seq_lens, out.
 */
mlra_status mlra_paged_gather(const void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size,
                              int32_t num_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, int32_t max_seq_len, int32_t batch, int32_t dtype,
                              void* out, uint32_t* error_flags, void* stream);

/*
 * Host check of a page table (all pointers host): for every sequence the
 * ceil(seq_lens[beta]/page_size) entries it uses must fit in max_pages, lie in
 * [0, num_pages) and be distinct across the whole table (one physical page backs
 * one logical page). Returns MLRA_OK or MLRA_ERR_INVALID_ARG with a message
 * naming the first bad entry.
 */
mlra_status mlra_page_table_check(const int32_t* page_table, int32_t batch, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t page_size, int32_t num_pages);

/*
 * Host page allocator: a deterministic LIFO free list of page ids
 * 0..num_pages-1 (a fresh pool hands out 0, 1, 2, ...). Not thread-safe; the
 * caller serialises use of one pool.
 *   create: MLRA_ERR_INVALID_ARG if num_pages < 1 or out is NULL.
 *   alloc:  writes n ids to ids (host); MLRA_ERR_NO_PAGES (and no change) when
 *           fewer than n pages are free.
 *   free:   returns n ids; MLRA_ERR_INVALID_ARG (and no change) if any id is out
 *           of range, not allocated, or repeated in the list.
 */
typedef struct mlra_page_pool mlra_page_pool;
mlra_status mlra_page_pool_create(int32_t num_pages, mlra_page_pool** out);
mlra_status mlra_page_pool_alloc(mlra_page_pool* pool, int32_t n, int32_t* ids);
mlra_status mlra_page_pool_free(mlra_page_pool* pool, int32_t n, const int32_t* ids);
int32_t mlra_page_pool_num_free(const mlra_page_pool* pool);
void mlra_page_pool_destroy(mlra_page_pool* pool);

/*
 * Measurement support: a streaming-read probe. Reads the `bytes` bytes at device
 * pointer `src` once with 16-byte nontemporal loads, each work-group streaming one
 * contiguous chunk, so that a caller can time the read rate this GPU reaches (the
 * practical ceiling next to the HBM peak, for reading the attention kernel's achieved
 * bandwidth). Writes
 * mlra_read_probe_words() 32-bit words to device buffer `out`: out[g] is the XOR of
 * the 32-bit words read by work-group g, so the XOR of all of them equals the XOR of
 * every 32-bit word of the buffer. Enqueued on `stream` without waiting.
 * Errors (no HIP call made): MLRA_ERR_INVALID_ARG if a pointer is NULL, `bytes` is 0
 * or not a multiple of 16, `src` is not 16-byte aligned, or `out_words` is smaller
 * than mlra_read_probe_words(); MLRA_ERR_HIP if the launch fails.
 */
int32_t mlra_read_probe_words(void);
mlra_status mlra_read_probe(const void* src, size_t bytes, uint32_t* out, int32_t out_words, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLRA_H_ */
