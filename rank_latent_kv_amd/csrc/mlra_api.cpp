// Host side of libmlra.so: argument validation (no HIP calls), launch planning,
// the page allocator, and the exported C ABI declared in include/mlra.h.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "mlra.h"
#include "mlra_internal.h"

namespace {

thread_local std::string g_last_error;

mlra_status fail(mlra_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mlra_status ok() {
  g_last_error.clear();
  return MLRA_OK;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The automatic split count aims for one work-group per compute unit (the MFMA kernel keeps
// one work-group per CU). The planner takes the device's CU and XCD counts as a parameter,
// so it stays free of HIP calls. The entry points that plan a real call (decode, workspace
// size, validation) read the counts of the current device once and keep them; without a
// usable device they plan for the largest gfx950 part, an MI355X with 256 CUs in 8 XCDs.
// (The splits are not monotone in the CU count: the shader-engine check below can grow the
// split on a larger device. So the workspace is sized for the device the call runs on, not
// for a bound over devices.)
struct Topology {
  int cus = 256;
  int xcds = 8;
};
constexpr Topology kLargestGfx950{};
constexpr int kMaxSplits = 4096;

struct Plan {
  int generic_reason = 0;   // MLRA_PLAN_* bits: why the generic kernel runs (0 on the MFMA path)
  int64_t groups = 0;       // attention work-groups that hold tokens
  int cus = 0;
  bool mfma = false;
  bool paged = false;
  int stage = 0;          // split granularity in tokens
  int split_tokens = 0;
  int num_splits = 0;
  size_t ws_o_bytes = 0;
  size_t ws_ml_bytes = 0;
  size_t ws_bytes = 0;
  bool f16_records = false;   // the attention kernel writes fp16 split records
};

int64_t total_tokens_estimate(const mlra_decode_args* a) {
  if (a->seq_lens_host) {
    int64_t t = 0;
    for (int i = 0; i < a->batch; ++i) t += std::min(std::max(a->seq_lens_host[i], 0), a->max_seq_len);
    return std::max<int64_t>(t, 1);
  }
  return (int64_t)a->batch * a->max_seq_len;
}

// Work-groups of a launch with `split`-token splits that hold tokens (groups past a
// sequence's end exit at once).
int64_t count_groups(const mlra_decode_args* a, int64_t split) {
  if (!a->seq_lens_host) return (int64_t)a->batch * cdiv(a->max_seq_len, split);
  int64_t g = 0;
  for (int i = 0; i < a->batch; ++i) g += cdiv(std::min(std::max(a->seq_lens_host[i], 1), a->max_seq_len), split);
  return g;
}

// The MFMA kernel's (splits, batch) grid as gfx950 places it: work-groups go to the XCDs in
// turn (linear id mod XCDs), and within an XCD to its 4 shader engines in turn, each engine
// with (CUs per XCD) / 4 CUs that hold one group apiece (8 on an MI355X). An engine given
// one more group than it has CUs runs it as a second pass (about twice the kernel time),
// however many groups of its XCD or of the whole launch are free; groups past a sequence's
// end exit at once and do not count. This placement matches every launch measured on ragged
// lengths of an MI355X: those with at most 8 working groups per engine ran in one pass,
// those with 9 in two. True when no engine gets more groups than CUs. A device whose CUs do
// not split evenly over 4 engines per XCD gets only the total-count check.
constexpr int kEnginesPerXcd = 4;
constexpr int kMaxEngines = 64;
bool one_pass_per_engine(const mlra_decode_args* a, int64_t split, const Topology& t) {
  if (!a->seq_lens_host) return true;   // without host lengths the group count alone decides
  if (t.xcds < 1 || t.cus % (t.xcds * kEnginesPerXcd) != 0 || t.xcds * kEnginesPerXcd > kMaxEngines) return true;
  const int engines = t.xcds * kEnginesPerXcd;
  const int64_t per_engine = t.cus / engines;
  const int64_t ns = cdiv(a->max_seq_len, split);
  int64_t working[kMaxEngines] = {};
  for (int b = 0; b < a->batch; ++b) {
    const int64_t L = std::min(std::max(a->seq_lens_host[b], 1), a->max_seq_len);
    for (int64_t s = 0; s * split < L; ++s) {
      const int64_t id = b * ns + s;
      ++working[(id % t.xcds) * kEnginesPerXcd + (id / t.xcds) % kEnginesPerXcd];
    }
  }
  for (int e = 0; e < engines; ++e)
    if (working[e] > per_engine) return false;
  return true;
}

// Validate the arguments and decide the launch for a device of topology `topo`. Pure host
// code: no HIP calls.
mlra_status make_plan(const mlra_decode_args* a, bool check_pointers, const Topology& topo, Plan* plan) {
  if (!a) return fail(MLRA_ERR_INVALID_ARG, "args is NULL");
  if (a->batch < 1) return fail(MLRA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", a->batch);
  if (a->num_heads < 1) return fail(MLRA_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", a->num_heads);
  if (a->num_branches < 1) return fail(MLRA_ERR_INVALID_ARG, "num_branches must be >= 1 (got %d)", a->num_branches);
  if (a->branch_dim < 1) return fail(MLRA_ERR_INVALID_ARG, "branch_dim must be >= 1 (got %d)", a->branch_dim);
  if (a->rope_dim < 0) return fail(MLRA_ERR_INVALID_ARG, "rope_dim must be >= 0 (got %d)", a->rope_dim);
  if (a->head_dim < 1) return fail(MLRA_ERR_INVALID_ARG, "head_dim must be >= 1 (got %d)", a->head_dim);
  if (a->dtype != MLRA_BF16 && a->dtype != MLRA_F32) return fail(MLRA_ERR_INVALID_ARG, "dtype %d is not a mlra_dtype", a->dtype);
  if (a->out_dtype != MLRA_BF16 && a->out_dtype != MLRA_F32)
    return fail(MLRA_ERR_INVALID_ARG, "out_dtype %d is not a mlra_dtype", a->out_dtype);
  if (!std::isfinite(a->sm_scale) || !std::isfinite(a->alpha))
    return fail(MLRA_ERR_INVALID_ARG, "sm_scale and alpha must be finite");
  if (!(a->sm_scale > 0.f)) return fail(MLRA_ERR_INVALID_ARG, "sm_scale must be > 0 (got %g)", (double)a->sm_scale);
  if (a->max_seq_len < 1) return fail(MLRA_ERR_INVALID_ARG, "max_seq_len must be >= 1 (got %d)", a->max_seq_len);
  if (a->num_splits < 0) return fail(MLRA_ERR_INVALID_ARG, "num_splits must be >= 0 (got %d)", a->num_splits);
  const int64_t dc = (int64_t)a->num_branches * a->branch_dim;
  const int64_t row_need = dc + a->rope_dim;
  if (a->row_stride < 1) return fail(MLRA_ERR_INVALID_ARG, "row_stride must be >= 1 (got %lld)", (long long)a->row_stride);
  if (check_pointers) {
    if (!a->q_lat || !a->q_rope || !a->kv_lat || !a->kv_rope || !a->seq_lens || !a->w_v || !a->out)
      return fail(MLRA_ERR_INVALID_ARG, "a required pointer (q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, out) is NULL");
  }
  if (a->seq_lens_host) {
    for (int i = 0; i < a->batch; ++i) {
      const int L = a->seq_lens_host[i];
      if (L < 1) return fail(MLRA_ERR_INVALID_ARG, "seq_lens[%d] = %d: an empty context has no softmax", i, L);
      if (L > a->max_seq_len) return fail(MLRA_ERR_INVALID_ARG, "seq_lens[%d] = %d exceeds max_seq_len %d", i, L, a->max_seq_len);
    }
  }
  const bool paged = a->page_table != nullptr;
  if (paged) {
    if (!is_pow2(a->page_size)) return fail(MLRA_ERR_INVALID_ARG, "page_size must be a power of two (got %d)", a->page_size);
    if (a->num_pages < 1) return fail(MLRA_ERR_INVALID_ARG, "num_pages must be >= 1 (got %d)", a->num_pages);
    if ((int64_t)a->max_pages * a->page_size < a->max_seq_len)
      return fail(MLRA_ERR_INVALID_ARG, "max_pages %d x page_size %d cannot hold max_seq_len %d", a->max_pages, a->page_size,
                  a->max_seq_len);
  } else {
    if (a->seq_stride < (int64_t)(a->max_seq_len - 1) * a->row_stride + 1 && a->batch > 1)
      return fail(MLRA_ERR_INVALID_ARG, "seq_stride %lld is smaller than max_seq_len rows of row_stride %lld",
                  (long long)a->seq_stride, (long long)a->row_stride);
  }
  // Rows may hold latent and RoPE parts anywhere; they must not overlap when they share one row.
  if (a->kv_lat && a->kv_rope) {
    const int64_t eb = a->dtype == MLRA_BF16 ? 2 : 4;
    const int64_t delta = (reinterpret_cast<const char*>(a->kv_rope) - reinterpret_cast<const char*>(a->kv_lat)) / eb;
    if (delta >= 0 && delta < dc && a->rope_dim > 0)
      return fail(MLRA_ERR_INVALID_ARG, "kv_rope overlaps the latent columns of kv_lat");
    if (delta == dc && a->row_stride < row_need)
      return fail(MLRA_ERR_INVALID_ARG, "row_stride %lld is smaller than d_c + d_R = %lld", (long long)a->row_stride,
                  (long long)row_need);
  }
  if (!mlra::merge_supported(a->num_branches, a->branch_dim, a->head_dim))
    return fail(MLRA_ERR_UNSUPPORTED, "latent width %lld is beyond the merge kernel's limit", (long long)dc);

  if (topo.cus < 1) return fail(MLRA_ERR_INVALID_ARG, "cu count must be >= 1 (got %d)", topo.cus);
  const int64_t kTargetGroups = topo.cus;
  Plan p;
  p.paged = paged;
  p.cus = topo.cus;
  const int st = (a->dtype == MLRA_BF16) ? mlra::mfma_stage_tokens(a->num_branches, a->branch_dim, a->rope_dim, a->num_heads) : 0;
  bool mfma = st > 0;
  if (a->dtype != MLRA_BF16) p.generic_reason |= MLRA_PLAN_GENERIC_DTYPE;
  else if (st == 0) p.generic_reason |= MLRA_PLAN_GENERIC_SHAPE;
  if (mfma) {
    // the MFMA path moves 16-byte chunks and reads 8-element query groups
    const bool al = aligned(a->q_lat, 16) && aligned(a->q_rope, 16) && aligned(a->kv_lat, 16) && aligned(a->kv_rope, 16) &&
                    a->row_stride % 8 == 0 && (paged || a->seq_stride % 8 == 0);
    if (!al) {
      mfma = false;
      p.generic_reason |= MLRA_PLAN_GENERIC_ALIGNMENT;
    }
    if (paged && a->page_size < mlra::mfma_min_page_size(a->num_branches, a->branch_dim, a->rope_dim, a->num_heads)) {
      mfma = false;
      p.generic_reason |= MLRA_PLAN_GENERIC_PAGE_SIZE;
    }
  }
  if (!mfma && !mlra::generic_supported(a->num_branches, a->branch_dim, a->rope_dim))
    return fail(MLRA_ERR_UNSUPPORTED, "no kernel for num_branches=%d branch_dim=%d rope_dim=%d dtype=%d", a->num_branches,
                a->branch_dim, a->rope_dim, a->dtype);
  p.mfma = mfma;
  p.stage = mfma ? st : mlra::kGenericStage;

  // split size: a multiple of the stage; automatic = about one group per CU over all tokens
  int64_t split;
  if (a->num_splits > 0) {
    split = cdiv(a->max_seq_len, a->num_splits);
  } else {
    const int64_t groups_per_pass = mfma ? kTargetGroups : kTargetGroups * 4;
    const int64_t heads_factor = mfma ? 1 : a->num_heads;   // the generic kernel has one group per head
    split = cdiv(total_tokens_estimate(a) * heads_factor, groups_per_pass);
  }
  split = std::max<int64_t>(round_up(std::max<int64_t>(split, 1), p.stage), p.stage);
  if (mfma && a->num_splits == 0) {
    // Ragged lengths round up per sequence, which can leave a few work-groups beyond
    // one per CU, or more than one per CU on one shader engine; those would run as a
    // second pass. The group count only falls as the split grows, so the smallest split
    // (in whole stages) whose groups fit one per CU is found by bisection; from there the
    // split grows one stage at a time until no shader engine gets a ninth group.
    if (split < a->max_seq_len && count_groups(a, split) > kTargetGroups) {
      int64_t lo = split / p.stage, hi = cdiv(a->max_seq_len, p.stage);   // count(hi) is the batch size
      if (count_groups(a, hi * p.stage) > kTargetGroups) {
        lo = hi;                                      // more sequences than CUs: one split each
      } else {
        while (lo < hi) {
          const int64_t mid = lo + (hi - lo) / 2;
          if (count_groups(a, mid * p.stage) > kTargetGroups) lo = mid + 1;
          else hi = mid;
        }
      }
      split = lo * p.stage;
    }
    while (split < a->max_seq_len && (count_groups(a, split) > kTargetGroups || !one_pass_per_engine(a, split, topo)))
      split += p.stage;
  }
  if (paged && mfma) {
    // the split's page ids must fit the kernel's page-id cache (one split starting mid-page
    // spans one page more than its length needs)
    const int cache = mlra::mfma_page_cache(a->num_branches, a->branch_dim, a->rope_dim, a->num_heads);
    const int64_t max_split = (int64_t)(cache - 1) * a->page_size / p.stage * p.stage;
    if (max_split < p.stage) return fail(MLRA_ERR_UNSUPPORTED, "page_size %d too small for the MFMA path", a->page_size);
    // the kernel forms a page's byte offset as a 32 x 32 -> 64-bit product
    const int64_t page_bytes = (int64_t)a->page_size * a->row_stride * (a->dtype == MLRA_BF16 ? 2 : 4);
    if (page_bytes >= ((int64_t)1 << 32))
      return fail(MLRA_ERR_UNSUPPORTED, "a page of %lld bytes is beyond the MFMA path's 4 GiB limit", (long long)page_bytes);
    split = std::min(split, max_split);
  }
  p.split_tokens = (int)std::min<int64_t>(split, a->max_seq_len + (int64_t)p.stage);
  p.num_splits = (int)cdiv(a->max_seq_len, p.split_tokens);
  p.groups = count_groups(a, p.split_tokens) * (mfma ? 1 : a->num_heads);
  if (p.num_splits > kMaxSplits)
    return fail(MLRA_ERR_UNSUPPORTED, "%d context splits exceed the limit %d", p.num_splits, kMaxSplits);
  // the vector-ALU merge keeps (m, l) of every split of a block of sequences in LDS
  if (!mlra::merge_uses_mfma(a->num_branches, a->branch_dim, a->head_dim, a->dtype, a->w_v) &&
      mlra::merge_lds_bytes(a->num_branches, a->branch_dim, p.num_splits) > mlra::kMergeLdsLimit)
    return fail(MLRA_ERR_UNSUPPORTED, "%d splits x %d branches exceed the merge kernel's LDS", p.num_splits, a->num_branches);
  const size_t recs = (size_t)a->batch * p.num_splits * a->num_heads * a->num_branches;
  // fp16 output records where the MFMA kernel writes them (see AttnParams), fp32 else
  p.f16_records = p.mfma && mlra::mfma_f16_records(a->num_branches, a->branch_dim, a->rope_dim, a->num_heads);
  p.ws_o_bytes = round_up(recs * a->branch_dim * (p.f16_records ? 2 : 4), 256);
  p.ws_ml_bytes = round_up(recs * 2 * sizeof(float), 256);
  p.ws_bytes = p.ws_o_bytes + p.ws_ml_bytes;
  *plan = p;
  return MLRA_OK;
}

mlra_status hip_fail(hipError_t e, const char* what) {
  return fail(MLRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// CU and XCD counts of the current device, read once per device and kept for the life of the
// process (the library's only global state). Without a usable device the largest gfx950 part
// is assumed.
constexpr int kMaxDevices = 64;
std::atomic<int> g_topo_cus[kMaxDevices];
std::atomic<int> g_topo_xcds[kMaxDevices];

Topology current_topology() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kLargestGfx950;
  }
  Topology t;
  const int cached = g_topo_cus[dev].load(std::memory_order_acquire);
  if (cached > 0) {
    t.cus = cached;
    t.xcds = g_topo_xcds[dev].load(std::memory_order_relaxed);
    return t;
  }
  int cus = 0, xcds = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    (void)hipGetLastError();
    return kLargestGfx950;
  }
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) {
    (void)hipGetLastError();
    xcds = 1;
  }
  t.cus = cus;
  t.xcds = xcds;
  g_topo_xcds[dev].store(xcds, std::memory_order_relaxed);
  g_topo_cus[dev].store(cus, std::memory_order_release);
  return t;
}

// Scratch of the allocation-free decode entry point: the split-partials workspace in a
// file-scope device array, one per GPU, held until the process ends. In host code `scratch`
// names a host-side stand-in, not a device address: its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that
// pointer is ever passed to kernels.
constexpr size_t kScratchBytes = MLRA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

mlra_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLRA_ERR_UNSUPPORTED, "device %d is beyond the library's %d devices", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p) return fail(MLRA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MLRA_OK;
}

mlra_status run_decode(const mlra_decode_args* a, void* stream_v) {
  Plan plan;
  mlra_status st = make_plan(a, true, current_topology(), &plan);
  if (st != MLRA_OK) return st;
  if (!a->workspace) return fail(MLRA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", plan.ws_bytes);
  if (a->workspace_bytes < plan.ws_bytes)
    return fail(MLRA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", a->workspace_bytes, plan.ws_bytes);
  if (!aligned(a->workspace, 256)) return fail(MLRA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  const int64_t eb = a->dtype == MLRA_BF16 ? 2 : 4;
  mlra::AttnParams p{};
  p.q_lat = a->q_lat;
  p.q_rope = a->q_rope;
  p.kv_lat = static_cast<const char*>(a->kv_lat);
  p.kv_rope = static_cast<const char*>(a->kv_rope);
  p.row_stride_b = a->row_stride * eb;
  p.seq_stride_b = a->seq_stride * eb;
  p.seq_lens = a->seq_lens;
  p.page_table = a->page_table;
  p.max_seq_len = a->max_seq_len;
  p.page_shift = plan.paged ? ilog2(a->page_size) : 0;
  p.max_pages = a->max_pages;
  p.num_pages = a->num_pages;
  p.B = a->batch;
  p.H = a->num_heads;
  p.NB = a->num_branches;
  p.DB = a->branch_dim;
  p.DR = a->rope_dim;
  p.q_scale = a->sm_scale * 1.4426950408889634f;
  p.split_tokens = plan.split_tokens;
  p.num_splits = plan.num_splits;
  p.ws_o = a->workspace;
  p.ws_o_f16 = plan.f16_records;
  p.ws_ml = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + plan.ws_o_bytes);
  p.error_flags = a->error_flags;

  hipError_t e;
  if (a->event_attn_begin) {
    e = hipEventRecord(static_cast<hipEvent_t>(a->event_attn_begin), stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(begin)");
  }
  if (plan.mfma) e = mlra::launch_attn_mfma(p, plan.paged, plan.num_splits, stream);
  else e = mlra::launch_attn_generic(p, plan.paged, a->dtype, plan.num_splits, stream);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  if (a->event_attn_end) {
    e = hipEventRecord(static_cast<hipEvent_t>(a->event_attn_end), stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(end)");
  }

  mlra::MergeParams m{};
  m.ws_o = p.ws_o;
  m.ws_o_f16 = p.ws_o_f16;
  m.ws_ml = p.ws_ml;
  m.seq_lens = a->seq_lens;
  m.w_v = a->w_v;
  m.out = a->out;
  m.max_seq_len = a->max_seq_len;
  m.B = a->batch;
  m.H = a->num_heads;
  m.NB = a->num_branches;
  m.DB = a->branch_dim;
  m.DH = a->head_dim;
  m.split_tokens = plan.split_tokens;
  m.num_splits = plan.num_splits;
  m.alpha = a->alpha;
  m.w_dtype = a->dtype;
  m.out_dtype = a->out_dtype;
  e = mlra::launch_merge(m, stream);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return ok();
}

}  // namespace

struct mlra_page_pool {
  int32_t num_pages;
  std::vector<int32_t> free_list;   // LIFO stack: back() is handed out next
  std::vector<uint8_t> allocated;
};

extern "C" {

const char* mlra_last_error(void) { return g_last_error.c_str(); }

const char* mlra_version(void) { return "mlra 0.1.0 (gfx950)"; }

size_t mlra_decode_workspace_size(const mlra_decode_args* args) {
  Plan plan;
  if (make_plan(args, false, current_topology(), &plan) != MLRA_OK) return 0;
  ok();
  return plan.ws_bytes;
}

mlra_status mlra_decode_plan(const mlra_decode_args* args, int32_t cu_count, mlra_plan_info* info) {
  if (!info) return fail(MLRA_ERR_INVALID_ARG, "info is NULL");
  if (cu_count < 0) return fail(MLRA_ERR_INVALID_ARG, "cu_count must be >= 0 (got %d)", cu_count);
  Topology t = kLargestGfx950;
  if (cu_count > 0) {
    t.cus = cu_count;
    // XCDs of 32 CUs where the count splits that way, else one
    t.xcds = cu_count % 32 == 0 ? cu_count / 32 : 1;
  } else {
    t = current_topology();
  }
  Plan plan;
  mlra_status st = make_plan(args, false, t, &plan);
  if (st != MLRA_OK) return st;
  info->kernel = plan.mfma ? MLRA_KERNEL_MFMA : MLRA_KERNEL_GENERIC;
  info->generic_reason = plan.generic_reason;
  info->num_splits = plan.num_splits;
  info->split_tokens = plan.split_tokens;
  info->work_groups = (int32_t)std::min<int64_t>(plan.groups, INT32_MAX);
  info->cu_count = plan.cus;
  info->workspace_bytes = plan.ws_bytes;
  return ok();
}

mlra_status mlra_decode_validate(const mlra_decode_args* args) {
  Plan plan;
  mlra_status st = make_plan(args, true, current_topology(), &plan);
  if (st != MLRA_OK) return st;
  if (!args->workspace) return fail(MLRA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", plan.ws_bytes);
  if (args->workspace_bytes < plan.ws_bytes)
    return fail(MLRA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", args->workspace_bytes, plan.ws_bytes);
  if (!aligned(args->workspace, 256)) return fail(MLRA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return ok();
}

mlra_status mlra_decode(const mlra_decode_args* args, void* stream) { return run_decode(args, stream); }

mlra_status mlra_decode_noalloc(const mlra_decode_args* args, void* stream) {
  if (!args) return fail(MLRA_ERR_INVALID_ARG, "args is NULL");
  Plan plan;
  mlra_status st = make_plan(args, true, current_topology(), &plan);
  if (st != MLRA_OK) return st;
  if (plan.ws_bytes > kScratchBytes)
    return fail(MLRA_ERR_WORKSPACE,
                "this call needs %zu bytes of split state, beyond the %zu-byte device array of the allocation-free "
                "entry point (use mlra_decode with a workspace)",
                plan.ws_bytes, kScratchBytes);
  void* p = nullptr;
  st = scratch_of_current_device(&p);
  if (st != MLRA_OK) return st;
  mlra_decode_args a = *args;
  a.workspace = p;
  a.workspace_bytes = kScratchBytes;
  return run_decode(&a, stream);
}

mlra_status mla_decode(const mlra_decode_args* args, void* stream) {
  if (!args) return fail(MLRA_ERR_INVALID_ARG, "args is NULL");
  if (args->num_branches != 1)
    return fail(MLRA_ERR_INVALID_ARG, "mla_decode needs num_branches == 1 (got %d)", args->num_branches);
  return run_decode(args, stream);
}

mlra_status mlra_decode_prepare(const mlra_prepare_args* a, void* stream) {
  if (!a) return fail(MLRA_ERR_INVALID_ARG, "args is NULL");
  if (a->batch < 1 || a->num_heads < 1 || a->num_branches < 1 || a->branch_dim < 1 || a->head_dim < 1)
    return fail(MLRA_ERR_INVALID_ARG, "batch, num_heads, num_branches, branch_dim and head_dim must be >= 1");
  if (a->rope_dim < 0 || a->rope_dim % 2 || a->rope_dim > 256)
    return fail(MLRA_ERR_INVALID_ARG, "rope_dim must be even, >= 0 and <= 256 (got %d)", a->rope_dim);
  if (a->dtype != MLRA_BF16 && a->dtype != MLRA_F32) return fail(MLRA_ERR_INVALID_ARG, "dtype %d is not a mlra_dtype", a->dtype);
  if (!std::isfinite(a->rope_base) || !(a->rope_base > 0.f))
    return fail(MLRA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (!a->q_nope || !a->q_pe || !a->w_uk || !a->c_new || !a->k_pe_new || !a->positions || !a->q_lat || !a->q_rope ||
      !a->kv_lat || !a->kv_rope)
    return fail(MLRA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (a->row_stride < 1) return fail(MLRA_ERR_INVALID_ARG, "row_stride must be >= 1");
  const bool paged = a->page_table != nullptr;
  int64_t capacity;
  if (paged) {
    if (!is_pow2(a->page_size)) return fail(MLRA_ERR_INVALID_ARG, "page_size must be a power of two (got %d)", a->page_size);
    if (a->num_pages < 1 || a->max_pages < 1) return fail(MLRA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
    capacity = (int64_t)a->max_pages * a->page_size;
  } else {
    if (a->max_seq_len < 1) return fail(MLRA_ERR_INVALID_ARG, "max_seq_len must be >= 1");
    if (a->batch > 1 && a->seq_stride < (int64_t)(a->max_seq_len - 1) * a->row_stride + 1)
      return fail(MLRA_ERR_INVALID_ARG, "seq_stride is smaller than max_seq_len rows");
    capacity = a->max_seq_len;
  }
  if (a->positions_host) {
    for (int i = 0; i < a->batch; ++i)
      if (a->positions_host[i] < 0 || a->positions_host[i] >= capacity)
        return fail(MLRA_ERR_INVALID_ARG, "positions[%d] = %d is outside the cache (capacity %lld)", i,
                    a->positions_host[i], (long long)capacity);
  }
  const int64_t dc = (int64_t)a->num_branches * a->branch_dim;
  const int64_t eb = a->dtype == MLRA_BF16 ? 2 : 4;
  mlra::PrepareParams p{};
  p.B = a->batch;
  p.H = a->num_heads;
  p.NB = a->num_branches;
  p.DB = a->branch_dim;
  p.DR = a->rope_dim;
  p.DH = a->head_dim;
  p.dtype = a->dtype;
  p.mfma = a->dtype == MLRA_BF16 && mlra::prepare_mfma_supported(a->head_dim, (int)dc) && aligned(a->q_nope, 16) &&
           aligned(a->w_uk, 16);
  p.rope_base = a->rope_base;
  p.q_nope = a->q_nope;
  p.q_pe = a->q_pe;
  p.w_uk = a->w_uk;
  p.c_new = a->c_new;
  p.k_pe_new = a->k_pe_new;
  p.positions = a->positions;
  p.q_lat = a->q_lat;
  p.q_rope = a->q_rope;
  p.kv_lat = a->kv_lat;
  p.kv_rope = a->kv_rope;
  p.row_stride_b = a->row_stride * eb;
  p.seq_stride_b = a->seq_stride * eb;
  p.max_seq_len = a->max_seq_len;
  p.page_shift = paged ? ilog2(a->page_size) : 0;
  p.page_table = a->page_table;
  p.max_pages = a->max_pages;
  p.num_pages = a->num_pages;
  p.error_flags = a->error_flags;
  hipError_t e = mlra::launch_prepare(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prepare kernel launch");
  return ok();
}

int32_t mlra_read_probe_words(void) { return mlra::kProbeBlocks; }

mlra_status mlra_read_probe(const void* src, size_t bytes, uint32_t* out, int32_t out_words, void* stream) {
  if (!src || !out) return fail(MLRA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (bytes == 0 || bytes % 16 != 0) return fail(MLRA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 (got %zu)", bytes);
  if (!aligned(src, 16)) return fail(MLRA_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (out_words < mlra::kProbeBlocks)
    return fail(MLRA_ERR_INVALID_ARG, "out holds %d words, needs %d", out_words, mlra::kProbeBlocks);
  hipError_t e = mlra::launch_read_probe(src, (int64_t)bytes, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read probe launch");
  return ok();
}

mlra_status mlra_paged_append(void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* positions, const void* rows,
                              int32_t batch, int32_t dtype, uint32_t* error_flags, void* stream) {
  if (!pool || !page_table || !positions || !rows) return fail(MLRA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (batch < 1) return fail(MLRA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (dtype != MLRA_BF16 && dtype != MLRA_F32) return fail(MLRA_ERR_INVALID_ARG, "dtype %d is not a mlra_dtype", dtype);
  if (!is_pow2(page_size)) return fail(MLRA_ERR_INVALID_ARG, "page_size must be a power of two (got %d)", page_size);
  if (num_pages < 1 || max_pages < 1) return fail(MLRA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
  if (row_elems < 1 || row_stride < row_elems)
    return fail(MLRA_ERR_INVALID_ARG, "need 1 <= row_elems <= row_stride (got %d, %lld)", row_elems, (long long)row_stride);
  const int eb = dtype == MLRA_BF16 ? 2 : 4;
  hipError_t e = mlra::launch_paged_append(pool, row_stride, row_elems, page_size, num_pages, page_table, max_pages, positions,
                                           rows, batch, eb, error_flags, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "paged append launch");
  return ok();
}

mlra_status mlra_paged_gather(const void* pool, int64_t row_stride, int32_t row_elems, int32_t page_size, int32_t num_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens, int32_t max_seq_len,
                              int32_t batch, int32_t dtype, void* out, uint32_t* error_flags, void* stream) {
  if (!pool || !page_table || !seq_lens || !out) return fail(MLRA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (batch < 1 || max_seq_len < 1) return fail(MLRA_ERR_INVALID_ARG, "batch and max_seq_len must be >= 1");
  if (dtype != MLRA_BF16 && dtype != MLRA_F32) return fail(MLRA_ERR_INVALID_ARG, "dtype %d is not a mlra_dtype", dtype);
  if (!is_pow2(page_size)) return fail(MLRA_ERR_INVALID_ARG, "page_size must be a power of two (got %d)", page_size);
  if (num_pages < 1 || max_pages < 1) return fail(MLRA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
  if (row_elems < 1 || row_stride < row_elems)
    return fail(MLRA_ERR_INVALID_ARG, "need 1 <= row_elems <= row_stride (got %d, %lld)", row_elems, (long long)row_stride);
  const int eb = dtype == MLRA_BF16 ? 2 : 4;
  hipError_t e = mlra::launch_paged_gather(pool, row_stride, row_elems, page_size, num_pages, page_table, max_pages, seq_lens,
                                           max_seq_len, batch, eb, out, error_flags, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "paged gather launch");
  return ok();
}

mlra_status mlra_page_table_check(const int32_t* page_table, int32_t batch, int32_t max_pages, const int32_t* seq_lens,
                                  int32_t page_size, int32_t num_pages) {
  if (!page_table || !seq_lens) return fail(MLRA_ERR_INVALID_ARG, "page_table and seq_lens must be host pointers");
  if (batch < 1 || max_pages < 1 || num_pages < 1) return fail(MLRA_ERR_INVALID_ARG, "batch, max_pages, num_pages must be >= 1");
  if (!is_pow2(page_size)) return fail(MLRA_ERR_INVALID_ARG, "page_size must be a power of two (got %d)", page_size);
  std::vector<int32_t> owner(num_pages, -1);
  for (int b = 0; b < batch; ++b) {
    const int L = seq_lens[b];
    if (L < 0) return fail(MLRA_ERR_INVALID_ARG, "seq_lens[%d] = %d is negative", b, L);
    const int64_t need = cdiv(L, page_size);
    if (need > max_pages)
      return fail(MLRA_ERR_INVALID_ARG, "sequence %d needs %lld pages, the table has %d", b, (long long)need, max_pages);
    for (int64_t j = 0; j < need; ++j) {
      const int32_t pg = page_table[(int64_t)b * max_pages + j];
      if (pg < 0 || pg >= num_pages)
        return fail(MLRA_ERR_INVALID_ARG, "page_table[%d][%lld] = %d is outside [0, %d)", b, (long long)j, pg, num_pages);
      const int32_t key = b * max_pages + (int32_t)j;
      if (owner[pg] != -1)
        return fail(MLRA_ERR_INVALID_ARG, "page %d backs both [%d][%d] and [%d][%lld]", pg, owner[pg] / max_pages,
                    owner[pg] % max_pages, b, (long long)j);
      owner[pg] = key;
    }
  }
  return ok();
}

mlra_status mlra_page_pool_create(int32_t num_pages, mlra_page_pool** out) {
  if (!out) return fail(MLRA_ERR_INVALID_ARG, "out is NULL");
  if (num_pages < 1) return fail(MLRA_ERR_INVALID_ARG, "num_pages must be >= 1 (got %d)", num_pages);
  mlra_page_pool* p = new (std::nothrow) mlra_page_pool;
  if (!p) return fail(MLRA_ERR_INVALID_ARG, "out of host memory");
  p->num_pages = num_pages;
  p->free_list.resize(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) p->free_list[i] = num_pages - 1 - i;   // page 0 on top
  p->allocated.assign(num_pages, 0);
  *out = p;
  return ok();
}

mlra_status mlra_page_pool_alloc(mlra_page_pool* pool, int32_t n, int32_t* ids) {
  if (!pool) return fail(MLRA_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return fail(MLRA_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (n > 0 && !ids) return fail(MLRA_ERR_INVALID_ARG, "ids is NULL");
  if ((size_t)n > pool->free_list.size())
    return fail(MLRA_ERR_NO_PAGES, "asked for %d pages, %zu free", n, pool->free_list.size());
  for (int32_t i = 0; i < n; ++i) {
    ids[i] = pool->free_list.back();
    pool->free_list.pop_back();
    pool->allocated[ids[i]] = 1;
  }
  return ok();
}

mlra_status mlra_page_pool_free(mlra_page_pool* pool, int32_t n, const int32_t* ids) {
  if (!pool) return fail(MLRA_ERR_INVALID_ARG, "pool is NULL");
  if (n < 0) return fail(MLRA_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
  if (n > 0 && !ids) return fail(MLRA_ERR_INVALID_ARG, "ids is NULL");
  std::vector<uint8_t> seen(pool->num_pages, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= pool->num_pages) return fail(MLRA_ERR_INVALID_ARG, "page id %d is outside [0, %d)", id, pool->num_pages);
    if (!pool->allocated[id]) return fail(MLRA_ERR_INVALID_ARG, "page %d is not allocated (double free?)", id);
    if (seen[id]) return fail(MLRA_ERR_INVALID_ARG, "page %d appears twice in one free call", id);
    seen[id] = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->allocated[ids[i]] = 0;
    pool->free_list.push_back(ids[i]);
  }
  return ok();
}

int32_t mlra_page_pool_num_free(const mlra_page_pool* pool) { return pool ? (int32_t)pool->free_list.size() : 0; }

void mlra_page_pool_destroy(mlra_page_pool* pool) { delete pool; }

}  // extern "C"
