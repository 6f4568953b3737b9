// Host-side driver of libmlra's C ABI for the sanitizer build: argument validation, launch
// planning (ragged, paged, many sequences, extreme lengths), the plan query with mocked CU
// counts, the page-table check and the page pool. It makes no GPU call: every entry point it
// uses runs on the host (a plan for the current device falls back to the largest gfx950 part
// when no device is present). Exit status 0 when every expectation holds; AddressSanitizer and
// UndefinedBehaviorSanitizer abort the process on any memory or UB error they catch.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "mlra.h"

static int g_fail = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static const uintptr_t kFake = uintptr_t(1) << 20;   // aligned stand-in device addresses, never dereferenced

static mlra_decode_args base(int B, int H, int NB, int DB, int DR, int DH, int L, int dtype) {
  mlra_decode_args a;
  std::memset(&a, 0, sizeof(a));
  a.batch = B; a.num_heads = H; a.num_branches = NB; a.branch_dim = DB; a.rope_dim = DR; a.head_dim = DH;
  a.dtype = a.out_dtype = dtype;
  a.sm_scale = 0.125f; a.alpha = 0.5f;
  const int eb = dtype == MLRA_BF16 ? 2 : 4;
  a.q_lat = (const void*)kFake; a.q_rope = (const void*)(2 * kFake);
  a.kv_lat = (const void*)(4 * kFake); a.kv_rope = (const void*)(4 * kFake + (uintptr_t)NB * DB * eb);
  a.row_stride = NB * DB + DR; a.seq_stride = (int64_t)L * a.row_stride;
  a.seq_lens = (const int32_t*)(8 * kFake); a.max_seq_len = L;
  a.w_v = (const void*)(16 * kFake); a.out = (void*)(32 * kFake);
  a.workspace = (void*)(64 * kFake);
  return a;
}

static void planning() {
  std::mt19937 rng(7);
  const int shapes[][6] = {{4, 32, 32, 64, 128, 0}, {1, 128, 32, 64, 128, 0}, {1, 32, 32, 16, 128, 0},
                           {2, 64, 32, 64, 128, 0}, {3, 16, 16, 8, 64, 1}, {4, 16, 16, 8, 64, 1}, {1, 128, 32, 16, 128, 0}};
  for (const auto& sh : shapes) {
    for (int trial = 0; trial < 40; ++trial) {
      const int B = 1 + (int)(rng() % (trial < 20 ? 64 : 2048));
      std::vector<int32_t> lens(B);
      int Lmax = 1;
      for (int b = 0; b < B; ++b) {
        const int kind = (int)(rng() % 4);
        lens[b] = kind == 0 ? 1 : kind == 1 ? 1 + (int)(rng() % 100) : kind == 2 ? 1 + (int)(rng() % 70000) : 1 << (10 + (int)(rng() % 10));
        Lmax = lens[b] > Lmax ? lens[b] : Lmax;
      }
      const int dtype = sh[5] ? MLRA_F32 : MLRA_BF16;
      mlra_decode_args a = base(B, sh[3], sh[0], sh[1], sh[2], sh[4], Lmax, dtype);
      a.seq_lens_host = lens.data();
      if (trial % 3 == 0) a.num_splits = 1 + (int)(rng() % 64);
      const size_t ws = mlra_decode_workspace_size(&a);
      mlra_plan_info info;
      for (int cus : {0, 1, 32, 80, 128, 200, 256}) {
        const mlra_status st = mlra_decode_plan(&a, cus, &info);
        if (st != MLRA_OK) continue;   // some random shapes exceed the split or merge limits on some devices
        if (cus == 0) EXPECT(info.workspace_bytes == ws);   // the call plans for the current device
        EXPECT(info.num_splits >= 1 && info.split_tokens >= 1);
        EXPECT((int64_t)info.num_splits * info.split_tokens >= Lmax);
        EXPECT(info.cu_count == (cus ? cus : 256));
        if (info.kernel == MLRA_KERNEL_MFMA && a.num_splits == 0 && info.num_splits > 1) EXPECT(info.work_groups <= info.cu_count);
      }
      a.workspace_bytes = ws;
      if (ws) EXPECT(mlra_decode_validate(&a) == MLRA_OK);
      // paged variant of the same lengths
      std::vector<int32_t> pt;
      const int ps = 1 << (4 + (int)(rng() % 7));
      const int max_pages = (Lmax + ps - 1) / ps;
      pt.assign((size_t)B * max_pages, -1);
      int next = 0;
      for (int b = 0; b < B; ++b)
        for (int j = 0; j < (lens[b] + ps - 1) / ps; ++j) pt[(size_t)b * max_pages + j] = next++;
      EXPECT(mlra_page_table_check(pt.data(), B, max_pages, lens.data(), ps, next) == MLRA_OK);
      if (next > 1) {
        pt[0] = next - 1;   // duplicate page
        EXPECT(mlra_page_table_check(pt.data(), B, max_pages, lens.data(), ps, next) != MLRA_OK || lens[0] == 0);
      }
      a.page_table = (const int32_t*)(128 * kFake);
      a.page_size = ps;
      a.max_pages = max_pages;
      a.num_pages = next > 0 ? next : 1;
      const size_t wsp = mlra_decode_workspace_size(&a);
      if (wsp) EXPECT(mlra_decode_plan(&a, 256, &info) == MLRA_OK);
    }
  }
  // invalid arguments: every path returns an error, none crashes
  mlra_decode_args a = base(2, 64, 4, 32, 32, 128, 4096, MLRA_BF16);
  std::vector<int32_t> bad = {0, 5000};
  a.seq_lens_host = bad.data();
  EXPECT(mlra_decode_validate(&a) == MLRA_ERR_INVALID_ARG);
  EXPECT(mlra_decode_workspace_size(&a) == 0);
  EXPECT(std::strlen(mlra_last_error()) > 0);
  mlra_plan_info info;
  EXPECT(mlra_decode_plan(nullptr, 256, &info) == MLRA_ERR_INVALID_ARG);
  EXPECT(mlra_decode_validate(nullptr) == MLRA_ERR_INVALID_ARG);
}

static void pages() {
  mlra_page_pool* pool = nullptr;
  EXPECT(mlra_page_pool_create(1000, &pool) == MLRA_OK);
  std::vector<int32_t> ids(1000);
  std::mt19937 rng(3);
  std::vector<int32_t> held;
  for (int it = 0; it < 2000; ++it) {
    if (rng() % 2 && !held.empty()) {
      const int n = 1 + (int)(rng() % held.size());
      std::vector<int32_t> back(held.end() - n, held.end());
      EXPECT(mlra_page_pool_free(pool, n, back.data()) == MLRA_OK);
      held.resize(held.size() - n);
      EXPECT(mlra_page_pool_free(pool, 1, back.data()) == MLRA_ERR_INVALID_ARG);   // double free
    } else {
      const int n = (int)(rng() % 64);
      const mlra_status st = mlra_page_pool_alloc(pool, n, ids.data());
      if (st == MLRA_OK) held.insert(held.end(), ids.begin(), ids.begin() + n);
      else EXPECT(st == MLRA_ERR_NO_PAGES);
    }
    EXPECT(mlra_page_pool_num_free(pool) == 1000 - (int)held.size());
  }
  int32_t oob = 1000;
  EXPECT(mlra_page_pool_free(pool, 1, &oob) == MLRA_ERR_INVALID_ARG);
  mlra_page_pool_destroy(pool);
}

int main() {
  planning();
  pages();
  std::printf("host sanitizer driver: %s (%d failures)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
