// The host layer of the library under AddressSanitizer and
// UndefinedBehaviorSanitizer. ts_api.cpp is built with host-side sanitizers
// and linked against stand-in launchers (stub_launchers.cpp), so every entry
// point runs its argument checks, planning, workspace carving and launch
// sequencing on the CPU. The "device" buffers handed in are a freed heap
// block: any host-side read or write of one is a use-after-free report.
//
// Swept: every *_workspace_size query over a grid of layouts, batch sizes and
// k (valid, invalid and extreme values, int32 limits included); for each
// valid plan the matching entry point with exactly that workspace (TS_OK, or
// TS_ERR_HIP where a HIP runtime call needs a device), one byte less
// (TS_ERR_WORKSPACE) and a missing tensor (TS_ERR_INVALID_ARG); the
// Selection-Cache and profiling calls with missing or out-of-range
// arguments. Exit status 0 when every call returned the expected class.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ts.h"

static int g_fail = 0, g_calls = 0;

#define EXPECT(cond, ...)                                          \
  do {                                                             \
    ++g_calls;                                                     \
    if (!(cond)) {                                                 \
      ++g_fail;                                                    \
      std::printf("FAIL line %d: ", __LINE__);                     \
      std::printf(__VA_ARGS__);                                    \
      std::printf(" (last error: %s)\n", ts_last_error());         \
    }                                                              \
  } while (0)

static bool ran(ts_status s) { return s == TS_OK || s == TS_ERR_HIP; }
static bool refused(ts_status s) { return s == TS_ERR_INVALID_ARG || s == TS_ERR_UNSUPPORTED; }

static void* g_dev = nullptr;   // freed heap block standing in for device memory

static ts_kv_layout layout(int Hq, int Hkv, int d, int dt, int ps, int max_len, int stride) {
  ts_kv_layout L;
  L.num_q_heads = Hq;
  L.num_kv_heads = Hkv;
  L.head_dim = d;
  L.dtype = dt;
  L.scale = 0.f;
  L.page_size = ps;
  L.max_len = max_len;
  L.page_table_stride = stride;
  return L;
}

// one (layout, batch, k) point: every sized entry point whose plan is valid
static void sweep_point(const ts_kv_layout& L, int batch, int k) {
  const int32_t* pt = L.page_size > 0 ? (const int32_t*)g_dev : nullptr;
  const int32_t* lens = (const int32_t*)g_dev;
  void* d = g_dev;
  size_t n = 0;
  ts_status st;

  st = ts_score_workspace_size(&L, batch, &n);
  if (st == TS_OK) {
    EXPECT(ran(ts_score(&L, batch, d, d, pt, lens, (float*)d, d, n, nullptr)), "score");
    if (n > 0) EXPECT(ts_score(&L, batch, d, d, pt, lens, (float*)d, d, n - 1, nullptr) == TS_ERR_WORKSPACE, "score ws-1");
    EXPECT(ts_score(&L, batch, nullptr, d, pt, lens, (float*)d, d, n, nullptr) == TS_ERR_INVALID_ARG, "score q null");
  } else {
    EXPECT(refused(st), "score_workspace_size status %d", st);
  }

  st = ts_sparse_attend_workspace_size(&L, batch, k, &n);
  if (st == TS_OK) {
    EXPECT(ran(ts_sparse_attend(&L, batch, d, d, d, pt, lens, (const int32_t*)d, k, (float*)d, d, n, nullptr)), "sparse_attend");
    if (n > 0) EXPECT(ts_sparse_attend(&L, batch, d, d, d, pt, lens, (const int32_t*)d, k, (float*)d, d, n - 1, nullptr) == TS_ERR_WORKSPACE, "sparse_attend ws-1");
    EXPECT(ts_sparse_attend(&L, batch, d, d, nullptr, pt, lens, (const int32_t*)d, k, (float*)d, d, n, nullptr) == TS_ERR_INVALID_ARG, "sparse_attend v null");
  } else {
    EXPECT(refused(st), "sparse_attend_workspace_size status %d", st);
  }

  st = ts_dense_attend_workspace_size(&L, batch, &n);
  if (st == TS_OK) {
    EXPECT(ran(ts_dense_attend(&L, batch, d, d, d, pt, lens, (float*)d, d, n, nullptr)), "dense_attend");
    if (n > 0) EXPECT(ts_dense_attend(&L, batch, d, d, d, pt, lens, (float*)d, d, n - 1, nullptr) == TS_ERR_WORKSPACE, "dense ws-1");
  } else {
    EXPECT(refused(st), "dense_attend_workspace_size status %d", st);
  }

  st = ts_decode_step_workspace_size(&L, batch, k, &n);
  EXPECT(st == TS_OK || refused(st), "decode_step_workspace_size status %d", st);
  EXPECT(ts_decode_step(nullptr, &L, batch, d, d, d, pt, lens, 0.9, (float*)d, nullptr, nullptr, d, n, nullptr) == TS_ERR_INVALID_ARG, "decode_step without a cache");
  EXPECT(ts_decode_step_noalloc(nullptr, &L, batch, d, d, d, pt, lens, 0.9, (float*)d, nullptr, nullptr, nullptr) == TS_ERR_INVALID_ARG, "noalloc without a cache");

  if (L.page_size > 0) {
    EXPECT(ran(ts_append_kv(&L, batch, d, d, d, d, pt, (int32_t*)d, nullptr)) || refused(ts_append_kv(&L, batch, d, d, d, d, pt, (int32_t*)d, nullptr)), "append paged");
    const int kp = k > 0 ? (int)(((long)k + L.page_size - 1) / L.page_size) : k;
    st = ts_quest_select_workspace_size(&L, batch, kp, &n);
    if (st == TS_OK) {
      EXPECT(ran(ts_quest_meta(&L, batch, d, pt, lens, 0, d, nullptr)), "quest_meta");
      EXPECT(ran(ts_quest_select(&L, batch, d, d, pt, lens, kp, (float*)d, (int32_t*)d, d, n, nullptr)), "quest_select");
      if (n > 0) EXPECT(ts_quest_select(&L, batch, d, d, pt, lens, kp, (float*)d, (int32_t*)d, d, n - 1, nullptr) == TS_ERR_WORKSPACE, "quest_select ws-1");
    } else {
      EXPECT(refused(st), "quest_select_workspace_size status %d", st);
    }
    st = ts_quest_attend_workspace_size(&L, batch, kp, &n);
    if (st == TS_OK) {
      EXPECT(ran(ts_quest_attend(&L, batch, d, d, d, pt, lens, (const int32_t*)d, kp, (float*)d, d, n, nullptr)), "quest_attend");
    } else {
      EXPECT(refused(st), "quest_attend_workspace_size status %d", st);
    }
  } else {
    st = ts_append_kv(&L, batch, d, d, d, d, nullptr, (int32_t*)d, nullptr);
    EXPECT(ran(st) || refused(st), "append status %d", st);
    // chunked prefill over a contiguous cache: a chunk at the end of the context
    const int n_ctx = L.max_len;
    const int chunk = batch;
    st = ts_score_prefill_workspace_size(&L, chunk, n_ctx, k, &n);
    if (st == TS_OK) {
      const int q0 = n_ctx - chunk;
      EXPECT(ran(ts_score_prefill(&L, chunk, q0, d, d, n_ctx, (float*)d, d, n, nullptr)), "score_prefill");
      EXPECT(ran(ts_select_prefill(&L, chunk, q0, d, d, n_ctx, k, (float*)d, (int32_t*)d, d, n, nullptr)), "select_prefill");
      if (n > 0) EXPECT(ts_select_prefill(&L, chunk, q0, d, d, n_ctx, k, (float*)d, (int32_t*)d, d, n - 1, nullptr) == TS_ERR_WORKSPACE, "select_prefill ws-1");
      if (q0 < INT_MAX)
        EXPECT(refused(ts_select_prefill(&L, chunk, q0 + 1, d, d, n_ctx, k, (float*)d, (int32_t*)d, d, n, nullptr)), "prefill past the context");
    } else {
      EXPECT(refused(st), "score_prefill_workspace_size status %d", st);
    }
    st = ts_sparse_attend_prefill_workspace_size(&L, chunk, k, &n);
    if (st == TS_OK && chunk <= n_ctx) {
      EXPECT(ran(ts_sparse_attend_prefill(&L, chunk, n_ctx - chunk, d, d, d, n_ctx, (const int32_t*)d, k, (float*)d, d, n, nullptr)), "sparse_attend_prefill");
    } else if (st != TS_OK) {
      EXPECT(refused(st), "sparse_attend_prefill_workspace_size status %d", st);
    }
  }
}

int main() {
  g_dev = std::malloc(4096);
  std::free(g_dev);   // poisoned from here on

  EXPECT(ts_abi_version() == TS_ABI_VERSION, "abi version");
  for (int s = -3; s < 12; ++s) EXPECT(ts_status_string(s) != nullptr, "status string %d", s);
  EXPECT(ts_last_error() != nullptr, "last error");

  const int Hqs[] = {1, 4, 7, 28, 32, 64, 128, 0, -4};
  const int Hkvs[] = {1, 2, 4, 8, 16, 3, 0};
  const int ds[] = {64, 128, 96, 0};
  const int dts[] = {TS_F32, TS_BF16, 7, -1};
  const int pss[] = {0, 1, 16, 64, 12, -16};
  const int lens[] = {1, 4096, 131072, 1 << 24, INT_MAX, 0, -1};
  const int batches[] = {1, 8, 512, 4096, 0, -1, INT_MAX};
  const int ks[] = {1, 2048, 1 << 20, INT_MAX, 0, -5};
  long points = 0;
  for (int Hq : Hqs)
    for (int Hkv : Hkvs)
      for (int d : ds)
        for (int dt : dts)
          for (int ps : pss)
            for (int ml : lens) {
              const long stride = ps > 0 ? ((long)ml + ps - 1) / ps : 0;
              const ts_kv_layout L = layout(Hq, Hkv, d, dt, ps, ml, stride > INT_MAX ? INT_MAX : (int)stride);
              // the full batch/k grid on the supported shapes, one point elsewhere
              const bool main_shape = (d == 64 || d == 128) && (dt == TS_F32 || dt == TS_BF16) && Hq > 0 &&
                                      Hkv > 0 && Hq % Hkv == 0;
              for (int b : batches)
                for (int k : ks) {
                  if (!main_shape && (b != 1 || k != 2048)) continue;
                  sweep_point(L, b, k);
                  ++points;
                }
            }
  // a paged layout whose page-table rows are too short for max_len
  {
    const ts_kv_layout L = layout(28, 4, 128, TS_BF16, 16, 4096, 8);
    size_t n = 0;
    EXPECT(refused(ts_score_workspace_size(&L, 1, &n)) || refused(ts_score(&L, 1, g_dev, g_dev, (const int32_t*)g_dev, (const int32_t*)g_dev, (float*)g_dev, g_dev, 1 << 30, nullptr)),
           "short page-table rows");
  }
  // top-k on its own
  for (int rows : {1, 8, 512, 0, -1, INT_MAX})
    for (int stride : {1, 1000, 131072, 1 << 24, 0, -3})
      for (int k : {1, 64, 4096, 1 << 20, 0, -1}) {
        size_t n = 0;
        const ts_status st = ts_topk_workspace_size(rows, stride, k, &n);
        if (st == TS_OK) {
          EXPECT(ran(ts_topk(rows, stride, (const float*)g_dev, (const int32_t*)g_dev, k, (int32_t*)g_dev, g_dev, n, nullptr)), "topk");
          if (n > 0) EXPECT(ts_topk(rows, stride, (const float*)g_dev, (const int32_t*)g_dev, k, (int32_t*)g_dev, g_dev, n - 1, nullptr) == TS_ERR_WORKSPACE, "topk ws-1");
        } else {
          EXPECT(refused(st), "topk_workspace_size status %d", st);
        }
      }
  // Selection Cache: missing or invalid arguments (creation itself needs a device)
  ts_sel_cache* c = nullptr;
  for (int mb : {0, -1}) EXPECT(refused(ts_sel_cache_create(mb, 28, 128, 2048, 0, &c)), "create batch %d", mb);
  EXPECT(refused(ts_sel_cache_create(1, 28, 96, 2048, 0, &c)), "create head_dim 96");
  EXPECT(refused(ts_sel_cache_create(1, 28, 128, 0, 0, &c)), "create k 0");
  EXPECT(refused(ts_sel_cache_create(1, 28, 128, 2048, 5, &c)), "create mode 5");
  EXPECT(refused(ts_sel_cache_create(INT_MAX, 28, 128, 2048, 0, &c)), "create batch INT_MAX");
  EXPECT(refused(ts_sel_cache_create(1, 4096, 128, 2048, 0, &c)), "create 4096 heads");
  EXPECT(refused(ts_sel_cache_create(1, 28, 128, INT_MAX, 0, &c)), "create k INT_MAX");
  EXPECT(refused(ts_sel_cache_create(1, 28, 128, 2048, 0, nullptr)), "create out null");
  EXPECT(refused(ts_sel_cache_reset(nullptr, nullptr, nullptr)), "reset null");
  EXPECT(ts_sel_cache_destroy(nullptr) == TS_OK, "destroy null (a no-op, like free)");
  int64_t h[4], m[4];
  EXPECT(refused(ts_sel_cache_stats(nullptr, 4, h, m, nullptr)), "stats null");
  // profiling: names and counters of every kernel kind, out-of-range ids refused
  const int nk = ts_profile_num_kernels();
  EXPECT(nk > 0, "profile kernels");
  for (int i = -2; i < nk + 3; ++i) {
    const char* nm = ts_profile_kernel_name(i);
    int64_t launches = 0;
    double ms = 0;
    const ts_status st = ts_profile_read(i, &launches, &ms);
    if (i >= 0 && i < nk) {
      EXPECT(nm != nullptr && nm[0] != 0, "kernel name %d", i);
      EXPECT(st == TS_OK, "profile_read %d", i);
    } else {
      EXPECT(refused(st), "profile_read out of range %d", i);
    }
  }
  EXPECT(refused(ts_profile_read(0, nullptr, nullptr)), "profile_read null");
  EXPECT(ts_profile_reset() == TS_OK, "profile_reset");

  std::printf("%d calls over %ld sweep points, %d failed\n", g_calls, points, g_fail);
  return g_fail ? 1 : 0;
}
