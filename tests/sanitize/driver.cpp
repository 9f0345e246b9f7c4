// Exercise the C ABI's host code under the address and undefined-behaviour
// sanitizers: the host slot table over long streams with manual evictions
// (checked against the closed form of the FIFO ring where it applies), the
// segment lists, argument validation of every entry point, and cache
// creation (which fails cleanly on a machine without a GPU).  Exit status 0
// on success; any sanitizer report aborts the run.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/kvc.h"
#include "../../include/kvc_tools.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                   \
    }                                                                 \
  } while (0)

static void table_stream(int W, int S, unsigned seed) {
  kvc_table_handle t = nullptr;
  CHECK(kvc_table_create(W, S, &t) == KVC_OK && t);
  std::vector<int64_t> slots(S + W + 3);
  bool manual = false;
  for (int c = 0; c < 400; ++c) {
    seed = seed * 1103515245u + 12345u;
    if ((seed >> 16) % 7 == 0 && c > S) {
      int64_t ids[64];
      int n = 0, occ = 0;
      CHECK(kvc_table_query(t, nullptr, &occ, nullptr, 0) == KVC_OK);
      const int win = occ - (c < S ? c : S);
      const int want = win > 0 ? 1 + (int)((seed >> 8) % win) : 0;
      CHECK(kvc_table_evict(t, want, ids, &n) == KVC_OK && n == want);
      for (int i = 1; i < n; ++i) CHECK(ids[i] > ids[i - 1]);
      CHECK(kvc_table_evict(t, win + 1 - n, ids, &n) == KVC_ERR_STATE);
      manual = manual || want > 0;
    }
    int64_t id = -2, ev = -2;
    int slot = -2;
    CHECK(kvc_table_append(t, &id, &slot, &ev) == KVC_OK);
    CHECK(id == c && slot >= 0 && slot < S + W);
    if (!manual) {  // closed form of the ring while no chunk was evicted by hand
      if (c < S) {
        CHECK(slot == c && ev == -1);
      } else {
        CHECK(slot == S + (c - S) % W);
        CHECK(ev == (c - S >= W ? c - W : -1));
      }
    }
    int64_t next = -1;
    int occ = -1;
    CHECK(kvc_table_query(t, &next, &occ, slots.data(), (int)slots.size()) == KVC_OK);
    CHECK(next == c + 1 && occ >= 1 && occ <= S + W);
    int32_t row0[80], len[80];
    int ns = -1;
    CHECK(kvc_table_segments(t, 100, 20, c & 1, row0, len, 80, &ns) == KVC_OK);
    CHECK(ns >= 1 && ns <= 1 + S + W);
    if (ns > 1) CHECK(kvc_table_segments(t, 100, 20, 0, row0, len, 0, &ns) == KVC_ERR_INVALID);
  }
  CHECK(kvc_table_reset(t) == KVC_OK);
  int occ = -1;
  CHECK(kvc_table_query(t, nullptr, &occ, nullptr, 0) == KVC_OK && occ == 0);
  CHECK(kvc_table_destroy(t) == KVC_OK);
}

int main() {
  const int ws[][2] = {{4, 1}, {8, 1}, {1, 1}, {3, 2}, {5, 0}, {63, 1}, {1, 0}};
  unsigned seed = 7;
  for (auto& p : ws) table_stream(p[0], p[1], seed++);
  kvc_table_handle t = nullptr;
  CHECK(kvc_table_create(0, 1, &t) == KVC_ERR_INVALID && t == nullptr);
  CHECK(kvc_table_create(64, 1, &t) == KVC_ERR_INVALID && t == nullptr);
  CHECK(kvc_table_create(2, 1, nullptr) == KVC_ERR_INVALID);
  CHECK(std::strlen(kvc_last_error()) > 0);
  CHECK(kvc_table_append(nullptr, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kvc_table_segments(nullptr, 1, 0, 1, nullptr, nullptr, 0, nullptr) == KVC_ERR_INVALID);

  // create: every rejected argument, then a valid one
  kvc_handle h = nullptr;
  const int bad[][7] = {{0, 4, 1, 0, 1, 128, 0},  {64, 0, 1, 0, 1, 128, 0}, {64, 4, -1, 0, 1, 128, 0},
                        {64, 4, 1, -1, 1, 128, 0}, {64, 4, 1, 0, 0, 128, 0}, {64, 64, 1, 0, 1, 128, 0},
                        {8, 63, 1, 1 << 30, 1, 128, 0}};
  for (auto& b : bad) {
    CHECK(kv_cache_create(b[0], b[1], b[2], b[3], b[4], b[5], b[6], &h) == KVC_ERR_INVALID && h == nullptr);
    CHECK(std::strlen(kvc_last_error()) > 0);
  }
  CHECK(kv_cache_create(64, 4, 1, 0, 1, 96, 0, &h) == KVC_ERR_UNSUPPORTED && h == nullptr);
  CHECK(kv_cache_create(64, 4, 1, 0, 1, 128, 7, &h) == KVC_ERR_UNSUPPORTED && h == nullptr);
  CHECK(kv_cache_create(60, 4, 1, 0, 1, 128, KVC_KV_FP8, &h) == KVC_ERR_UNSUPPORTED && h == nullptr);
  CHECK(kv_cache_create_layers(64, 4, 1, 0, 1, 128, 0, 0, &h) == KVC_ERR_INVALID && h == nullptr);
  CHECK(kv_cache_create_layers(64, 4, 1, 0, 1 << 11, 128, 0, 1 << 10, &h) == KVC_ERR_INVALID && h == nullptr);
  const int rc = kv_cache_create(64, 4, 1, 16, 2, 128, 0, &h);
  if (rc == KVC_OK) {  // a machine with a GPU: the handle is usable and frees cleanly
    int64_t next = -1;
    CHECK(kv_cache_query(h, &next, nullptr, nullptr, 0) == KVC_OK && next == 0);
    CHECK(kv_cache_destroy(h) == KVC_OK);
  } else {
    CHECK((rc == KVC_ERR_HIP || rc == KVC_ERR_OOM) && h == nullptr);
  }
  // every entry point rejects a NULL handle without touching anything
  int i = -3;
  size_t n = 7;
  CHECK(kv_cache_destroy(nullptr) == KVC_OK);
  CHECK(kv_cache_evict(nullptr, 1, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_reset(nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_query(nullptr, nullptr, nullptr, nullptr, 0) == KVC_ERR_INVALID);
  CHECK(kv_cache_set_condition(nullptr, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_set_condition_rows(nullptr, 0, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_append_chunk(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_write_chunk(nullptr, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_append_commit(nullptr, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_layer(nullptr, 0, nullptr) == KVC_ERR_INVALID);
  CHECK(sink_window_attention(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f, nullptr) ==
        KVC_ERR_INVALID);
  CHECK(sink_window_attention_rows(nullptr, 5, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f, nullptr) ==
        KVC_ERR_INVALID);
  CHECK(sink_window_attention_chunks(nullptr, 2, nullptr, nullptr, nullptr, nullptr, nullptr, 0.f, nullptr, 0,
                                     nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_config_count(nullptr, &i) == KVC_ERR_INVALID && i == -3);
  CHECK(kv_cache_config_info(nullptr, 0, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kv_cache_set_config(nullptr, 0) == KVC_ERR_INVALID);
  CHECK(kv_cache_get_config(nullptr, &i) == KVC_ERR_INVALID && i == -3);
  CHECK(kv_cache_autotune(nullptr, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, nullptr) ==
        KVC_ERR_INVALID);
  CHECK(kvc_chunks_workspace_bytes(nullptr, 2, &n) == KVC_ERR_INVALID && n == 7);
  CHECK(kv_cache_pool_view(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == KVC_ERR_INVALID);
  CHECK(kvc_probe_copy(nullptr, nullptr, 16, nullptr) == KVC_ERR_INVALID);
  CHECK(kvc_probe_mfma_bf16(nullptr, 1, 1, nullptr) == KVC_ERR_INVALID);
  std::printf("sanitized host checks passed\n");
  return 0;
}
