// Host-only check of the cache planning code (plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_host.py. Exits non-zero on the first failure.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "plan.h"

#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                      \
    }                                                                    \
  } while (0)

static rswa_cache_desc desc(int B, const std::vector<int32_t>& m, const std::vector<int32_t>& cap,
                            int mode, int paged, int dtype) {
  rswa_cache_desc d{};
  d.batch = B;
  d.num_heads = 16;
  d.head_dim = 128;
  d.kv_dtype = dtype;
  d.mode = mode;
  d.prefix_len = m.data();
  d.window = mode == RSWA_MODE_RSWA ? cap.data() : nullptr;
  d.max_steps = mode == RSWA_MODE_FULL_CAUSAL ? cap.data() : nullptr;
  d.prefix_paged = paged;
  return d;
}

int main() {
  std::mt19937 rng(7);
  // layouts: offsets back to back, rows, prefix table offsets, bytes
  for (int it = 0; it < 2000; ++it) {
    const int B = 1 + (int)(rng() % 64);
    std::vector<int32_t> m(B), cap(B);
    for (int b = 0; b < B; ++b) {
      m[b] = (int32_t)(rng() % 3000);
      cap[b] = 1 + (int32_t)(rng() % 600);
    }
    const int mode = (rng() & 1) ? RSWA_MODE_RSWA : RSWA_MODE_FULL_CAUSAL;
    const int paged = (int)(rng() & 1);
    const int dtype = (rng() & 1) ? RSWA_BF16 : RSWA_F32;
    const rswa_cache_desc d = desc(B, m, cap, mode, paged, dtype);
    rswa::Plan p;
    std::string why;
    CHECK(rswa::make_plan(&d, &p, &why) == RSWA_OK);
    const int64_t e = dtype == RSWA_F32 ? 4 : 2;
    int64_t off = 0, pre = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t R = paged ? cap[b] : (int64_t)m[b] + cap[b];
      CHECK(p.rows[b] == R);
      CHECK(p.seq_off[b] == off);
      CHECK(p.prefix_row0[b] == pre);
      CHECK(p.prefix[b] == m[b] && p.cap[b] == cap[b]);
      off += 2 * 16 * R * 128;
      pre += m[b];
    }
    CHECK(p.total_prefix_rows == pre);
    CHECK(p.bytes == (uint64_t)(off * e) + rswa::kStorageTailBytes);
  }
  // invalid descriptions are rejected with a reason
  {
    std::vector<int32_t> m{5, -1}, cap{4, 4};
    rswa_cache_desc d = desc(2, m, cap, RSWA_MODE_RSWA, 0, RSWA_BF16);
    rswa::Plan p;
    std::string why;
    CHECK(rswa::make_plan(&d, &p, &why) == RSWA_E_INVALID && !why.empty());
    m[1] = 3;
    cap[0] = 0;
    CHECK(rswa::make_plan(&d, &p, &why) == RSWA_E_INVALID);
    cap[0] = 4;
    d.prefix_paged = 3;
    CHECK(rswa::make_plan(&d, &p, &why) == RSWA_E_INVALID);
    d.prefix_paged = 0;
    d.head_dim = 64;
    CHECK(rswa::make_plan(&d, &p, &why) == RSWA_E_UNSUPPORTED);
    d.head_dim = 128;
    d.batch = rswa::kMaxBatch + 1;
    CHECK(rswa::make_plan(&d, &p, &why) == RSWA_E_INVALID);
    CHECK(rswa::make_plan(nullptr, &p, &why) == RSWA_E_INVALID);
  }
  // decode split: pieces cover every row, the grid fits the workspace, aligned only when uniform
  for (int it = 0; it < 20000; ++it) {
    const int B = 1 + (int)(rng() % 200);
    const int H = 1 + (int)(rng() % 32);
    const bool uniform = rng() % 3 == 0;
    std::vector<int64_t> L(B);
    const int64_t base = (int64_t)(rng() % 9000);
    for (int b = 0; b < B; ++b) L[b] = uniform ? base : (int64_t)(rng() % 9000);
    const int64_t resident = 1 + (int64_t)(rng() % 4096);
    const int64_t grid_max = 1 + (int64_t)(rng() % 4096);
    const int32_t min_rows = (rng() % 4 == 0) ? 1 + (int32_t)(rng() % 512) : 0;
    const int32_t grid_user = (rng() % 4 == 0) ? 1 + (int32_t)(rng() % 5000) : 0;
    const bool masked = rng() % 5 == 0;
    const rswa::DecodePlan dp =
        rswa::plan_decode(L, H, resident, grid_max, min_rows, grid_user, masked);
    int64_t total = 0;
    for (int b = 0; b < B; ++b) total += H * L[b];
    if (total == 0) {
      CHECK(dp.grid == 0);
      continue;
    }
    CHECK(dp.grid >= 1);
    if (dp.aligned) {
      CHECK(!masked && min_rows == 0 && grid_user == 0);
      for (int b = 0; b < B; ++b) CHECK(L[b] == L[0]);
      CHECK(dp.grid == (int64_t)B * H && !dp.stream_k && dp.split == 0);
      CHECK(dp.grid <= std::min(resident, grid_max));
    } else if (dp.split > 0) {
      CHECK(!masked && min_rows == 0 && grid_user == 0 && !dp.stream_k);
      for (int b = 0; b < B; ++b) CHECK(L[b] == L[0]);
      CHECK(dp.split >= 2 && dp.grid == (int64_t)B * H * dp.split);
      CHECK(dp.grid <= std::min(resident, grid_max));
      CHECK(L[0] >= 64 * (int64_t)dp.split);  // every piece holds at least the minimum rows
    } else {
      CHECK(dp.stream_k);
      CHECK(dp.rows_per_piece >= (min_rows > 0 ? min_rows : 64));
      CHECK(dp.grid * dp.rows_per_piece >= total);
      CHECK((dp.grid - 1) * dp.rows_per_piece < total);
      CHECK(dp.grid <= grid_max);
    }
  }
  std::puts("plan host check: ok");
  return 0;
}
