// Host-only cache planning: descriptor validation, storage layout and decode split policy.
// Pure C++ (no HIP calls), so it is also built and sanitizer-tested on the CPU.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "rswa.h"

namespace rswa {

constexpr int32_t kMaxBatch = 4096;
constexpr int32_t kMaxHeads = 1024;
constexpr int32_t kPlanHeadDim = 128;

struct Plan {
  std::vector<int64_t> seq_off;   // element offset of sequence b's K block
  std::vector<int32_t> rows;      // R_b = m_b + cap_b
  std::vector<int32_t> prefix;    // m_b
  std::vector<int32_t> cap;       // n_b (R-SWA) or max_steps_b (full causal)
  std::vector<int64_t> prefix_row0; // first packed prefix row of sequence b
  int64_t total_prefix_rows = 0;
  int32_t max_prefix = 0;
  uint64_t bytes = 0;
  int32_t elem = 0;
};

// Validates `d` and fills `p`. On failure returns the status and a reason in `why`.
rswa_status make_plan(const rswa_cache_desc* d, Plan* p, std::string* why);

// Decode items (one per (b, h, chunk)) for the given live row counts.
int64_t decode_items(const std::vector<int64_t>& live_rows, int32_t heads, int32_t chunk);

// Automatic chunk size: the largest of 512, 256, 128, 64 rows that still yields at least
// `min_items` items at the cache's full size, else 64.
int32_t auto_chunk(const Plan& p, int32_t heads, int64_t min_items);

// Split slots per (b, h) that the workspace must hold for chunks of `chunk` rows.
int32_t split_slots(const Plan& p, int32_t chunk);

}  // namespace rswa
