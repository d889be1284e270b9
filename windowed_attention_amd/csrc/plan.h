// Host-only cache planning: descriptor validation, storage layout and decode split policy.
// Pure C++ (no HIP calls), so it is also built and sanitizer-tested on the CPU.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "rswa.h"

namespace rswa {

constexpr int32_t kMaxBatch = 2048;
constexpr int32_t kMaxHeads = 1024;
constexpr int32_t kPlanHeadDim = 128;
// Bytes after the last row of the storage that the decode kernel may read but never uses: its
// loads cover whole row tiles, and the last tile of the last range can pass the final row.
constexpr uint64_t kStorageTailBytes = 4096;
// MI355X's last-level cache (Infinity Cache, shared by all XCDs): a decode step whose rows exceed
// it reads them with non-temporal loads.
constexpr int64_t kLastLevelCacheBytes = 256LL << 20;

struct Plan {
  std::vector<int64_t> seq_off;   // element offset of sequence b's K block
  std::vector<int32_t> rows;      // R_b = m_b + cap_b (cap_b with a paged prefix)
  std::vector<int32_t> prefix;    // m_b
  std::vector<int32_t> cap;       // n_b (R-SWA) or max_steps_b (full causal)
  std::vector<int64_t> prefix_row0; // first packed prefix row (page-table entry) of sequence b
  int64_t total_prefix_rows = 0;
  int32_t max_prefix = 0;
  uint64_t bytes = 0;
  int32_t elem = 0;
};

// Validates `d` and fills `p`. On failure returns the status and a reason in `why`.
rswa_status make_plan(const rswa_cache_desc* d, Plan* p, std::string* why);

// How one decode launch splits its work (see decode.hip).
struct DecodePlan {
  bool aligned = false;  // one workgroup per (b, h) key range
  int64_t grid = 0;      // workgroups to launch (0: nothing to do)
  int64_t rows_per_piece = 0;  // stream-K piece size for the host's row counts
  bool stream_k = false;    // ranges cut into pieces (split ranges merged in the same launch)
  int32_t split = 0;        // > 1: every range cut into `split` equal pieces (grid = ranges x split)
};

// live_rows: per-sequence live rows (upper bounds) after the launch's append; resident: decode
// workgroups that fit the GPU at once; grid_max: workgroups the workspace holds; min_rows /
// grid_user: user settings (0 = automatic); masked: an active mask is in use (row counts are then
// only upper bounds, so the aligned and split layouts, which need equal ranges, are not chosen).
// Equal ranges that fill one round of resident workgroups get one workgroup each (aligned); fewer
// equal ranges are cut into k = min(resident / ranges, rows / minimum rows) >= 2 equal pieces each
// (split: every piece holds rows of one range only, so it publishes its partial once, at its end);
// anything else is cut into equal stream-K pieces.
DecodePlan plan_decode(const std::vector<int64_t>& live_rows, int32_t heads, int64_t resident,
                       int64_t grid_max, int32_t min_rows, int32_t grid_user, bool masked);

}  // namespace rswa
