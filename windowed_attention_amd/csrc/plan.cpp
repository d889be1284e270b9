// Host-only cache planning (see plan.h). The row counts follow the pages' cache sizes:
// R-SWA holds m + n rows at most (deep dive "Unlimited-OCR", N(t) code block: C(T) = L_m +
// min(n, T) <= L_m + n); full causal holds m + T (GeekNews "Unlimited OCR", KV cache management).
#include "plan.h"

#include <algorithm>
#include <limits>

namespace rswa {

rswa_status make_plan(const rswa_cache_desc* d, Plan* p, std::string* why) {
  auto bad = [&](rswa_status s, const char* msg) {
    if (why) *why = msg;
    return s;
  };
  if (!d || !p) return bad(RSWA_E_INVALID, "null descriptor");
  if (d->batch < 1 || d->batch > kMaxBatch) return bad(RSWA_E_INVALID, "batch out of range");
  if (d->num_heads < 1 || d->num_heads > kMaxHeads)
    return bad(RSWA_E_INVALID, "num_heads out of range");
  if (d->head_dim < 1) return bad(RSWA_E_INVALID, "head_dim must be positive");
  if (d->head_dim != kPlanHeadDim) return bad(RSWA_E_UNSUPPORTED, "head_dim must be 128");
  if (d->kv_dtype != RSWA_BF16 && d->kv_dtype != RSWA_F32)
    return bad(RSWA_E_INVALID, "kv_dtype must be RSWA_BF16 or RSWA_F32");
  if (d->mode != RSWA_MODE_RSWA && d->mode != RSWA_MODE_FULL_CAUSAL)
    return bad(RSWA_E_INVALID, "mode must be RSWA_MODE_RSWA or RSWA_MODE_FULL_CAUSAL");
  if (!d->prefix_len) return bad(RSWA_E_INVALID, "prefix_len is NULL");
  const bool full = d->mode == RSWA_MODE_FULL_CAUSAL;
  if (!full && !d->window) return bad(RSWA_E_INVALID, "window is NULL in R-SWA mode");
  if (full && !d->max_steps) return bad(RSWA_E_INVALID, "max_steps is NULL in full-causal mode");
  if (d->prefix_paged != 0 && d->prefix_paged != 1)
    return bad(RSWA_E_INVALID, "prefix_paged must be 0 or 1");
  const bool paged = d->prefix_paged == 1;

  const int B = d->batch;
  const int64_t H = d->num_heads, D = d->head_dim;
  p->elem = d->kv_dtype == RSWA_F32 ? 4 : 2;
  p->seq_off.assign(B, 0);
  p->rows.assign(B, 0);
  p->prefix.assign(B, 0);
  p->cap.assign(B, 0);
  p->prefix_row0.assign(B, 0);
  p->total_prefix_rows = 0;
  p->max_prefix = 0;
  int64_t off = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t m = d->prefix_len[b];
    const int64_t cap = full ? d->max_steps[b] : d->window[b];
    if (m < 0) return bad(RSWA_E_INVALID, "prefix_len must be >= 0");
    if (cap < 1) return bad(RSWA_E_INVALID, full ? "max_steps must be >= 1" : "window must be >= 1");
    const int64_t R = paged ? cap : m + cap;  // a paged prefix is not stored in the cache
    if (R > std::numeric_limits<int32_t>::max() / 2)
      return bad(RSWA_E_INVALID, "prefix_len + capacity too large");
    p->seq_off[b] = off;
    p->rows[b] = (int32_t)R;
    p->prefix[b] = (int32_t)m;
    p->cap[b] = (int32_t)cap;
    p->prefix_row0[b] = p->total_prefix_rows;
    p->total_prefix_rows += m;
    p->max_prefix = std::max<int32_t>(p->max_prefix, (int32_t)m);
    const int64_t elems = 2 * H * R * D;
    if (off > std::numeric_limits<int64_t>::max() / 8 - elems)
      return bad(RSWA_E_INVALID, "cache too large");
    off += elems;
  }
  p->bytes = (uint64_t)off * (uint64_t)p->elem + kStorageTailBytes;
  return RSWA_OK;
}

DecodePlan plan_decode(const std::vector<int64_t>& live_rows, int32_t heads, int64_t resident,
                       int64_t grid_max, int32_t min_rows, int32_t grid_user, bool masked) {
  DecodePlan p;
  const int64_t nseg = (int64_t)live_rows.size() * heads;
  int64_t total = 0;
  bool uniform = !masked;
  for (size_t b = 0; b < live_rows.size(); ++b) {
    total += (int64_t)heads * live_rows[b];
    if (live_rows[b] != live_rows[0]) uniform = false;
  }
  if (total == 0) return p;
  resident = std::max<int64_t>(1, std::min(resident, grid_max));
  const bool user = min_rows > 0 || grid_user > 0;
  if (!user && uniform && nseg <= resident && 2 * nseg >= resident) {
    p.aligned = true;
    p.grid = nseg;
    p.rows_per_piece = live_rows[0];
    return p;
  }
  const int64_t w_min = min_rows > 0 ? min_rows : 64;
  if (!user && uniform && 2 * nseg <= resident) {
    const int64_t k = std::min(resident / nseg, live_rows[0] / w_min);
    if (k >= 2) {
      p.split = (int32_t)k;
      p.grid = nseg * k;
      p.rows_per_piece = (live_rows[0] + k - 1) / k;
      return p;
    }
  }
  const int64_t g_req = grid_user > 0 ? std::min<int64_t>(grid_user, grid_max) : resident;
  p.rows_per_piece = std::max<int64_t>(w_min, (total + g_req - 1) / g_req);
  p.grid = (total + p.rows_per_piece - 1) / p.rows_per_piece;
  p.stream_k = true;
  return p;
}

}  // namespace rswa
