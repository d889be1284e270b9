// C ABI of the R-SWA library (declared in include/rswa.h): argument validation, cache ownership,
// per-sequence metadata on the device, and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "plan.h"
#include "rswa.h"

namespace {

thread_local std::string g_last_error;

rswa_status fail(rswa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

rswa_status hip_fail(hipError_t e, const char* what) {
  return fail(RSWA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct DeviceGuard {
  int prev = -1;
  bool switched = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
      switched = hipSetDevice(dev) == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

// Metadata errors that the prefill and backward kernels find on the device (a sequence longer
// than its launch's max_seqlen, a prefix longer than its sequence, a window below 1), OR-ed
// together until rswa_prefill_check() reads and clears them. Each device holds its own copy of
// this word; host code uses the address hipGetSymbolAddress gives for the current device, never
// the variable's name (which is only a host-side stand-in).
__device__ __align__(256) int32_t g_prefill_err;

// Work array of rswa_prefill_bwd_noalloc: lse * log2(e) and -delta of every (token, head) row,
// kNoAllocRows rows each (8 MiB), held by each device the library runs on until the process ends.
// Host code uses the address hipGetSymbolAddress gives for the current device (kept per device in
// g_scratch_ptr), never the array's name.
constexpr int64_t kNoAllocRows = int64_t{1} << 20;
__device__ __align__(256) float scratch[2 * kNoAllocRows];

constexpr int kMaxDevices = 64;
int32_t* g_prefill_err_ptr[kMaxDevices] = {};
float* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_statics_mutex;

// Device address of the current device's scratch array, or nullptr (reason in *e).
float* scratch_ptr(hipError_t* e) {
  int dev = -1;
  *e = hipGetDevice(&dev);
  if (*e != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *e = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_statics_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    *e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*e != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = reinterpret_cast<float*>(ptr);
  }
  return g_scratch_ptr[dev];
}

// Device address of the current device's error word, or nullptr (reason in *e).
int32_t* prefill_err_word(hipError_t* e) {
  int dev = -1;
  *e = hipGetDevice(&dev);
  if (*e != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *e = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_statics_mutex);
  if (!g_prefill_err_ptr[dev]) {
    void* ptr = nullptr;
    *e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_prefill_err));
    if (*e != hipSuccess) return nullptr;
    g_prefill_err_ptr[dev] = reinterpret_cast<int32_t*>(ptr);
  }
  return g_prefill_err_ptr[dev];
}

}  // namespace

struct rswa_cache {
  int32_t B = 0, H = 0, D = 0, kv_dtype = 0, mode = 0;
  rswa::Plan plan;
  std::vector<int64_t> calls;  // appends enqueued per sequence: an upper bound of t_b
  bool masked = false;         // an active mask has been used: calls[] may overstate t_b, so the
                               // full-causal capacity check is left to the device
  bool equal_t = true;         // every t_b is the same (false after a fill from sequences of
                               // unequal output counts); the host-known decode plan needs it
  int graphs = 0;              // live step graphs that reference this cache
  void* storage = nullptr;
  bool owns_storage = false;
  void* meta_dev = nullptr;
  rswa::CacheMeta meta{};
  int32_t* steps_dev[2] = {nullptr, nullptr};  // double-buffered step counters
  int cur = 0;                                 // steps_dev[cur] holds the current t_b
  int64_t* prefix_row0_dev = nullptr;
  void* ws_dev = nullptr;
  float* ws_acc = nullptr;
  float* ws_ml = nullptr;
  int32_t* ws_cnt = nullptr;
  bool uniform = false;  // every sequence has the same m and capacity (a host-known plan applies)
  int32_t grid_max = 0;  // stream-K workgroups the workspace is sized for
  int32_t min_rows = 0;  // user setting (0 = automatic)
  int32_t grid_user = 0; // user setting (0 = automatic)
  int device = 0;
  int num_cus = 0;
  int blocks_per_cu = 0; // resident decode workgroups per CU

  bool full() const { return mode == RSWA_MODE_FULL_CAUSAL; }
  // Upper bound of each sequence's live rows after `extra` more appends, from the host count of
  // append calls (exact when no active mask has been used).
  std::vector<int64_t> live_upper(int extra) const {
    std::vector<int64_t> L(B);
    for (int b = 0; b < B; ++b)
      L[b] = plan.prefix[b] + std::min<int64_t>(plan.cap[b], calls[b] + extra);
    return L;
  }
  // Whether a decode over live rows L reads more than the last-level cache holds: then none of
  // its rows is found there at the next step anyway, and the step streams them.
  bool exceeds_llc(const std::vector<int64_t>& L) const {
    int64_t rows = 0;
    for (int b = 0; b < B; ++b) rows += L[b];
    return rows * H * 2 * D * (kv_dtype == RSWA_F32 ? 4 : 2) > rswa::kLastLevelCacheBytes;
  }
  // Non-temporal loads for such a step, except over paged prefixes: their rows are shared by
  // several sequences and do get reused within the step.
  bool streams(const std::vector<int64_t>& L) const { return !meta.table && exceeds_llc(L); }
  // Workgroups the decode plan spreads a launch over. A streamed step keeps at most
  // kStreamBlocksPerCu of them per CU: three workgroups of 4 waves per CU, each on a larger share
  // of the rows (fewer concurrent row streams), read 346 MB per step 1.6 % faster than four did
  // (57.3 vs 58.2 us). A paged cache keeps all of them: its prefix rows are looked up one by one
  // from a pool that the last-level cache holds, which needs the extra waves to cover the latency
  // (three per CU made such a step 39 % slower).
  static constexpr int kStreamBlocksPerCu = 3;
  int64_t decode_resident(const std::vector<int64_t>& L) const {
    return (int64_t)num_cus *
           (streams(L) ? std::min(blocks_per_cu, kStreamBlocksPerCu) : blocks_per_cu);
  }
};

namespace {

void release(rswa_cache* c) {
  if (!c) return;
  if (c->owns_storage && c->storage) (void)hipFree(c->storage);
  if (c->meta_dev) (void)hipFree(c->meta_dev);
  if (c->ws_dev) (void)hipFree(c->ws_dev);
  delete c;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

const char* rswa_status_str(int32_t s) {
  switch (s) {
    case RSWA_OK: return "RSWA_OK";
    case RSWA_E_INVALID: return "RSWA_E_INVALID";
    case RSWA_E_UNSUPPORTED: return "RSWA_E_UNSUPPORTED";
    case RSWA_E_CAPACITY: return "RSWA_E_CAPACITY";
    case RSWA_E_OOM: return "RSWA_E_OOM";
    case RSWA_E_HIP: return "RSWA_E_HIP";
    case RSWA_E_INTERNAL: return "RSWA_E_INTERNAL";
    default: return "RSWA_E_UNKNOWN";
  }
}

const char* rswa_last_error(void) { return g_last_error.c_str(); }

rswa_status rswa_cache_plan(const rswa_cache_desc* desc, int64_t* seq_offset_host,
                            int32_t* rows_host, uint64_t* storage_bytes_host) {
  try {
    rswa::Plan p;
    std::string why;
    const rswa_status s = rswa::make_plan(desc, &p, &why);
    if (s != RSWA_OK) return fail(s, why);
    for (int b = 0; b < desc->batch; ++b) {
      if (seq_offset_host) seq_offset_host[b] = p.seq_off[b];
      if (rows_host) rows_host[b] = p.rows[b];
    }
    if (storage_bytes_host) *storage_bytes_host = p.bytes;
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_cache_plan");
  }
}

uint64_t rswa_cache_bytes(const rswa_cache_desc* desc) {
  uint64_t bytes = 0;
  if (rswa_cache_plan(desc, nullptr, nullptr, &bytes) != RSWA_OK) return 0;
  return bytes;
}

}  // extern "C"

namespace {

// Shared by rswa_cache_create (prefix copied into the cache) and rswa_cache_create_paged (prefix
// looked up in the caller's pool through the page table).
struct PagedPrefix {
  const void* pool_k = nullptr;
  const void* pool_v = nullptr;
  int64_t pool_rows = 0;
  const int32_t* table = nullptr;
};

// rswa_cache_create_from_prefill: packed prefix + output segments of a prefill batch.
struct PrefillSource {
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* cu = nullptr;  // host [B + 1]
};

rswa_status create_cache(const rswa_cache_desc* desc, const void* prefix_k_dev,
                         const void* prefix_v_dev, const PagedPrefix* pg, void* stream,
                         rswa_cache** out, const PrefillSource* fill = nullptr) {
  if (!out) return fail(RSWA_E_INVALID, "out is NULL");
  *out = nullptr;
  rswa_cache* c = nullptr;
  try {
    rswa::Plan p;
    std::string why;
    rswa_status s = rswa::make_plan(desc, &p, &why);
    if (s != RSWA_OK) return fail(s, why);
    const bool paged = pg != nullptr;
    if (paged != (desc->prefix_paged == 1))
      return fail(RSWA_E_INVALID, paged ? "rswa_cache_create_paged needs desc->prefix_paged = 1"
                                        : "desc->prefix_paged = 1 needs rswa_cache_create_paged");
    if (paged) {
      if (p.total_prefix_rows > 0 && (!pg->pool_k || !pg->pool_v || !pg->table))
        return fail(RSWA_E_INVALID, "pool_k / pool_v / prefix_table is NULL but some m_b > 0");
      if (p.total_prefix_rows > 0 && pg->pool_rows < 1)
        return fail(RSWA_E_INVALID, "pool_rows must be >= 1");
      if ((reinterpret_cast<uintptr_t>(pg->pool_k) % 16) != 0 ||
          (reinterpret_cast<uintptr_t>(pg->pool_v) % 16) != 0)
        return fail(RSWA_E_INVALID, "pool_k / pool_v must be 16-byte aligned");
    } else if (!fill && p.total_prefix_rows > 0 && (!prefix_k_dev || !prefix_v_dev)) {
      return fail(RSWA_E_INVALID, "prefix_k_dev / prefix_v_dev are NULL but some m_b > 0");
    }
    // a fill from a prefill batch: sequence b is the segment [cu[b], cu[b + 1]), its first m_b
    // rows the prefix, the other t_b rows its outputs
    std::vector<int32_t> fill_t;
    int64_t fill_rows = 0;
    int fill_live = 0;
    if (fill) {
      if (!fill->cu) return fail(RSWA_E_INVALID, "cu_seqlens_host is NULL");
      if (fill->cu[0] < 0) return fail(RSWA_E_INVALID, "cu_seqlens[0] < 0");
      fill_t.resize(desc->batch);
      for (int b = 0; b < desc->batch; ++b) {
        const int64_t S = (int64_t)fill->cu[b + 1] - fill->cu[b];
        if (S < p.prefix[b])
          return fail(RSWA_E_INVALID, "a segment of cu_seqlens is shorter than its prefix");
        const int64_t t = S - p.prefix[b];
        if (desc->mode == RSWA_MODE_FULL_CAUSAL && t > p.cap[b])
          return fail(RSWA_E_CAPACITY, "a segment holds more outputs than max_steps");
        fill_t[b] = (int32_t)t;
        fill_rows += S;
        const int live = desc->mode == RSWA_MODE_FULL_CAUSAL ? (int)t : (int)std::min<int64_t>(t, p.cap[b]);
        fill_live = std::max(fill_live, live);
      }
      if (fill_rows > 0 && (!fill->k || !fill->v))
        return fail(RSWA_E_INVALID, "k_dev / v_dev are NULL but the segments hold rows");
      if ((reinterpret_cast<uintptr_t>(fill->k) % 16) != 0 ||
          (reinterpret_cast<uintptr_t>(fill->v) % 16) != 0)
        return fail(RSWA_E_INVALID, "k_dev / v_dev must be 16-byte aligned");
    }
    if (desc->storage_dev && desc->storage_bytes < p.bytes)
      return fail(RSWA_E_CAPACITY, "storage_bytes smaller than rswa_cache_bytes()");
    if (desc->storage_dev && (reinterpret_cast<uintptr_t>(desc->storage_dev) % 16) != 0)
      return fail(RSWA_E_INVALID, "storage_dev must be 16-byte aligned");

    c = new rswa_cache();
    c->B = desc->batch;
    c->H = desc->num_heads;
    c->D = desc->head_dim;
    c->kv_dtype = desc->kv_dtype;
    c->mode = desc->mode;
    c->plan = p;
    c->calls.assign(c->B, 0);
    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipGetDevice");
    }
    e = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, c->device);
    if (e != hipSuccess || c->num_cus <= 0) {
      release(c);
      return hip_fail(e, "hipDeviceGetAttribute(multiProcessorCount)");
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    // storage
    if (desc->storage_dev) {
      c->storage = desc->storage_dev;
    } else {
      e = hipMalloc(&c->storage, std::max<uint64_t>(p.bytes, 256));
      if (e != hipSuccess) {
        c->storage = nullptr;
        release(c);
        return fail(RSWA_E_OOM, std::string("hipMalloc(storage): ") + hipGetErrorString(e));
      }
      c->owns_storage = true;
      e = hipMemsetAsync(c->storage, 0, p.bytes, st);
      if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "hipMemsetAsync(storage)");
      }
    }

    // device metadata: seq_off[B], prefix_row0[B] (int64); rows, prefix, cap, steps [B], err[1]
    const int B = c->B;
    const size_t off_i64 = 0;
    const size_t off_row0 = align_up(off_i64 + 8 * (size_t)B, 256);
    const size_t off_rows = align_up(off_row0 + 8 * (size_t)B, 256);
    const size_t off_pref = align_up(off_rows + 4 * (size_t)B, 256);
    const size_t off_cap = align_up(off_pref + 4 * (size_t)B, 256);
    const size_t off_steps = align_up(off_cap + 4 * (size_t)B, 256);
    const size_t off_steps2 = align_up(off_steps + 4 * (size_t)B, 256);
    const size_t off_err = align_up(off_steps2 + 4 * (size_t)B, 256);
    const size_t meta_bytes = off_err + 256;
    std::vector<unsigned char> host(meta_bytes, 0);
    std::memcpy(host.data() + off_i64, p.seq_off.data(), 8 * (size_t)B);
    if (fill) {
      std::vector<int64_t> row0(B);
      for (int b = 0; b < B; ++b) row0[b] = fill->cu[b];
      std::memcpy(host.data() + off_row0, row0.data(), 8 * (size_t)B);
      std::memcpy(host.data() + off_steps, fill_t.data(), 4 * (size_t)B);
    } else {
      std::memcpy(host.data() + off_row0, p.prefix_row0.data(), 8 * (size_t)B);
    }
    std::memcpy(host.data() + off_rows, p.rows.data(), 4 * (size_t)B);
    std::memcpy(host.data() + off_pref, p.prefix.data(), 4 * (size_t)B);
    std::memcpy(host.data() + off_cap, p.cap.data(), 4 * (size_t)B);
    e = hipMalloc(&c->meta_dev, meta_bytes);
    if (e != hipSuccess) {
      c->meta_dev = nullptr;
      release(c);
      return fail(RSWA_E_OOM, std::string("hipMalloc(meta): ") + hipGetErrorString(e));
    }
    e = hipMemcpyAsync(c->meta_dev, host.data(), meta_bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipMemcpyAsync(meta)");
    }
    unsigned char* mb = reinterpret_cast<unsigned char*>(c->meta_dev);
    c->meta.seq_off = reinterpret_cast<const int64_t*>(mb + off_i64);
    c->prefix_row0_dev = reinterpret_cast<int64_t*>(mb + off_row0);
    c->meta.rows = reinterpret_cast<const int32_t*>(mb + off_rows);
    c->meta.prefix_len = reinterpret_cast<const int32_t*>(mb + off_pref);
    c->meta.cap = reinterpret_cast<const int32_t*>(mb + off_cap);
    c->steps_dev[0] = reinterpret_cast<int32_t*>(mb + off_steps);
    c->steps_dev[1] = reinterpret_cast<int32_t*>(mb + off_steps2);
    c->meta.err = reinterpret_cast<int32_t*>(mb + off_err);
    int32_t* table_bad = reinterpret_cast<int32_t*>(mb + off_err + 4);  // zeroed with the rest
    if (paged) {
      c->meta.table = pg->table;
      c->meta.table_off = c->prefix_row0_dev;
      c->meta.pool_k = pg->pool_k;
      c->meta.pool_v = pg->pool_v;
    }

    // decode plan: resident workgroups per CU, and a workspace sized for the largest stream-K
    // grid (partial slot = workgroup index + (b, h) index, see decode.hip)
    c->blocks_per_cu = rswa::decode_blocks_per_cu(c->kv_dtype == RSWA_F32, 1, B);
    c->grid_max = std::max(1, c->num_cus * std::max(c->blocks_per_cu, 8));
    const size_t ws_slots = (size_t)c->grid_max + (size_t)B * c->H;
    const size_t ws_acc_bytes = align_up(ws_slots * rswa::kPlanHeadDim * sizeof(float), 256);
    const size_t ws_ml_bytes = align_up(ws_slots * 2 * sizeof(float), 256);
    const size_t ws_cnt_bytes = align_up((size_t)B * c->H * sizeof(int32_t), 256);
    const size_t ws_bytes = ws_acc_bytes + ws_ml_bytes + ws_cnt_bytes;
    e = hipMalloc(&c->ws_dev, ws_bytes);
    if (e != hipSuccess) {
      c->ws_dev = nullptr;
      release(c);
      return fail(RSWA_E_OOM, std::string("hipMalloc(workspace): ") + hipGetErrorString(e));
    }
    unsigned char* wb = reinterpret_cast<unsigned char*>(c->ws_dev);
    c->ws_acc = reinterpret_cast<float*>(wb);
    c->ws_ml = reinterpret_cast<float*>(wb + ws_acc_bytes);
    c->ws_cnt = reinterpret_cast<int32_t*>(wb + ws_acc_bytes + ws_ml_bytes);
    // the split-range counters start at zero; every launch leaves them at zero
    e = hipMemsetAsync(c->ws_cnt, 0, ws_cnt_bytes, st);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipMemsetAsync(workspace counters)");
    }
    c->uniform = true;
    for (int b = 1; b < B; ++b)
      if (p.prefix[b] != p.prefix[0] || p.cap[b] != p.cap[0]) c->uniform = false;

    if (paged) {
      // every page-table entry must name a pool row: checked once here, so decode never reads
      // outside the pool
      e = rswa::launch_table_check(pg->table, p.total_prefix_rows, pg->pool_rows, table_bad, st);
      if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "page-table check launch");
      }
    } else {
      rswa::PrefixCopyArgs pa{};
      pa.storage = c->storage;
      pa.meta = c->meta;
      pa.pk = fill ? fill->k : prefix_k_dev;
      pa.pv = fill ? fill->v : prefix_v_dev;
      pa.prefix_row0 = c->prefix_row0_dev;
      pa.heads = c->H;
      pa.batch = B;
      e = rswa::launch_prefix_copy(pa, c->kv_dtype == RSWA_F32, p.max_prefix, st);
      if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "prefix copy launch");
      }
      if (fill) {
        rswa::FillArgs fa{};
        fa.storage = c->storage;
        fa.meta = c->meta;
        fa.k = fill->k;
        fa.v = fill->v;
        fa.row0 = c->prefix_row0_dev;
        fa.steps = c->steps_dev[0];
        fa.heads = c->H;
        fa.batch = B;
        fa.full_causal = c->full() ? 1 : 0;
        e = rswa::launch_fill_outputs(fa, c->kv_dtype == RSWA_F32, fill_live, st);
        if (e != hipSuccess) {
          release(c);
          return hip_fail(e, "fill launch");
        }
        for (int b = 0; b < B; ++b) {
          c->calls[b] = fill_t[b];
          if (fill_t[b] != fill_t[0]) c->equal_t = false;
        }
      }
    }
    // the host metadata buffer must outlive the async copy
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipStreamSynchronize(create)");
    }
    if (paged) {
      int32_t bad = 0;
      e = hipMemcpy(&bad, table_bad, sizeof(bad), hipMemcpyDeviceToHost);
      if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "hipMemcpy(page-table check)");
      }
      if (bad) {
        release(c);
        return fail(RSWA_E_INVALID, "a page-table entry lies outside [0, pool_rows)");
      }
    }
    *out = c;
    return RSWA_OK;
  } catch (const std::bad_alloc&) {
    release(c);
    return fail(RSWA_E_OOM, "host allocation failed");
  } catch (...) {
    release(c);
    return fail(RSWA_E_INTERNAL, "exception in rswa_cache_create");
  }
}

}  // namespace

extern "C" {

rswa_status rswa_cache_create(const rswa_cache_desc* desc, const void* prefix_k_dev,
                              const void* prefix_v_dev, void* stream, rswa_cache** out) {
  return create_cache(desc, prefix_k_dev, prefix_v_dev, nullptr, stream, out);
}

rswa_status rswa_cache_create_from_prefill(const rswa_cache_desc* desc, const void* k_dev,
                                           const void* v_dev, const int32_t* cu_seqlens_host,
                                           void* stream, rswa_cache** out) {
  if (desc && desc->prefix_paged)
    return fail(RSWA_E_INVALID, "a cache filled from a prefill holds its prefixes (prefix_paged = 0)");
  PrefillSource src;
  src.k = k_dev;
  src.v = v_dev;
  src.cu = cu_seqlens_host;
  return create_cache(desc, nullptr, nullptr, nullptr, stream, out, &src);
}

rswa_status rswa_cache_create_paged(const rswa_cache_desc* desc, const void* pool_k_dev,
                                    const void* pool_v_dev, int64_t pool_rows,
                                    const int32_t* prefix_table_dev, void* stream,
                                    rswa_cache** out) {
  PagedPrefix pg;
  pg.pool_k = pool_k_dev;
  pg.pool_v = pool_v_dev;
  pg.pool_rows = pool_rows;
  pg.table = prefix_table_dev;
  return create_cache(desc, nullptr, nullptr, &pg, stream, out);
}

rswa_status rswa_append_kv(rswa_cache* c, const void* k_dev, const void* v_dev,
                           const uint8_t* active_dev, void* stream) {
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  if (!k_dev || !v_dev) return fail(RSWA_E_INVALID, "k_dev / v_dev is NULL");
  try {
    if (c->full() && !active_dev && !c->masked) {
      for (int b = 0; b < c->B; ++b)
        if (c->calls[b] >= c->plan.cap[b])
          return fail(RSWA_E_CAPACITY, "full-causal append past max_steps");
    }
    DeviceGuard g(c->device);
    rswa::AppendArgs a{};
    a.storage = c->storage;
    a.meta = c->meta;
    a.steps_in = c->steps_dev[c->cur];
    a.steps_out = c->steps_dev[c->cur ^ 1];
    a.k_new = k_dev;
    a.v_new = v_dev;
    a.active = active_dev;
    a.heads = c->H;
    a.full_causal = c->full();
    const hipError_t e = rswa::launch_append(a, c->B, c->kv_dtype == RSWA_F32,
                                             reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "append launch");
    c->cur ^= 1;
    for (int b = 0; b < c->B; ++b) c->calls[b] += 1;
    if (active_dev) c->masked = true;
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_append_kv");
  }
}

namespace {

// Shared body of rswa_decode_attn (k_dev == NULL) and rswa_decode_step (append fused in).
// How a decode launch is enqueued: eagerly, or into a step graph that reads every sequence's
// counter, or into one that reads the step count all sequences share.
constexpr int kEager = 0, kCaptureGeneral = 1, kCaptureUniform = 2;

rswa_status decode_launch(rswa_cache* c, const void* q_dev, const void* k_dev, const void* v_dev,
                          void* out_dev, int32_t out_dtype, float softmax_scale,
                          const uint8_t* active_dev, void* stream, const char* what,
                          int capture = kEager) {
  const bool capturing = capture != kEager;
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  if (!q_dev || !out_dev) return fail(RSWA_E_INVALID, "q_dev / out_dev is NULL");
  if (out_dtype != RSWA_BF16 && out_dtype != RSWA_F32)
    return fail(RSWA_E_INVALID, "out_dtype must be RSWA_BF16 or RSWA_F32");
  if (!(softmax_scale <= 0.f) && !std::isfinite(softmax_scale))
    return fail(RSWA_E_INVALID, "softmax_scale must be finite");
  const bool append = k_dev != nullptr;
  try {
    if (append && c->full() && !active_dev && !c->masked) {
      for (int b = 0; b < c->B; ++b)
        if (c->calls[b] >= c->plan.cap[b])
          return fail(RSWA_E_CAPACITY, "full-causal append past max_steps");
    }
    const std::vector<int64_t> L = c->live_upper(append ? 1 : 0);
    if (!active_dev) {
      for (int b = 0; b < c->B; ++b)
        if (L[b] == 0)
          return fail(RSWA_E_INVALID, "empty key set: a sequence with m = 0 has no output yet");
    }
    DeviceGuard g(c->device);
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)c->D);
    rswa::DecodeArgs a{};
    a.storage = c->storage;
    a.meta = c->meta;
    a.steps_in = c->steps_dev[c->cur];
    a.steps_out = append ? c->steps_dev[c->cur ^ 1] : nullptr;
    a.k_new = k_dev;
    a.v_new = v_dev;
    a.q = q_dev;
    a.out = out_dev;
    a.active = active_dev;
    a.ws_acc = c->ws_acc;
    a.ws_ml = c->ws_ml;
    a.ws_cnt = c->ws_cnt;
    // The host knows every t_b exactly while no active mask has been used (each call appends to
    // every sequence); with equal m and capacity the plan then needs no metadata loads. Captured
    // launches are replayed at later steps, so they read the step counts from the device: the
    // shared one (kUniFromCounters) when the graph is captured for a cache in that state, else
    // every sequence's.
    a.uni_t = -1;
    if (c->uniform && c->equal_t && !c->masked && !active_dev && capture != kCaptureGeneral) {
      a.uni_t = capture == kCaptureUniform ? rswa::kUniFromCounters : (int32_t)c->calls[0];
      a.uni_m = c->plan.prefix[0];
      a.uni_cap = c->plan.cap[0];
      a.uni_rows = c->plan.rows[0];
    }
    a.batch = c->B;
    a.heads = c->H;
    a.full_causal = c->full();
    a.min_rows = c->min_rows > 0 ? c->min_rows : 64;
    a.stream_loads = c->streams(L) ? 1 : 0;
    a.scale_log2 = scale * 1.4426950408889634f;

    const int64_t resident = c->decode_resident(L);
    const rswa::DecodePlan plan = rswa::plan_decode(L, c->H, resident, c->grid_max, c->min_rows,
                                                    c->grid_user, active_dev != nullptr);
    a.aligned = plan.aligned ? 1 : 0;
    a.split = plan.split;
    const hipError_t e = rswa::launch_decode(a, c->kv_dtype == RSWA_F32, out_dtype == RSWA_F32,
                                             (int)plan.grid, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, what);
    if (append) {
      c->cur ^= 1;
      for (int b = 0; b < c->B; ++b) c->calls[b] += 1;
      if (active_dev) c->masked = true;
    }
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, std::string("exception in ") + what);
  }
}

}  // namespace

rswa_status rswa_decode_attn(rswa_cache* c, const void* q_dev, void* out_dev, int32_t out_dtype,
                             float softmax_scale, const uint8_t* active_dev, void* stream) {
  return decode_launch(c, q_dev, nullptr, nullptr, out_dev, out_dtype, softmax_scale, active_dev,
                       stream, "rswa_decode_attn");
}

rswa_status rswa_decode_step(rswa_cache* c, const void* q_dev, const void* k_dev,
                             const void* v_dev, void* out_dev, int32_t out_dtype,
                             float softmax_scale, const uint8_t* active_dev, void* stream) {
  if (c && (!k_dev || !v_dev)) return fail(RSWA_E_INVALID, "k_dev / v_dev is NULL");
  return decode_launch(c, q_dev, k_dev, v_dev, out_dev, out_dtype, softmax_scale, active_dev,
                       stream, "rswa_decode_step");
}

struct rswa_step_graph {
  rswa_cache* c = nullptr;
  hipGraph_t graph = nullptr;      // steps that read every sequence's counter
  hipGraphExec_t exec = nullptr;
  hipGraph_t graph_uni = nullptr;  // the same steps reading the one count all sequences share
  hipGraphExec_t exec_uni = nullptr;  // (captured when the cache was in that state)
  int32_t steps = 0;
  int cur0 = 0;  // counter buffer the captured steps start from (and, steps being even, end in)
};

namespace {

void release_graph(rswa_step_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->exec_uni) (void)hipGraphExecDestroy(g->exec_uni);
  if (g->graph_uni) (void)hipGraphDestroy(g->graph_uni);
  delete g;
}

// All sequences share m, capacity and step count, and no active mask has been used.
bool shares_counts(const rswa_cache* c) { return c->uniform && c->equal_t && !c->masked; }

}  // namespace

rswa_status rswa_step_graph_create(rswa_cache* c, int32_t steps, const void* q_slots,
                                   const void* k_slots, const void* v_slots, void* out_slots,
                                   int32_t out_dtype, float softmax_scale,
                                   rswa_step_graph** out) {
  if (!out) return fail(RSWA_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  if (steps < 2 || steps > 4096 || (steps & 1))
    return fail(RSWA_E_INVALID, "steps must be even, in [2, 4096]");
  if (!q_slots || !k_slots || !v_slots || !out_slots)
    return fail(RSWA_E_INVALID, "q / k / v / out slot pointer is NULL");
  if (out_dtype != RSWA_BF16 && out_dtype != RSWA_F32)
    return fail(RSWA_E_INVALID, "out_dtype must be RSWA_BF16 or RSWA_F32");
  rswa_step_graph* g = nullptr;
  hipStream_t cs = nullptr;
  const std::vector<int64_t> calls = c->calls;
  const int cur = c->cur;
  try {
    DeviceGuard dg(c->device);
    g = new rswa_step_graph();
    g->c = c;
    g->steps = steps;
    g->cur0 = cur;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) {
      release_graph(g);
      return hip_fail(e, "hipStreamCreateWithFlags(capture)");
    }
    const size_t elem = c->kv_dtype == RSWA_F32 ? 4 : 2;
    const size_t slot = (size_t)c->B * c->H * c->D;
    const size_t oelem = out_dtype == RSWA_F32 ? 4 : 2;
    // capture the steps in one mode into (graph, exec)
    auto capture = [&](int mode, hipGraph_t* graph, hipGraphExec_t* exec) -> rswa_status {
      hipError_t ce = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
      if (ce != hipSuccess) return hip_fail(ce, "hipStreamBeginCapture");
      rswa_status st = RSWA_OK;
      for (int i = 0; i < steps && st == RSWA_OK; ++i) {
        const char* q = reinterpret_cast<const char*>(q_slots) + i * slot * elem;
        const char* k = reinterpret_cast<const char*>(k_slots) + i * slot * elem;
        const char* v = reinterpret_cast<const char*>(v_slots) + i * slot * elem;
        char* o = reinterpret_cast<char*>(out_slots) + i * slot * oelem;
        st = decode_launch(c, q, k, v, o, out_dtype, softmax_scale, nullptr, cs,
                           "rswa_step_graph_create", mode);
      }
      ce = hipStreamEndCapture(cs, graph);
      // capture enqueues nothing: the host view of the cache stays where it was
      c->calls = calls;
      c->cur = cur;
      if (st != RSWA_OK) return st;
      if (ce != hipSuccess) return hip_fail(ce, "hipStreamEndCapture");
      ce = hipGraphInstantiate(exec, *graph, nullptr, nullptr, 0);
      if (ce != hipSuccess) {
        *exec = nullptr;
        return hip_fail(ce, "hipGraphInstantiate");
      }
      return RSWA_OK;
    };
    rswa_status st = capture(kCaptureGeneral, &g->graph, &g->exec);
    if (st == RSWA_OK && shares_counts(c))
      st = capture(kCaptureUniform, &g->graph_uni, &g->exec_uni);
    (void)hipStreamDestroy(cs);
    cs = nullptr;
    if (st != RSWA_OK) {
      release_graph(g);
      return st;
    }
    *out = g;
    c->graphs += 1;
    return RSWA_OK;
  } catch (...) {
    c->calls = calls;
    c->cur = cur;
    if (cs) (void)hipStreamDestroy(cs);
    release_graph(g);
    return fail(RSWA_E_INTERNAL, "exception in rswa_step_graph_create");
  }
}

rswa_status rswa_step_graph_launch(rswa_step_graph* g, void* stream) {
  if (!g) return fail(RSWA_E_INVALID, "graph is NULL");
  rswa_cache* c = g->c;
  try {
    if (c->full() && !c->masked) {
      for (int b = 0; b < c->B; ++b)
        if (c->calls[b] + g->steps > c->plan.cap[b])
          return fail(RSWA_E_CAPACITY, "full-causal append past max_steps");
    }
    DeviceGuard dg(c->device);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // The captured kernels read the counters from buffer cur0. After an odd number of eager
    // appends since the capture the current counters sit in the other buffer: move them first.
    if (c->cur != g->cur0) {
      const hipError_t e = hipMemcpyAsync(c->steps_dev[g->cur0], c->steps_dev[c->cur],
                                          sizeof(int32_t) * (size_t)c->B,
                                          hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(step counters)");
      c->cur = g->cur0;
    }
    // the steps that read the shared count while the cache is still in that state
    hipGraphExec_t exec = g->exec_uni && shares_counts(c) ? g->exec_uni : g->exec;
    const hipError_t e = hipGraphLaunch(exec, st);
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    for (int b = 0; b < c->B; ++b) c->calls[b] += g->steps;
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_step_graph_launch");
  }
}

rswa_status rswa_step_graph_destroy(rswa_step_graph* g) {
  if (!g) return RSWA_OK;
  DeviceGuard dg(g->c->device);
  g->c->graphs -= 1;
  release_graph(g);
  return RSWA_OK;
}

rswa_status rswa_cache_steps(rswa_cache* c, int32_t* steps_host, void* stream) {
  if (!c || !steps_host) return fail(RSWA_E_INVALID, "cache / steps_host is NULL");
  try {
    DeviceGuard g(c->device);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int32_t err = 0;
    hipError_t e = hipMemcpyAsync(steps_host, c->steps_dev[c->cur], 4 * (size_t)c->B,
                                  hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(&err, c->meta.err, 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "reading step counters");
    if (err) return fail(RSWA_E_CAPACITY, "a full-causal append past max_steps was skipped");
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_cache_steps");
  }
}

rswa_status rswa_cache_info(const rswa_cache* c, void** storage_dev, int64_t* seq_offset_host,
                            int32_t* rows_host) {
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  if (storage_dev) *storage_dev = c->storage;
  for (int b = 0; b < c->B; ++b) {
    if (seq_offset_host) seq_offset_host[b] = c->plan.seq_off[b];
    if (rows_host) rows_host[b] = c->plan.rows[b];
  }
  return RSWA_OK;
}

rswa_status rswa_cache_decode_plan(const rswa_cache* c, int32_t appending, int32_t* grid_blocks,
                                  int32_t* launches) {
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  try {
    const std::vector<int64_t> L = c->live_upper(appending ? 1 : 0);
    const rswa::DecodePlan plan =
        rswa::plan_decode(L, c->H, c->decode_resident(L), c->grid_max,
                          c->min_rows, c->grid_user, false);
    if (grid_blocks) *grid_blocks = (int32_t)plan.grid;
    if (launches) *launches = plan.grid > 0 ? 1 : 0;
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_cache_decode_plan");
  }
}

rswa_status rswa_cache_set_decode_split(rswa_cache* c, int32_t chunk_rows, int32_t grid_blocks) {
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  if (chunk_rows < 0) return fail(RSWA_E_INVALID, "chunk_rows must be >= 0");
  if (grid_blocks < 0) return fail(RSWA_E_INVALID, "grid_blocks must be >= 0");
  c->min_rows = chunk_rows;
  c->grid_user = grid_blocks;
  return RSWA_OK;
}

rswa_status rswa_cache_destroy(rswa_cache* c) {
  if (!c) return RSWA_OK;
  if (c->graphs > 0)
    return fail(RSWA_E_INVALID, "destroy every step graph of this cache before the cache");
  DeviceGuard g(c->device);
  // The cache may have been used on any stream; freeing device memory waits for the whole
  // device anyway, so wait for it once, explicitly, and report its status.
  const hipError_t e = hipDeviceSynchronize();
  release(c);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize(destroy)");
  return RSWA_OK;
}

rswa_status rswa_cache_query(rswa_cache* c, void** storage_dev, int64_t* k_offset_host,
                             int64_t* v_offset_host, int32_t* rows_host, int32_t* steps_host,
                             void* stream) {
  if (!c) return fail(RSWA_E_INVALID, "cache is NULL");
  if (storage_dev) *storage_dev = c->storage;
  for (int b = 0; b < c->B; ++b) {
    const int64_t k0 = c->plan.seq_off[b];
    if (k_offset_host) k_offset_host[b] = k0;
    if (v_offset_host) v_offset_host[b] = k0 + (int64_t)c->H * c->plan.rows[b] * c->D;
    if (rows_host) rows_host[b] = c->plan.rows[b];
  }
  if (!steps_host) return RSWA_OK;
  return rswa_cache_steps(c, steps_host, stream);
}

namespace {

// Host-checkable arguments shared by the prefill entry points.
rswa_status check_prefill(const void* q, const void* k, const void* v, const void* out,
                          int32_t out_dtype, const int32_t* cu, const int32_t* pl,
                          const int32_t* win, int32_t nseq, int32_t num_heads, int32_t head_dim,
                          int32_t max_seqlen, int32_t prefix_causal, float softmax_scale) {
  if (!q || !k || !v || !out) return fail(RSWA_E_INVALID, "q/k/v/out pointer is NULL");
  if (!cu || !pl || !win) return fail(RSWA_E_INVALID, "sequence metadata pointer is NULL");
  if (nseq < 1) return fail(RSWA_E_INVALID, "nseq must be >= 1");
  if (num_heads < 1 || num_heads > rswa::kMaxHeads)
    return fail(RSWA_E_INVALID, "num_heads out of range");
  if (head_dim < 1) return fail(RSWA_E_INVALID, "head_dim must be positive");
  if (head_dim != rswa::kPlanHeadDim) return fail(RSWA_E_UNSUPPORTED, "head_dim must be 128");
  if (max_seqlen < 0) return fail(RSWA_E_INVALID, "max_seqlen must be >= 0");
  if (out_dtype != RSWA_BF16 && out_dtype != RSWA_F32)
    return fail(RSWA_E_INVALID, "out_dtype must be RSWA_BF16 or RSWA_F32");
  if (prefix_causal != 0 && prefix_causal != 1)
    return fail(RSWA_E_INVALID, "prefix_causal must be 0 or 1");
  if (!(softmax_scale <= 0.f) && !std::isfinite(softmax_scale))
    return fail(RSWA_E_INVALID, "softmax_scale must be finite");
  return RSWA_OK;
}

float resolve_scale(float softmax_scale, int32_t head_dim) {
  return softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
}

rswa_status prefill_forward(const void* q_dev, const void* k_dev, const void* v_dev,
                            void* out_dev, int32_t out_dtype, float* lse_dev,
                            const int32_t* cu_seqlens_dev, const int32_t* prefix_len_dev,
                            const int32_t* window_dev, int32_t nseq, int32_t num_heads,
                            int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                            float softmax_scale, void* stream, const char* what) {
  const rswa_status st = check_prefill(q_dev, k_dev, v_dev, out_dev, out_dtype, cu_seqlens_dev,
                                       prefix_len_dev, window_dev, nseq, num_heads, head_dim,
                                       max_seqlen, prefix_causal, softmax_scale);
  if (st != RSWA_OK) return st;
  if (max_seqlen == 0) return RSWA_OK;
  try {
    const float scale = resolve_scale(softmax_scale, head_dim);
    rswa::PrefillArgs a{};
    a.q = reinterpret_cast<const uint16_t*>(q_dev);
    a.k = reinterpret_cast<const uint16_t*>(k_dev);
    a.v = reinterpret_cast<const uint16_t*>(v_dev);
    a.out = out_dev;
    a.lse = lse_dev;
    a.cu_seqlens = cu_seqlens_dev;
    a.prefix_len = prefix_len_dev;
    a.window = window_dev;
    a.nseq = nseq;
    a.heads = num_heads;
    a.max_seqlen = max_seqlen;
    a.prefix_causal = prefix_causal;
    a.scale_log2 = scale * 1.4426950408889634f;
    hipError_t e = hipSuccess;
    a.err = prefill_err_word(&e);
    if (!a.err) return hip_fail(e, "hipGetSymbolAddress(error word)");
    e = rswa::launch_prefill(a, out_dtype == RSWA_F32, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, what);
  }
}

}  // namespace

rswa_status rswa_prefill_attn(const void* q_dev, const void* k_dev, const void* v_dev,
                              void* out_dev, int32_t out_dtype, const int32_t* cu_seqlens_dev,
                              const int32_t* prefix_len_dev, const int32_t* window_dev,
                              int32_t nseq, int32_t num_heads, int32_t head_dim,
                              int32_t max_seqlen, int32_t prefix_causal, float softmax_scale,
                              void* stream) {
  return prefill_forward(q_dev, k_dev, v_dev, out_dev, out_dtype, nullptr, cu_seqlens_dev,
                         prefix_len_dev, window_dev, nseq, num_heads, head_dim, max_seqlen,
                         prefix_causal, softmax_scale, stream, "exception in rswa_prefill_attn");
}

rswa_status rswa_prefill_fwd(const void* q_dev, const void* k_dev, const void* v_dev,
                             void* out_dev, int32_t out_dtype, float* lse_dev,
                             const int32_t* cu_seqlens_dev, const int32_t* prefix_len_dev,
                             const int32_t* window_dev, int32_t nseq, int32_t num_heads,
                             int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                             float softmax_scale, void* stream) {
  if (!lse_dev) return fail(RSWA_E_INVALID, "lse pointer is NULL");
  return prefill_forward(q_dev, k_dev, v_dev, out_dev, out_dtype, lse_dev, cu_seqlens_dev,
                         prefix_len_dev, window_dev, nseq, num_heads, head_dim, max_seqlen,
                         prefix_causal, softmax_scale, stream, "exception in rswa_prefill_fwd");
}

}  // extern "C"

namespace {

// Shared body of rswa_prefill_bwd (caller's work array) and rswa_prefill_bwd_noalloc (the
// library's scratch array).
rswa_status prefill_backward(const void* q_dev, const void* k_dev, const void* v_dev,
                             const void* out_dev, int32_t out_dtype, const void* dout_dev,
                             const float* lse_dev, float* work_dev, void* dq_dev, void* dk_dev,
                             void* dv_dev, int32_t grad_dtype, const int32_t* cu_seqlens_dev,
                             const int32_t* prefix_len_dev, const int32_t* window_dev,
                             int32_t nseq, int32_t total_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                             float softmax_scale, void* stream) {
  const float scale = resolve_scale(softmax_scale, head_dim);
  rswa::BwdArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q_dev);
  a.k = reinterpret_cast<const uint16_t*>(k_dev);
  a.v = reinterpret_cast<const uint16_t*>(v_dev);
  a.out = out_dev;
  a.dout = reinterpret_cast<const uint16_t*>(dout_dev);
  a.lse = lse_dev;
  a.work = work_dev;
  a.rows = (int64_t)total_tokens * num_heads;
  a.dq = dq_dev;
  a.dk = dk_dev;
  a.dv = dv_dev;
  a.cu_seqlens = cu_seqlens_dev;
  a.prefix_len = prefix_len_dev;
  a.window = window_dev;
  a.nseq = nseq;
  a.heads = num_heads;
  a.max_seqlen = max_seqlen;
  a.prefix_causal = prefix_causal;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = hipSuccess;
  a.err = prefill_err_word(&e);
  if (!a.err) return hip_fail(e, "hipGetSymbolAddress(error word)");
  e = rswa::launch_prefill_bwd(a, out_dtype == RSWA_F32, grad_dtype == RSWA_F32,
                               reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill backward launch");
  return RSWA_OK;
}

// Host-checkable arguments of the backward entry points (the work array checked by the caller).
rswa_status check_backward(const void* q_dev, const void* k_dev, const void* v_dev,
                           const void* out_dev, int32_t out_dtype, const void* dout_dev,
                           const float* lse_dev, void* dq_dev, void* dk_dev, void* dv_dev,
                           int32_t grad_dtype, const int32_t* cu_seqlens_dev,
                           const int32_t* prefix_len_dev, const int32_t* window_dev,
                           int32_t nseq, int32_t total_tokens, int32_t num_heads,
                           int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                           float softmax_scale) {
  const rswa_status st = check_prefill(q_dev, k_dev, v_dev, out_dev, out_dtype, cu_seqlens_dev,
                                       prefix_len_dev, window_dev, nseq, num_heads, head_dim,
                                       max_seqlen, prefix_causal, softmax_scale);
  if (st != RSWA_OK) return st;
  if (!dout_dev || !lse_dev) return fail(RSWA_E_INVALID, "dout/lse pointer is NULL");
  if (!dq_dev || !dk_dev || !dv_dev) return fail(RSWA_E_INVALID, "dq/dk/dv pointer is NULL");
  if (grad_dtype != RSWA_BF16 && grad_dtype != RSWA_F32)
    return fail(RSWA_E_INVALID, "grad_dtype must be RSWA_BF16 or RSWA_F32");
  if (total_tokens < 0) return fail(RSWA_E_INVALID, "total_tokens must be >= 0");
  return RSWA_OK;
}

}  // namespace

extern "C" {

rswa_status rswa_prefill_bwd(const void* q_dev, const void* k_dev, const void* v_dev,
                             const void* out_dev, int32_t out_dtype, const void* dout_dev,
                             const float* lse_dev, float* work_dev, void* dq_dev, void* dk_dev,
                             void* dv_dev, int32_t grad_dtype, const int32_t* cu_seqlens_dev,
                             const int32_t* prefix_len_dev, const int32_t* window_dev,
                             int32_t nseq, int32_t total_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t max_seqlen, int32_t prefix_causal,
                             float softmax_scale, void* stream) {
  const rswa_status st = check_backward(q_dev, k_dev, v_dev, out_dev, out_dtype, dout_dev, lse_dev,
                                        dq_dev, dk_dev, dv_dev, grad_dtype, cu_seqlens_dev,
                                        prefix_len_dev, window_dev, nseq, total_tokens, num_heads,
                                        head_dim, max_seqlen, prefix_causal, softmax_scale);
  if (st != RSWA_OK) return st;
  if (!work_dev) return fail(RSWA_E_INVALID, "work pointer is NULL");
  if (max_seqlen == 0 || total_tokens == 0) return RSWA_OK;
  try {
    return prefill_backward(q_dev, k_dev, v_dev, out_dev, out_dtype, dout_dev, lse_dev, work_dev,
                            dq_dev, dk_dev, dv_dev, grad_dtype, cu_seqlens_dev, prefix_len_dev,
                            window_dev, nseq, total_tokens, num_heads, head_dim, max_seqlen,
                            prefix_causal, softmax_scale, stream);
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_prefill_bwd");
  }
}

rswa_status rswa_prefill_bwd_noalloc(const void* q_dev, const void* k_dev, const void* v_dev,
                                     const void* out_dev, int32_t out_dtype, const void* dout_dev,
                                     const float* lse_dev, void* dq_dev, void* dk_dev,
                                     void* dv_dev, int32_t grad_dtype,
                                     const int32_t* cu_seqlens_dev,
                                     const int32_t* prefix_len_dev, const int32_t* window_dev,
                                     int32_t nseq, int32_t total_tokens, int32_t num_heads,
                                     int32_t head_dim, int32_t max_seqlen,
                                     int32_t prefix_causal, float softmax_scale, void* stream) {
  const rswa_status st = check_backward(q_dev, k_dev, v_dev, out_dev, out_dtype, dout_dev, lse_dev,
                                        dq_dev, dk_dev, dv_dev, grad_dtype, cu_seqlens_dev,
                                        prefix_len_dev, window_dev, nseq, total_tokens, num_heads,
                                        head_dim, max_seqlen, prefix_causal, softmax_scale);
  if (st != RSWA_OK) return st;
  if ((int64_t)total_tokens * num_heads > kNoAllocRows)
    return fail(RSWA_E_INVALID, "total_tokens * num_heads exceeds the scratch array of "
                                "rswa_prefill_bwd_noalloc (1048576 rows)");
  if (max_seqlen == 0 || total_tokens == 0) return RSWA_OK;
  try {
    hipError_t e = hipSuccess;
    float* work = scratch_ptr(&e);
    if (!work) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    return prefill_backward(q_dev, k_dev, v_dev, out_dev, out_dtype, dout_dev, lse_dev, work,
                            dq_dev, dk_dev, dv_dev, grad_dtype, cu_seqlens_dev, prefix_len_dev,
                            window_dev, nseq, total_tokens, num_heads, head_dim, max_seqlen,
                            prefix_causal, softmax_scale, stream);
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_prefill_bwd_noalloc");
  }
}

rswa_status rswa_prefill_check(void* stream) {
  try {
    hipError_t e = hipSuccess;
    int32_t* word = prefill_err_word(&e);
    if (!word) return hip_fail(e, "hipGetSymbolAddress(error word)");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int32_t err = 0;
    e = hipMemcpyAsync(&err, word, sizeof(err), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess && err) {
      const int32_t zero = 0;
      e = hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, st);
      if (e == hipSuccess) e = hipStreamSynchronize(st);
    }
    if (e != hipSuccess) return hip_fail(e, "reading the prefill error word");
    if (err)
      return fail(RSWA_E_INVALID,
                  "a prefill or backward launch found a sequence longer than its max_seqlen (rows "
                  "past it were not written), a prefix longer than its sequence, or a window < 1");
    return RSWA_OK;
  } catch (...) {
    return fail(RSWA_E_INTERNAL, "exception in rswa_prefill_check");
  }
}

}  // extern "C"
