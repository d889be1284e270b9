// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rswa {

// Per-sequence metadata of a decode cache, resident on the device (written once at creation).
struct CacheMeta {
  const int64_t* seq_off;    // [B] element offset of sequence b's K block
  const int32_t* rows;       // [B] R_b = m_b + cap_b rows per head
  const int32_t* prefix_len; // [B] m_b
  const int32_t* cap;        // [B] n_b (R-SWA ring slots) or max_steps_b (full causal)
  int32_t* err;              // [1] sticky flag: a full-causal append found no free row
  // Paged prefix (table != nullptr): cache row r < m_b is pool row table[table_off[b] + r] of the
  // token-major pools [rows][H][D]; storage row r' holds cache row m_b + r'.
  const int32_t* table;
  const int64_t* table_off;  // [B]
  const void* pool_k;
  const void* pool_v;
};

// Step counters t_b are double-buffered: a launch that appends reads steps_in and writes
// steps_out (= steps_in + appended), so no workgroup of that launch races on them; the host
// swaps the two buffers after every appending launch.
struct AppendArgs {
  void* storage;
  CacheMeta meta;
  const int32_t* steps_in;
  int32_t* steps_out;
  const void* k_new;        // [B][H][D]
  const void* v_new;        // [B][H][D]
  const uint8_t* active;    // [B] or nullptr
  int32_t heads;
  int32_t full_causal;
};

constexpr int32_t kUniFromCounters = -2;

struct DecodeArgs {
  void* storage;
  CacheMeta meta;
  const int32_t* steps_in;
  int32_t* steps_out;       // nullptr unless this launch appends
  const void* k_new;        // [B][H][D] or nullptr: decode only, no append
  const void* v_new;
  const void* q;            // [B][H][D]
  void* out;                // [B][H][D]
  const uint8_t* active;    // [B] or nullptr
  float* ws_acc;            // [slots][D] partial numerators
  float* ws_ml;             // [slots][2] partial (max, sum), log2 domain
  int32_t* ws_cnt;          // [B * H] pieces of each split range done in this launch (zero
                            // between launches: the last piece resets it)
  int32_t batch;
  int32_t heads;
  int32_t full_causal;
  int32_t aligned;          // 1: one workgroup per (b, h) key range; 0: balanced stream-K ranges
  int32_t split;            // > 1 (and not aligned): workgroup w takes piece w % split of range
                            // w / split, rows [i L / split, (i + 1) L / split)
  int32_t min_rows;         // stream-K: fewest rows a workgroup takes
  int32_t stream_loads;     // 1: cache rows are read with non-temporal loads (the step's rows do
                            // not fit the last-level cache, so keeping them there gains nothing)
  float scale_log2;         // softmax scale * log2(e)
  // Host-known plan: when every sequence has the same m, capacity and step count and no active
  // mask is involved, the host passes them (uni_t >= 0) and the kernel reads no per-sequence
  // metadata. uni_t = kUniFromCounters: the same, but the shared step count is read from
  // steps_in[0] on the device (captured steps, replayed at later counts). Otherwise (-1)
  // everything comes from the device arrays (masks, ragged, unequal counts).
  int32_t uni_t;            // t_b before this launch
  int32_t uni_m;            // m_b
  int32_t uni_cap;          // cap_b
  int32_t uni_rows;         // R_b (storage rows per head)
};

struct PrefixCopyArgs {
  void* storage;
  CacheMeta meta;
  const void* pk;           // [sum m][H][D]
  const void* pv;
  const int64_t* prefix_row0; // [B] first packed row of sequence b
  int32_t heads;
  int32_t batch;
};

// Output rows of a cache filled from a packed prefill batch: sequence b's segment starts at packed
// row row0[b] (its prefix), its outputs follow at row0[b] + m_b, and it holds steps[b] of them.
struct FillArgs {
  void* storage;
  CacheMeta meta;
  const void* k;            // [total][H][D], kv dtype
  const void* v;
  const int64_t* row0;      // [B]
  const int32_t* steps;     // [B] t_b
  int32_t heads;
  int32_t batch;
  int32_t full_causal;
};

struct PrefillArgs {
  const uint16_t* q;        // [total][H][D] bf16
  const uint16_t* k;
  const uint16_t* v;
  void* out;                // [total][H][D]
  float* lse;               // [total][H] natural log-sum-exp of the scaled scores, or nullptr
  const int32_t* cu_seqlens;
  const int32_t* prefix_len;
  const int32_t* window;
  int32_t nseq;
  int32_t heads;
  int32_t max_seqlen;
  int32_t prefix_causal;
  float scale_log2;
  int32_t* err;             // [1] set to 1 when the device finds metadata the launch cannot serve
};

struct BwdArgs {
  const uint16_t* q;        // [total][H][D] bf16
  const uint16_t* k;
  const uint16_t* v;
  const void* out;          // [total][H][D] forward output (bf16 or float32)
  const uint16_t* dout;     // [total][H][D] bf16 gradient of the output
  const float* lse;         // [total][H] natural log-sum-exp from the forward
  float* work;              // [2][H][total] written: lse * log2(e), then -rowsum(dout * out)
  int64_t rows;             // total * H
  void* dq;                 // [total][H][D] gradients (bf16 or float32)
  void* dk;
  void* dv;
  const int32_t* cu_seqlens;
  const int32_t* prefix_len;
  const int32_t* window;
  int32_t nseq;
  int32_t heads;
  int32_t max_seqlen;
  int32_t prefix_causal;
  float scale;
  float scale_log2;
  int32_t* err;             // [1] set to 1 when the device finds metadata the launch cannot serve
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_prefix_copy(const PrefixCopyArgs& a, int kv_f32, int max_rows, hipStream_t s);
// max_rows: the most output rows any sequence holds (min(n_b, t_b), or t_b in full-causal mode).
hipError_t launch_fill_outputs(const FillArgs& a, int kv_f32, int max_rows, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, int batch, int kv_f32, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int kv_f32, int out_f32, int grid_blocks,
                         hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int out_f32, hipStream_t s);
// Sets *bad = 1 if any of the n table entries lies outside [0, pool_rows).
hipError_t launch_table_check(const int32_t* table, int64_t n, int64_t pool_rows, int32_t* bad,
                              hipStream_t s);
hipError_t launch_prefill_bwd(const BwdArgs& a, int out_f32, int grad_f32, hipStream_t s);
// Resident 256-thread decode workgroups per CU (occupancy of the decode kernel for a batch of B).
int decode_blocks_per_cu(int kv_f32, int out_f32, int batch);
size_t decode_lds_bytes(int batch);

}  // namespace rswa
