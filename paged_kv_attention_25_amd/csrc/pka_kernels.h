// Launchers of the gfx950 kernels (internal C++ interface between the C ABI and
// the kernels). Arguments are already validated by the caller; each launcher only
// enqueues work on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pka {

struct StoreArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* out_loc;
  int32_t num_tokens;
  int32_t row_chunks;  // 16-byte chunks per pool row (Hkv * D * 2 / 16)
  int64_t num_slots;
  void* k_pool;
  void* v_pool;
};
hipError_t launch_store_kv(const StoreArgs& a, hipStream_t stream);

// Plan of the decode kernel: `groups` groups of Hkv wavefronts (`waves` in all) share
// the batch's 64-key blocks, each group an equal contiguous range of the requests'
// blocks, one wavefront per kv head; `splits` when a (request, kv head) pair can have
// two or more blocks and so be split between groups (then a merge pass runs).
struct DecodePlan {
  int32_t groups;
  int32_t waves;
  bool splits;
  // One launch: a workgroup per (request, kv head), a wavefront per 64-key block of it
  // (small_waves of them), the blocks merged in LDS; the workspace is not used.
  bool small;
  int32_t small_waves;
};
DecodePlan plan_decode(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_seq_len);
// Whether the decode kernel supports this shape: batch, group size (q heads per kv
// head) and total block count (batch * Hkv * ceil(max_seq_len / 64) below 2^31).
bool decode_supported(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_seq_len);
size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              const DecodePlan& plan);

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* out;
  void* workspace;
  int64_t num_pages;
  int32_t page_size;
  int32_t pt_stride;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_seq_len;  // keys past it are not attended
  float scale;
  // With k_new non-null the launch also stores request b's new rows k_new[b], v_new[b]
  // into slot out_loc[b] of k_dst / v_dst (the same pools as k_pool / v_pool).
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* out_loc = nullptr;
  void* k_dst = nullptr;
  void* v_dst = nullptr;
};
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// Query rows (token, q head of the kv head's group) one prefill workgroup owns; a
// request gets ceil(max_extend * G / kPrefillRowsPerBlock) work items per kv head.
constexpr int kPrefillRowsPerBlock = 256;

struct PrefillArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* prefix_lens;
  const int32_t* extend_lens;
  const int32_t* cu_extend;
  void* out;
  int64_t num_pages;
  int32_t page_size;
  int32_t pt_stride;
  int32_t batch;
  int32_t num_tokens;
  int32_t max_extend;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  float scale;
  void* workspace;  // prefill_workspace_bytes(...) bytes (dispatch order), may be null when 0
};
// Workspace of a prefill launch: the dispatch order of its (request, q tile) items,
// one int32 each, when there is more than one request (a single request's items are
// already dispatched heaviest first); 0 otherwise.
size_t prefill_workspace_bytes(int32_t batch, int32_t group, int32_t max_extend);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Static device scratch (scratch.hip) for the decode entry point that allocates
// nothing: its address on the stream's device (which must be the current device),
// looked up on the first call on that device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch(hipStream_t stream, void** ptr);

inline int32_t page_shift_of(int32_t page_size) {
  if (page_size <= 0 || (page_size & (page_size - 1)) != 0) return -1;
  int32_t s = 0;
  while ((1 << s) < page_size) ++s;
  return s;
}

}  // namespace pka
