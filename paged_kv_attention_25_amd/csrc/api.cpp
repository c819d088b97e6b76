// C ABI of the paged KV-cache attention library: host-side argument checks, the
// decode split plan, and kernel launches. Nothing here waits for the device or
// reads device memory, so every call is safe to capture into a HIP graph.
#include <hip/hip_runtime.h>

#include "../../include/pka.h"
#include "../../include/pka_sched.h"
#include "pka_kernels.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool geom_ok(const pka_geom* g) {
  if (g->num_q_heads < 1 || g->num_kv_heads < 1) return false;
  if (g->num_q_heads % g->num_kv_heads != 0) return false;
  if (g->head_dim < 1 || g->page_size < 1 || g->num_pages < 1) return false;
  // slots are 32-bit signed on the device
  if (g->num_pages * (int64_t)g->page_size > (int64_t)0x7fffffff) return false;
  return true;
}

int attn_geom_status(const pka_geom* g) {
  if (!geom_ok(g)) return PKA_E_SHAPE;
  if (g->head_dim != 128) return PKA_E_UNSUPPORTED;
  return PKA_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// The kernels move bf16 rows and workspace entries in 16-byte vector accesses (and
// copy pool rows straight into LDS in 16-byte pieces), and read index arrays as int32.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? PKA_OK : PKA_E_HIP; }

}  // namespace

extern "C" {

int pka_version(void) { return kVersion; }

const char* pka_status_string(int status) {
  switch (status) {
    case PKA_OK: return "ok";
    case PKA_E_NULLPTR: return "a required pointer is NULL";
    case PKA_E_SHAPE: return "invalid size or geometry";
    case PKA_E_UNSUPPORTED: return "unsupported by these kernels";
    case PKA_E_WORKSPACE: return "workspace missing or too small";
    case PKA_E_HIP: return "HIP runtime error";
    case PKA_E_STATE: return "unknown request or wrong request state";
    case PKA_E_CAPACITY: return "output array or page-table row too small";
    case PKA_E_NOMEM: return "host memory allocation failed";
    case PKA_E_SCRATCH: return "call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int pka_store_kv(const pka_geom* geom, const void* k_new, const void* v_new,
                 const int32_t* out_loc, int32_t num_tokens, void* k_pool, void* v_pool,
                 void* stream) {
  if (!geom) return PKA_E_NULLPTR;
  if (!geom_ok(geom) || num_tokens < 0) return PKA_E_SHAPE;
  if (geom->head_dim % 8 != 0) return PKA_E_UNSUPPORTED;
  if (num_tokens == 0) return PKA_OK;
  if (!k_new || !v_new || !out_loc || !k_pool || !v_pool) return PKA_E_NULLPTR;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(out_loc))
    return PKA_E_UNSUPPORTED;
  pka::StoreArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out_loc = out_loc;
  a.num_tokens = num_tokens;
  a.row_chunks = geom->num_kv_heads * geom->head_dim * 2 / 16;
  a.num_slots = geom->num_pages * (int64_t)geom->page_size;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  return launch_status(pka::launch_store_kv(a, as_stream(stream)));
}

size_t pka_decode_workspace_bytes(const pka_geom* geom, int32_t batch, int32_t max_seq_len) {
  if (!geom || !geom_ok(geom) || batch < 0 || max_seq_len < 0) return 0;
  const int32_t group = geom->num_q_heads / geom->num_kv_heads;
  const pka::DecodePlan plan = pka::plan_decode(batch, geom->num_kv_heads, group, max_seq_len);
  return pka::decode_workspace_bytes(batch, geom->num_q_heads, geom->num_kv_heads, plan);
}

}  // extern "C"

namespace {

// Checks and launch shared by the decode entry points; `store` non-null adds the
// new tokens' store (k_new, v_new, out_loc) to the launch; `use_static` takes the
// split partials' buffer from the library's static scratch instead of `workspace`.
struct NewRows {
  const void* k_new;
  const void* v_new;
  const int32_t* out_loc;
};

int decode_impl(const pka_geom* geom, const void* q, const void* k_pool, const void* v_pool,
                const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
                int32_t batch, int32_t max_seq_len, float scale, void* out, void* workspace,
                size_t workspace_bytes, void* stream, const NewRows* store,
                bool use_static = false) {
  if (!geom) return PKA_E_NULLPTR;
  const int gs = attn_geom_status(geom);
  if (gs != PKA_OK) return gs;
  if (batch < 0 || max_seq_len < 0 || page_table_stride < 0) return PKA_E_SHAPE;
  if (batch == 0) return PKA_OK;
  if (max_seq_len < 1) return PKA_E_SHAPE;
  const int32_t group = geom->num_q_heads / geom->num_kv_heads;
  if (!pka::decode_supported(batch, geom->num_kv_heads, group, max_seq_len))
    return PKA_E_UNSUPPORTED;
  const int64_t pages_needed = ((int64_t)max_seq_len + geom->page_size - 1) / geom->page_size;
  if (page_table_stride < pages_needed) return PKA_E_SHAPE;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !out) return PKA_E_NULLPTR;
  if (store && (!store->k_new || !store->v_new || !store->out_loc)) return PKA_E_NULLPTR;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      !aligned4(page_table) || !aligned4(seq_lens) || !aligned16(workspace))
    return PKA_E_UNSUPPORTED;
  if (store && (!aligned16(store->k_new) || !aligned16(store->v_new) ||
                !aligned4(store->out_loc)))
    return PKA_E_UNSUPPORTED;
  const pka::DecodePlan plan = pka::plan_decode(batch, geom->num_kv_heads, group, max_seq_len);
  const size_t need =
      pka::decode_workspace_bytes(batch, geom->num_q_heads, geom->num_kv_heads, plan);
  if (use_static) {
    if (need > pka::kStaticScratchBytes) return PKA_E_SCRATCH;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      if (pka::static_scratch(as_stream(stream), &workspace) != hipSuccess) return PKA_E_HIP;
      workspace_bytes = pka::kStaticScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKA_E_WORKSPACE;
  pka::DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.workspace = workspace;
  a.num_pages = geom->num_pages;
  a.page_size = geom->page_size;
  a.pt_stride = page_table_stride;
  a.batch = batch;
  a.num_q_heads = geom->num_q_heads;
  a.num_kv_heads = geom->num_kv_heads;
  a.max_seq_len = max_seq_len;
  a.scale = scale;
  if (store) {
    a.k_new = store->k_new;
    a.v_new = store->v_new;
    a.out_loc = store->out_loc;
    a.k_dst = const_cast<void*>(k_pool);
    a.v_dst = const_cast<void*>(v_pool);
  }
  return launch_status(pka::launch_decode(a, plan, as_stream(stream)));
}

}  // namespace

extern "C" {

int pka_paged_attn_decode(const pka_geom* geom, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* page_table,
                          int32_t page_table_stride, const int32_t* seq_lens, int32_t batch,
                          int32_t max_seq_len, float scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_impl(geom, q, k_pool, v_pool, page_table, page_table_stride, seq_lens, batch,
                     max_seq_len, scale, out, workspace, workspace_bytes, stream, nullptr);
}

int pka_paged_attn_decode_store(const pka_geom* geom, const void* q, const void* k_new,
                                const void* v_new, const int32_t* out_loc, void* k_pool,
                                void* v_pool, const int32_t* page_table,
                                int32_t page_table_stride, const int32_t* seq_lens,
                                int32_t batch, int32_t max_seq_len, float scale, void* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const NewRows rows{k_new, v_new, out_loc};
  return decode_impl(geom, q, k_pool, v_pool, page_table, page_table_stride, seq_lens, batch,
                     max_seq_len, scale, out, workspace, workspace_bytes, stream, &rows);
}

int pka_paged_attn_decode_store_noalloc(const pka_geom* geom, const void* q, const void* k_new,
                                        const void* v_new, const int32_t* out_loc, void* k_pool,
                                        void* v_pool, const int32_t* page_table,
                                        int32_t page_table_stride, const int32_t* seq_lens,
                                        int32_t batch, int32_t max_seq_len, float scale,
                                        void* out, void* stream) {
  const NewRows rows{k_new, v_new, out_loc};
  return decode_impl(geom, q, k_pool, v_pool, page_table, page_table_stride, seq_lens, batch,
                     max_seq_len, scale, out, nullptr, 0, stream, &rows, true);
}

size_t pka_prefill_workspace_bytes(const pka_geom* geom, int32_t batch, int32_t num_tokens,
                                   int32_t max_extend) {
  (void)num_tokens;
  if (!geom || !geom_ok(geom) || batch < 0 || max_extend < 0) return 0;
  return pka::prefill_workspace_bytes(batch, geom->num_q_heads / geom->num_kv_heads, max_extend);
}

int pka_paged_attn_prefill(const pka_geom* geom, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* page_table,
                           int32_t page_table_stride, const int32_t* seq_lens,
                           const int32_t* prefix_lens, const int32_t* extend_lens,
                           const int32_t* cu_extend, int32_t batch, int32_t num_tokens,
                           int32_t max_extend, int32_t max_seq_len, float scale, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!geom) return PKA_E_NULLPTR;
  const int gs = attn_geom_status(geom);
  if (gs != PKA_OK) return gs;
  if (batch < 0 || num_tokens < 0 || max_extend < 0 || max_seq_len < 0 ||
      page_table_stride < 0)
    return PKA_E_SHAPE;
  if (batch == 0 || num_tokens == 0) return PKA_OK;
  if (max_extend < 1 || max_extend > num_tokens || max_seq_len < max_extend)
    return PKA_E_SHAPE;
  const int64_t pages_needed = ((int64_t)max_seq_len + geom->page_size - 1) / geom->page_size;
  if (page_table_stride < pages_needed) return PKA_E_SHAPE;
  const int64_t group = geom->num_q_heads / geom->num_kv_heads;
  const int64_t tiles =
      ((int64_t)max_extend * group + pka::kPrefillRowsPerBlock - 1) / pka::kPrefillRowsPerBlock;
  if (tiles * batch * geom->num_kv_heads > 0x7fffffffLL) return PKA_E_UNSUPPORTED;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !prefix_lens || !extend_lens ||
      !cu_extend || !out)
    return PKA_E_NULLPTR;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      !aligned4(page_table) || !aligned4(seq_lens) || !aligned4(prefix_lens) ||
      !aligned4(extend_lens) || !aligned4(cu_extend) || !aligned16(workspace))
    return PKA_E_UNSUPPORTED;
  const size_t need = pka::prefill_workspace_bytes(batch, (int32_t)group, max_extend);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKA_E_WORKSPACE;
  pka::PrefillArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.prefix_lens = prefix_lens;
  a.extend_lens = extend_lens;
  a.cu_extend = cu_extend;
  a.out = out;
  a.num_pages = geom->num_pages;
  a.page_size = geom->page_size;
  a.pt_stride = page_table_stride;
  a.batch = batch;
  a.num_tokens = num_tokens;
  a.max_extend = max_extend;
  a.num_q_heads = geom->num_q_heads;
  a.num_kv_heads = geom->num_kv_heads;
  a.scale = scale;
  a.workspace = need > 0 ? workspace : nullptr;
  return launch_status(pka::launch_prefill(a, as_stream(stream)));
}

}  // extern "C"
