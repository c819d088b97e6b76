// store_kv: scatter the step's new K/V rows into their pool slots (bit copies).
//
// New keys and values join the pool history before attention reads them
// ("miniSGLang intro blog", section 1.3); the slot is a token position inside a
// page ("Mini-SGLang deployment guide", section 6.2).
//
// HBM-bound copy: each thread moves one 16-byte chunk of a K row and the same
// chunk of the V row. Consecutive threads cover consecutive chunks of a row, so
// both the reads of the new rows and the writes into a slot are fully coalesced
// (a row is Hkv*D*2 bytes: 2 KiB at 8 kv heads).
#include "pka_device.h"
#include "pka_kernels.h"

namespace pka {

__global__ __launch_bounds__(256) void store_kv_kernel(const u32x4* __restrict__ k_new,
                                                       const u32x4* __restrict__ v_new,
                                                       const int32_t* __restrict__ out_loc,
                                                       int64_t total_chunks, int32_t row_chunks,
                                                       int64_t num_slots, u32x4* __restrict__ k_pool,
                                                       u32x4* __restrict__ v_pool) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += stride) {
    const int64_t t = i / row_chunks;
    const int64_t c = i - t * row_chunks;
    const int32_t slot = out_loc[t];
    if (slot < 0 || (int64_t)slot >= num_slots) continue;  // outside the pool: skipped
    const int64_t dst = (int64_t)slot * row_chunks + c;
    k_pool[dst] = k_new[i];
    v_pool[dst] = v_new[i];
  }
}

hipError_t launch_store_kv(const StoreArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_tokens * a.row_chunks;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(store_kv_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)a.k_new, (const u32x4*)a.v_new, a.out_loc, total,
                     a.row_chunks, a.num_slots, (u32x4*)a.k_pool, (u32x4*)a.v_pool);
  return hipGetLastError();
}

}  // namespace pka
