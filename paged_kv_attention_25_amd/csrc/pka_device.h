// Device-side helpers shared by the gfx950 kernels: vector types, bf16 packing,
// MFMA wrappers and page-table slot lookup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pka {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16). Lane l supplies row (l % 16) of A
// and column (l % 16) of B, reduction elements 8*(l/16) .. 8*(l/16)+7; it receives
// column (l % 16), rows 4*(l/16) .. 4*(l/16)+3 of D.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16). Lane l supplies row (l % 32) of A
// and column (l % 32) of B, reduction elements 8*(l/32) .. 8*(l/32)+7; register r of
// lane l receives D[8*(r/4) + 4*(l/32) + (r%4)][l % 32].
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even) in one dword, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Low (or high) 16-bit halves of two dwords, x's half in the low half of the result.
__device__ __forceinline__ uint32_t lo_halves(uint32_t x, uint32_t y) {
  return (x & 0xffffu) | (y << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t x, uint32_t y) {
  return (x >> 16) | (y & 0xffff0000u);
}

// Keep the compiler from using (and so waiting for) a loaded value `x` before this
// point: the load's latency overlaps with whatever comes before.
template <typename T>
__device__ __forceinline__ void hold(T& x) {
  asm volatile("" : "+v"(x));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Page-table geometry: token j of a request lives in slot table[j / P] * P + j % P.
struct PageGeom {
  int32_t page_size;
  int32_t page_shift;   // log2(page_size) when it is a power of two, else -1
  int32_t table_width;  // entries per page-table row
  int64_t num_pages;
  uint32_t div_magic;   // key / page_size == (key * div_magic) >> div_shift, 0 <= key < 2^31
  int32_t div_shift;
};

// Host: the geometry of a pool of `num_pages` pages of `page_size` slots read through
// page-table rows of `table_width` entries. Division by the page size becomes a
// multiply and a shift: with l = ceil(log2 P), shift = 31 + l and magic =
// ceil(2^shift / P) < 2^32, the error magic*P - 2^shift is below P <= 2^l, so for
// key < 2^31 it adds less than 1/P to key/P and the floor is exact.
inline PageGeom make_page_geom(int32_t page_size, int32_t table_width, int64_t num_pages) {
  PageGeom g;
  g.page_size = page_size;
  g.table_width = table_width;
  g.num_pages = num_pages;
  int32_t l = 0;
  while ((int64_t(1) << l) < page_size) ++l;
  g.page_shift = (int64_t(1) << l) == page_size ? l : -1;
  g.div_shift = 31 + l;
  g.div_magic = (uint32_t)(((uint64_t(1) << g.div_shift) + page_size - 1) / (uint64_t)page_size);
  return g;
}

// Page-table index of logical token `key` (0 <= key < 2^31).
__device__ __forceinline__ int32_t page_index(int32_t key, const PageGeom& pg) {
  return (int32_t)(((uint64_t)(uint32_t)key * pg.div_magic) >> pg.div_shift);
}

// Slot of logical token `key` of the request whose page-table row is `row`, or -1
// when the entry lies past the row or the page id is outside the pool (such a key
// is treated as absent; nothing outside the table or the pool is touched).
__device__ __forceinline__ int32_t slot_of(const int32_t* __restrict__ row, int32_t key,
                                           const PageGeom& pg) {
  int32_t idx, off;
  if (pg.page_shift >= 0) {
    idx = key >> pg.page_shift;
    off = key & (pg.page_size - 1);
  } else {
    idx = key / pg.page_size;
    off = key - idx * pg.page_size;
  }
  if (idx < 0 || idx >= pg.table_width) return -1;
  const int32_t page = row[idx];
  if (page < 0 || (int64_t)page >= pg.num_pages) return -1;
  return page * pg.page_size + off;
}

}  // namespace pka
