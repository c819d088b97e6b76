// Paged causal extend (chunked) prefill for gfx950.
//
// New token i of request b sits at absolute position p_b + i and attends to keys
// 0 .. p_b + i of its request, read from the paged pool through the page table
// (chunked prefill over a cached prefix: "Mini-SGLang deployment guide", sections
// 6.1 and 6.5; keys located through page-table metadata: "miniSGLang intro blog",
// section 1.3).
//
// Tiling. A workgroup of 8 wavefronts (two per SIMD) owns 256 query rows of one
// (request, kv head). Rows are (token, head-in-group) pairs, row r = i*G + hh, so the
// G q heads that share a kv head share every K/V tile. Each wavefront owns 32 rows. Keys are
// processed in tiles of 64, copied through the page table straight from the pool
// into LDS (no registers in between) by four of the wavefronts: four stages, one
// barrier per tile, a tile's loads issued between two and three tiles before its first
// use. The page-table entries the loads need are copied into LDS the same way two
// tiles earlier, so every global access of the loop is one in-order stream per loader
// with exact waits.
//
// Dispatch order. Work items are (request, 256-row q tile); with several requests a
// one-workgroup plan kernel first counting-sorts them by their number of key tiles,
// heaviest first, and the blocks take their items in that order (a single request's
// items already come in that order).
//
// LDS layout: K and V tiles are row-major (one 256-byte row per key) with the 16-byte
// chunks of row r XOR-swizzled, by r % 16 for K and by 2*(r % 8) for V, so that the K
// operand reads (16 bytes per lane) and the transposing V reads (8 bytes per lane)
// spread over all banks.
//
// Per wavefront and tile, with 32x32x16 bf16 MFMAs:
//   S^T[key][row] = K . Q^T   (A = K rows from LDS, B = Q held in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T from LDS by transposing reads, B = P^T taken
//                              straight from S^T's registers)
// Index choices:
//  * QK reduction order: lane l feeds d = 16c + 8*(l/32) + j to MFMA c.
//  * PV key order: MFMA u contracts the 16 keys 16u + 8*(j/4) + 4*(l/32) + (j%4),
//    the scores lane l already holds, so P^T needs no data movement; the transposing
//    reads fetch V rows in that order.
// Softmax runs in the log2 domain with the scale folded into one FMA per score. The
// running max comes from the first tile; later tiles exponentiate against it without
// computing their own maxima, and only a tile whose exponentials grow large (a lane's
// sum of 32 past 2^32) takes its row maxima, raises the max, rescales and redoes them.
// Probabilities therefore stay below 2^32 (bf16 and fp32 hold such values with the
// same relative precision as values in [0, 1]). Causal masking only on tiles that
// cross a wavefront's diagonal.
#include "pka_device.h"
#include "pka_kernels.h"

namespace pka {

namespace {

constexpr int kRowsPerWave = 32;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // 256
static_assert(kRowsPerBlock == kPrefillRowsPerBlock, "work items are sized by the launcher");
constexpr int kKeysPerTile = 64;
constexpr int kLoaders = kWaves / 2;                   // wavefronts that load tiles
constexpr int kKeysPerWave = kKeysPerTile / kLoaders;  // keys of a tile each loader loads
constexpr int kTileElems = kKeysPerTile * kHeadDim;   // one K or V tile: 16 KB
constexpr int kStages = 4;  // power of two
constexpr float kRedoSum = 0x1p32f;  // exponential sum that makes a tile raise the max
constexpr float kNegInf = -__builtin_huge_valf();

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

struct PrefillKernelArgs {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k_pool;
  const uint16_t* __restrict__ v_pool;
  const int32_t* __restrict__ page_table;
  const int32_t* __restrict__ prefix_lens;
  const int32_t* __restrict__ extend_lens;
  const int32_t* __restrict__ cu_extend;
  uint16_t* __restrict__ out;
  PageGeom pg;
  int32_t pt_stride;
  int32_t batch;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t tiles_per_seq;  // ceil(max_extend * G / 256)
  float scale_log2;
  // Item order (heaviest first), or null: entry i = {item, prefix_lens[b],
  // extend_lens[b], cu_extend[b]} of the i-th item to run (b = its request).
  const i32x4* __restrict__ schedule;
};

// Work item r (0 .. tiles_per_seq*batch-1) is q tile tiles_per_seq-1 - r/batch of request
// r % batch; with no schedule, items go out in that order (the highest q tiles, with
// the most keys, first) and the kv head varies fastest across consecutive blocks.
__device__ __forceinline__ int item_tiles(int item, const int32_t* __restrict__ prefix_lens,
                                          const int32_t* __restrict__ extend_lens, int batch,
                                          int group, int tiles_per_seq) {
  const int b = item % batch;
  const int tile = tiles_per_seq - 1 - item / batch;
  const int nrows = extend_lens[b] * group;
  const int row0 = tile * kRowsPerBlock;
  if (row0 >= nrows) return 0;
  const int key_end = prefix_lens[b] + (min(row0 + kRowsPerBlock, nrows) - 1) / group + 1;
  return (key_end + kKeysPerTile - 1) / kKeysPerTile;
}

constexpr int kPlanThreads = 1024;
constexpr int kPlanBins = 4096;  // work beyond 4095 tiles shares the last bin

// Dispatch order for several requests: one workgroup counting-sorts the work items by
// their number of key tiles, heaviest first (longest-processing-time-first list
// scheduling onto the CUs), so that long items do not start last and leave a tail.
// The order of items with equal work is arbitrary; it only affects timing. Each entry
// carries its request's lengths and row offset, so a block gets all it needs to start
// in one load.
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(
    const int32_t* __restrict__ prefix_lens, const int32_t* __restrict__ extend_lens,
    const int32_t* __restrict__ cu_extend, int32_t batch, int32_t group,
    int32_t tiles_per_seq, i32x4* __restrict__ schedule) {
  __shared__ int32_t start[kPlanBins];  // histogram, then first position of each bin
  __shared__ int32_t wave_tot[kPlanThreads / 64];
  const int tid = threadIdx.x;
  const int items = tiles_per_seq * batch;
  for (int i = tid; i < kPlanBins; i += kPlanThreads) start[i] = 0;
  __syncthreads();
  for (int it = tid; it < items; it += kPlanThreads) {
    const int w = min(item_tiles(it, prefix_lens, extend_lens, batch, group, tiles_per_seq),
                      kPlanBins - 1);
    atomicAdd(&start[w], 1);
  }
  __syncthreads();
  // Exclusive scan in descending work: thread t owns bins 4095-4t .. 4092-4t.
  constexpr int kPer = kPlanBins / kPlanThreads;
  int cnt[kPer];
  int local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    cnt[j] = start[kPlanBins - 1 - (kPer * tid + j)];
    local += cnt[j];
  }
  int incl = local;  // inclusive scan across the wavefront
  const int lane = tid & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[tid >> 6] = incl;
  __syncthreads();
  int before = incl - local;
  for (int w = 0; w < (tid >> 6); ++w) before += wave_tot[w];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    start[kPlanBins - 1 - (kPer * tid + j)] = before;
    before += cnt[j];
  }
  __syncthreads();
  for (int it = tid; it < items; it += kPlanThreads) {
    const int w = min(item_tiles(it, prefix_lens, extend_lens, batch, group, tiles_per_seq),
                      kPlanBins - 1);
    const int b = it % batch;
    schedule[atomicAdd(&start[w], 1)] = i32x4{it, prefix_lens[b], extend_lens[b], cu_extend[b]};
  }
}

// Element offset of 16-byte chunk c (0..15) of key row r in a K (or V) tile.
__device__ __forceinline__ int k_chunk(int r, int c) { return r * kHeadDim + 8 * (c ^ (r & 15)); }
__device__ __forceinline__ int v_chunk(int r, int c) {
  return r * kHeadDim + 8 * (c ^ (2 * (r & 7)));
}

// Transposing LDS read: within each 16-lane group, lane i receives element i % 4 of
// the four 8-byte chunks addressed by lanes 4j + i/4 (j = 0..3), in that order.
__device__ __forceinline__ u32x2 tr_read(const uint16_t* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Global -> LDS copies, no registers in between: lane l's 16 (or 4) bytes from `src`
// land at `lds_dst` + 16*l (4*l); `lds_dst` is the same for the whole wavefront and
// goes in M0 (one wait state before the load reads it). Completion is counted by
// vmcnt like any other vector load. They are issued from inline assembly so that the
// compiler adds no waits of its own before later LDS reads (it cannot tell the ring
// stages apart); the kernel waits for exactly the copies it needs (wait_vmcnt) and
// its own vmcnt waits stay correct, only more conservative, with these in flight.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}
__device__ __forceinline__ void global_to_lds(const uint16_t* src, uint16_t* lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_address(lds_dst)) : "memory", "m0");
}
__device__ __forceinline__ void global_to_lds_b32(const int32_t* src, int32_t* lds_dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_address(lds_dst)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  // vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their
  // maxima (no wait).
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence. The loads into LDS it orders are waited
// for explicitly (wait_vmcnt) before it.
__device__ __forceinline__ void lds_barrier() { __builtin_amdgcn_s_barrier(); }

// Instruction-scheduling hints: ask for a group of `n` instructions of one kind at
// this point of the scheduling region (groups are placed in program order).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
#define sched_group(kind, n) __builtin_amdgcn_sched_group_barrier((kind), (n), 0)

// max(x of this lane, x of lane l ^ 32).
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, r[0]), __builtin_bit_cast(float, r[1]));
}

// Two wavefronts per SIMD: while one runs its MFMAs the other runs its softmax or
// waits on LDS.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillKernelArgs p) {
  // Block id -> (work item, kv head), kv head fastest (all heads of an item run
  // together); the item comes from the schedule when there is one.
  const int id = blockIdx.x;
  const int g = id % p.num_kv_heads;
  int rest, e, prefix, q_row0;
  if (p.schedule) {
    const i32x4 entry = p.schedule[id / p.num_kv_heads];
    rest = entry[0];
    prefix = entry[1];
    e = entry[2];
    q_row0 = entry[3];
  } else {
    rest = id / p.num_kv_heads;
    const int b1 = rest % p.batch;
    e = p.extend_lens[b1];
    prefix = p.prefix_lens[b1];
    q_row0 = p.cu_extend[b1];
  }
  const int b = rest % p.batch;
  const int tile = p.tiles_per_seq - 1 - rest / p.batch;

  const int G = p.group;
  const int nrows = e * G;
  const int row0 = tile * kRowsPerBlock;
  if (row0 >= nrows) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31;   // MFMA column: this lane's query row
  const int hgrp = lane >> 5;  // MFMA reduction group

  // Keys the block needs: 0 .. prefix + (token of its last row).
  const int last_row_blk = min(row0 + kRowsPerBlock, nrows) - 1;
  const int key_end = prefix + last_row_blk / G + 1;
  const int n_tiles = (key_end + kKeysPerTile - 1) / kKeysPerTile;

  // This lane's query row.
  const int r = row0 + wave * kRowsPerWave + col;
  const bool row_in = r < nrows;
  const int tok = row_in ? r / G : 0;
  const int hh = row_in ? r - tok * G : 0;
  const bool row_ok = row_in && q_row0 + tok >= 0 && q_row0 + tok < p.num_tokens;
  const int lim = prefix + tok;  // last visible key of this row
  // The wavefront's smallest limit (rows are in token order).
  const int wrow_first = row0 + wave * kRowsPerWave;
  const int wave_lim_lo = prefix + (wrow_first < nrows ? wrow_first / G : 0);
  const bool active = wrow_first < nrows;  // the wavefront has rows of the block

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kStages * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kStages * kTileElems];
  __shared__ __attribute__((aligned(16))) int32_t ids_lds[kStages][kLoaders][64];

  // K/V tiles go from the pool straight into LDS (no registers in between). Only the
  // first kLoaders wavefronts load (they get issue priority on their SIMDs and so have
  // slack before each barrier); loader w loads keys 16w .. 16w+15 of a tile:
  // instruction i covers keys 16w + 4i + l/16, and lane l writes LDS bytes 16l .. 16l+15
  // of its 1 KB, i.e. chunk position l % 16 of key row 16w + 4i + l/16, so it fetches
  // the chunk the swizzle puts there.
  const bool loader = wave < kLoaders;
  const int64_t row_elems = (int64_t)p.num_kv_heads * kHeadDim;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_stride;
  const uint16_t* kbase = p.k_pool + (int64_t)g * kHeadDim;
  const uint16_t* vbase = p.v_pool + (int64_t)g * kHeadDim;
  // Key of instruction i of a tile starting at kt; keys past the block's last key are
  // clamped to it (loaded, never used).
  auto dma_key = [&](int kt, int i) {
    return min(kt + kKeysPerWave * wave + 4 * i + (lane >> 4), key_end - 1);
  };
  // Page-table entries of a tile's keys also go straight into LDS, into a ring of
  // kStages slots per loader: lane p (of the first 16) fetches the entry of the
  // loader's key 4*(p%4) + p/4, so lane l later reads the entries of its four keys
  // 4i + l/16 (i = 0..3) as one 16-byte word at position 4*(l/16). A table index past
  // the row reads the row's last entry.
  auto ids_dma = [&](int kt, int slot) {
    const int p16 = lane & 15;
    const int key = min(kt + kKeysPerWave * wave + 4 * (p16 & 3) + (p16 >> 2), key_end - 1);
    const int idx = min(page_index(key, p.pg), p.pg.table_width - 1);
    global_to_lds_b32(pt_row + idx, &ids_lds[slot][wave][0]);
  };
  // Issue the K/V loads of the tile at kt into `stage` from its page-table entries in
  // ring slot `slot`. A page id outside the pool reads slot 0 (that request's result
  // is then unspecified); every access stays in bounds.
  const uint32_t pages_u = (uint32_t)p.pg.num_pages;  // slots (so pages) < 2^31
  const uint32_t row_bytes = (uint32_t)row_elems * 2u;
  auto dma_tile = [&](int kt, int stage, int slot) {
    const i32x4 page = *(const i32x4*)&ids_lds[slot][wave][4 * (lane >> 4)];
    uint16_t* kd = k_lds + stage * kTileElems + kKeysPerWave * wave * kHeadDim;
    uint16_t* vd = v_lds + stage * kTileElems + kKeysPerWave * wave * kHeadDim;
    uint32_t slot_i[4];
    if (p.pg.page_shift >= 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        slot_i[i] = ((uint32_t)page[i] << p.pg.page_shift) +
                    (uint32_t)(dma_key(kt, i) & (p.pg.page_size - 1));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = dma_key(kt, i);
        slot_i[i] = (uint32_t)page[i] * p.pg.page_size +
                    (uint32_t)(key - page_index(key, p.pg) * p.pg.page_size);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t ro = (uint64_t)((uint32_t)page[i] < pages_u ? slot_i[i] : 0u) * row_bytes;
      const int rr = (4 * i + (lane >> 4)) & 15;  // key row mod 16 (16w is a multiple of 16)
      global_to_lds((const uint16_t*)((const char*)(kbase + 8 * ((lane & 15) ^ rr)) + ro),
                    kd + 4 * i * kHeadDim);
      global_to_lds((const uint16_t*)((const char*)(vbase + 8 * ((lane & 15) ^ (2 * (rr & 7)))) + ro),
                    vd + 4 * i * kHeadDim);
    }
  };

  // K operand reads: row 32*kb2 + col, chunk 2c + hgrp (swizzled by col % 16).
  int k_rd[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) k_rd[c] = k_chunk(col, 2 * c + hgrp);
  // V^T operand reads for d block t4 (d = 32*t4 + l % 32), key chunk u, half h: lane
  // (group gq = l/16, s = l%16) addresses key 16u + 8h + 4*(gq/2) + s/4 at
  // d = 32*t4 + 16*(gq%2) + 4*(s%4); the key part 16u + 8h is a whole number of rows.
  const int gq = lane >> 4;
  const int sq = lane & 15;
  int v_rd[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
    const int rv = 4 * (gq >> 1) + (sq >> 2);
    const int d = 32 * t4 + 16 * (gq & 1) + 4 * (sq & 3);
    v_rd[t4] = v_chunk(rv, d >> 3) + (d & 7);
  }

  float m = kNegInf;
  float lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t4][i] = 0.f;

  // Prologue. The loaders' copies of the page-table entries of tiles 0..3 go out
  // together with Q's loads, and one wait covers both.
  if (loader) {
#pragma unroll
    for (int t = 0; t < 4; ++t) ids_dma(t * kKeysPerTile, t);
  }
  // Q^T operands: 8 MFMAs over D, lane feeds d = 16c + 8*hgrp .. +8 of its row.
  u32x4 qv[8];
  if (row_ok) {
    const u32x4* src = (const u32x4*)(p.q + ((int64_t)(q_row0 + tok) * p.num_q_heads +
                                              (int64_t)g * G + hh) * kHeadDim + 8 * hgrp);
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[c] = src[2 * c];
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) qv[c] = u32x4{0, 0, 0, 0};
  }
  // Q has landed before any tile copy is issued: the compiler does not see those
  // copies, so a wait it placed for Q after them would also wait for them.
  wait_vmcnt<0>();
  // Then the K/V of tiles 0..2 and the entries of tile 4 (ring slot 0: tile 0's entries
  // have been read by then). Only tile 0 (the first 8 of these 25 copies) has landed
  // before the first barrier; the loop's first wait covers the rest.
  if (loader) {
#pragma unroll
    for (int t = 0; t < 3; ++t) dma_tile(t * kKeysPerTile, t, t);
    ids_dma(4 * kKeysPerTile, 0);
    wait_vmcnt<17>();
  }
  lds_barrier();

  f32x16 s[2];  // S^T of the current tile: two 32-key blocks
  u32x4 pb[4];  // P^T operands, one per 16-key chunk

  for (int t = 0; t < n_tiles; ++t) {
    const int kt = t * kKeysPerTile;
    const int stage = t & (kStages - 1);
    const uint16_t* kt_lds = k_lds + stage * kTileElems;
    const uint16_t* vt_lds = v_lds + stage * kTileElems;

    // A wavefront whose 32 rows all lie past the block's rows (the last q tile of a
    // request) skips the compute and only copies and waits, leaving its SIMD to the
    // other wavefront.
    if (active) {
      // S^T = K Q^T for the tile's two 32-key blocks. The K operands are read 8 MFMAs
      // ahead of their use (the schedule below), so LDS latency stays hidden.
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb2][i] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4 a = *(const u32x4*)(kt_lds + 32 * kb2 * kHeadDim + k_rd[c]);
          s[kb2] = mfma_32x32x16(a, qv[c], s[kb2]);
        }
      }
      sched_group(kSchedDsRead, 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sched_group(kSchedMfma, 1);
        sched_group(kSchedDsRead, 1);
      }
      sched_group(kSchedMfma, 8);
      // Causal mask only where the tile crosses this wavefront's diagonal: register i
      // of block kb2 holds key kt + 32*kb2 + 8*(i/4) + 4*hgrp + (i%4).
      if (kt + kKeysPerTile - 1 > wave_lim_lo) {
        const int dl = lim - kt - 4 * hgrp;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb2 + 8 * (i >> 2) + (i & 3) > dl) s[kb2][i] = kNegInf;
      }
      // Exponentials against the running max as it stands. Only the first tile, or a
      // tile where some lane's sum of 32 exponentials passes 2^32 (a row max above the
      // running one by more than ~27 in log2 units), computes the tile's row maxima,
      // raises the running max, rescales and redoes them; every other tile skips the max.
      auto exps = [&](float neg_m) {
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float pr[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pr[j] = fast_exp2(fmaf(s[u >> 1][8 * (u & 1) + j], p.scale_log2, neg_m));
            ps += pr[j];
          }
          pb[u][0] = pack_bf16x2(pr[0], pr[1]);
          pb[u][1] = pack_bf16x2(pr[2], pr[3]);
          pb[u][2] = pack_bf16x2(pr[4], pr[5]);
          pb[u][3] = pack_bf16x2(pr[6], pr[7]);
        }
        return ps;
      };
      float ps = 0.f;
      bool redo = t == 0;
      if (!redo) {
        ps = exps(-m * p.scale_log2);
        redo = __any(ps > kRedoSum);
      }
      if (redo) {
        float mx = kNegInf;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb2][i]);
        mx = max_across_halves(mx);
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2((m - m_new) * p.scale_log2);  // 0 when m = -inf
        lsum *= alpha;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) o[t4] = o[t4] * alpha;
        m = m_new;
        ps = exps(-m * p.scale_log2);
      }
      lsum += ps;
      // O^T += V^T P^T: d block t4, 16-key chunk u; the V^T operands are read 4 MFMAs
      // ahead of their use.
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const uint16_t* src = vt_lds + 16 * u * kHeadDim + v_rd[t4];
          const u32x2 lo = tr_read(src);
          const u32x2 hi = tr_read(src + 8 * kHeadDim);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          o[t4] = mfma_32x32x16(a, pb[u], o[t4]);
        }
      }
      sched_group(kSchedDsRead, 8);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        sched_group(kSchedMfma, 1);
        sched_group(kSchedDsRead, 2);
      }
      sched_group(kSchedMfma, 4);
    }
    if (loader) {
      // Tile t+3 into the stage tile t-1 used (every wavefront finished tile t-1 before
      // the last barrier), then the page-table entries of tile t+5 (its ring slot held
      // tile t+1's, read last iteration). Issued before this iteration's barrier, while
      // the other wavefront of the SIMD still computes.
      if (t + 3 < n_tiles)
        dma_tile(kt + 3 * kKeysPerTile, (t + 3) & (kStages - 1), (t + 3) & (kStages - 1));
      if (t + 5 < n_tiles) ids_dma(kt + 5 * kKeysPerTile, (t + 5) & (kStages - 1));
      // Before the barrier: tile t+1 (issued two iterations ago) and the entries of tile
      // t+4 (last iteration, after tile t+2) have landed. Issued after those entries:
      // this iteration's 8 loads of tile t+3 and one load of entries, each only if that
      // tile exists.
      if (t + 5 < n_tiles)
        wait_vmcnt<9>();
      else if (t + 3 < n_tiles)
        wait_vmcnt<8>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
  }

  if (!row_ok) return;
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / ltot;
  // Register r of tile t4 holds d = 32*t4 + 8*(r/4) + 4*hgrp + (r%4).
  uint16_t* dst = p.out + ((int64_t)(q_row0 + tok) * p.num_q_heads + (int64_t)g * G + hh) *
                              kHeadDim + 4 * hgrp;
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      u32x2 w;
      w[0] = pack_bf16x2(o[t4][4 * a4 + 0] * inv, o[t4][4 * a4 + 1] * inv);
      w[1] = pack_bf16x2(o[t4][4 * a4 + 2] * inv, o[t4][4 * a4 + 3] * inv);
      *(u32x2*)(dst + 32 * t4 + 8 * a4) = w;
    }
  }
}

}  // namespace

size_t prefill_workspace_bytes(int32_t batch, int32_t group, int32_t max_extend) {
  if (batch <= 1 || max_extend <= 0 || group <= 0) return 0;
  const int64_t tiles = ((int64_t)max_extend * group + kRowsPerBlock - 1) / kRowsPerBlock;
  return (size_t)(tiles * batch) * sizeof(i32x4);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.num_tokens == 0 || a.max_extend == 0) return hipSuccess;
  PrefillKernelArgs k;
  k.q = (const uint16_t*)a.q;
  k.k_pool = (const uint16_t*)a.k_pool;
  k.v_pool = (const uint16_t*)a.v_pool;
  k.page_table = a.page_table;
  k.prefix_lens = a.prefix_lens;
  k.extend_lens = a.extend_lens;
  k.cu_extend = a.cu_extend;
  k.out = (uint16_t*)a.out;
  k.pg = make_page_geom(a.page_size, a.pt_stride, a.num_pages);
  k.pt_stride = a.pt_stride;
  k.batch = a.batch;
  k.num_tokens = a.num_tokens;
  k.num_q_heads = a.num_q_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.group = a.num_q_heads / a.num_kv_heads;
  const int64_t rows = (int64_t)a.max_extend * k.group;
  k.tiles_per_seq = (int32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  k.scale_log2 = a.scale * kLog2e;
  k.schedule = nullptr;
  if (prefill_workspace_bytes(a.batch, k.group, a.max_extend) > 0) {
    i32x4* sched = (i32x4*)a.workspace;
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a.prefix_lens,
                       a.extend_lens, a.cu_extend, a.batch, k.group, k.tiles_per_seq, sched);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    k.schedule = sched;
  }
  const int64_t blocks = (int64_t)k.tiles_per_seq * a.batch * a.num_kv_heads;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, k);
  return hipGetLastError();
}

}  // namespace pka
