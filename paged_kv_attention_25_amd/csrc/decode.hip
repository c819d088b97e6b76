// Paged GQA decode for gfx950: persistent wavefronts over equal shares of the batch's
// key blocks, then a merge pass for the (request, kv head) pairs split between them.
//
// Batched decode reads every request's keys from the paged pool through its page
// table ("miniSGLang intro blog", section 1.3; "Mini-SGLang deployment guide",
// sections 6.2 and 6.3, where decode has its own kernel).
//
// Work decomposition. Request b's keys form nb_b = ceil(L_b / 64) blocks of 64, the
// same for each of its kv heads. The requests' blocks are laid end to end (NBh blocks
// per kv head) and cut into C equal contiguous ranges [c*NBh/C, (c+1)*NBh/C) (C at
// most NBh, so no range is empty). Range c goes to a group of Hkv wavefronts,
// wavefronts c*Hkv + g, one per kv head g, so every wavefront streams the same number
// of blocks (+-1) and the Hkv wavefronts of a group read the kv-head pieces of the
// same pool rows at about the same time (the rows reach HBM as whole rows rather than
// as Hkv separate gathers: long_decode -6%, decode_b256 -2% against ranges over the
// (request, kv head) pairs laid end to end). Each workgroup first builds, in LDS, the
// prefix sums of nb_b over the batch (and a copy of seq_lens) to map a block index to
// its (request, block). The part of one pair inside a wavefront's range is a
// segment: a segment that is the whole pair is written to `out` directly (bf16);
// otherwise it is a split of its pair, and its normalised partial output (f32) and
// log2-sum-exp go to the workspace slot 2w (the wavefront's first segment) or 2w+1
// (its last), and the merge kernel combines the splits of that pair:
//   LSE = log2 sum_s 2^lse_s,  out = sum_s 2^(lse_s - LSE) * o_s.
// Nothing synchronises the wavefronts, and moving to the next segment reads only LDS.
//
// Streaming. A wavefront holds one 64-key block (32 KB of K/V at 256-byte head
// rows) in registers. The next block's K (and q) go out as soon as this block's
// scores are computed, its V as soon as this block's PV is done (each into the
// registers just freed); the wavefront then moves its cursor (LDS only) and issues
// the page-table entries of the block after that (one entry per lane covers 64 keys).
// Page-table entries are consumed only after the next block's scores, so waiting for
// them never drains K/V loads issued after them (vmcnt counts vector memory
// operations in issue order).
//
// Per block, the G q heads of kv head g are the columns of 16x16x32 bf16 MFMA
// tiles (padded to 16 with zero queries):
//   S^T[key][head] = K . Q^T   (A = K rows, B = Q; 16 MFMAs per 64 keys)
//   O^T[d][head] += V^T . P^T  (A = V^T, B = P^T; 16 MFMAs per 64 keys)
// Index choices that make every operand a plain load:
//  * QK: MFMA c reduces over d = 32c .. 32c+31; lane group l/16 feeds d = 32c +
//    8*(l/16) .. +8, so one load instruction reads a whole 64-byte sector of each of
//    16 key rows.
//  * PV key order: in each 32-key half, lane group l/16 feeds keys {4*(l/16)+j,
//    16+4*(l/16)+j}, exactly the keys whose scores it holds after QK, so P^T needs
//    no data movement.
//  * Output rows: row m of O^T tile t is d = 8m + t, so lane l loads 16 contiguous
//    bytes V[key][8*(l%16) .. +8] per key (16 lanes read one 256-byte row) and an
//    in-register 8x8 transpose of bf16 pairs forms the operands.
// Softmax is online in the log2 domain (scale*log2(e) folded into one multiply).
//
// Workspace layout (only when a pair can have more than one block): partial outputs
// [2W, G, D] f32, their log2-sum-exps [2W, G] f32, then the block prefix sums over
// the batch [B + 1] int32 (written by workgroup 0 for the merge kernel).
#include "pka_device.h"
#include "pka_kernels.h"

namespace pka {

namespace {

constexpr int kBlock = 64;        // keys per wavefront block
constexpr int kWaves = 4;         // wavefronts per workgroup (sharing the LDS tables)
constexpr int kMaxBatchLds = 4096;
constexpr int kMaxGroup = 16;
// Wavefronts of the split kernel: one per SIMD (256 CUs x 4), one 4-wavefront workgroup
// per CU. Measured on decode_b256 / long_decode / tp4_mixed: 1024 beats 2048 (two per
// SIMD) by 1-2%; 1536 (half the CUs with two workgroups) and 512 are 11% and 35% slower.
constexpr int kMaxDecodeWaves = 1024;
constexpr float kNegInf = -__builtin_huge_valf();

// The pool pointers carry no __restrict__: with the store (kStore) the same pools are
// written through k_dst / v_dst in the same launch.
struct DecodeKernelArgs {
  const uint16_t* __restrict__ q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* __restrict__ page_table;
  const int32_t* __restrict__ seq_lens;
  uint16_t* __restrict__ out;
  float* __restrict__ part_o;        // [2W, G, D]
  float* __restrict__ part_lse;      // [2W, G]
  int32_t* __restrict__ req_blocks;  // [B + 1] block prefix sums (for the merge), or null
  PageGeom pg;
  int32_t pt_stride;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_seq_len;  // keys past it are not attended
  int32_t groups;       // C: groups of Hkv wavefronts sharing the blocks
  float scale_log2;
  // Store of the new tokens' rows (null k_new: none): request b's row goes to slot
  // out_loc[b] of k_dst / v_dst (the pools).
  const uint16_t* __restrict__ k_new;  // [B, Hkv, D]
  const uint16_t* __restrict__ v_new;
  const int32_t* __restrict__ out_loc;  // [B]
  uint16_t* k_dst;
  uint16_t* v_dst;
  int64_t num_slots;
};

struct Lds {
  int32_t prefix[kMaxBatchLds + 1];  // prefix sums of blocks per request
  int32_t seq_len[kMaxBatchLds];     // seq_lens, clamped to max_seq_len
  int32_t wave_tot[kWaves];
};

// Register-resident q, K and V of one 64-key block.
struct Block {
  u32x4 q[4];      // Q^T operand: q head n, d = 32c + 8*grp .. +8 (zero for n >= G)
  u32x4 k[4][4];   // [16-key group s][c]: key 16s + n, d = 32c + 8*grp .. +8
  u32x4 v[2][8];   // [32-key half h][j]: key 32h + {4grp+j | 16+4grp+(j-4)}, d = 8n .. +8
};

// One block of a wavefront's stream.
struct Desc {
  int32_t valid;
  int32_t b, g;
  int32_t k0, end, L;  // block start key, end of its segment's keys, request length
  int32_t last;        // last block of its segment
  int32_t slot;        // partial-output slot of its segment, or -1: written directly
  int32_t tail;        // the block holds the request's key L - 1 (its pair's last block)
};

struct SoftmaxState {
  float m;     // running max of this lane's column (log2 domain)
  float lsum;  // this lane's share of the running sum
  f32x4 o[8];  // O^T tiles: lane holds d = 32*grp + 8v + t in o[t][v]
};

__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int32_t blocks_of(int32_t L) { return L > 0 ? (L + kBlock - 1) / kBlock : 0; }

// First block of range c of `parts` equal ranges over n blocks (c = parts gives n).
__device__ __forceinline__ int32_t range_start(int32_t c, int32_t n, int32_t parts) {
  return (int32_t)(((int64_t)c * n) / parts);
}

// The wavefront's cursor: the next block x of its range [x, hi) and the segment x
// lies in.
struct Cursor {
  int32_t x, lo, hi;
  int32_t b, g, L;
  int32_t seg_end;  // end of the segment in the flattened block order
  int32_t slot;     // -1 when the segment is its whole pair
  int32_t j;        // block index of x within its pair
};

// Locate block x (lo <= x < hi) of the wavefront's kv head and set up its segment.
__device__ __forceinline__ void locate(Cursor& c, int32_t wave_id, const DecodeKernelArgs& p,
                                       const Lds& lds) {
  // largest b with prefix[b] <= x (requests without blocks have empty ranges)
  int32_t lo = 0, hi = p.batch;  // prefix[lo] <= x < prefix[hi]
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (uniform(lds.prefix[mid]) <= c.x) lo = mid; else hi = mid;
  }
  c.b = lo;
  c.L = uniform(lds.seq_len[lo]);
  const int32_t pair_start = uniform(lds.prefix[lo]);
  const int32_t pair_end = pair_start + blocks_of(c.L);
  c.seg_end = min(pair_end, c.hi);
  if (pair_start >= c.lo && pair_end <= c.hi)
    c.slot = -1;
  else
    c.slot = 2 * wave_id + (c.x == c.lo ? 0 : 1);
  c.j = c.x - pair_start;
}

__device__ __forceinline__ Desc cursor_next(Cursor& c, int32_t wave_id, const DecodeKernelArgs& p,
                                            const Lds& lds) {
  Desc d;
  d.valid = c.x < c.hi;
  d.b = c.b;
  // The kv head is the same for the whole stream; hidden from the compiler so that the
  // head's pool pointers are formed per block instead of held in registers.
  int32_t g = c.g;
  asm volatile("" : "+s"(g));
  d.g = g;
  d.L = c.L;
  d.slot = c.slot;
  if (!d.valid) {
    d.k0 = d.end = 0;
    d.last = 0;
    d.tail = 0;
    return d;
  }
  d.k0 = c.j * kBlock;
  d.end = min(c.L, (c.j + (c.seg_end - c.x)) * kBlock);
  d.last = c.x + 1 >= c.seg_end;
  d.tail = d.end == c.L && c.L <= d.k0 + kBlock;
  c.x += 1;
  c.j += 1;
  if (c.x >= c.seg_end && c.x < c.hi) locate(c, wave_id, p, lds);
  return d;
}

// Page-table entry of key (block start + lane), loaded but not yet used: the slot
// arithmetic runs in resolve(), after the current block's compute.
struct RawSlot {
  int32_t page;  // loaded page id
  int32_t off;   // offset in the page; -1 when the key's table index is past the row
  // (store, the pair's last block) the request's out_loc and this lane's 4 bytes of
  // the new token's K and V rows of kv head g
  int32_t loc;
  uint32_t krow, vrow;
};

template <bool kStore>
__device__ __forceinline__ RawSlot lookup_raw(const Desc& d, int lane, const DecodeKernelArgs& p) {
  RawSlot r;
  r.page = 0;
  r.off = -1;
  r.loc = -1;
  r.krow = r.vrow = 0u;
  if (!d.valid) return r;
  if (kStore && d.tail) {
    r.loc = p.out_loc[d.b];
    // (lane offset hidden from the compiler: per-lane pointers formed outside the
    // loop would cost registers for the whole stream)
    int32_t lo = 2 * lane;
    asm volatile("" : "+v"(lo));
    const int64_t e = ((int64_t)d.b * p.num_kv_heads + d.g) * kHeadDim;
    r.krow = *(const uint32_t*)(p.k_new + e + lo);
    r.vrow = *(const uint32_t*)(p.v_new + e + lo);
  }
  // keys past the block's end are clamped to the last valid key (loaded, masked)
  const int32_t key = min(d.k0 + lane, d.end - 1);
  int32_t idx;
  if (p.pg.page_shift >= 0) {
    idx = key >> p.pg.page_shift;
    r.off = key & (p.pg.page_size - 1);
  } else {
    idx = key / p.pg.page_size;
    r.off = key - idx * p.pg.page_size;
  }
  if (idx < 0 || idx >= p.pg.table_width) {
    r.off = -1;
  } else {
    r.page = p.page_table[(int64_t)d.b * p.pt_stride + idx];
  }
  return r;
}

__device__ __forceinline__ int32_t resolve(RawSlot r, const DecodeKernelArgs& p) {
  hold(r.page);
  const bool ok = r.off >= 0 && r.page >= 0 && (int64_t)r.page < p.pg.num_pages;
  return ok ? r.page * p.pg.page_size + r.off : -1;
}

// (store) Before the loads of a pair's last block: write the new token's row of kv
// head d.g to slot out_loc[b] when that slot is inside the pool. The wavefront's own
// loads issued after these stores see them, so the block's key L - 1 reads the new
// row when the page table maps it to that slot.
__device__ __forceinline__ void store_new_row(const Desc& d, RawSlot r, int lane,
                                              const DecodeKernelArgs& p) {
  if (!d.tail) return;
  hold(r.loc);
  hold(r.krow);
  hold(r.vrow);
  const int32_t loc = uniform(r.loc);
  if (loc < 0 || (int64_t)loc >= p.num_slots) return;
  int32_t lo = 2 * lane;
  asm volatile("" : "+v"(lo));
  const int64_t e = ((int64_t)loc * p.num_kv_heads + d.g) * kHeadDim;
  *(uint32_t*)(p.k_dst + e + lo) = r.krow;
  *(uint32_t*)(p.v_dst + e + lo) = r.vrow;
}

// Issue the loads of one block: K and q (kKQ) and/or V (kV). `slot` is this lane's
// slot of key (block start + lane). A key whose page id is outside the pool (slot -1) reads slot 0 instead: the
// access stays in bounds and that request's result is unspecified.
template <bool kKQ, bool kV>
__device__ __forceinline__ void load_block(Block& blk, const Desc& d, int32_t slot, int n, int grp,
                                           const DecodeKernelArgs& p) {
  const int64_t row_elems = (int64_t)p.num_kv_heads * kHeadDim;
  const uint16_t* kbase = p.k_pool + (int64_t)d.g * kHeadDim + 8 * grp;
  const uint16_t* vbase = p.v_pool + (int64_t)d.g * kHeadDim + 8 * n;
  if (kKQ) {
    if (n < p.group) {
      const uint16_t* qrow =
          p.q + ((int64_t)d.b * p.num_q_heads + d.g * p.group + n) * kHeadDim + 8 * grp;
#pragma unroll
      for (int c = 0; c < 4; ++c) blk.q[c] = *(const u32x4*)(qrow + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) blk.q[c] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int32_t sk = max(__shfl(slot, 16 * s + n), 0);
      const uint16_t* kp = kbase + (int64_t)sk * row_elems;
#pragma unroll
      for (int c = 0; c < 4; ++c) blk.k[s][c] = *(const u32x4*)(kp + 32 * c);
    }
  }
  if (kV) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kl = 32 * h + ((j < 4) ? (4 * grp + j) : (16 + 4 * grp + (j - 4)));
        const int32_t sv = max(__shfl(slot, kl), 0);
        blk.v[h][j] = *(const u32x4*)(vbase + (int64_t)sv * row_elems);
      }
    }
  }
}

__device__ __forceinline__ void reset_state(SoftmaxState& st) {
  st.m = kNegInf;
  st.lsum = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Scores and softmax of one block (K and q only): P^T operands in pb, running state
// updated (O rescaled).
__device__ __forceinline__ void scores_softmax(const Block& blk, const Desc& d, int grp,
                                               float scale_log2, SoftmaxState& st,
                                               u32x4 (&pbs)[2]) {
  // Scores: lane holds column n (q head), keys k0 + 16s + 4*grp + v in sacc[s][v].
  f32x4 sacc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc[s] = mfma_16x16x32(blk.k[s][c], blk.q[c], sacc[s]);
  }
  float sc[16];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int key = d.k0 + 16 * s + 4 * grp + v;
      sc[4 * s + v] = (key < d.end) ? sacc[s][v] * scale_log2 : kNegInf;
    }
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);  // finite: key k0 is always valid
  const float alpha = fast_exp2(st.m - m_new);
  float pr[16];
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pr[i] = fast_exp2(sc[i] - m_new);
    ps += pr[i];
  }
  st.lsum = st.lsum * alpha + ps;
  st.m = m_new;
#pragma unroll
  for (int t = 0; t < 8; ++t) st.o[t] = st.o[t] * alpha;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // P^T operand of half h: slots j<4 -> group 2h, j>=4 -> group 2h+1
    pbs[h][0] = pack_bf16x2(pr[8 * h + 0], pr[8 * h + 1]);
    pbs[h][1] = pack_bf16x2(pr[8 * h + 2], pr[8 * h + 3]);
    pbs[h][2] = pack_bf16x2(pr[8 * h + 4], pr[8 * h + 5]);
    pbs[h][3] = pack_bf16x2(pr[8 * h + 6], pr[8 * h + 7]);
  }
}

// O^T += V^T P^T for one block (V only).
__device__ __forceinline__ void pv_block(const Block& blk, const u32x4 (&pbs)[2],
                                         SoftmaxState& st) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 pb = pbs[h];
    const u32x4* vv = blk.v[h];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int w = t >> 1;
      u32x4 a;
      if ((t & 1) == 0) {
        a[0] = lo_halves(vv[0][w], vv[1][w]);
        a[1] = lo_halves(vv[2][w], vv[3][w]);
        a[2] = lo_halves(vv[4][w], vv[5][w]);
        a[3] = lo_halves(vv[6][w], vv[7][w]);
      } else {
        a[0] = hi_halves(vv[0][w], vv[1][w]);
        a[1] = hi_halves(vv[2][w], vv[3][w]);
        a[2] = hi_halves(vv[4][w], vv[5][w]);
        a[3] = hi_halves(vv[6][w], vv[7][w]);
      }
      st.o[t] = mfma_16x16x32(a, pb, st.o[t]);
    }
  }
}

// Write one segment's result: bf16 output when the segment is its whole pair, else
// the normalised partial output and its log2-sum-exp in the segment's slot.
__device__ __forceinline__ void finish_segment(const Desc& d, SoftmaxState& st, int n, int grp,
                                               const DecodeKernelArgs& p) {
  // (lane indices hidden from the compiler: output pointers formed outside the loop
  // would hold registers for the whole stream)
  asm volatile("" : "+v"(n), "+v"(grp));
  float ltot = st.lsum + __shfl_xor(st.lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  const float inv = 1.f / ltot;
  if (n < p.group) {
    if (d.slot < 0) {
      const int h = d.g * p.group + n;
      uint16_t* dst = p.out + ((int64_t)d.b * p.num_q_heads + h) * kHeadDim + 32 * grp;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        u32x4 w;
        w[0] = pack_bf16x2(st.o[0][v] * inv, st.o[1][v] * inv);
        w[1] = pack_bf16x2(st.o[2][v] * inv, st.o[3][v] * inv);
        w[2] = pack_bf16x2(st.o[4][v] * inv, st.o[5][v] * inv);
        w[3] = pack_bf16x2(st.o[6][v] * inv, st.o[7][v] * inv);
        *(u32x4*)(dst + 8 * v) = w;
      }
    } else {
      const int64_t row = (int64_t)d.slot * p.group + n;
      float* dst = p.part_o + row * kHeadDim + 32 * grp;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        *(f32x4*)(dst + 8 * v) =
            f32x4{st.o[0][v] * inv, st.o[1][v] * inv, st.o[2][v] * inv, st.o[3][v] * inv};
        *(f32x4*)(dst + 8 * v + 4) =
            f32x4{st.o[4][v] * inv, st.o[5][v] * inv, st.o[6][v] * inv, st.o[7][v] * inv};
      }
      if (grp == 0) p.part_lse[row] = st.m + __builtin_log2f(ltot);
    }
  }
  reset_state(st);
}

// Two wavefronts per SIMD (256 registers each). kStore: the launch also stores the new
// tokens' rows (p.k_new non-null).
template <bool kStore>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_split_kernel(DecodeKernelArgs p) {
  __shared__ Lds lds;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;   // MFMA row/column index of this lane
  const int grp = lane >> 4; // MFMA reduction group of this lane

  // Prefix sums of blocks per request (blocked scan: each thread owns a run of
  // consecutive requests) and a copy of seq_lens clamped to max_seq_len.
  const int per = (p.batch + kWaves * 64 - 1) / (kWaves * 64);
  const int b0 = tid * per;
  int32_t run = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < p.batch) {
      const int32_t L = min(p.seq_lens[b], p.max_seq_len);
      lds.seq_len[b] = L;
      run += blocks_of(L);
    }
  }
  int32_t incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds.wave_tot[wave] = incl;
  __syncthreads();
  int32_t base = 0;
  for (int w = 0; w < wave; ++w) base += lds.wave_tot[w];
  int32_t excl = base + incl - run;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < p.batch) {
      lds.prefix[b] = excl;
      if (blockIdx.x == 0 && p.req_blocks) p.req_blocks[b] = excl;
      excl += blocks_of(lds.seq_len[b]);
    }
  }
  if (tid == kWaves * 64 - 1) {
    lds.prefix[p.batch] = excl;
    if (blockIdx.x == 0 && p.req_blocks) p.req_blocks[p.batch] = excl;
  }
  __syncthreads();
  const int32_t nb_head = uniform(lds.prefix[p.batch]);

  // No more groups than blocks of one kv head, so that every range is non-empty.
  const int32_t groups = min(p.groups, nb_head);
  const int32_t wave_id = (int32_t)blockIdx.x * kWaves + wave;
  if (wave_id >= groups * p.num_kv_heads) return;
  const int32_t grp_id = uniform(wave_id / p.num_kv_heads);
  Cursor cur;
  cur.g = uniform(wave_id - grp_id * p.num_kv_heads);
  cur.lo = uniform(range_start(grp_id, nb_head, groups));
  cur.hi = uniform(range_start(grp_id + 1, nb_head, groups));
  cur.x = cur.lo;
  if (cur.x >= cur.hi) return;
  locate(cur, wave_id, p, lds);

  SoftmaxState st;
  reset_state(st);
  Block blk;
  Desc d = cursor_next(cur, wave_id, p, lds);
  {
    const RawSlot raw = lookup_raw<kStore>(d, lane, p);
    const int32_t slot = resolve(raw, p);
    if (kStore) store_new_row(d, raw, lane, p);
    load_block<true, true>(blk, d, slot, n, grp, p);
  }
  Desc dn = cursor_next(cur, wave_id, p, lds);
  RawSlot raw_n = lookup_raw<kStore>(dn, lane, p);

  while (d.valid) {
    // The next block's K and q go out as soon as this block's scores are computed, its
    // V as soon as this block's PV is done; then the cursor (LDS only), the page-table
    // entries of the block after (and, with the store, the new token's row when that
    // block is its pair's last) and this segment's stores.
    u32x4 pbs[2];
    scores_softmax(blk, d, grp, p.scale_log2, st, pbs);
    const int32_t slot_n = resolve(raw_n, p);
    if (kStore) store_new_row(dn, raw_n, lane, p);
    if (dn.valid) load_block<true, false>(blk, dn, slot_n, n, grp, p);
    pv_block(blk, pbs, st);
    if (dn.valid) load_block<false, true>(blk, dn, slot_n, n, grp, p);
    const Desc dnn = cursor_next(cur, wave_id, p, lds);
    raw_n = lookup_raw<kStore>(dnn, lane, p);
    if (d.last) finish_segment(d, st, n, grp, p);
    d = dn;
    dn = dnn;
  }
}

// Small launches (a pair has at most kSmallWaves blocks and the whole batch fits in
// one round of resident wavefronts): one workgroup per (request, kv head) pair, one
// wavefront per 64-key block of it. Each wavefront runs its block like a split-kernel
// segment, leaves the normalised partial output and log2-sum-exp of its q heads in LDS,
// and the workgroup merges them (the same combination as the merge kernel), so the step
// needs neither the batch-wide block scan nor a second launch.
constexpr int kSmallWaves = 8;  // 256 VGPRs per wavefront: two per SIMD
constexpr int kSmallMaxTotalWaves = 2048;

template <bool kStore>
__global__ __launch_bounds__(kSmallWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void decode_small_kernel(DecodeKernelArgs p) {
  __shared__ float s_o[kSmallWaves * kMaxGroup][kHeadDim];
  __shared__ float s_lse[kSmallWaves * kMaxGroup];
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;
  const int grp = lane >> 4;
  const int32_t b = uniform((int32_t)blockIdx.x / p.num_kv_heads);
  const int32_t g = uniform((int32_t)blockIdx.x - b * p.num_kv_heads);
  // The page-table entry of key k0 + lane (and, for the store, the request's out_loc
  // and new rows) load together with the request's length, as none of them depends on
  // it: the block's keys past the length are redirected to key L - 1 afterwards. The
  // kernel arguments these loads need are in registers first, so that no wait for one
  // of those arguments also waits for a load already in flight.
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_stride;
  const int32_t* len_at = p.seq_lens + b;
  const int32_t* loc_at = p.out_loc + b;
  asm volatile("" ::"s"(pt_row), "s"(len_at), "s"(loc_at), "s"(p.pg.page_shift),
               "s"(p.pg.page_size), "s"(p.pg.table_width), "s"(p.pg.div_magic),
               "s"(p.pg.div_shift), "s"(p.max_seq_len));
  Desc d;
  d.b = b;
  d.g = g;
  d.k0 = wave * kBlock;
  RawSlot raw;
  raw.page = 0;
  raw.loc = -1;
  raw.krow = raw.vrow = 0u;
  {
    const int32_t key = d.k0 + lane;
    int32_t idx;
    if (p.pg.page_shift >= 0) {
      idx = key >> p.pg.page_shift;
      raw.off = key & (p.pg.page_size - 1);
    } else {
      idx = (int32_t)(((uint64_t)(uint32_t)key * p.pg.div_magic) >> p.pg.div_shift);
      raw.off = key - idx * p.pg.page_size;
    }
    if (idx >= p.pg.table_width) raw.off = -1;
    else raw.page = pt_row[idx];
  }
  const int32_t L = uniform(min(*len_at, p.max_seq_len));
  if (kStore) {
    raw.loc = *loc_at;
    // (lane offset hidden from the compiler, as in the split path)
    int32_t lo = 2 * lane;
    asm volatile("" : "+v"(lo));
    const int64_t e = ((int64_t)b * p.num_kv_heads + g) * kHeadDim;
    raw.krow = *(const uint32_t*)(p.k_new + e + lo);
    raw.vrow = *(const uint32_t*)(p.v_new + e + lo);
  }
  if (L <= 0) {
    // No keys: the output row is not written (as in the split path). (The loads above
    // are consumed on this path too, so that the compiler keeps them ahead of the
    // length's wait.)
    hold(raw.page);
    hold(raw.krow);
    return;
  }
  d.L = L;
  d.end = L;
  d.valid = d.k0 < L;
  d.last = 1;
  d.slot = -1;
  d.tail = d.valid && L <= d.k0 + kBlock;
  SoftmaxState st;
  reset_state(st);
  if (d.valid) {
    // Keys past L - 1 read key L - 1's slot (held by lane L - 1 - k0), as the clamped
    // lookup of the split path does.
    int32_t slot = resolve(raw, p);
    const int32_t slot_last = __shfl(slot, min(L - 1 - d.k0, kBlock - 1));
    if (d.k0 + lane >= L) slot = slot_last;
    if (kStore) store_new_row(d, raw, lane, p);
    Block blk;
    load_block<true, true>(blk, d, slot, n, grp, p);
    u32x4 pbs[2];
    scores_softmax(blk, d, grp, p.scale_log2, st, pbs);
    pv_block(blk, pbs, st);
    float ltot = st.lsum + __shfl_xor(st.lsum, 16);
    ltot += __shfl_xor(ltot, 32);
    if (n < p.group) {
      // lane (n, grp) holds d = 32*grp + 8v + t of q head n in o[t][v]
      const int row = wave * p.group + n;
      const float inv = 1.f / ltot;
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int t = 0; t < 8; ++t) s_o[row][32 * grp + 8 * v + t] = st.o[t][v] * inv;
      if (grp == 0) s_lse[row] = st.m + __builtin_log2f(ltot);
    }
  }
  __syncthreads();
  // Merge: thread i combines output element i of the pair's G x D (two per thread).
  const int nblk = blocks_of(L);  // wavefronts that wrote a partial (>= 1)
  const int pairs = p.group * (kHeadDim / 2);
  for (int i = tid; i < pairs; i += (int)blockDim.x) {
    const int hn = i / (kHeadDim / 2);
    const int dd = 2 * (i - hn * (kHeadDim / 2));
    float mx = kNegInf;
    for (int w = 0; w < nblk; ++w) mx = fmaxf(mx, s_lse[w * p.group + hn]);
    float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int w = 0; w < nblk; ++w) {
      const int row = w * p.group + hn;
      const float wt = fast_exp2(s_lse[row] - mx);
      wsum += wt;
      acc0 += wt * s_o[row][dd];
      acc1 += wt * s_o[row][dd + 1];
    }
    const float inv = 1.f / wsum;
    uint16_t* dst = p.out + ((int64_t)b * p.num_q_heads + (int64_t)g * p.group + hn) * kHeadDim + dd;
    *(uint32_t*)dst = pack_bf16x2(acc0 * inv, acc1 * inv);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// The group whose range holds block x of a kv head: the largest c with
// floor(c*NBh/C) <= x, i.e. ceil((x+1)*C/NBh) - 1.
__device__ __forceinline__ int32_t group_of(int32_t x, int32_t nb_head, int32_t groups) {
  return (int32_t)((((int64_t)x + 1) * groups + nb_head - 1) / nb_head) - 1;
}

// Merge of up to K splits with one round of loads: lane s loads split s's
// log2-sum-exp while every lane loads its part (d = 2l, 2l+1) of all splits' outputs.
template <int K, typename RowOf>
__device__ __forceinline__ void merge_one_round(const float* __restrict__ part_o,
                                                const float* __restrict__ part_lse,
                                                const RowOf& row_of, int nsplit, int lane,
                                                uint32_t* dst) {
  const float lse_l = lane < nsplit ? part_lse[row_of(lane)] : kNegInf;
  float2 v[K];
#pragma unroll
  for (int i = 0; i < K; ++i)
    v[i] = i < nsplit ? *(const float2*)(part_o + row_of(i) * kHeadDim + 2 * lane)
                      : float2{0.f, 0.f};
  const float mx = wave_max(lse_l);
  const float w_l = lane < nsplit ? fast_exp2(lse_l - mx) : 0.f;
  const float inv = 1.f / wave_sum(w_l);
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const float w = __shfl(w_l, i);  // 0 past nsplit
    acc0 += w * v[i].x;
    acc1 += w * v[i].y;
  }
  dst[lane] = pack_bf16x2(acc0 * inv, acc1 * inv);
}

// One wavefront per (request, q head) of a pair (b, g) split between the ranges of
// groups c0 .. c1, four per workgroup: split i comes from wavefront w = (c0 + i) * Hkv
// + g, in slot 2w (that wavefront's first segment) except for i = 0 when its range
// began before the pair (slot 2w + 1). Lane l combines d = 2l, 2l+1. Up to 32 splits
// (the usual case) are merged with one round of loads; longer rows go through a loop
// of 64 splits at a time.
constexpr int kMergeWaves = 4;
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse,
    const int32_t* __restrict__ req_blocks, uint16_t* __restrict__ out, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t groups) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= (int64_t)batch * num_q_heads) return;
  const int b = (int)(row / num_q_heads);
  const int h = (int)(row - (int64_t)b * num_q_heads);
  const int G = num_q_heads / num_kv_heads;
  const int g = h / G;
  const int nq = h - g * G;
  // The pair's blocks from the prefix sums alone (they count min(seq_len, max_seq_len)),
  // so that its three loads go out together.
  const int32_t S = req_blocks[b];
  const int32_t nb = req_blocks[b + 1] - S;
  const int32_t nb_head = req_blocks[batch];
  if (nb <= 0) return;
  groups = min(groups, nb_head);  // as in the split kernel
  const int32_t c0 = group_of(S, nb_head, groups);
  const int32_t c1 = group_of(S + nb - 1, nb_head, groups);
  if (c0 == c1) return;  // written directly by the split kernel
  const int32_t first0 = range_start(c0, nb_head, groups) == S ? 0 : 1;
  const int nsplit = c1 - c0 + 1;
  // row of split i in part_o / part_lse: wavefront (c0 + i) * Hkv + g
  auto row_of = [&](int i) -> int64_t {
    const int32_t w = (c0 + i) * num_kv_heads + g;
    const int32_t slot = 2 * w + (i == 0 ? first0 : 0);
    return (int64_t)slot * G + nq;
  };
  uint32_t* dst = (uint32_t*)(out + ((int64_t)b * num_q_heads + h) * kHeadDim);
  if (nsplit <= 16) {
    merge_one_round<16>(part_o, part_lse, row_of, nsplit, lane, dst);
    return;
  }
  if (nsplit <= 32) {
    merge_one_round<32>(part_o, part_lse, row_of, nsplit, lane, dst);
    return;
  }
  float mx = kNegInf;
  for (int s0 = 0; s0 < nsplit; s0 += 64)
    mx = fmaxf(mx, s0 + lane < nsplit ? part_lse[row_of(s0 + lane)] : kNegInf);
  mx = wave_max(mx);
  float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int my = s0 + lane;
    const float w_l = my < nsplit ? fast_exp2(part_lse[row_of(my)] - mx) : 0.f;
    wsum += w_l;
    const int cnt = min(64, nsplit - s0);
    // 16 splits' loads in flight at a time: a long row's merge is a chain of
    // dependent memory latencies otherwise.
    int s = 0;
    for (; s + 16 <= cnt; s += 16) {
      float2 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = *(const float2*)(part_o + row_of(s0 + s + i) * kHeadDim + 2 * lane);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float w = __shfl(w_l, s + i);
        acc0 += w * v[i].x;
        acc1 += w * v[i].y;
      }
    }
    for (; s < cnt; ++s) {
      const float2 v = *(const float2*)(part_o + row_of(s0 + s) * kHeadDim + 2 * lane);
      const float w = __shfl(w_l, s);
      acc0 += w * v.x;
      acc1 += w * v.y;
    }
  }
  const float inv = 1.f / wave_sum(wsum);
  dst[lane] = pack_bf16x2(acc0 * inv, acc1 * inv);
}

}  // namespace

bool decode_supported(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_seq_len) {
  const int64_t blocks = (int64_t)batch * num_kv_heads * ((max_seq_len + kBlock - 1) / kBlock);
  return batch <= kMaxBatchLds && group <= kMaxGroup && blocks < ((int64_t)1 << 31);
}

DecodePlan plan_decode(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_seq_len) {
  // As many groups of Hkv wavefronts as fit resident (at least one), but no more than
  // the most blocks one kv head of the batch can have; a pair can be split only when
  // it can have two or more blocks.
  DecodePlan plan;
  const int64_t per_pair = max_seq_len > 0 ? ((int64_t)max_seq_len + kBlock - 1) / kBlock : 0;
  const int64_t head_blocks = (int64_t)batch * per_pair;
  int64_t groups = kMaxDecodeWaves / num_kv_heads;
  if (groups > head_blocks) groups = head_blocks;
  if (groups < 1) groups = 1;
  plan.groups = (int32_t)groups;
  plan.waves = (int32_t)(groups * num_kv_heads);
  plan.splits = per_pair > 1;
  plan.small_waves = (int32_t)per_pair;
  plan.small = per_pair >= 1 && per_pair <= kSmallWaves && group <= kMaxGroup &&
               (int64_t)batch * num_kv_heads * per_pair <= kSmallMaxTotalWaves;
  return plan;
}

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              const DecodePlan& plan) {
  if (!plan.splits) return 0;
  const size_t rows = (size_t)2 * plan.waves * (num_q_heads / num_kv_heads);
  return rows * (kHeadDim + 1) * sizeof(float) + ((size_t)batch + 1) * sizeof(int32_t);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  DecodeKernelArgs k;
  k.q = (const uint16_t*)a.q;
  k.k_pool = (const uint16_t*)a.k_pool;
  k.v_pool = (const uint16_t*)a.v_pool;
  k.page_table = a.page_table;
  k.seq_lens = a.seq_lens;
  k.out = (uint16_t*)a.out;
  const int32_t group = a.num_q_heads / a.num_kv_heads;
  const size_t rows = (size_t)2 * plan.waves * group;
  k.part_o = plan.splits ? (float*)a.workspace : nullptr;
  k.part_lse = plan.splits ? k.part_o + rows * kHeadDim : nullptr;
  k.req_blocks = plan.splits ? (int32_t*)(k.part_lse + rows) : nullptr;
  k.pg = make_page_geom(a.page_size, a.pt_stride, a.num_pages);
  k.pt_stride = a.pt_stride;
  k.batch = a.batch;
  k.num_q_heads = a.num_q_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.group = group;
  k.max_seq_len = a.max_seq_len;
  k.groups = plan.groups;
  k.scale_log2 = a.scale * kLog2e;
  k.k_new = (const uint16_t*)a.k_new;
  k.v_new = (const uint16_t*)a.v_new;
  k.out_loc = a.out_loc;
  k.k_dst = (uint16_t*)a.k_dst;
  k.v_dst = (uint16_t*)a.v_dst;
  k.num_slots = a.num_pages * (int64_t)a.page_size;
  if (plan.small) {
    const dim3 grid((unsigned)((int64_t)a.batch * a.num_kv_heads));
    const dim3 block((unsigned)(plan.small_waves * 64));
    if (k.k_new)
      hipLaunchKernelGGL(decode_small_kernel<true>, grid, block, 0, stream, k);
    else
      hipLaunchKernelGGL(decode_small_kernel<false>, grid, block, 0, stream, k);
    return hipGetLastError();
  }
  const int grid = (plan.waves + kWaves - 1) / kWaves;
  if (k.k_new)
    hipLaunchKernelGGL(decode_split_kernel<true>, dim3((unsigned)grid), dim3(kWaves * 64), 0,
                       stream, k);
  else
    hipLaunchKernelGGL(decode_split_kernel<false>, dim3((unsigned)grid), dim3(kWaves * 64), 0,
                       stream, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !plan.splits) return err;
  const int64_t merge_rows = (int64_t)a.batch * a.num_q_heads;
  hipLaunchKernelGGL(decode_merge_kernel,
                     dim3((unsigned)((merge_rows + kMergeWaves - 1) / kMergeWaves)),
                     dim3(64 * kMergeWaves), 0, stream,
                     k.part_o, k.part_lse, k.req_blocks, (uint16_t*)a.out, a.batch,
                     a.num_q_heads, a.num_kv_heads, plan.groups);
  return hipGetLastError();
}

}  // namespace pka
