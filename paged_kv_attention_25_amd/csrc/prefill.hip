// Paged causal extend (chunked) prefill for gfx950.
//
// New token i of request b sits at absolute position p_b + i and attends to keys
// 0 .. p_b + i of its request, read from the paged pool through the page table
// (chunked prefill over a cached prefix: "Mini-SGLang deployment guide", sections
// 6.1 and 6.5; keys located through page-table metadata: "miniSGLang intro blog",
// section 1.3).
//
// Tiling. A workgroup of 4 wavefronts owns 128 query rows of one (request, kv head).
// Rows are (token, head-in-group) pairs, row r = i*G + hh, so the G q heads that
// share a kv head share every K/V tile. Each wavefront owns 32 rows. Keys are
// processed in tiles of 64: the tile's K rows are gathered through the page table
// into LDS row-major (272-byte pitch), its V rows transposed into LDS (V^T, one row
// per d, 144-byte pitch, 16-byte chunks XOR-swizzled by row), with the next tile's
// global loads in flight while the current tile is computed.
//
// Per wavefront and tile, with 32x32x16 bf16 MFMAs:
//   S^T[key][row] = K . Q^T   (A = K from LDS, B = Q held in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T from LDS, B = P^T straight from S^T's registers)
// Index choices:
//  * QK reduction order: lane l feeds d = 16c + 8*(l/32) + j to MFMA c, a 16-byte
//    LDS read of K and a 16-byte global read of Q.
//  * PV key order: MFMA u takes keys 16u + 8*(j/4) + 4*(l/32) + (j%4), which are
//    exactly the scores lane l already holds, so P^T needs no data movement. V^T
//    stores key k of a 16-key group at position k with bits 2 and 3 swapped, which
//    makes those 8 keys contiguous: each V^T operand is one 16-byte LDS read.
// Softmax runs in the log2 domain with the scale folded into one FMA per score. The
// running max is only raised (and the output rescaled) when it grows by more than
// 2^8, so most tiles skip the rescale; probabilities stay below 2^8 in between.
// Causal masking only on tiles that cross a wavefront's diagonal; tiles past the
// last row's position are skipped.
#include "pka_device.h"
#include "pka_kernels.h"

namespace pka {

namespace {

constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // 128
constexpr int kKeysPerTile = 64;
constexpr int kLdsPitch = kHeadDim + 8;     // K rows: elements; 272 bytes per row
constexpr int kVtPitch = kKeysPerTile + 8;  // V^T rows: elements; 144 bytes per row
constexpr float kRescaleLog2 = 8.f;         // raise the running max past 2^8 growth
constexpr float kNegInf = -__builtin_huge_valf();

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
  int32_t tiles_per_seq;  // ceil(max_extend * G / 128)
  float scale_log2;
};

// Position of key k (0..63) of a tile in the V^T rows: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}
// V^T row d keeps its eight 16-byte chunks XOR-swizzled by (d / 16) % 8, so that both
// the transposing 8-byte writes and the 16-byte operand reads spread over all banks.

// Two workgroups (8 wavefronts) per CU.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void prefill_kernel(PrefillKernelArgs p) {
  // Block id -> (q tile, request, kv head); the highest q tiles (the most keys)
  // are dispatched first, and with the kv head fastest all tiles of one
  // (request, kv head) land on the same XCD when the head count divides 8.
  const int id = blockIdx.x;
  const int g = id % p.num_kv_heads;
  const int rest = id / p.num_kv_heads;
  const int b = rest % p.batch;
  const int tile = p.tiles_per_seq - 1 - rest / p.batch;

  const int e = p.extend_lens[b];
  const int G = p.group;
  const int nrows = e * G;
  const int row0 = tile * kRowsPerBlock;
  if (row0 >= nrows) return;
  const int prefix = p.prefix_lens[b];
  const int q_row0 = p.cu_extend[b];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;  // MFMA column: this lane's query row within the wave
  const int hgrp = lane >> 5; // MFMA reduction group

  // Keys the block needs: 0 .. prefix + (token of its last row).
  const int last_row_blk = min(row0 + kRowsPerBlock, nrows) - 1;
  const int key_end = prefix + last_row_blk / G + 1;

  // This lane's query row.
  const int r = row0 + wave * kRowsPerWave + col;
  const bool row_in = r < nrows;
  const int tok = row_in ? r / G : 0;
  const bool row_ok = row_in && q_row0 + tok >= 0 && q_row0 + tok < p.num_tokens;  // in bounds
  const int hh = row_in ? r - tok * G : 0;
  const int lim = prefix + tok;  // last visible key of this row
  // The wave's smallest and largest limits (rows are in token order).
  const int wrow_first = row0 + wave * kRowsPerWave;
  const int wrow_last = min(wrow_first + kRowsPerWave, nrows) - 1;
  const bool wave_live = wrow_first < nrows;
  const int wave_lim_lo = prefix + (wave_live ? wrow_first / G : 0);
  const int wave_lim_hi = prefix + (wave_live ? wrow_last / G : 0);

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKeysPerTile * kLdsPitch];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kHeadDim * kVtPitch];

  // Q^T operand: 8 MFMAs over D, lane feeds d = 16c + 8*hgrp .. +8 of its row.
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

  // Global -> LDS staging: thread covers 16-byte chunk m = tid % 16 (d = 8m .. 8m+7)
  // of the four keys 4a .. 4a+3, a = tid / 16.
  const int64_t row_elems = (int64_t)p.num_kv_heads * kHeadDim;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_stride;
  const int ld_m = tid & 15;
  const int ld_a = tid >> 4;
  const uint16_t* kbase = p.k_pool + (int64_t)g * kHeadDim + 8 * ld_m;
  const uint16_t* vbase = p.v_pool + (int64_t)g * kHeadDim + 8 * ld_m;
  // Page-table entries of this thread's four keys of a tile are loaded one tile ahead
  // of the K/V loads that use them, so no load waits on another in the loop. Every
  // load is unconditional and in bounds: keys past the block's last key are clamped to
  // it, a table index past the row to the row's last entry, and a page id outside the
  // pool reads slot 0 (that request's result is then unspecified).
  int32_t raw_page[4], raw_off[4];
  auto lookup = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(kt + 4 * ld_a + i, key_end - 1);
      int idx;
      if (p.pg.page_shift >= 0) {
        idx = key >> p.pg.page_shift;
        raw_off[i] = key & (p.pg.page_size - 1);
      } else {
        idx = key / p.pg.page_size;
        raw_off[i] = key - idx * p.pg.page_size;
      }
      raw_page[i] = pt_row[min(idx, p.pg.table_width - 1)];
    }
  };
  u32x4 kst[4], vst[4];
  auto load_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hold(raw_page[i]);
      const int32_t page = raw_page[i];
      const int32_t slot =
          (uint32_t)page < (uint64_t)p.pg.num_pages ? page * p.pg.page_size + raw_off[i] : 0;
      kst[i] = *(const u32x4*)(kbase + (int64_t)slot * row_elems);
      vst[i] = *(const u32x4*)(vbase + (int64_t)slot * row_elems);
    }
  };
  // K: row-major, key row at 272-byte pitch.
  uint16_t* const k_st = k_lds + 4 * ld_a * kLdsPitch + 8 * ld_m;
  // V^T: row d = 8m + j; the four keys land at positions vt_pos(4a) .. +3 of 16-byte
  // chunk c = vt_pos(4a)/8, stored at chunk c ^ vt_swz(d) (8 bytes per row and key quad).
  const int vq = vt_pos(4 * ld_a);
  uint16_t* const vt_st = vt_lds + 8 * ld_m * kVtPitch + 8 * ((vq >> 3) ^ (ld_m >> 1)) + (vq & 7);
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(k_st + i * kLdsPitch) = kst[i];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x2 lo, hi;  // d = 8m + 2w and 8m + 2w + 1, keys 4a .. 4a+3
      lo[0] = lo_halves(vst[0][w], vst[1][w]);
      lo[1] = lo_halves(vst[2][w], vst[3][w]);
      hi[0] = hi_halves(vst[0][w], vst[1][w]);
      hi[1] = hi_halves(vst[2][w], vst[3][w]);
      *(u32x2*)(vt_st + (2 * w) * kVtPitch) = lo;
      *(u32x2*)(vt_st + (2 * w + 1) * kVtPitch) = hi;
    }
  };
  // PV operand read base: V^T row col (+32t), chunk (2u + hgrp) ^ vt_swz(32t + col)
  // = 2(u ^ t) + (hgrp ^ (col / 16)).
  const uint16_t* const vt_rd = vt_lds + col * kVtPitch + 8 * (hgrp ^ (col >> 4));

  float m = kNegInf;
  float lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;

  lookup(0);
  load_tile();
  store_tile();
  lookup(kKeysPerTile);
  __syncthreads();

  for (int kt = 0; kt < key_end; kt += kKeysPerTile) {
    const bool has_next = kt + kKeysPerTile < key_end;
    // Next tile's K/V and the page ids of the one after (past the end: clamped reloads).
    load_tile();
    lookup(kt + 2 * kKeysPerTile);

    if (wave_live && kt <= wave_lim_hi) {
      // S^T for two 32-key blocks.
      f32x16 sblk[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sblk[kb2][i] = 0.f;
        const uint16_t* krow = k_lds + (kb2 * 32 + col) * kLdsPitch + 8 * hgrp;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const u32x4 a = *(const u32x4*)(krow + 16 * c);
          sblk[kb2] = mfma_32x32x16(a, qv[c], sblk[kb2]);
        }
      }
      // Causal mask only where the tile crosses this wavefront's diagonal: register i
      // of block kb2 holds key kt + 32*kb2 + 8*(i/4) + 4*hgrp + (i%4).
      if (kt + kKeysPerTile - 1 > wave_lim_lo) {
        const int dl = lim - kt - 4 * hgrp;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kb2 + 8 * (i >> 2) + (i & 3) > dl) sblk[kb2][i] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sblk[kb2][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // Raw-score max; the scale is applied inside the exponent. Rescale only when
      // some row's max grew by more than 2^kRescaleLog2 (or has no value yet).
      const bool grow = (mx - m) * p.scale_log2 > kRescaleLog2;
      if (__any(grow)) {
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2((m - m_new) * p.scale_log2);  // 0 when m = -inf
        lsum *= alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = o[t] * alpha;
        m = m_new;
      }
      const float neg_m = (m == kNegInf) ? 0.f : -m * p.scale_log2;
      float ps = 0.f;
      u32x4 pb[4];  // P^T operands for the 4 PV MFMAs (16 keys each)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb2 = u >> 1;
        const int r0 = 8 * (u & 1);
        float pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pr[j] = fast_exp2(fmaf(sblk[kb2][r0 + j], p.scale_log2, neg_m));
          ps += pr[j];
        }
        pb[u][0] = pack_bf16x2(pr[0], pr[1]);
        pb[u][1] = pack_bf16x2(pr[2], pr[3]);
        pb[u][2] = pack_bf16x2(pr[4], pr[5]);
        pb[u][3] = pack_bf16x2(pr[6], pr[7]);
      }
      lsum += ps;

      // O^T += V^T P^T: tile t covers d = 32t .. 32t+31; MFMA u takes the 16 keys at
      // V^T positions 16u .. 16u+15, lane group hgrp the 8 at 16u + 8*hgrp.
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4 a = *(const u32x4*)(vt_rd + 32 * t * kVtPitch + 16 * (u ^ t));
          o[t] = mfma_32x32x16(a, pb[u], o[t]);
        }
      }
    }

    if (has_next) {
      __syncthreads();  // every wave is done reading this tile
      store_tile();
      __syncthreads();
    }
  }

  if (!row_ok) return;
  float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.f / ltot;
  // Register r of tile t holds d = 32t + 8*(r/4) + 4*hgrp + (r%4).
  uint16_t* dst = p.out + ((int64_t)(q_row0 + tok) * p.num_q_heads + (int64_t)g * G + hh) *
                              kHeadDim + 4 * hgrp;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      u32x2 w;
      w[0] = pack_bf16x2(o[t][4 * a4 + 0] * inv, o[t][4 * a4 + 1] * inv);
      w[1] = pack_bf16x2(o[t][4 * a4 + 2] * inv, o[t][4 * a4 + 3] * inv);
      *(u32x2*)(dst + 32 * t + 8 * a4) = w;
    }
  }
}

}  // namespace

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
  k.pg.page_size = a.page_size;
  k.pg.page_shift = page_shift_of(a.page_size);
  k.pg.num_pages = a.num_pages;
  k.pg.table_width = a.pt_stride;
  k.pt_stride = a.pt_stride;
  k.batch = a.batch;
  k.num_tokens = a.num_tokens;
  k.num_q_heads = a.num_q_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.group = a.num_q_heads / a.num_kv_heads;
  const int64_t rows = (int64_t)a.max_extend * k.group;
  k.tiles_per_seq = (int32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  k.scale_log2 = a.scale * kLog2e;
  const int64_t blocks = (int64_t)k.tiles_per_seq * a.batch * a.num_kv_heads;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k);
  return hipGetLastError();
}

}  // namespace pka
