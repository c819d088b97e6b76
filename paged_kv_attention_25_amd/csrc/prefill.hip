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
// processed in tiles of 64: the tile's K and V rows are gathered through the page
// table into LDS (row pitch 272 bytes to spread LDS banks), with the next tile's
// global loads in flight while the current tile is computed.
//
// Per wavefront and tile, with 32x32x16 bf16 MFMAs:
//   S^T[key][row] = K . Q^T   (A = K from LDS, B = Q held in registers)
//   O^T[d][row]  += V^T . P^T (A = V^T from LDS, B = P^T straight from S^T's registers)
// Index choices:
//  * QK reduction order: lane l feeds d = 16c + 8*(l/32) + j to MFMA c, a 16-byte
//    LDS read of K and a 16-byte global read of Q.
//  * PV key order: MFMA u takes keys 16u + 8*(j/4) + 4*(l/32) + (j%4), which are
//    exactly the scores lane l already holds, so P^T needs no data movement.
//  * Output rows: row m of O^T tile t is d = 4m + t, so a lane reads 8 bytes
//    V[key][4*(l%32) .. +4] per key and transposes 4x8 bf16 in registers.
// Online softmax in the log2 domain, causal mask only on tiles that cross the
// diagonal, tiles past the last row's position skipped.
#include "pka_device.h"
#include "pka_kernels.h"

namespace pka {

namespace {

constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = kRowsPerWave * kWaves;  // 128
constexpr int kKeysPerTile = 64;
constexpr int kLdsPitch = kHeadDim + 8;  // elements; 272 bytes per row
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

__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillKernelArgs p) {
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
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kKeysPerTile * kLdsPitch];

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

  // Global -> LDS staging: thread covers 16-byte chunk (tid % 16) of keys tid/16 + 16i.
  const int64_t row_elems = (int64_t)p.num_kv_heads * kHeadDim;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_stride;
  const uint16_t* kbase = p.k_pool + (int64_t)g * kHeadDim + 8 * (tid & 15);
  const uint16_t* vbase = p.v_pool + (int64_t)g * kHeadDim + 8 * (tid & 15);
  const int ld_key = tid >> 4;
  u32x4 kst[4], vst[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(kt + ld_key + 16 * i, key_end - 1);
      const int32_t slot = slot_of(pt_row, key, p.pg);
      if (slot >= 0) {
        kst[i] = *(const u32x4*)(kbase + (int64_t)slot * row_elems);
        vst[i] = *(const u32x4*)(vbase + (int64_t)slot * row_elems);
      } else {
        kst[i] = u32x4{0, 0, 0, 0};
        vst[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = (ld_key + 16 * i) * kLdsPitch + 8 * (tid & 15);
      *(u32x4*)(k_lds + off) = kst[i];
      *(u32x4*)(v_lds + off) = vst[i];
    }
  };

  float m = kNegInf;
  float lsum = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;

  load_tile(0);
  store_tile();
  __syncthreads();

  for (int kt = 0; kt < key_end; kt += kKeysPerTile) {
    const bool has_next = kt + kKeysPerTile < key_end;
    if (has_next) load_tile(kt + kKeysPerTile);

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
      // Scale, causal mask (only where the tile crosses the wave's diagonal), max.
      const bool need_mask = kt + kKeysPerTile - 1 > wave_lim_lo;
      float mx = kNegInf;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = sblk[kb2][i] * p.scale_log2;
          if (need_mask) {
            const int key = kt + kb2 * 32 + 8 * (i >> 2) + 4 * hgrp + (i & 3);
            x = (key <= lim) ? x : kNegInf;
          }
          sblk[kb2][i] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float ps = 0.f;
      u32x4 pb[4];  // P^T operands for the 4 PV MFMAs (16 keys each)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kb2 = u >> 1;
        const int r0 = 8 * (u & 1);
        float pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pr[j] = fast_exp2(sblk[kb2][r0 + j] - m_use);
          ps += pr[j];
        }
        pb[u][0] = pack_bf16x2(pr[0], pr[1]);
        pb[u][1] = pack_bf16x2(pr[2], pr[3]);
        pb[u][2] = pack_bf16x2(pr[4], pr[5]);
        pb[u][3] = pack_bf16x2(pr[6], pr[7]);
      }
      lsum = lsum * alpha + ps;
      m = m_new;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = o[t] * alpha;

      // O^T += V^T P^T. MFMA u covers keys 16u + 8*(j/4) + 4*hgrp + (j%4).
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x2 vk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = 16 * u + 8 * (j >> 2) + 4 * hgrp + (j & 3);
          vk[j] = *(const u32x2*)(v_lds + key * kLdsPitch + 4 * col);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int w = t >> 1;
          u32x4 a;
          if ((t & 1) == 0) {
            a[0] = lo_halves(vk[0][w], vk[1][w]);
            a[1] = lo_halves(vk[2][w], vk[3][w]);
            a[2] = lo_halves(vk[4][w], vk[5][w]);
            a[3] = lo_halves(vk[6][w], vk[7][w]);
          } else {
            a[0] = hi_halves(vk[0][w], vk[1][w]);
            a[1] = hi_halves(vk[2][w], vk[3][w]);
            a[2] = hi_halves(vk[4][w], vk[5][w]);
            a[3] = hi_halves(vk[6][w], vk[7][w]);
          }
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
  // Register i of tile t holds d = 32*(i/4) + 16*hgrp + 4*(i%4) + t: for fixed i/4
  // the lane owns 16 contiguous d values.
  uint16_t* dst = p.out + ((int64_t)(q_row0 + tok) * p.num_q_heads + (int64_t)g * G + hh) *
                              kHeadDim + 16 * hgrp;
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4) {
    u32x4 w0, w1;
    // d offsets 0..7 -> (i%4 = 0, t=0..3), (i%4 = 1, t=0..3)
    w0[0] = pack_bf16x2(o[0][4 * a4 + 0] * inv, o[1][4 * a4 + 0] * inv);
    w0[1] = pack_bf16x2(o[2][4 * a4 + 0] * inv, o[3][4 * a4 + 0] * inv);
    w0[2] = pack_bf16x2(o[0][4 * a4 + 1] * inv, o[1][4 * a4 + 1] * inv);
    w0[3] = pack_bf16x2(o[2][4 * a4 + 1] * inv, o[3][4 * a4 + 1] * inv);
    w1[0] = pack_bf16x2(o[0][4 * a4 + 2] * inv, o[1][4 * a4 + 2] * inv);
    w1[1] = pack_bf16x2(o[2][4 * a4 + 2] * inv, o[3][4 * a4 + 2] * inv);
    w1[2] = pack_bf16x2(o[0][4 * a4 + 3] * inv, o[1][4 * a4 + 3] * inv);
    w1[3] = pack_bf16x2(o[2][4 * a4 + 3] * inv, o[3][4 * a4 + 3] * inv);
    *(u32x4*)(dst + 32 * a4) = w0;
    *(u32x4*)(dst + 32 * a4 + 8) = w1;
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
