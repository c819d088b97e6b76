// Paged GQA decode for gfx950: split over the key axis, then a merge pass.
//
// Batched decode reads every request's keys from the paged pool through its page
// table ("miniSGLang intro blog", section 1.3; "Mini-SGLang deployment guide",
// sections 6.2 and 6.3, where decode has its own kernel).
//
// Work unit = (request b, kv head g, split s): one wavefront attends the G q heads
// of kv head g to keys [s*chunk, min((s+1)*chunk, L_b)). The G q heads are the
// columns of 16x16x32 bf16 MFMA tiles (padded to 16 with zero queries), 32 keys at
// a time:
//   S^T[key][head] = K . Q^T   (A = K rows, B = Q; 4 MFMAs per 16 keys over D=128)
//   O^T[d][head] += V^T . P^T  (A = V^T, B = P^T; 8 MFMAs over 32 keys)
// Index choices that make every operand a plain load:
//  * QK reduction order: lane l feeds d = 32*(l/16) + 8c + j to MFMA c, so each
//    lane reads 64 contiguous bytes of one key row (K) and of one query row (Q).
//  * PV key order: the 32 keys of a step are fed so that lane group l/16 takes keys
//    {4*(l/16)+j, 16+4*(l/16)+j}, exactly the keys whose scores it holds after QK,
//    so P^T needs no data movement.
//  * Output rows: row m of O^T tile t is d = 8m + t, so lane l loads 16 contiguous
//    bytes V[key][8*(l%16) .. +8] per key (16 lanes read one 256-byte row: fully
//    coalesced) and an in-register 8x8 transpose of bf16 pairs forms the operands.
// Softmax is online in the log2 domain (scale*log2(e) folded into one multiply);
// the running sum stays a per-lane partial until the end.
//
// A request whose keys fit in one chunk is written to `out` directly (bf16).
// Otherwise each split writes its normalised partial output (f32) and its
// log2-sum-exp to the workspace and the merge kernel combines them:
//   LSE = log2 sum_s 2^lse_s,  out = sum_s 2^(lse_s - LSE) * o_s.
#include "pka_device.h"
#include "pka_kernels.h"

namespace pka {

namespace {

constexpr int kKeysPerStep = 32;
constexpr float kNegInf = -__builtin_huge_valf();

struct DecodeKernelArgs {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k_pool;
  const uint16_t* __restrict__ v_pool;
  const int32_t* __restrict__ page_table;
  const int32_t* __restrict__ seq_lens;
  uint16_t* __restrict__ out;
  float* __restrict__ part_o;    // [B, Hq, S, D]
  float* __restrict__ part_lse;  // [B, Hq, S]
  PageGeom pg;
  int32_t pt_stride;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t chunk;
  int32_t num_splits;
  float scale_log2;
};

__global__ __launch_bounds__(64) void decode_split_kernel(DecodeKernelArgs p) {
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int n = lane & 15;   // MFMA row/column index of this lane
  const int grp = lane >> 4; // MFMA reduction group of this lane

  const int L = p.seq_lens[b];
  const int start = s * p.chunk;
  if (start >= L) return;
  const int end = min(start + p.chunk, L);
  const bool single = L <= p.chunk;

  const int64_t row_elems = (int64_t)p.num_kv_heads * kHeadDim;
  const int32_t* pt_row = p.page_table + (int64_t)b * p.pt_stride;
  const uint16_t* kbase = p.k_pool + (int64_t)g * kHeadDim;
  const uint16_t* vbase = p.v_pool + (int64_t)g * kHeadDim;

  // Q^T operand: column n is q head g*G + n (zero for n >= G).
  const int h = g * p.group + n;
  u32x4 qv[4];
  if (n < p.group) {
    const u32x4* qrow =
        (const u32x4*)(p.q + ((int64_t)b * p.num_q_heads + h) * kHeadDim + 32 * grp);
#pragma unroll
    for (int c = 0; c < 4; ++c) qv[c] = qrow[c];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qv[c] = u32x4{0, 0, 0, 0};
  }

  float m = kNegInf;  // running max of this column (log2 domain)
  float lsum = 0.f;   // this lane's share of the running sum
  f32x4 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = start; kb < end; kb += 2 * kKeysPerStep) {
    // One page-table lookup per lane covers 64 keys; keys past `end` are clamped to
    // the last valid key (loaded but masked out of the softmax).
    const int32_t my_slot = slot_of(pt_row, min(kb + lane, end - 1), p.pg);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k0 = kb + half * kKeysPerStep;
      if (k0 >= end) break;
      const int base_lane = half * kKeysPerStep;
      // K rows of keys k0+n and k0+16+n: 64 bytes each, d from 32*grp.
      const int32_t sk0 = __shfl(my_slot, base_lane + n);
      const int32_t sk1 = __shfl(my_slot, base_lane + 16 + n);
      u32x4 k0r[4], k1r[4];
      if (sk0 >= 0) {
        const u32x4* src = (const u32x4*)(kbase + (int64_t)sk0 * row_elems + 32 * grp);
#pragma unroll
        for (int c = 0; c < 4; ++c) k0r[c] = src[c];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) k0r[c] = u32x4{0, 0, 0, 0};
      }
      if (sk1 >= 0) {
        const u32x4* src = (const u32x4*)(kbase + (int64_t)sk1 * row_elems + 32 * grp);
#pragma unroll
        for (int c = 0; c < 4; ++c) k1r[c] = src[c];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) k1r[c] = u32x4{0, 0, 0, 0};
      }
      // V rows of this lane's 8 PV keys: 16 bytes each, d = 8n .. 8n+7.
      u32x4 vr[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kl = (j < 4) ? (4 * grp + j) : (16 + 4 * grp + (j - 4));
        const int32_t sv = __shfl(my_slot, base_lane + kl);
        if (sv >= 0) {
          vr[j] = *(const u32x4*)(vbase + (int64_t)sv * row_elems + 8 * n);
        } else {
          vr[j] = u32x4{0, 0, 0, 0};
        }
      }

      // Scores: lane holds column n (q head), keys k0 + 4*grp + v and k0 + 16 + 4*grp + v.
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s0 = mfma_16x16x32(k0r[c], qv[c], s0);
        s1 = mfma_16x16x32(k1r[c], qv[c], s1);
      }
      float sc[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int key0 = k0 + 4 * grp + v;
        sc[v] = (key0 < end) ? s0[v] * p.scale_log2 : kNegInf;
        sc[4 + v] = (key0 + 16 < end) ? s1[v] * p.scale_log2 : kNegInf;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);  // finite: key k0 is always valid
      const float alpha = fast_exp2(m - m_new);
      float pr[8];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = fast_exp2(sc[i] - m_new);
        ps += pr[i];
      }
      lsum = lsum * alpha + ps;
      m = m_new;
      u32x4 pb;
      pb[0] = pack_bf16x2(pr[0], pr[1]);
      pb[1] = pack_bf16x2(pr[2], pr[3]);
      pb[2] = pack_bf16x2(pr[4], pr[5]);
      pb[3] = pack_bf16x2(pr[6], pr[7]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int w = t >> 1;
        u32x4 a;
        if ((t & 1) == 0) {
          a[0] = lo_halves(vr[0][w], vr[1][w]);
          a[1] = lo_halves(vr[2][w], vr[3][w]);
          a[2] = lo_halves(vr[4][w], vr[5][w]);
          a[3] = lo_halves(vr[6][w], vr[7][w]);
        } else {
          a[0] = hi_halves(vr[0][w], vr[1][w]);
          a[1] = hi_halves(vr[2][w], vr[3][w]);
          a[2] = hi_halves(vr[4][w], vr[5][w]);
          a[3] = hi_halves(vr[6][w], vr[7][w]);
        }
        o[t] = o[t] * alpha;
        o[t] = mfma_16x16x32(a, pb, o[t]);
      }
    }
  }

  float ltot = lsum + __shfl_xor(lsum, 16);
  ltot += __shfl_xor(ltot, 32);
  if (n >= p.group) return;
  const float inv = 1.f / ltot;
  // Lane holds d = 32*grp + 8v + t for t = 0..7 in o[t][v].
  if (single) {
    uint16_t* dst = p.out + ((int64_t)b * p.num_q_heads + h) * kHeadDim + 32 * grp;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x4 w;
      w[0] = pack_bf16x2(o[0][v] * inv, o[1][v] * inv);
      w[1] = pack_bf16x2(o[2][v] * inv, o[3][v] * inv);
      w[2] = pack_bf16x2(o[4][v] * inv, o[5][v] * inv);
      w[3] = pack_bf16x2(o[6][v] * inv, o[7][v] * inv);
      *(u32x4*)(dst + 8 * v) = w;
    }
  } else {
    const int64_t unit = ((int64_t)b * p.num_q_heads + h) * p.num_splits + s;
    float* dst = p.part_o + unit * kHeadDim + 32 * grp;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      f32x4 lo = {o[0][v] * inv, o[1][v] * inv, o[2][v] * inv, o[3][v] * inv};
      f32x4 hi = {o[4][v] * inv, o[5][v] * inv, o[6][v] * inv, o[7][v] * inv};
      *(f32x4*)(dst + 8 * v) = lo;
      *(f32x4*)(dst + 8 * v + 4) = hi;
    }
    if (grp == 0) p.part_lse[unit] = m + __builtin_log2f(ltot);
  }
}

// One wavefront per (request, q head): lane l combines d = 2l, 2l+1 over the splits.
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const int32_t* __restrict__ seq_lens,
                                                          uint16_t* __restrict__ out,
                                                          int32_t num_q_heads, int32_t chunk,
                                                          int32_t num_splits) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = seq_lens[b];
  // Keys past num_splits * chunk (a length above the planned maximum) were not
  // attended, so only the planned splits exist in the workspace.
  const int nsplit = min((L + chunk - 1) / chunk, num_splits);
  if (L <= chunk) return;  // written directly by the split kernel
  const int64_t unit0 = ((int64_t)b * num_q_heads + h) * num_splits;
  float mx = kNegInf;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part_lse[unit0 + s]);
  float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = fast_exp2(part_lse[unit0 + s] - mx);
    const float2 v = *(const float2*)(part_o + (unit0 + s) * kHeadDim + 2 * lane);
    wsum += w;
    acc0 += w * v.x;
    acc1 += w * v.y;
  }
  const float inv = 1.f / wsum;
  uint32_t* dst = (uint32_t*)(out + ((int64_t)b * num_q_heads + h) * kHeadDim);
  dst[lane] = pack_bf16x2(acc0 * inv, acc1 * inv);
}

}  // namespace

DecodePlan plan_decode(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  // Aim for about 8192 work units (32 per CU on 256 CUs) counted against the upper
  // bound batch * max_seq_len, with chunks a multiple of 64 keys in [64, 4096].
  DecodePlan plan;
  const int64_t work = (int64_t)batch * num_kv_heads * (int64_t)(max_seq_len > 0 ? max_seq_len : 1);
  int64_t chunk = 64;
  while (chunk < 4096 && work / chunk > 8192) chunk *= 2;
  plan.chunk = (int32_t)chunk;
  plan.num_splits = (int32_t)((max_seq_len + chunk - 1) / chunk);
  if (plan.num_splits < 1) plan.num_splits = 1;
  return plan;
}

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, const DecodePlan& plan) {
  if (plan.num_splits <= 1) return 0;
  const size_t units = (size_t)batch * num_q_heads * plan.num_splits;
  return units * (kHeadDim + 1) * sizeof(float);
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
  const size_t units = (size_t)a.batch * a.num_q_heads * plan.num_splits;
  k.part_o = (float*)a.workspace;
  k.part_lse = plan.num_splits > 1 ? k.part_o + units * kHeadDim : nullptr;
  k.pg.page_size = a.page_size;
  k.pg.page_shift = page_shift_of(a.page_size);
  k.pg.num_pages = a.num_pages;
  k.pg.table_width = a.pt_stride;
  k.pt_stride = a.pt_stride;
  k.num_q_heads = a.num_q_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.group = a.num_q_heads / a.num_kv_heads;
  k.chunk = plan.chunk;
  k.num_splits = plan.num_splits;
  k.scale_log2 = a.scale * kLog2e;
  hipLaunchKernelGGL(decode_split_kernel, dim3(plan.num_splits, a.num_kv_heads, a.batch),
                     dim3(64), 0, stream, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.num_splits <= 1) return err;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.num_q_heads, a.batch), dim3(64), 0, stream,
                     k.part_o, k.part_lse, a.seq_lens, (uint16_t*)a.out, a.num_q_heads,
                     plan.chunk, plan.num_splits);
  return hipGetLastError();
}

}  // namespace pka
