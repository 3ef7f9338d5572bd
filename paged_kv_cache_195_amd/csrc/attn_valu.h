// Split-KV paged attention on the vector ALUs (gfx950, wave64).
//
// One workgroup computes MR query rows that share one kv head over one split
// of one sequence's pages.  A row is a (query position, head of the group)
// pair, so the same kernel runs grouped-query decode (one position, MR heads)
// and prefill (several positions).  The softmax is the online
// (running max / running sum) form, kept in base 2.
//
// Work split inside the workgroup:
//  * NW waves take the split's pages round-robin; each wave streams one whole
//    page (its kv head's rows) at a time and prefetches the next page into
//    registers while it computes the current one.
//  * Inside a wave, LPT = D*sizeof(T)/16 lanes hold one token row (16 bytes
//    each) and TPL = 64/LPT tokens sit side by side, so a wave load of
//    16 bytes per lane reads TPL whole rows: each row is one contiguous run of
//    D*sizeof(T) bytes.
//  * q.k is a 16-byte dot per lane, summed over the LPT lanes of the token
//    with DPP moves (no LDS).  Every lane then holds the scores of its own
//    token for all MR rows and keeps its own running max, sum and partial
//    output for its Dims chunk; lanes merge once at the end (first across the
//    tokens of the wave, then across waves through LDS).
//
// Guards (rocMLIR "Fix split-kv attention masking and sweep RMS", Technical
// Details): a running max of -inf is replaced by 0 before it is subtracted,
// so a fully masked split never forms -inf - (-inf) and contributes exactly
// nothing; a row whose sum is 0 stores output 0 and LSE -inf instead of 0/0.
// Split ranges use ceiling division with clamped ends.  V rows of tokens past
// the sequence length are zeroed before use, so garbage (even NaN) in a last
// page's tail never reaches the output.
#pragma once

#include "device_common.h"
#include "pa_internal.h"
#include "page_table.h"

namespace pa {

template <typename T, int D, int PS, int MR, int NW>
__global__ __launch_bounds__(NW * 64) void attn_valu_kernel(const AttnParams p) {
  constexpr int kEpc = Chunk<T>::kElems;  // elements per 16-byte chunk
  constexpr int kLpt = D / kEpc;          // lanes per token row
  constexpr int kTpl = 64 / kLpt;         // tokens per wave load
  constexpr int kNl = PS / kTpl;          // wave loads per page (K or V)
  static_assert(D % kEpc == 0 && 64 % kLpt == 0 && kLpt <= 64, "row must split into lanes");
  static_assert(PS % kTpl == 0, "a page must hold whole wave loads");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = lane / kLpt;  // token slot inside a wave load
  const int ch = lane % kLpt;  // 16-byte chunk inside the row

  const int S = p.num_splits;
  const int split = blockIdx.x % S;
  const int rg = blockIdx.x / S;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;

  const int seq_len = p.seq_lens[b];
  const int n_pages = (seq_len + PS - 1) / PS;

  // ---- rows of this workgroup: query, key limit (causal: bottom-right)
  u32x4 qv[MR];
  int lim[MR];
  int row_id[MR];  // flat (b, i, h) row index, -1 when past the last row
  int max_lim = 0;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const int r_lin = rg * MR + r;
    if (r_lin < p.rows_per_kvh) {
      const int i = r_lin / G;
      const int h = kvh * G + (r_lin - i * G);
      int l = seq_len;
      if (p.causal) {
        l = seq_len - Sq + i + 1;
        l = l < 0 ? 0 : (l > seq_len ? seq_len : l);
      }
      lim[r] = l;
      row_id[r] = (b * Sq + i) * Hq + h;
      const T* qp = static_cast<const T*>(p.q) + static_cast<int64_t>(row_id[r]) * D + ch * kEpc;
      qv[r] = *reinterpret_cast<const u32x4*>(qp);
      max_lim = l > max_lim ? l : max_lim;
    } else {
      lim[r] = -1;
      row_id[r] = -1;
      qv[r] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  int min_lim = max_lim;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if (row_id[r] < 0) lim[r] = max_lim;  // unused rows never force the masked path
    min_lim = lim[r] < min_lim ? lim[r] : min_lim;
  }

  // ---- this split's page range: ceil-divided, clamped, and cut at the last
  // page any row of the workgroup can see
  const int per = (n_pages + S - 1) / S;
  const int first = min(split * per, n_pages);
  int end = min(first + per, n_pages);
  end = min(end, (max_lim + PS - 1) / PS);

  PageTable pt;
  pt.row = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  pt.page_bytes = static_cast<int64_t>(PS) * Hkv * D * static_cast<int64_t>(sizeof(T));
  pt.n_pages = n_pages;

  // Byte offset of this lane's chunk for wave load j, the same on every page.
  uint32_t off[kNl];
#pragma unroll
  for (int j = 0; j < kNl; ++j)
    off[j] = static_cast<uint32_t>(((j * kTpl + tl) * Hkv + kvh) * D + ch * kEpc) *
             static_cast<uint32_t>(sizeof(T));

  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);

  float m[MR], l[MR], acc[MR][kEpc];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < kEpc; ++e) acc[r][e] = 0.f;
  }

  u32x4 kc[kNl], vc[kNl];
  int slot = first + wave;
  if (slot < end) {
    const int64_t base = pt.base(slot);
#pragma unroll
    for (int j = 0; j < kNl; ++j) kc[j] = *reinterpret_cast<const u32x4*>(kbase + base + off[j]);
#pragma unroll
    for (int j = 0; j < kNl; ++j) vc[j] = *reinterpret_cast<const u32x4*>(vbase + base + off[j]);
  }

  while (slot < end) {
    // prefetch the wave's next page
    const int next = slot + NW;
    u32x4 kn[kNl], vn[kNl];
    if (next < end) {
      const int64_t base = pt.base(next);
#pragma unroll
      for (int j = 0; j < kNl; ++j) kn[j] = *reinterpret_cast<const u32x4*>(kbase + base + off[j]);
#pragma unroll
      for (int j = 0; j < kNl; ++j) vn[j] = *reinterpret_cast<const u32x4*>(vbase + base + off[j]);
    }

    // scores of this lane's tokens, base 2
    float x[kNl][MR];
#pragma unroll
    for (int j = 0; j < kNl; ++j)
#pragma unroll
      for (int r = 0; r < MR; ++r)
        x[j][r] = group_sum<kLpt>(chunk_dot<T>(qv[r], kc[j], 0.f)) * p.scale_log2;

    const int tok0 = slot * PS;
    if (tok0 + PS > min_lim) {  // wave-uniform: only pages that hold a masked key
#pragma unroll
      for (int j = 0; j < kNl; ++j) {
        const int tok = tok0 + j * kTpl + tl;
#pragma unroll
        for (int r = 0; r < MR; ++r) x[j][r] = tok < lim[r] ? x[j][r] : kNegInf;
        if (tok >= seq_len) vc[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    float vf[kNl][kEpc];
#pragma unroll
    for (int j = 0; j < kNl; ++j) chunk_to_float<T>(vc[j], vf[j]);

#pragma unroll
    for (int r = 0; r < MR; ++r) {
      float mt = x[0][r];
#pragma unroll
      for (int j = 1; j < kNl; ++j) mt = __builtin_fmaxf(mt, x[j][r]);
      const float mn = __builtin_fmaxf(m[r], mt);
      const float msub = mn == kNegInf ? 0.f : mn;  // no -inf - (-inf)
      const float alpha = fast_exp2(m[r] - msub);
      m[r] = mn;
      float pj[kNl];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < kNl; ++j) {
        pj[j] = fast_exp2(x[j][r] - msub);
        psum += pj[j];
      }
      l[r] = l[r] * alpha + psum;
#pragma unroll
      for (int e = 0; e < kEpc; ++e) {
        float a = acc[r][e] * alpha;
#pragma unroll
        for (int j = 0; j < kNl; ++j) a = __builtin_fmaf(pj[j], vf[j][e], a);
        acc[r][e] = a;
      }
    }

    if (next < end) {
#pragma unroll
      for (int j = 0; j < kNl; ++j) {
        kc[j] = kn[j];
        vc[j] = vn[j];
      }
    }
    slot = next;
  }

  // ---- merge the token slots of this wave (lanes with the same chunk)
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const float mw = strided_max<kLpt>(m[r]);
    const float msub = mw == kNegInf ? 0.f : mw;
    const float f = fast_exp2(m[r] - msub);
    l[r] = strided_sum<kLpt>(l[r] * f);
#pragma unroll
    for (int e = 0; e < kEpc; ++e) acc[r][e] = strided_sum<kLpt>(acc[r][e] * f);
    m[r] = mw;
  }

  // ---- merge the waves through LDS and finish
  __shared__ float sm_acc[NW][MR][D];
  __shared__ float sm_m[NW][MR];
  __shared__ float sm_l[NW][MR];
  if (tl == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int e = 0; e < kEpc; ++e) sm_acc[wave][r][ch * kEpc + e] = acc[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      sm_m[wave][r] = m[r];
      sm_l[wave][r] = l[r];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < MR * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx - r * D;
    int rid = -1;
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) rid = rr == r ? row_id[rr] : rid;
    if (rid < 0) continue;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = __builtin_fmaxf(mx, sm_m[w][r]);
    const float msub = mx == kNegInf ? 0.f : mx;
    float lsum = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm_m[w][r] - msub);
      lsum += f * sm_l[w][r];
      a += f * sm_acc[w][r][d];
    }
    float o, lse;
    if (lsum > 0.f) {
      o = a / lsum;
      lse = (mx + log2f(lsum)) * kLn2;
    } else {  // no valid key: 0 instead of 0/0
      o = 0.f;
      lse = kNegInf;
    }
    if (S == 1) {
      static_cast<T*>(p.out)[static_cast<int64_t>(rid) * D + d] = from_float<T>(o);
      if (d == 0 && p.lse != nullptr) p.lse[rid] = lse;
    } else {
      const int64_t prow = static_cast<int64_t>(rid) * S + split;
      p.part_out[prow * D + d] = o;
      if (d == 0) p.part_lse[prow] = lse;
    }
  }
}

}  // namespace pa
