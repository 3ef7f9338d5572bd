// Split-KV paged attention on the vector ALUs (gfx950, wave64).  The library
// instantiates it for f32 caches; 16-bit and 8-bit caches run faster on the
// matrix cores.
//
// A workgroup computes, for kpw kv heads of one sequence and one split of its
// pages, MR query rows per kv head.  A row is a (query position, head of the
// group) pair, so the same kernel runs grouped-query decode (one position,
// MR heads) and prefill (several positions).  The softmax is the online
// (running max / running sum) form, kept in base 2.
//
// Work split inside the workgroup:
//  * wph = NW / kpw waves serve each of the kpw kv heads; the waves of a head
//    take the split's pages round-robin.  With kpw = Hkv the workgroup reads
//    whole pages (every kv head) close together in time, which the HBM serves
//    faster than scattered 256-byte rows.
//  * A wave streams one page of its kv head per step and keeps PF further
//    pages in flight in a register ring, so PF + 1 pages of loads are
//    outstanding while it computes.
//  * Inside a wave, LPT = D*sizeof(T)/16 lanes hold one token row (16 bytes
//    each) and TPL = 64/LPT tokens sit side by side, so a wave load of
//    16 bytes per lane reads TPL whole rows: each row is one contiguous run of
//    D*sizeof(T) bytes.
//  * q.k is a 16-byte dot per lane, summed over the LPT lanes of the token
//    with DPP moves (no LDS).  Every lane then holds the scores of its own
//    token for all MR rows and keeps its own running max, sum and partial
//    output for its 16-byte slice of the head dimension; lanes merge once at
//    the end (first across the tokens of the wave, then across waves through
//    LDS).
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

// T: element type; D: head dim (= Dv); PS: tokens per page; MR: rows per kv
// head; NW: waves per workgroup; PF: pages in flight beyond the one being
// computed; NT: non-temporal K/V loads (the cache is streamed once).  The
// number of kv heads per workgroup, p.heads_per_wg, divides both NW and Hkv.
template <typename T, int D, int PS, int MR, int NW, int PF, bool NT>
__global__ __launch_bounds__(NW * 64) void attn_valu_kernel(const AttnParams p) {
  constexpr int kEpc = Chunk<T>::kElems;  // elements per 16-byte chunk
  constexpr int kLpt = D / kEpc;          // lanes per token row
  constexpr int kTpl = 64 / kLpt;         // tokens per wave load
  constexpr int kNl = PS / kTpl;          // wave loads per page (K or V)
  constexpr int kStages = PF + 1;
  static_assert(D % kEpc == 0 && 64 % kLpt == 0 && kLpt <= 64, "row must split into lanes");
  static_assert(PS % kTpl == 0, "a page must hold whole wave loads");
  static_assert(PF >= 0 && PF <= 3, "ring depth");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = lane / kLpt;  // token slot inside a wave load
  const int ch = lane % kLpt;  // 16-byte chunk inside the row

  const int S = p.num_splits;
  const int split = blockIdx.x % S;
  const int rg = blockIdx.x / S;
  const int kpw = p.heads_per_wg;
  const int wph = NW / kpw;                  // waves per kv head
  const int kg = wave / wph;                 // kv head of this wave, inside the workgroup
  const int sub = wave - kg * wph;           // this wave's share of the head's pages
  const int kvh = blockIdx.y * kpw + kg;
  const int b = blockIdx.z;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;

  const int seq_len = p.seq_lens[b];
  const int n_pages = (seq_len + PS - 1) / PS;
  const int64_t pos0 = causal_row0(p.prefix_offset, b, seq_len, Sq);

  // ---- rows of this wave's kv head: query, key limit (causal: bottom-right
  // or from the prefix offset)
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
      const int l = p.causal ? causal_key_limit(seq_len, pos0, i) : seq_len;
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
  // page any row of the workgroup can see (the same for every kv head)
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

  // The scale is applied inside the exponent: p = exp2(x * c - msub) with
  // c = |scale| * log2(e); a negative scale is folded into q by flipping its
  // sign bits (exact), so scores can be compared unscaled.  c is at least
  // FLT_MIN so a masked score (-inf) times c stays -inf when the scale is 0;
  // every valid weight then still rounds to exactly 1.
  const float c = __builtin_fmaxf(__builtin_fabsf(p.scale_log2), 1.17549435e-38f);
  if (p.scale_log2 < 0.f) {
    const uint32_t sign = sizeof(T) == 4 ? 0x80000000u : 0x80008000u;
#pragma unroll
    for (int r = 0; r < MR; ++r) qv[r] ^= u32x4{sign, sign, sign, sign};
  }

  // Per lane and row: ref = reference max of the scaled scores seen so far
  // (-inf before the first valid key), msub = ref or 0 when ref is -inf (the
  // value actually subtracted, so -inf - (-inf) never occurs), l and acc
  // relative to msub.  ref is raised only when a page's max exceeds it by
  // more than kSlack (log2 units), so weights stay <= 2^kSlack and the
  // rescale of l and acc is skipped on most pages.
  constexpr float kSlack = 8.f;
  float ref[MR], msub[MR], l[MR], acc[MR][kEpc];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    ref[r] = kNegInf;
    msub[r] = 0.f;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < kEpc; ++e) acc[r][e] = 0.f;
  }

  auto load_page = [&](int slot, u32x4* kk, u32x4* vv) __attribute__((always_inline)) {
    const int64_t base = pt.base(slot);
#pragma unroll
    for (int j = 0; j < kNl; ++j) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kbase + base + off[j]);
      kk[j] = NT ? __builtin_nontemporal_load(src) : *src;
    }
#pragma unroll
    for (int j = 0; j < kNl; ++j) {
      const u32x4* src = reinterpret_cast<const u32x4*>(vbase + base + off[j]);
      vv[j] = NT ? __builtin_nontemporal_load(src) : *src;
    }
  };

  auto consume_page = [&](int slot, const u32x4* kk, u32x4* vv) __attribute__((always_inline)) {
    // unscaled scores q.k of this lane's tokens
    float x[kNl][MR];
#pragma unroll
    for (int j = 0; j < kNl; ++j)
#pragma unroll
      for (int r = 0; r < MR; ++r) x[j][r] = group_sum<kLpt>(chunk_dot<T>(qv[r], kk[j], 0.f));

    const int tok0 = slot * PS;
    if (tok0 + PS > min_lim) {  // wave-uniform: only pages that hold a masked key
#pragma unroll
      for (int j = 0; j < kNl; ++j) {
        const int tok = tok0 + j * kTpl + tl;
#pragma unroll
        for (int r = 0; r < MR; ++r) x[j][r] = tok < lim[r] ? x[j][r] : kNegInf;
        if (tok >= seq_len) vv[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }

    float ymax[MR];
    bool raise = false;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      float mt = x[0][r];
#pragma unroll
      for (int j = 1; j < kNl; ++j) mt = __builtin_fmaxf(mt, x[j][r]);
      ymax[r] = mt * c;
      raise |= ymax[r] > ref[r] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float nref = __builtin_fmaxf(ref[r], ymax[r]);
        const float nsub = nref == kNegInf ? 0.f : nref;
        const float alpha = fast_exp2(msub[r] - nsub);  // l, acc are 0 while ref is -inf
        l[r] *= alpha;
#pragma unroll
        for (int e = 0; e < kEpc; ++e) acc[r][e] *= alpha;
        ref[r] = nref;
        msub[r] = nsub;
      }
    }

    float vf[kNl][kEpc];
#pragma unroll
    for (int j = 0; j < kNl; ++j) chunk_to_float<T>(vv[j], vf[j]);

#pragma unroll
    for (int r = 0; r < MR; ++r) {
      float pj[kNl];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < kNl; ++j) {
        pj[j] = fast_exp2(__builtin_fmaf(x[j][r], c, -msub[r]));  // x = -inf gives 0
        psum += pj[j];
      }
      l[r] += psum;
#pragma unroll
      for (int e = 0; e < kEpc; ++e) {
        float a = acc[r][e];
#pragma unroll
        for (int j = 0; j < kNl; ++j) a = __builtin_fmaf(pj[j], vf[j][e], a);
        acc[r][e] = a;
      }
    }
  };

  // ---- stream this wave's pages through a ring of kStages register buffers
  u32x4 kb[kStages][kNl], vb[kStages][kNl];
  int slot = first + sub;
#pragma unroll
  for (int s = 0; s < PF; ++s)
    if (slot + s * wph < end) load_page(slot + s * wph, kb[s], vb[s]);
  for (; slot < end; slot += kStages * wph) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int cur = slot + st * wph;
      const int ahead = cur + PF * wph;
      if (ahead < end) load_page(ahead, kb[(st + PF) % kStages], vb[(st + PF) % kStages]);
      if (cur < end) consume_page(cur, kb[st], vb[st]);
    }
  }

  // ---- merge the token slots of this wave (lanes with the same chunk).
  // A lane without a valid key has ref = -inf and contributes weight 0.
  float m[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const float mw = strided_max<kLpt>(ref[r]);
    const float wsub = mw == kNegInf ? 0.f : mw;
    const float f = ref[r] == kNegInf ? 0.f : fast_exp2(msub[r] - wsub);
    l[r] = strided_sum<kLpt>(l[r] * f);
#pragma unroll
    for (int e = 0; e < kEpc; ++e) acc[r][e] = strided_sum<kLpt>(acc[r][e] * f);
    m[r] = mw;
  }

  // ---- merge the waves of each kv head through LDS and finish
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

  for (int idx = threadIdx.x; idx < kpw * MR * D; idx += NW * 64) {
    const int g = idx / (MR * D);
    const int r = (idx / D) % MR;
    const int d = idx % D;
    const int r_lin = rg * MR + r;
    if (r_lin >= p.rows_per_kvh) continue;
    const int i = r_lin / G;
    const int rid = (b * Sq + i) * Hq + (blockIdx.y * kpw + g) * G + (r_lin - i * G);
    float mx = kNegInf;
    for (int w = g * wph; w < (g + 1) * wph; ++w) mx = __builtin_fmaxf(mx, sm_m[w][r]);
    const float msub = mx == kNegInf ? 0.f : mx;
    float lsum = 0.f, a = 0.f;
    for (int w = g * wph; w < (g + 1) * wph; ++w) {
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
