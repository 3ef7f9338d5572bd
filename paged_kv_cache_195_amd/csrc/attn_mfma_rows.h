// The matrix-core paged attention kernel of attn_mfma.h with RB blocks of 16
// query rows per wave.  Used with RB = 2 when a kv head carries 17 to 32
// rows (decode at group sizes 17..32, and 8-bit caches up to 63 rows): all
// of a wave's row blocks share each staged K/V tile, so a kv head's pages
// are read once per 32 rows instead of once per 16.  Everything else -- the
// page walk, staging, the running softmax per row, the split ranges, the
// merge of the waves of a kv head -- is that kernel's, done per row block.
// (The RB = 1 case stays in attn_mfma.h: folding both into one template
// changed the one-block code enough to slow the Qwen3-235B decode step
// from 630 to 715 us.)
#pragma once

#include "attn_mfma.h"

namespace pa {

// T: bf16_t or f16_t (q, out and the MFMA operands); KV: KvSame (caches of
// T) or KvI8 / KvFp8 (8-bit codes with p.k_scale / p.v_scale); D: head dim
// (= Dv, a multiple of 32; >= 64 for codes); PS: tokens per page (a multiple
// of 16); NW: waves per workgroup; RB: blocks of 16 rows per wave, which
// share each staged K/V tile (RB = 2 serves 17 to 32 rows per kv head with
// one read of the pages instead of two).  p.heads_per_wg kv heads per
// workgroup, NW / heads_per_wg waves per head; each workgroup covers 16 RB
// rows per kv head (row group rg = blockIdx.x / S).
// Static LDS of one workgroup: per wave, a K and a V tile of 16 staged rows,
// reused for the final merge of its 16 RB rows.
template <int D, int NW, int RB>
constexpr int mfma_rows_static_lds() {
  return NW * ((2 * 16 * D * 2) > (16 * RB * D * 4 + 2 * 16 * RB * 4)
                   ? (2 * 16 * D * 2)
                   : (16 * RB * D * 4 + 2 * 16 * RB * 4));
}

template <typename T, typename KV, int D, int PS, int NW, int RB>
__global__ __launch_bounds__(NW * 64) void attn_mfma_rows_kernel(const AttnParams p) {
  static_assert(D % 32 == 0 && PS % 16 == 0, "tile shape");
  constexpr bool kQuant = KvTraits<KV>::quant;
  constexpr int kKSteps = D / 32;         // 16x16x32 steps for q.k
  constexpr int kNBlocks = D / 16;        // 16-dim output blocks
  constexpr int kTiles = PS / 16;         // 16-token tiles per page
  constexpr int kRowBytes = D * 2;        // a staged row (operand type)
  constexpr int kCacheRowBytes = kQuant ? D : D * 2;  // a row in the cache
  constexpr float kSlack = 8.f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // 16-lane group
  const int li = lane & 15;  // index inside the group

  const int S = p.num_splits;
  const int split = blockIdx.x % S;
  const int rg = blockIdx.x / S;
  const int kpw = p.heads_per_wg;
  const int wph = NW / kpw;
  const int kg = wave / wph;
  const int sub = wave - kg * wph;
  const int kvh = blockIdx.y * kpw + kg;
  const int b = blockIdx.z;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;

  const int seq_len = p.seq_lens[b];
  const int n_pages = (seq_len + PS - 1) / PS;
  const int64_t pos0 = causal_row0(p.prefix_offset, b, seq_len, Sq);

  // ---- this lane's rows (row li of each block of 16) and the key limits of
  // the group
  auto row_limit = [&](int r_lin) __attribute__((always_inline)) {
    return p.causal ? causal_key_limit(seq_len, pos0, r_lin / G) : seq_len;
  };
  constexpr int kRows = 16 * RB;  // rows of a row group
  int my_r[RB];
  bool my_valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    my_r[rb] = rg * kRows + 16 * rb + li;
    my_valid[rb] = my_r[rb] < p.rows_per_kvh;
  }
  // rows of this group: limits are the same for every kv head
  int max_lim = 0, min_lim = 0x7fffffff;
  for (int r = 0; r < kRows; ++r) {
    const int r_lin = rg * kRows + r;
    if (r_lin >= p.rows_per_kvh) break;
    const int l = row_limit(r_lin);
    max_lim = l > max_lim ? l : max_lim;
    min_lim = l < min_lim ? l : min_lim;
  }
  int my_lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) my_lim[rb] = my_valid[rb] ? row_limit(my_r[rb]) : max_lim;

  // Q^T as the B operand: lane l holds q[row li of block rb][32 s + 8 g .. +8]
  u32x4 qb[RB][kKSteps];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = my_r[rb] / G;
    const int h = kvh * G + (my_r[rb] - i * G);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qb[rb][s] = u32x4{0u, 0u, 0u, 0u};
    if (my_valid[rb]) {  // padding rows past the last row never touch q
      const T* qrow =
          static_cast<const T*>(p.q) + (static_cast<int64_t>(b * Sq + i) * Hq + h) * D;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        qb[rb][s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
    }
  }
  const float c = __builtin_fmaxf(__builtin_fabsf(p.scale_log2), 1.17549435e-38f);
  if (p.scale_log2 < 0.f) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        qb[rb][s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  // ---- split range (ceil-divided, clamped, cut at the last visible page)
  const int per = (n_pages + S - 1) / S;
  const int first = min(split * per, n_pages);
  int end = min(first + per, n_pages);
  end = min(end, (max_lim + PS - 1) / PS);

  PageTable pt;
  pt.row = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  pt.page_bytes = static_cast<int64_t>(PS) * Hkv * kCacheRowBytes;
  pt.n_pages = n_pages;

  // Whole-row loads: wave load j covers rows j * kRowsPerLoad .. +kRowsPerLoad
  // of the tile; lane l takes 16-byte chunk lc of row lr.
  constexpr int kChunks = D / 8;                      // 16-byte chunks per staged row
  constexpr int kCacheChunks = kCacheRowBytes / 16;   // 16-byte chunks per cache row
  constexpr int kRowsPerLoad = 64 / kCacheChunks;     // rows per wave load
  constexpr int kLoads = 16 / kRowsPerLoad;           // wave loads per tile
  static_assert(kRowsPerLoad <= 16 && 16 % kRowsPerLoad == 0, "whole rows per tile");
  const int lr = lane / kCacheChunks;
  const int lc = lane % kCacheChunks;
  const uint32_t lane_off = static_cast<uint32_t>((lr * Hkv + kvh) * kCacheRowBytes + 16 * lc);
  const uint32_t load_step = static_cast<uint32_t>(kRowsPerLoad * Hkv * kCacheRowBytes);
  const uint32_t tile_step = static_cast<uint32_t>(16 * Hkv * kCacheRowBytes);
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);

  // LDS: per wave, a K tile and a V tile of 16 swizzled rows; reused for the
  // final merge
  constexpr int kTileLds = 2 * 16 * kRowBytes;
  constexpr int kMergeLds = kRows * D * 4 + 2 * kRows * 4;
  constexpr int kPerWave = kTileLds > kMergeLds ? kTileLds : kMergeLds;
  static_assert(NW * kPerWave == mfma_rows_static_lds<D, NW, RB>(), "LDS size");
  __shared__ __attribute__((aligned(16))) char smem[NW * kPerWave];
  char* my_lds = smem + wave * kPerWave;
  lds_char* my_lds3 = (lds_char*)(smem) + wave * kPerWave;
  char* lds_k = my_lds;
  char* lds_v = my_lds + 16 * kRowBytes;
  lds_char* lds_v3 = my_lds3 + 16 * kRowBytes;
  // byte offset in a tile of 16-byte chunk c of row r
  auto swz = [](int r, int c) __attribute__((always_inline)) { return r * kRowBytes + 16 * (c ^ ((2 * r) & (kChunks - 1))); };

  float ref[RB], msub[RB], lsum[RB];
  f32x4 o[RB][kNBlocks];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    ref[rb] = kNegInf;
    msub[rb] = 0.f;
    lsum[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto load_tile = [&](int64_t base, int t, u32x4* kk, u32x4* vv) __attribute__((always_inline)) {
    const uint32_t off = lane_off + t * tile_step;
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      kk[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + base + off + j * load_step));
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      vv[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(vbase + base + off + j * load_step));
  };

  auto consume_tile = [&](int tok0, const u32x4* kk, u32x4* vv, float ks, float vs)
                          __attribute__((always_inline)) {
    // stage K and V rows; V rows of tokens past the sequence become zero
    const bool tail = tok0 + 16 > min_lim;  // wave-uniform
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int r = j * kRowsPerLoad + lr;
      u32x4 vrow = vv[j];
      if (tail && tok0 + r >= seq_len) vrow = u32x4{0u, 0u, 0u, 0u};
      if constexpr (kQuant) {
        u32x4 lo, hi;
        widen16<T, KV>(kk[j], lo, hi);
        *reinterpret_cast<u32x4*>(lds_k + swz(r, 2 * lc)) = lo;
        *reinterpret_cast<u32x4*>(lds_k + swz(r, 2 * lc + 1)) = hi;
        widen16<T, KV>(vrow, lo, hi);
        *reinterpret_cast<u32x4*>(lds_v + swz(r, 2 * lc)) = lo;
        *reinterpret_cast<u32x4*>(lds_v + swz(r, 2 * lc + 1)) = hi;
      } else {
        *reinterpret_cast<u32x4*>(lds_k + swz(r, lc)) = kk[j];
        *reinterpret_cast<u32x4*>(lds_v + swz(r, lc)) = vrow;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // S^T: lane holds S[row li of block rb][token tok0 + 4 g + e]
    f32x4 sacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(lds_k + swz(li, 4 * s + g));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb] = Mfma<T>::k32(ka, qb[rb][s], sacc[rb]);
    }

    // weights, split into high and low 16-bit parts.  For 8-bit caches with
    // bf16 operands the V scale folds into the weights (bf16 keeps float's
    // exponent range and the split keeps the sign); f16 weights could overflow,
    // so there the scale multiplies each tile's P.V product instead.
    constexpr bool kFoldV = kQuant && __is_same(T, bf16_t);
    s16x4 phi[RB], plo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float x[4] = {sacc[rb][0], sacc[rb][1], sacc[rb][2], sacc[rb][3]};
      if constexpr (kQuant) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] *= ks;
      }
      if (tail) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = tok0 + 4 * g + e < my_lim[rb] ? x[e] : kNegInf;
      }

      float tmax = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), __builtin_fmaxf(x[2], x[3]));
      const bool raise = tmax * c > ref[rb] + kSlack;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
        float rmax = __builtin_fmaxf(tmax, shfl_xor(tmax, 16));
        rmax = __builtin_fmaxf(rmax, shfl_xor(rmax, 32));  // max of row li over the tile
        const float nref = __builtin_fmaxf(ref[rb], rmax * c);
        const float nsub = nref == kNegInf ? 0.f : nref;
        const float alpha = fast_exp2(msub[rb] - nsub);
        ref[rb] = nref;
        msub[rb] = nsub;
        lsum[rb] *= alpha;
        // O rows 4 g + e need the factor of those rows, held by lanes 4 g + e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = __builtin_bit_cast(
              float, __builtin_amdgcn_ds_bpermute((4 * g + e) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
          for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb][e] *= ae;
        }
      }

      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = fast_exp2(__builtin_fmaf(x[e], c, -msub[rb]));  // x = -inf gives 0
        lsum[rb] += pe[e];
        if constexpr (kFoldV) pe[e] *= vs;
      }
      uint32_t h01, l01, h23, l23;
      Mfma<T>::split2(pe[0], pe[1], h01, l01);
      Mfma<T>::split2(pe[2], pe[3], h23, l23);
      phi[rb] = __builtin_bit_cast(s16x4, uint64_t(h01) | (uint64_t(h23) << 32));
      plo[rb] = __builtin_bit_cast(s16x4, uint64_t(l01) | (uint64_t(l23) << 32));
    }

    // B operand for block nb: tokens 4 g .. 4 g + 3 of dimension 16 nb + li;
    // source lane li points at row 4 g + li / 4, dimensions 16 nb + 4 (li % 4) ..
    const int tr_row = 4 * g + (li >> 2);
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb) {
      const int chunk = 2 * nb + ((li & 3) >> 1);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(lds_v3 + swz(tr_row, chunk) + 8 * (li & 1)));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (kQuant && !kFoldV) {
          f32x4 t = Mfma<T>::k16(phi[rb], vb, f32x4{0.f, 0.f, 0.f, 0.f});
          t = Mfma<T>::k16(plo[rb], vb, t);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[rb][nb][e] = __builtin_fmaf(vs, t[e], o[rb][nb][e]);
        } else {
          o[rb][nb] = Mfma<T>::k16(phi[rb], vb, o[rb][nb]);
          o[rb][nb] = Mfma<T>::k16(plo[rb], vb, o[rb][nb]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Scales of a page: [page][kv head], read as wave-uniform scalars.
  auto page_scales = [&](uint32_t pid, float& ks, float& vs) __attribute__((always_inline)) {
    if constexpr (kQuant) {
      const int64_t si = static_cast<int64_t>(pid) * Hkv + kvh;
      ks = p.k_scale[si];
      vs = p.v_scale[si];
    }
  };
  if constexpr (!kQuant) {
    // ---- stream, 16-bit caches: the wave takes pages first + sub,
    // first + sub + wph, ...; each page is kTiles tiles; the next tile's
    // loads are issued before the current tile is computed.
    int slot = first + sub;
    if (slot < end) {
      int64_t base = pt.base(slot);
      u32x4 kc[kLoads], vc[kLoads];
      int t = 0;
      load_tile(base, 0, kc, vc);
      while (true) {
        const int tok0 = slot * PS + 16 * t;
        int nslot = slot, nt = t + 1;
        if (nt == kTiles) {
          nslot = slot + wph;
          nt = 0;
        }
        const bool more = nslot < end;
        int64_t nbase = base;
        u32x4 kn[kLoads], vn[kLoads];
        if (more) {
          if (nslot != slot) nbase = pt.base(nslot);
          load_tile(nbase, nt, kn, vn);
        }
        consume_tile(tok0, kc, vc, 1.f, 1.f);
        if (!more) break;
#pragma unroll
        for (int s = 0; s < kLoads; ++s) {
          kc[s] = kn[s];
          vc[s] = vn[s];
        }
        slot = nslot;
        t = nt;
        base = nbase;
      }
    }
  } else {
    // ---- stream, 8-bit caches: the same tile order (tile k is tile
    // k % kTiles of the page in slot first + sub + (k / kTiles) * wph), with
    // loads kAhead tiles ahead of the compute through a ring of kAhead + 1
    // register buffers indexed by compile-time stages.  An 8-bit tile holds
    // half the bytes of a 16-bit one, so more of them stay in flight (one
    // ahead: 452 us, three ahead: 356 us on the Llama-3-8B decode shape).
    constexpr int kAhead = PA_QUANT_AHEAD;
    constexpr int kRing = kAhead + 1;
    const int my_first = first + sub;
    const int my_pages = my_first < end ? (end - my_first + wph - 1) / wph : 0;
    const int n_tiles = my_pages * kTiles;
    u32x4 kr[kRing][kLoads], vr[kRing][kLoads];
    float rks[kRing], rvs[kRing];
    int64_t cur_base = 0;
    float cur_ks = 1.f, cur_vs = 1.f;
    // issue the loads of tile k into one ring stage
    auto issue = [&](int k, u32x4* kk, u32x4* vv, float& ks, float& vs)
                     __attribute__((always_inline)) {
      const int pg = k / kTiles;
      const int t = k - pg * kTiles;
      if (t == 0) {
        const uint32_t pid = pt.id(my_first + pg * wph);
        cur_base = pt.base_of(pid);
        page_scales(pid, cur_ks, cur_vs);
      }
      ks = cur_ks;
      vs = cur_vs;
      load_tile(cur_base, t, kk, vv);
    };
#pragma unroll
    for (int st = 0; st < kAhead; ++st)
      if (st < n_tiles) issue(st, kr[st], vr[st], rks[st], rvs[st]);
    for (int k0 = 0; k0 < n_tiles; k0 += kRing) {
#pragma unroll
      for (int st = 0; st < kRing; ++st) {
        const int k = k0 + st;
        if (k < n_tiles) {  // wave-uniform
          const int ns = (st + kAhead) % kRing;
          if (k + kAhead < n_tiles) issue(k + kAhead, kr[ns], vr[ns], rks[ns], rvs[ns]);
          const int pg = k / kTiles;
          const int tok0 = (my_first + pg * wph) * PS + 16 * (k - pg * kTiles);
          consume_tile(tok0, kr[st], vr[st], rks[st], rvs[st]);
        }
      }
    }
  }

  // ---- finish this wave: row sums over the four token groups
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lsum[rb] += shfl_xor(lsum[rb], 16);
    lsum[rb] += shfl_xor(lsum[rb], 32);
  }

  // ---- merge the waves of each kv head through LDS, then write
  __syncthreads();  // every wave is done with its V tiles
  float* mo = reinterpret_cast<float*>(my_lds);  // [16 RB rows][D]
  float* mref = mo + kRows * D;                  // [16 RB]
  float* ml = mref + kRows;                      // [16 RB]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mo[(16 * rb + 4 * g + e) * D + 16 * nb + li] = o[rb][nb][e];
    if (g == 0) {
      mref[16 * rb + li] = ref[rb];
      ml[16 * rb + li] = lsum[rb];
    }
  }
  __syncthreads();

  merge_wave_states<T, D, kRows, NW, kPerWave>(p, smem, kpw, rg, b, split);
}

}  // namespace pa
