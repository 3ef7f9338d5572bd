// Paged prefill attention on the matrix cores (gfx950 MFMA) with two teams
// of waves in opposite phases ("ping-pong").
//
// A workgroup of 8 waves owns 256 rows of one kv head (a row is a (query
// position, head of the group) pair); each wave owns two blocks of 16 rows.
// The waves form two teams of four, one wave of each team on every SIMD.
// Every wave alternates two phases, separated by workgroup barriers:
//
//   M(t): O += P(t-1) . V(t-1) and S(t) = K(t) . Q^T  (matrix cores, LDS reads)
//   V(t): softmax of S(t) into the f16 weights P(t), and loads of a later
//         tile                                         (vector ALUs, memory)
//
// Team 1 starts one phase late, so while one team's wave on a SIMD issues
// MFMAs the other team's wave issues vector instructions, and the SIMD runs
// both at once (a probe of independent MFMA and exp/FMA streams in two waves
// of one SIMD: 166 us together against 148 and 106 us alone).  Within one
// wave the two kinds would run mostly one after the other.
//
// K/V tiles of 64 tokens sit in three LDS buffers: a tile is read by the two
// teams one phase apart (K in M(t), V in M(t+1)), so a buffer is busy for
// four phases.  Team 0 loads rows 0-31 of tile t+1 during its V(t), team 1
// rows 32-63 of tile t+2 during its V(t); each wave 8 rows, K straight into
// LDS (global_load_lds_dwordx4); V of f16 caches straight into LDS as well
// (a buffer load whose range ends at the split's last token, so rows past it
// arrive as zeros), V of bf16 caches through registers to be converted.  The
// V phase reads no LDS, so those loads overlap the softmax and the barrier
// that ends the phase is the first wait for them.
//
// The arithmetic per tile is that of the single-team prefill kernel: S^T =
// K . Q^T with v_mfma_f32_16x16x32 (K from LDS, Q^T in registers), the mask
// only on tiles that cross a row's last key or the split's end, one
// lazy-rescale decision per row block per tile (exponents y = x c - msub; the
// reference max rises only when some y exceeds the slack, which the main
// loop detects on the sum of a lane's weights), weights rounded
// once to f16, P . V on the f16 matrix cores with the transposing LDS read
// (bf16 V converted to f16 on its way into LDS).  A bf16 V value beyond f16
// range leaves a non-finite accumulator; a workgroup that ends with one
// recomputes its rows with high and low bf16 weights and the unconverted V
// (one tile at a time, no phases).  Masks, the -inf - (-inf) and 0/0 guards
// and the split ranges follow rocMLIR "Fix split-kv attention masking and
// sweep RMS" (Technical Details).
#pragma once

#include <type_traits>

#include "attn_prefill.h"

namespace pa {

template <typename T, int D, int PS>
__global__ __launch_bounds__(512, 1) void attn_prefill_pp_kernel(const AttnParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(PS == 16 || PS == 32, "page size");
  constexpr int NW = 8;                          // waves per workgroup
  constexpr int RB = 2;                          // 16-row blocks per wave
  constexpr int kTile = 64;                      // tokens per tile
  constexpr int kKSteps = D / 32;
  constexpr int kNBlocks = D / 16;
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  constexpr int kRowsPerLoad = 64 / kChunks;     // rows per wave load
  constexpr int kRowsPerWave = 8;                // tile rows each wave loads
  constexpr int kLoads = kRowsPerWave / kRowsPerLoad;
  static_assert(kRowsPerWave % kRowsPerLoad == 0 && kLoads >= 1, "load split");
  static_assert(PS % kRowsPerWave == 0, "a wave's rows stay inside one page");
  constexpr int kRowsPerWaveQ = 16 * RB;         // query rows per wave
  constexpr int kBuf = kTile * kRowBytes;        // one K or V tile in LDS
  constexpr int kNBuf = 3;
  constexpr float kSlack = 8.f;
  constexpr bool kConvertV = std::is_same<T, bf16_t>::value;
  // V already f16 in memory: straight into LDS like K, no registers
  constexpr bool kVDma = !kConvertV;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // waves are placed on the 4 SIMDs in turn: waves w and w + 4 share one
  const int team = wave >> 2;
  const int wt = wave & 3;
  const int g = lane >> 4;
  const int li = lane & 15;

  // XCD-aware order, as in the single-team kernel: XCD x runs a contiguous
  // range of (row group, kv head, sequence), heaviest row groups first.
  constexpr uint32_t kXcds = 8;
  const uint32_t gx = gridDim.x, gy = gridDim.y;
  const uint32_t n_wg = gx * gy * gridDim.z;
  const uint32_t lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const uint32_t xcd = lin % kXcds;
  const uint32_t per_xcd = n_wg / kXcds, extra = n_wg % kXcds;
  const uint32_t x_first =
      xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd;
  const uint32_t j = lin / kXcds;
  uint32_t logical = x_first + j;
  if (extra == 0 && per_xcd % gx == 0) {
    const uint32_t pairs = per_xcd / gx;
    logical = x_first + (j % pairs) * gx + j / pairs;
  }
  const int bx = static_cast<int>(logical % gx);
  const int by = static_cast<int>((logical / gx) % gy);
  const int bz = static_cast<int>(logical / (gx * gy));
  const int S = p.num_splits;
  const int split = bx % S;
  const int n_rg = gridDim.x / S;
  const int rg = n_rg - 1 - bx / S;
  const int kvh = by;
  const int b = bz;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;

  PageTable pt;
  pt.row = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  // With one split the prologue's rows of this wave (tile 0, and tile 1 for
  // team 1; see the loads below) sit in fixed slots: their ids are read
  // beside the sequence length instead of after it.
  const uint32_t early_id0 =
      pt.id_early((32 * team + 8 * wt) / PS, p.table_width, p.seq_lens + b);
  const uint32_t early_id1 =
      pt.id_early((64 + 32 * team + 8 * wt) / PS, p.table_width, p.seq_lens + b);
  // rows of the workgroup: [wg_first, +256); team 0 owns the first 128
  const int wg_first = rg * kRowsPerWaveQ * NW;
  const int wave_first = wg_first + kRowsPerWaveQ * (4 * team + wt);
  // Q^T as the B operand, loaded first: nothing here waits for the
  // sequence length
  u32x4 qb[RB][kKSteps];
  const float c = __builtin_fmaxf(__builtin_fabsf(p.scale_log2), 1.17549435e-38f);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave_first + 16 * rb + li;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qb[rb][s] = u32x4{0u, 0u, 0u, 0u};
    if (r < p.rows_per_kvh) {
      const int i = div_by(r, p.group_div);
      const int h = kvh * G + (r - i * G);
      const T* qrow = static_cast<const T*>(p.q) + (static_cast<int64_t>(b * Sq + i) * Hq + h) * D;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        qb[rb][s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
    }
  }

  const int seq_len = p.seq_lens[b];
  const int n_pages = (seq_len + PS - 1) / PS;
  const int64_t pos0 = causal_row0(p.prefix_offset, b, seq_len, Sq);

  auto row_limit = [&](int r_lin) __attribute__((always_inline)) {
    return p.causal ? causal_key_limit(seq_len, pos0, div_by(r_lin, p.group_div)) : seq_len;
  };
  const int wg_last = min(wg_first + kRowsPerWaveQ * NW, p.rows_per_kvh) - 1;
  const int wg_max_lim = row_limit(wg_last);

  // ---- split range in pages, cut at the last page the workgroup can see
  const int per = (n_pages + S - 1) / S;
  const int first = min(split * per, n_pages);
  int end = min(first + per, n_pages);
  end = min(end, (wg_max_lim + PS - 1) / PS);
  const int tok_begin = first * PS;
  const int tok_end = min(end * PS, seq_len);
  const int n_tiles = tok_end > tok_begin ? (tok_end - tok_begin + kTile - 1) / kTile : 0;

  pt.page_bytes = static_cast<int64_t>(PS) * Hkv * kRowBytes;
  pt.n_pages = n_pages;

  // ---- LDS: three K/V tile buffers (swizzled rows)
  __shared__ __attribute__((aligned(16))) char smem[kNBuf * 2 * kBuf];
  lds_char* smem3 = (lds_char*)(smem);
  auto swz = [](int r, int cidx) __attribute__((always_inline)) {
    return r * kRowBytes + 16 * (cidx ^ ((2 * r) & (kChunks - 1)));
  };

  const int lr = lane / kChunks;
  const int lc = lane % kChunks;
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);
  typedef __attribute__((address_space(1))) const void* global_ptr;
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // this wave's 8 rows of a tile: team 0 rows 0-31, team 1 rows 32-63
  const int row0 = 32 * team + kRowsPerWave * wt;

  // Issue this wave's loads of one tile: K straight into buffer buf, V into
  // vr.  Lane l fills LDS position lc of row lr of each wave load (its place
  // is fixed by the lane index), so it fetches the chunk the swizzle puts there.
  typedef u32x4 VRegs[kLoads];
  auto load_rows = [&](int tile_tok0, int buf, VRegs& vr, bool early = false,
                       uint32_t early_id = 0) __attribute__((always_inline)) {
    const int tok = tile_tok0 + row0;
    if (tok < tok_end) {                                     // wave-uniform
      const int64_t base = early ? pt.base_of(early_id) : pt.base(tok / PS);
      const int in_page = tok % PS;
#pragma unroll
      for (int jl = 0; jl < kLoads; ++jl) {
        const int r = row0 + jl * kRowsPerLoad + lr;
        const int chunk = lc ^ ((2 * r) & (kChunks - 1));
        const uint32_t off = static_cast<uint32_t>(
            ((in_page + jl * kRowsPerLoad + lr) * Hkv + kvh) * kRowBytes + 16 * chunk);
        const int lds_off = buf * 2 * kBuf + (row0 + jl * kRowsPerLoad) * kRowBytes;
        __builtin_amdgcn_global_load_lds((global_ptr)(kbase + base + off),
                                         (lds_ptr)(smem3 + lds_off), 16, 0, 0);
        if constexpr (!kVDma) vr[jl] = *reinterpret_cast<const u32x4*>(vbase + base + off);
      }
      if constexpr (kVDma) {
        // a buffer resource whose range ends at tok_end: rows past it land
        // in LDS as zeros (the sequence's last page may hold anything there)
        const int rows = min(kRowsPerWave, tok_end - tok);
        const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(vbase) + base + static_cast<int64_t>(in_page) * Hkv * kRowBytes, 0,
            rows * Hkv * kRowBytes, 0x00020000);
#pragma unroll
        for (int jl = 0; jl < kLoads; ++jl) {
          const int r = row0 + jl * kRowsPerLoad + lr;
          const int chunk = lc ^ ((2 * r) & (kChunks - 1));
          const int voff = ((jl * kRowsPerLoad + lr) * Hkv + kvh) * kRowBytes + 16 * chunk;
          const int lds_off = buf * 2 * kBuf + kBuf + (row0 + jl * kRowsPerLoad) * kRowBytes;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr)(smem3 + lds_off), 16, voff, 0,
                                                   0, 0);
        }
      }
    }
  };
  // Store vr where the direct load would have put it; V rows at or past
  // tok_end (past the sequence end, in a page of the next split, or never
  // loaded) become zeros, so no garbage meets a zero weight.  K rows there
  // are harmless: their scores are masked by a select.  With f16v, bf16 V
  // goes to f16.
  auto store_v = [&](auto f16v, int tile_tok0, int buf, const VRegs& vr)
                     __attribute__((always_inline)) {
    constexpr bool kConv = decltype(f16v)::value && kConvertV;
    char* vb = smem + buf * 2 * kBuf + kBuf;
    auto conv = [](u32x4 w) __attribute__((always_inline)) {
      if constexpr (kConv) {
        u32x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = bf16x2_to_f16x2(w[i]);
        return h;
      } else {
        return w;
      }
    };
    if constexpr (kVDma && decltype(f16v)::value) {
      // loaded straight into LDS; a wave that loaded nothing writes zeros
      if (tile_tok0 + row0 >= tok_end) {
#pragma unroll
        for (int jl = 0; jl < kLoads; ++jl)
          *reinterpret_cast<u32x4*>(vb + (row0 + jl * kRowsPerLoad) * kRowBytes + 16 * lane) =
              u32x4{0u, 0u, 0u, 0u};
      }
    } else if (__builtin_expect(tile_tok0 + row0 + kRowsPerWave <= tok_end, 1)) {  // wave-uniform
#pragma unroll
      for (int jl = 0; jl < kLoads; ++jl)
        *reinterpret_cast<u32x4*>(vb + (row0 + jl * kRowsPerLoad) * kRowBytes + 16 * lane) =
            conv(vr[jl]);
    } else if (tile_tok0 + row0 >= tok_end) {  // nothing was loaded
#pragma unroll
      for (int jl = 0; jl < kLoads; ++jl)
        *reinterpret_cast<u32x4*>(vb + (row0 + jl * kRowsPerLoad) * kRowBytes + 16 * lane) =
            u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int jl = 0; jl < kLoads; ++jl) {
        const bool keep = tile_tok0 + row0 + jl * kRowsPerLoad + lr < tok_end;
        *reinterpret_cast<u32x4*>(vb + (row0 + jl * kRowsPerLoad) * kRowBytes + 16 * lane) =
            keep ? conv(vr[jl]) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // prologue loads: tile 0 (both halves) and team 1's half of tile 1, all
  // issued before the first store and before the rest of the set-up; with
  // one split tok_begin is 0 and the rows' page ids were read early
  VRegs vr, vr1;
  if (n_tiles > 0) {
    static_assert(kRowsPerWave == 8 && kTile == 64, "the early page-id slots");
    load_rows(tok_begin, 0, vr, S == 1, early_id0);
    if (team == 1 && n_tiles > 1) load_rows(tok_begin + kTile, 1, vr1, S == 1, early_id1);
  }
  const int wave_last = min(wave_first + kRowsPerWaveQ - 1, p.rows_per_kvh - 1);
  const int wave_min_lim = row_limit(min(wave_first, p.rows_per_kvh - 1));
  const int wave_max_lim = wave_first < p.rows_per_kvh ? row_limit(wave_last) : 0;
  int my_lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave_first + 16 * rb + li;
    my_lim[rb] = r < p.rows_per_kvh ? row_limit(r) : 0;
  }

  float ref[RB], msub[RB];
  f32x4 o[RB][kNBlocks];
  float lsum[RB];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ref[rb] = kNegInf;
      msub[rb] = 0.f;
      lsum[rb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

  // Scores of a tile: x[h][rb][q2][e] is row block rb, row li, token
  // tile_tok0 + 32 h + 16 q2 + 4 g + e.
  typedef float Scores[2][RB][2][4];
  auto qk = [&](int buf, Scores& x) __attribute__((always_inline)) {
    const char* kb = smem + buf * 2 * kBuf;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        f32x4 sacc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kKSteps; ++s) {
          const u32x4 ka =
              *reinterpret_cast<const u32x4*>(kb + swz(32 * h + 16 * q2 + li, 4 * s + g));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) sacc[rb] = Mfma<T>::k32(ka, qb[rb][s], sacc[rb]);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[h][rb][q2][e] = sacc[rb][e];
      }
  };
  // Scores to exponents y = x c - msub in place (the recompute path): the
  // mask (only on tiles that cross a row's last key or the split's end), then
  // one lazy-rescale decision per row block for the tile (an FMA's result is
  // a canonical float, so the maximum runs as v_max3 with no quieting of its
  // inputs).
  auto exponents = [&](int tile_tok0, Scores& x) __attribute__((always_inline)) {
    if (__builtin_expect(tile_tok0 + kTile > wave_min_lim || tile_tok0 + kTile > tok_end, 0)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int lim = min(my_lim[rb], tok_end);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[h][rb][q2][e] =
                  tile_tok0 + 32 * h + 16 * q2 + 4 * g + e < lim ? x[h][rb][q2][e] : kNegInf;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int e = 0; e < 4; ++e) x[h][rb][q2][e] = __builtin_fmaf(x[h][rb][q2][e], c, -msub[rb]);
      float tmax = __builtin_fmaxf(__builtin_fmaxf(x[0][rb][0][0], x[0][rb][0][1]), x[0][rb][0][2]);
#pragma unroll
      for (int k = 3; k + 1 < 16; k += 2)
        tmax = __builtin_fmaxf(__builtin_fmaxf(tmax, x[k >> 3][rb][(k >> 2) & 1][k & 3]),
                               x[(k + 1) >> 3][rb][((k + 1) >> 2) & 1][(k + 1) & 3]);
      tmax = __builtin_fmaxf(tmax, x[1][rb][1][3]);
      const bool raise = tmax > (ref[rb] == kNegInf ? kNegInf : kSlack);
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform, rare
        float rmax = __builtin_fmaxf(tmax, shfl_xor(tmax, 16));
        rmax = __builtin_fmaxf(rmax, shfl_xor(rmax, 32));
        const float nref = __builtin_fmaxf(ref[rb], rmax + msub[rb]);
        const float nsub = nref == kNegInf ? 0.f : nref;
        const float shift = msub[rb] - nsub;
        const float alpha = fast_exp2(shift);
        ref[rb] = nref;
        msub[rb] = nsub;
        lsum[rb] *= alpha;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[h][rb][q2][e] += shift;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ae = __builtin_bit_cast(
              float,
              __builtin_amdgcn_ds_bpermute((4 * g + e) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
          for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb][e] *= ae;
        }
      }
    }
  };
  typedef u32x4 Weights[2][RB];
  // O += P . V for one 32-token half (lane l's eight A values are its weights
  // of the half's two 16-token sub-tiles; its eight B values the two
  // transposing LDS reads of those sub-tiles).  kHiLo: weights as high and
  // low bf16 parts over unconverted bf16 V; else f16 weights over f16 V.
  auto pv_half = [&](auto hilo, int buf, int h, const u32x4 (&phi)[RB], const u32x4 (&plo)[RB])
                     __attribute__((always_inline)) {
    constexpr bool kHiLo = decltype(hilo)::value;
    lds_char* vb3 = smem3 + buf * 2 * kBuf + kBuf;
    const int tr_row = 4 * g + (li >> 2);
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb) {
      const int chunk = 2 * nb + ((li & 3) >> 1);
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(vb3 + swz(32 * h + tr_row, chunk) + 8 * (li & 1)));
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(vb3 + swz(32 * h + 16 + tr_row, chunk) + 8 * (li & 1)));
      const u32x4 vv =
          __builtin_bit_cast(u32x4, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if constexpr (kHiLo) {
          o[rb][nb] = Mfma<T>::k32(phi[rb], vv, o[rb][nb]);
          o[rb][nb] = Mfma<T>::k32(plo[rb], vv, o[rb][nb]);
        } else {
          o[rb][nb] = Mfma<f16_t>::k32(phi[rb], vv, o[rb][nb]);
        }
      }
    }
  };
  // The main loop's softmax of one tile: exponents, weights 2^y as packed
  // f16, row sums.  The lazy rescale needs to know whether some y exceeds
  // the slack (a weight above 2^kSlack); a lane's weights can only hold one
  // if their sum does, so the tile is checked on that sum, which the row sum
  // needs anyway, instead of on a maximum taken before the exponentials.  A
  // lane over the limit, or a row with no reference yet, sends the wave to
  // the exact test: the maximum, the raise of exponents() above, and the
  // weights again.
  auto softmax_f16 = [&](int tile_tok0, Scores& xs, Weights& pw) __attribute__((always_inline)) {
    if (__builtin_expect(tile_tok0 + kTile > wave_min_lim || tile_tok0 + kTile > tok_end, 0)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int lim = min(my_lim[rb], tok_end);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              xs[h][rb][q2][e] =
                  tile_tok0 + 32 * h + 16 * q2 + 4 * g + e < lim ? xs[h][rb][q2][e] : kNegInf;
      }
    }
    // both row blocks' exponentials first (one stream of independent
    // instructions), then one wave-wide test for the rare cases
    float pe[RB][16];
    float tsum[RB];
    bool check = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float& y = xs[k >> 3][rb][(k >> 2) & 1][k & 3];
        y = __builtin_fmaf(y, c, -msub[rb]);
        pe[rb][k] = fast_exp2(y);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // the 16 weights summed as a tree: a serial chain of 16 dependent
      // additions left the wave stalled on each one
      float s8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) s8[k] = pe[rb][2 * k] + pe[rb][2 * k + 1];
      tsum[rb] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
      check = check || ref[rb] == kNegInf || !(tsum[rb] <= 256.f);  // 2^kSlack
    }
    if (__builtin_amdgcn_ballot_w64(check) != 0) {  // wave-uniform, rare
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bool check_rb = ref[rb] == kNegInf || !(tsum[rb] <= 256.f);
        if (__builtin_amdgcn_ballot_w64(check_rb) == 0) continue;
        float tmax = kNegInf;
#pragma unroll
        for (int k = 0; k < 16; ++k) tmax = __builtin_fmaxf(tmax, xs[k >> 3][rb][(k >> 2) & 1][k & 3]);
        const bool raise = tmax > (ref[rb] == kNegInf ? kNegInf : kSlack);
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
          float rmax = __builtin_fmaxf(tmax, shfl_xor(tmax, 16));
          rmax = __builtin_fmaxf(rmax, shfl_xor(rmax, 32));
          const float nref = __builtin_fmaxf(ref[rb], rmax + msub[rb]);
          const float nsub = nref == kNegInf ? 0.f : nref;
          const float shift = msub[rb] - nsub;
          const float alpha = fast_exp2(shift);
          ref[rb] = nref;
          msub[rb] = nsub;
          lsum[rb] *= alpha;
          tsum[rb] = 0.f;
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            float& y = xs[k >> 3][rb][(k >> 2) & 1][k & 3];
            y += shift;
            pe[rb][k] = fast_exp2(y);
            tsum[rb] += pe[rb][k];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ae = __builtin_bit_cast(
                float,
                __builtin_amdgcn_ds_bpermute((4 * g + e) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
            for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb][e] *= ae;
          }
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lsum[rb] += tsum[rb];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pw[h][rb][w] = f32x2_to_f16x2(pe[rb][8 * h + 2 * w], pe[rb][8 * h + 2 * w + 1]);
    }
  };
  const std::true_type f16v;
  const std::false_type unconverted;
  const u32x4 no_lo[RB] = {};
  auto active = [&](int t) __attribute__((always_inline)) {
    return tok_begin + t * kTile < wave_max_lim;  // this wave's rows see some key of tile t
  };

  // ---- the two-team tile loop
  reset();
  Scores x;
  Weights pw;
  if (p.scale_log2 < 0.f) {  // a negative scale flips the scores' sign through Q
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        qb[rb][s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }
  if (n_tiles > 0) {
    store_v(f16v, tok_begin, 0, vr);
    if (team == 1 && n_tiles > 1) store_v(f16v, tok_begin + kTile, 1, vr1);
  }
  __syncthreads();
  if (team == 1) __syncthreads();  // team 1 runs one phase behind
  // M(t): P(t-1) . V(t-1), then S(t).  The buffer of tile t is t mod 3, a
  // compile-time constant in the unrolled loop below, so every LDS read
  // takes its buffer as an immediate offset.
  auto m_phase = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int kB = decltype(bufc)::value;
    if (t > 0 && active(t - 1)) {
      pv_half(std::false_type(), (kB + kNBuf - 1) % kNBuf, 0, pw[0], no_lo);
      pv_half(std::false_type(), (kB + kNBuf - 1) % kNBuf, 1, pw[1], no_lo);
      // LDS reads 8 ahead of the MFMAs that use them (32 transposing reads,
      // 32 MFMAs): left to itself the scheduler kept two reads in flight and
      // each pair of MFMAs waited for its operands
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 24; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    if (t < n_tiles && active(t)) {
      qk(kB, x);
      // 16 K-operand reads, 32 MFMAs (two per read), reads 4 ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };
  // V(t): this team's loads of a later tile (team 0 rows 0-31 of tile t+1,
  // team 1 rows 32-63 of tile t+2), then the softmax of tile t
  auto v_phase = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int kB = decltype(bufc)::value;
    const int lt = t + 1 + team;
    const int lbuf = team == 0 ? (kB + 1) % kNBuf : (kB + 2) % kNBuf;
    const bool load = lt < n_tiles;
    if (load) load_rows(tok_begin + lt * kTile, lbuf, vr);
    if (active(t)) softmax_f16(tok_begin + t * kTile, x, pw);
    if (load) store_v(f16v, tok_begin + lt * kTile, lbuf, vr);
  };
  for (int t = 0;; t += kNBuf) {
    m_phase(t, std::integral_constant<int, 0>());
    __syncthreads();
    if (t == n_tiles) break;
    v_phase(t, std::integral_constant<int, 0>());
    __syncthreads();
    m_phase(t + 1, std::integral_constant<int, 1>());
    __syncthreads();
    if (t + 1 == n_tiles) break;
    v_phase(t + 1, std::integral_constant<int, 1>());
    __syncthreads();
    m_phase(t + 2, std::integral_constant<int, 2>());
    __syncthreads();
    if (t + 2 == n_tiles) break;
    v_phase(t + 2, std::integral_constant<int, 2>());
    __syncthreads();
  }
  if (team == 0) __syncthreads();  // the barrier team 1 spent at the start

  if constexpr (kConvertV) {
    // a V value beyond f16 range (or a non-finite input) left a non-finite
    // accumulator: 0 * inf and 0 * NaN are NaN
    float z = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) z = __builtin_fmaf(o[rb][nb][e], 0.f, z);
    int* flags = reinterpret_cast<int*>(smem);  // the tile buffers are free after the last barrier
    const bool bad = __builtin_amdgcn_ballot_w64(z != z) != 0;
    if (lane == 0) flags[wave] = bad;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= flags[w];
    if (redo) {  // workgroup-uniform, rare: one tile at a time, bf16 high/low weights
      __syncthreads();  // every wave has read the flags before the loads reuse the buffers
      reset();
      for (int t = 0; t < n_tiles; ++t) {
        const int tok0 = tok_begin + t * kTile;
        load_rows(tok0, 0, vr);  // the 8 waves' rows cover the tile
        store_v(unconverted, tok0, 0, vr);
        __syncthreads();
        if (active(t)) {
          qk(0, x);
          exponents(tok0, x);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 phi[RB], plo[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
              float pe[8];
#pragma unroll
              for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                for (int e = 0; e < 4; ++e) pe[4 * q2 + e] = fast_exp2(x[h][rb][q2][e]);
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                uint32_t hi, lo;
                Mfma<T>::split2(pe[2 * w], pe[2 * w + 1], hi, lo);
                phi[rb][w] = hi;
                plo[rb][w] = lo;
              }
#pragma unroll
              for (int w = 0; w < 8; ++w) lsum[rb] += pe[w];
            }
            pv_half(std::true_type(), 0, h, phi, plo);
          }
        }
        __syncthreads();  // every wave is done with the tile before the next one's loads
      }
    }
  }

  // ---- finish: normalize and write.  After the two exchanges every lane
  // holds row li's sum and reference, so it forms that row's 1/l and LSE
  // once; row 4 g + e of the O layout takes its 1/l from lane 4 g + e.  Two
  // rows' values are rounded to the output type in one packed conversion.
  typedef __attribute__((ext_vector_type(2))) float f32x2v;
  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2v;
  auto pack2 = [](float a, float b) __attribute__((always_inline)) {
    const f32x2v v = {a, b};
    if constexpr (std::is_same<T, bf16_t>::value)
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
    else
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v));
  };
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lsum[rb] += shfl_xor(lsum[rb], 16);
    lsum[rb] += shfl_xor(lsum[rb], 32);
    const bool any = lsum[rb] > 0.f;  // no valid key: (0, -inf) instead of 0/0
    const float inv_row = any ? 1.f / lsum[rb] : 0.f;
    const float lse_row = any ? (ref[rb] + log2f(lsum[rb])) * kLn2 : kNegInf;
    auto row_id = [&](int r_lin) __attribute__((always_inline)) {
      const int i = div_by(r_lin, p.group_div);
      return (b * Sq + i) * Hq + kvh * G + (r_lin - i * G);
    };
    {
      const int r_lin = wave_first + 16 * rb + li;
      if (g == 0 && r_lin < p.rows_per_kvh) {
        const int rid = row_id(r_lin);
        if (S == 1) {
          if (p.lse != nullptr) p.lse[rid] = lse_row;
        } else {
          p.part_lse[static_cast<int64_t>(rid) * S + split] = lse_row;
        }
      }
    }
    float inv[4];
    int rid[4];
    bool valid[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      inv[e] = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute((4 * g + e) << 2, __builtin_bit_cast(int, inv_row)));
      const int r_lin = wave_first + 16 * rb + 4 * g + e;
      valid[e] = r_lin < p.rows_per_kvh;
      rid[e] = valid[e] ? row_id(r_lin) : 0;
    }
    if (S == 1) {
      // Every row of the block exists except in a tail row group: the stores
      // then need no per-row guard (each guard cost a branch and an address
      // rebuild around every 2-byte store).
      const bool all_rows = wave_first + 16 * rb + 15 < p.rows_per_kvh;  // wave-uniform
#pragma unroll
      for (int ep = 0; ep < 2; ++ep) {
        uint16_t* d0 = reinterpret_cast<uint16_t*>(static_cast<T*>(p.out) +
                                                   static_cast<int64_t>(rid[2 * ep]) * D) + li;
        uint16_t* d1 = reinterpret_cast<uint16_t*>(static_cast<T*>(p.out) +
                                                   static_cast<int64_t>(rid[2 * ep + 1]) * D) + li;
        if (__builtin_expect(all_rows, 1)) {
#pragma unroll
          for (int nb = 0; nb < kNBlocks; ++nb) {
            const uint32_t pk = pack2(o[rb][nb][2 * ep] * inv[2 * ep],
                                      o[rb][nb][2 * ep + 1] * inv[2 * ep + 1]);
            d0[16 * nb] = static_cast<uint16_t>(pk);
            d1[16 * nb] = static_cast<uint16_t>(pk >> 16);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < kNBlocks; ++nb) {
            const uint32_t pk = pack2(o[rb][nb][2 * ep] * inv[2 * ep],
                                      o[rb][nb][2 * ep + 1] * inv[2 * ep + 1]);
            if (valid[2 * ep]) d0[16 * nb] = static_cast<uint16_t>(pk);
            if (valid[2 * ep + 1]) d1[16 * nb] = static_cast<uint16_t>(pk >> 16);
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!valid[e]) continue;
        float* dst = p.part_out + (static_cast<int64_t>(rid[e]) * S + split) * D;
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb) dst[16 * nb + li] = o[rb][nb][e] * inv[e];
      }
    }
  }
}

}  // namespace pa
