// Paged prefill attention on the matrix cores (gfx950 MFMA), when one kv
// head carries many query rows (a row is a (query position, head of the
// group) pair).  Serves 16-bit caches at D = 64 (D = 128 takes the two-team
// kernel of attn_prefill_pp.h, which also uses this file's helpers) and
// 8-bit K/V codes at D = 64 and 128.
//
// A workgroup owns 16 * RB * NW rows of one kv head; wave w owns RB blocks of
// 16 rows.  The workgroup walks its split's keys in 64-token tiles.  Each
// tile of K and V is loaded once, cooperatively (every wave loads whole rows
// of it; K, and V of f16 caches, with global_load_lds_dwordx4 straight into
// LDS), into one of two LDS buffers, and every wave computes its rows against
// it, so each K/V byte read from memory serves 16 * RB * NW rows and each
// operand read from LDS serves RB row blocks.  The next tile's loads are
// issued before the current tile is computed.
//
// Per 16-token sub-tile and row block, S^T = K . Q^T is the decode MFMA
// kernel's product (v_mfma_f32_16x16x32, K from LDS, Q^T in registers); its
// accumulator holds, per lane, row l%16 and tokens 4*(l/16)..+3.  O += P . V
// runs on 32-token halves with v_mfma_f32_16x16x32 as well: the order of the
// 32 tokens along K is free as long as both operands agree, so lane l's eight
// A values are its four weights from each of the two sub-tiles, and its
// eight B values are the two transposing LDS reads (ds_read_b64_tr_b16) of
// those sub-tiles -- no data moves between lanes.  LDS rows use the same XOR
// swizzle as the decode kernel.
//
// P . V runs in f16: each weight is rounded once to f16 (11 significant bits,
// relative error <= 2^-12; a weight is at most 2^8 under the lazy rescale).
// f16 caches need nothing more.  For bf16 caches the V tile passes through
// registers and is converted to f16 on its way into LDS (exact for values of
// magnitude 2^-14 .. 65504; smaller ones keep an absolute error <= 2^-25).  A
// V value beyond f16 range becomes infinite and leaves a non-finite
// accumulator behind, so a workgroup that ends with one recomputes its rows
// with the bf16 operands: each weight as a high and a low bf16 part (two
// MFMAs per product, 16 significant bits), V loaded unchanged.  One bf16
// weight alone (8 bits) is not accurate enough for the bf16 error bound.
//
// Causal masking is bottom-right (row i of Sq sits at key position
// L - Sq + i); tiles past the last key any row of the workgroup can see are
// skipped.  The running state, the guards against -inf - (-inf) and 0/0, and
// the split ranges follow rocMLIR "Fix split-kv attention masking and sweep
// RMS" (Technical Details), as in the decode kernels.  Every wave owns
// distinct rows, so no cross-wave merge is needed.
#pragma once

#include <type_traits>

#include "attn_mfma.h"

namespace pa {

// Two floats as a packed f16 pair, each rounded to nearest even (one
// v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
// A packed bf16 pair as a packed f16 pair: exact for magnitudes 2^-14 ..
// 65504, rounded to nearest even below, infinite above.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return f32x2_to_f16x2(__builtin_bit_cast(float, w << 16),
                        __builtin_bit_cast(float, w & 0xffff0000u));
}

typedef __attribute__((address_space(3))) float lds_float;

// LDS of the kernel: two K/V tile buffers of 64 rows.
template <int D>
constexpr int prefill_tile_lds() {
  return 2 * 2 * 64 * D * 2;
}

// The whole computation of one workgroup.  kExact (8-bit codes only) adds the
// per-tile test for V factors far below the running reference.  Without it,
// a workgroup whose pages' V scales lie more than 2^6 apart returns false
// before any tile is read, and the kernel runs it again with kExact.
template <typename T, int D, int PS, int NW, int RB, typename KV, bool kExact>
__device__ __forceinline__ bool prefill_body(const AttnParams& p, lds_char* smem3,
                                             lds_float* sub_scale) {
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(PS == 16 || PS == 32, "page size");
  // 8-bit K/V codes (KvI8, KvFp8): both tiles pass through registers and are
  // decoded exactly on their way into LDS -- K to the query type, V to f16 --
  // so the LDS layout and the MFMA steps are those of 16-bit caches.  A
  // 16-token sub-tile always lies in one page, so its K scale multiplies its
  // scores, and its V scale joins its f16 weights as vs / vref, where vref is
  // the largest |V scale| the wave has met (the accumulators are rescaled when
  // it grows, like the running max), so a weight never exceeds its unscaled
  // value and no scale overflows f16; the output is multiplied by vref at the
  // end.  While every sub-tile of a tile has |vs / vref| >= 2^-6, its weights
  // down to 2^-8 stay normal f16 numbers, exact to 2^-12.  A tile holding a
  // sub-tile further below (a wave-uniform test on the scales) adds that
  // sub-tile on its own: with vs / vref = m 2^E (|m| in [1, 2)), O is scaled
  // by 2^-E, takes the sub-tile's P . V with its weights times m, and is
  // scaled back by 2^E (exact in f32) -- so the weights keep f16's relative
  // precision however far apart the V scales lie.
  constexpr bool kQuant = KvTraits<KV>::quant;
  constexpr int kTile = 64;                      // tokens per tile
  constexpr int kSub = kTile / 16;               // 16-token sub-tiles
  constexpr int kKSteps = D / 32;
  constexpr int kNBlocks = D / 16;
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  constexpr int kRowsPerLoad = 64 / kChunks;     // rows per wave load
  constexpr int kRowsPerWave = kTile / NW;       // tile rows each wave loads
  constexpr int kLoads = kRowsPerWave / kRowsPerLoad;
  static_assert(kRowsPerWave % kRowsPerLoad == 0 && kLoads >= 1, "load split");
  static_assert(kRowsPerWave <= PS, "a wave's rows stay inside one page");
  constexpr int kRowsPerWaveQ = 16 * RB;         // query rows per wave
  constexpr int kBuf = kTile * kRowBytes;        // one K or V tile in LDS
  constexpr float kSlack = 8.f;
  constexpr float kFarScale = 1.f / 64.f;  // 8-bit codes: V factors below this take half_pv_sub
  constexpr bool kConvertV = !kQuant && std::is_same<T, bf16_t>::value;  // bf16 V goes to f16
  constexpr int kCacheRowBytes = kQuant ? D : kRowBytes;  // a K or V row in the cache
  constexpr int kCodeChunks = D / 16;                     // 16-byte chunks of a code row
  constexpr int kRowsPerLoadQ = 64 / kCodeChunks;         // code rows per wave load
  constexpr int kLoadsQ = kRowsPerWave / kRowsPerLoadQ;
  static_assert(!kQuant || (kRowsPerWave % kRowsPerLoadQ == 0 && kLoadsQ >= 1 &&
                            kRowsPerWave % 16 == 0),
                "8-bit loads: whole code rows, whole 16-token sub-tiles per wave");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int li = lane & 15;

  // XCD-aware order.  An MI355X dispatches workgroups round-robin over its 8
  // XCDs, each with its own L2, and every row group of a (sequence, kv head)
  // reads the same K/V tiles.  Renumbered so that XCD x runs a contiguous
  // range of (row group, kv head, sequence), a kv head's tiles stay in one
  // L2 instead of being fetched by all eight (B=4, Sq=L=1024: 102 -> 78 us;
  // B=1, Sq=L=4096: 436 -> 376 us).  The renumbering is a bijection for any
  // grid size; the XCD count only tunes locality and order.
  constexpr uint32_t kXcds = 8;
  const uint32_t gx = gridDim.x, gy = gridDim.y;
  const uint32_t n_wg = gx * gy * gridDim.z;
  const uint32_t lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const uint32_t xcd = lin % kXcds;
  const uint32_t per_xcd = n_wg / kXcds, extra = n_wg % kXcds;
  const uint32_t x_first =
      xcd < extra ? xcd * (per_xcd + 1) : extra * (per_xcd + 1) + (xcd - extra) * per_xcd;
  const uint32_t j = lin / kXcds;  // this workgroup's place in its XCD's dispatch order
  uint32_t logical = x_first + j;
  if (extra == 0 && per_xcd % gx == 0) {
    // the XCD's range holds whole (kv head, sequence) pairs: dispatch it row
    // group by row group across its pairs, heaviest row groups first, so no
    // pair's heavy groups wait behind another pair's light ones (B=4,
    // Sq=L=1024: 75 -> 63 us; B=16: 256 -> 231 us)
    const uint32_t pairs = per_xcd / gx;
    logical = x_first + (j % pairs) * gx + j / pairs;
  }
  const int bx = static_cast<int>(logical % gx);
  const int by = static_cast<int>((logical / gx) % gy);
  const int bz = static_cast<int>(logical / (gx * gy));
  const int S = p.num_splits;
  const int split = bx % S;
  // heaviest (latest) row groups first: they see the most keys
  const int n_rg = gridDim.x / S;
  const int rg = n_rg - 1 - bx / S;
  const int kvh = by;
  const int b = bz;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;

  const int seq_len = p.seq_lens[b];
  const int n_pages = (seq_len + PS - 1) / PS;
  const int64_t pos0 = causal_row0(p.prefix_offset, b, seq_len, Sq);

  auto row_limit = [&](int r_lin) __attribute__((always_inline)) {
    return p.causal ? causal_key_limit(seq_len, pos0, div_by(r_lin, p.group_div)) : seq_len;
  };
  // rows of the workgroup: [wg_first, +16 RB NW); the last one sees the most keys
  const int wg_first = rg * kRowsPerWaveQ * NW;
  const int wg_last = min(wg_first + kRowsPerWaveQ * NW, p.rows_per_kvh) - 1;
  const int wg_max_lim = row_limit(wg_last);
  // this wave's rows: [wave_first, +16 RB); block rb, lane row li is wave_first + 16 rb + li
  const int wave_first = wg_first + kRowsPerWaveQ * wave;
  const int wave_last = min(wave_first + kRowsPerWaveQ - 1, p.rows_per_kvh - 1);
  const int wave_min_lim = row_limit(min(wave_first, p.rows_per_kvh - 1));
  const int wave_max_lim = wave_first < p.rows_per_kvh ? row_limit(wave_last) : 0;
  int my_lim[RB];
  u32x4 qb[RB][kKSteps];
  const float c = __builtin_fmaxf(__builtin_fabsf(p.scale_log2), 1.17549435e-38f);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = wave_first + 16 * rb + li;
    const bool valid = r < p.rows_per_kvh;
    my_lim[rb] = valid ? row_limit(r) : 0;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qb[rb][s] = u32x4{0u, 0u, 0u, 0u};
    if (valid) {
      const int i = div_by(r, p.group_div);
      const int h = kvh * G + (r - i * G);
      const T* qrow = static_cast<const T*>(p.q) + (static_cast<int64_t>(b * Sq + i) * Hq + h) * D;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        qb[rb][s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
    }
    if (p.scale_log2 < 0.f) {
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        qb[rb][s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
  }

  // ---- split range in pages, cut at the last page the workgroup can see
  const int per = (n_pages + S - 1) / S;
  const int first = min(split * per, n_pages);
  int end = min(first + per, n_pages);
  end = min(end, (wg_max_lim + PS - 1) / PS);
  const int tok_begin = first * PS;
  const int tok_end = min(end * PS, seq_len);  // keys of this split (and no further)

  PageTable pt;
  pt.row = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  pt.page_bytes = static_cast<int64_t>(PS) * Hkv * kCacheRowBytes;
  pt.n_pages = n_pages;

  if constexpr (kQuant && !kExact) {
    // The largest and the smallest nonzero |V scale| of the split's pages
    // (this kv head): only when they lie more than 2^6 apart can a sub-tile's
    // factor vs / vref fall below 2^-6, so only then is the exact form run.
    // Every wave finds the same answer, so the return is uniform over the
    // workgroup (and comes before any barrier).
    float vhi = 0.f, vlo = __builtin_inff();
    for (int slot = first + lane; slot < end; slot += 64) {
      const uint32_t pid = static_cast<uint32_t>(pt.row[slot]);
      const float a = __builtin_fabsf(p.v_scale[static_cast<int64_t>(pid) * Hkv + kvh]);
      vhi = __builtin_fmaxf(vhi, a);
      if (a > 0.f) vlo = __builtin_fminf(vlo, a);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      vhi = __builtin_fmaxf(vhi, shfl_xor(vhi, m));
      vlo = __builtin_fminf(vlo, shfl_xor(vlo, m));
    }
    if (__builtin_amdgcn_readfirstlane(vlo < vhi * kFarScale ? 1 : 0)) return false;
  }

  // ---- LDS (the kernel's): two K/V tile buffers (swizzled rows); for 8-bit
  // codes also the K and V scales of each buffer's 16-token sub-tiles,
  // sub_scale[buf][K, V][sub-tile]
  static_assert(2 * 2 * kBuf == prefill_tile_lds<D>(), "LDS size");
  char* smem = (char*)smem3;
  auto swz = [](int r, int cidx) __attribute__((always_inline)) {
    return r * kRowBytes + 16 * (cidx ^ ((2 * r) & (kChunks - 1)));
  };

  // this wave loads tile rows [kRowsPerWave * wave, +kRowsPerWave): lane l
  // writes LDS position lc of row lr of each wave load (its place is fixed by
  // the lane index), so it fetches the chunk that the swizzle puts there
  const int lr = lane / kChunks;
  const int lc = lane % kChunks;
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);
  typedef __attribute__((address_space(1))) const void* global_ptr;
  typedef __attribute__((address_space(3))) void* lds_ptr;

  // Issue this wave's loads of a tile; returns true when some of its rows lie
  // at or past tok_end (their V rows must then be zeroed once the loads land).
  // With kViaRegs the V chunks go to vr instead of LDS (store_v converts and
  // stores them).
  typedef u32x4 VRegs[kLoads];
  auto load_tile = [&](auto via_regs, int buf, int tile_tok0, VRegs& vr)
                       __attribute__((always_inline)) {
    constexpr bool kViaRegs = decltype(via_regs)::value;
    const int row0 = kRowsPerWave * wave;                    // first tile row of this wave
    const int tok = tile_tok0 + row0;
    if (tok < tok_end) {                                     // wave-uniform
      const int64_t base = pt.base(tok / PS);                // one page per wave
      const int in_page = tok % PS;
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int r = row0 + j * kRowsPerLoad + lr;          // tile row of this lane
        const int chunk = lc ^ ((2 * r) & (kChunks - 1));
        const uint32_t off = static_cast<uint32_t>(
            ((in_page + j * kRowsPerLoad + lr) * Hkv + kvh) * kRowBytes + 16 * chunk);
        const int lds_off = buf * 2 * kBuf + (row0 + j * kRowsPerLoad) * kRowBytes;
        __builtin_amdgcn_global_load_lds((global_ptr)(kbase + base + off),
                                         (lds_ptr)(smem3 + lds_off), 16, 0, 0);
        if constexpr (kViaRegs)
          vr[j] = *reinterpret_cast<const u32x4*>(vbase + base + off);
        else
          __builtin_amdgcn_global_load_lds((global_ptr)(vbase + base + off),
                                           (lds_ptr)(smem3 + lds_off + kBuf), 16, 0, 0);
      }
    }
    return tok + kRowsPerWave > tok_end;
  };
  // The V chunks of load_tile's register path, as f16, where the direct load
  // would have put them (lane l's 16 bytes at l * 16 of each wave load); rows
  // at or past tok_end are stored as zeros.
  auto store_v = [&](int buf, int tile_tok0, const VRegs& vr) __attribute__((always_inline)) {
    char* vb = smem + buf * 2 * kBuf + kBuf;
    if (__builtin_expect(tile_tok0 + kRowsPerWave * (wave + 1) <= tok_end, 1)) {  // wave-uniform
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        u32x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = bf16x2_to_f16x2(vr[j][i]);
        *reinterpret_cast<u32x4*>(vb + (kRowsPerWave * wave + j * kRowsPerLoad) * kRowBytes +
                                  16 * lane) = h;
      }
    } else if (tile_tok0 + kRowsPerWave * wave >= tok_end) {  // nothing was loaded
#pragma unroll
      for (int j = 0; j < kLoads; ++j)
        *reinterpret_cast<u32x4*>(vb + (kRowsPerWave * wave + j * kRowsPerLoad) * kRowBytes +
                                  16 * lane) = u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int r0 = kRowsPerWave * wave + j * kRowsPerLoad;
        const bool keep = tile_tok0 + r0 + lr < tok_end;
        u32x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = keep ? bf16x2_to_f16x2(vr[j][i]) : 0u;
        *reinterpret_cast<u32x4*>(vb + r0 * kRowBytes + 16 * lane) = h;
      }
    }
  };
  // Zero this wave's V rows at or past tok_end (past the sequence end, in a
  // page of the next split, or never loaded), after its loads have landed, so
  // no garbage meets a zero weight in the MFMA.  K rows there are harmless:
  // their scores are masked.
  auto zero_tail = [&](int buf, int tile_tok0) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads are in LDS
    char* vb = smem + buf * 2 * kBuf + kBuf;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int r = kRowsPerWave * wave + j * kRowsPerLoad + lr;
      if (tile_tok0 + r >= tok_end)
        *reinterpret_cast<u32x4*>(vb + r * kRowBytes + 16 * lc) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // 8-bit codes: this wave's rows of a tile into registers (K and V codes,
  // 16 per lane and load), with the K and V scales of their page; nothing is
  // read (and the scales are 0) when the rows lie at or past tok_end.
  typedef u32x4 QRegs[kLoadsQ];
  const int lrq = lane / kCodeChunks;
  const int lcq = lane % kCodeChunks;
  auto load_tile_q = [&](int tile_tok0, QRegs& kr, QRegs& vr, float& ks, float& vs)
                         __attribute__((always_inline)) {
    const int row0 = kRowsPerWave * wave;
    const int tok = tile_tok0 + row0;
    ks = 0.f;
    vs = 0.f;
    if (tok < tok_end) {  // wave-uniform; one page per wave
      const uint32_t pid = pt.id(tok / PS);
      const int64_t base = pt.base_of(pid);
      const int64_t si = static_cast<int64_t>(pid) * Hkv + kvh;
      ks = p.k_scale[si];
      vs = p.v_scale[si];
      const int in_page = tok % PS;
#pragma unroll
      for (int j = 0; j < kLoadsQ; ++j) {
        const uint32_t off = static_cast<uint32_t>(
            ((in_page + j * kRowsPerLoadQ + lrq) * Hkv + kvh) * D + 16 * lcq);
        kr[j] = *reinterpret_cast<const u32x4*>(kbase + base + off);
        vr[j] = *reinterpret_cast<const u32x4*>(vbase + base + off);
      }
    }
  };
  // ... and from registers into LDS buffer `buf`, decoded (K to T, V to f16);
  // rows at or past tok_end become zeros.  The wave that loaded a sub-tile's
  // first row stores that sub-tile's scales.
  auto store_tile_q = [&](int buf, int tile_tok0, const QRegs& kr, const QRegs& vr, float ks,
                          float vs) __attribute__((always_inline)) {
    if constexpr (kQuant) {
      char* kb = smem + buf * 2 * kBuf;
      char* vb = kb + kBuf;
      const int row0 = kRowsPerWave * wave;
#pragma unroll
      for (int j = 0; j < kLoadsQ; ++j) {
        const int r = row0 + j * kRowsPerLoadQ + lrq;
        const bool keep = tile_tok0 + r < tok_end;
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (keep) widen16<T, KV>(kr[j], lo, hi);
        *reinterpret_cast<u32x4*>(kb + swz(r, 2 * lcq)) = lo;
        *reinterpret_cast<u32x4*>(kb + swz(r, 2 * lcq + 1)) = hi;
        lo = u32x4{0u, 0u, 0u, 0u};
        hi = u32x4{0u, 0u, 0u, 0u};
        if (keep) widen16<f16_t, KV>(vr[j], lo, hi);
        *reinterpret_cast<u32x4*>(vb + swz(r, 2 * lcq)) = lo;
        *reinterpret_cast<u32x4*>(vb + swz(r, 2 * lcq + 1)) = hi;
      }
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < kRowsPerWave / 16; ++k) {
          sub_scale[(buf * 2 + 0) * kSub + row0 / 16 + k] = ks;
          sub_scale[(buf * 2 + 1) * kSub + row0 / 16 + k] = vs;
        }
      }
    }
  };
  float vref = 0.f, inv_vref = 0.f;  // 8-bit codes: largest |V scale| met so far

  // lsum[rb]: lane (g, li) sums row li's weights over its own tokens (the
  // four token groups are added at the end).  Summing on the vector ALUs
  // instead of with MFMAs against a block of ones saves 8 of 104 MFMAs per
  // tile (B=1, Sq=L=4096: 381 -> 371 us); it normalises by the float weights,
  // within 2^-12 of the rounded weights the P . V MFMAs use.
  float ref[RB], msub[RB];
  f32x4 o[RB][kNBlocks];
  float lsum[RB];

  // A 64-token tile in two 32-token halves.  Scores of row block rb, row li,
  // tokens tile_tok0 + 32 h + 16 q2 + 4 g + e.
  typedef float Scores[RB][2][4];
  // the S MFMAs of one half, both row blocks
  auto half_scores = [&](const char* kb, int h, Scores& x) __attribute__((always_inline)) {
    const int buf = (kb - smem) / (2 * kBuf);
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
      float ks = 1.f;
      if constexpr (kQuant) ks = sub_scale[(buf * 2 + 0) * kSub + 2 * h + q2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[rb][q2][e] = kQuant ? sacc[rb][e] * ks : sacc[rb][e];
    }
  };
  // keys a row may not see, or outside the split, become -inf (a select, so
  // stale rows of the LDS tile never reach the arithmetic)
  auto half_mask = [&](int tok0, Scores& x) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int lim = min(my_lim[rb], tok_end);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[rb][q2][e] = tok0 + 16 * q2 + 4 * g + e < lim ? x[rb][q2][e] : kNegInf;
    }
  };
  // weights 2^x of one half's exponents, 8 per row block (as f16, or as high
  // and low bf16 parts), their row sums, and O += P . V
  auto half_pv = [&](auto f16pv, lds_char* vb3, int h, Scores& x, const float* vfac,
                     bool add_sums = true) __attribute__((always_inline)) {
    constexpr bool kF16 = decltype(f16pv)::value;
    u32x4 phi[RB], plo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float pe[8], pw[8];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[4 * q2 + e] = fast_exp2(x[rb][q2][e]);  // x holds the exponent
          pw[4 * q2 + e] = kQuant ? pe[4 * q2 + e] * vfac[2 * h + q2] : pe[4 * q2 + e];
        }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (kF16) {
          hi[w] = f32x2_to_f16x2(pw[2 * w], pw[2 * w + 1]);
          lo[w] = 0u;
        } else {
          Mfma<T>::split2(pw[2 * w], pw[2 * w + 1], hi[w], lo[w]);
        }
      }
      phi[rb] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      plo[rb] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      if (add_sums)  // as a tree: a serial chain of dependent additions stalls the wave
        lsum[rb] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
    }
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
        if constexpr (kF16) {
          o[rb][nb] = Mfma<f16_t>::k32(phi[rb], vv, o[rb][nb]);
        } else {
          o[rb][nb] = Mfma<T>::k32(phi[rb], vv, o[rb][nb]);
          o[rb][nb] = Mfma<T>::k32(plo[rb], vv, o[rb][nb]);
        }
      }
    }
  };
  auto scale_o = [&](float f) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[rb][nb][e] *= f;
  };

  // One tile: both halves' score MFMAs; the mask (only on tiles that cross a
  // row's last key or the split's end); one lazy-rescale decision per row
  // block for the whole tile (the reference max is raised only when some
  // score of the tile exceeds it by more than kSlack); then the weights and
  // P . V of both halves as one straight-line block, so the compiler can
  // interleave the first half's MFMAs with the second half's exponentials
  // (iglp_opt(1) steers that interleave).  A wave's last, partial tile
  // computes its second half too, fully masked: fewer branches beat the
  // skipped MFMAs (B=1, Sq=L=4096: 455 -> 429 us).  Each wave issues in order,
  // so without such an interleave the matrix cores and the vector ALUs of a
  // SIMD were busy together only 8% of the time.
  auto compute_tile = [&](auto f16pv, int buf, int tile_tok0) __attribute__((always_inline)) {
    const char* kb = smem + buf * 2 * kBuf;
    lds_char* vb3 = smem3 + buf * 2 * kBuf + kBuf;
    Scores x0, x1;
    half_scores(kb, 0, x0);
    half_scores(kb, 1, x1);
    // wave-uniform and rare; the hint keeps the compiler from turning the mask
    // into selects that every tile would execute (64 vector instructions)
    if (__builtin_expect(tile_tok0 + kTile > wave_min_lim || tile_tok0 + kTile > tok_end, 0)) {
      half_mask(tile_tok0, x0);
      half_mask(tile_tok0 + 32, x1);
    }
    // scores become exponents y = x c - msub in place (an FMA's result is a
    // canonical float, so the max below needs no quieting of its inputs and
    // runs as v_max3); the tile raises the reference when some y exceeds
    // kSlack, or when the reference is still -inf and some key is visible
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float yv[16];
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x0[rb][q2][e] = __builtin_fmaf(x0[rb][q2][e], c, -msub[rb]);
          x1[rb][q2][e] = __builtin_fmaf(x1[rb][q2][e], c, -msub[rb]);
          yv[4 * q2 + e] = x0[rb][q2][e];
          yv[8 + 4 * q2 + e] = x1[rb][q2][e];
        }
      float tmax = __builtin_fmaxf(__builtin_fmaxf(yv[0], yv[1]), yv[2]);
#pragma unroll
      for (int k = 3; k + 1 < 16; k += 2)
        tmax = __builtin_fmaxf(__builtin_fmaxf(tmax, yv[k]), yv[k + 1]);
      tmax = __builtin_fmaxf(tmax, yv[15]);
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
        for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[rb][q2][e] += shift;
            x1[rb][q2][e] += shift;
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
    float vfac[kSub];
#pragma unroll
    for (int k = 0; k < kSub; ++k) vfac[k] = 1.f;
    if constexpr (kQuant) {
      // the tile's V scales relative to the largest |V scale| so far; when a
      // larger one arrives, the accumulators move to the new reference
      float vs[kSub], vmax = vref;
#pragma unroll
      for (int k = 0; k < kSub; ++k) {
        vs[k] = sub_scale[(buf * 2 + 1) * kSub + k];
        vmax = __builtin_fmaxf(vmax, __builtin_fabsf(vs[k]));
      }
      if (vmax > vref) {  // wave-uniform
        const float ratio = vref / vmax;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[rb][nb][e] *= ratio;
        vref = vmax;
        inv_vref = 1.f / vmax;
      }
      bool far[kSub], any_far = false;
#pragma unroll
      for (int k = 0; k < kSub; ++k) {
        vfac[k] = vs[k] * inv_vref;
        far[k] = kExact && vfac[k] != 0.f && __builtin_fabsf(vfac[k]) < kFarScale;
        any_far |= far[k];
      }
      if (kExact && any_far) {  // wave-uniform (the scales are)
        // the near sub-tiles (and every row sum) as usual, the far ones zeroed;
        // then each far sub-tile alone, its exponents computed again from LDS:
        // its factor f = m 2^E with |m| in [1, 2) (E at least -60, below which
        // its share is negligible); O is taken to 2^-E times itself, gets
        // P . V with weights times m, and comes back -- powers of two, exact
        // in f32 at these magnitudes
        float vz[kSub];
#pragma unroll
        for (int k = 0; k < kSub; ++k) vz[k] = far[k] ? 0.f : vfac[k];
        half_pv(f16pv, vb3, 0, x0, vz);
        half_pv(f16pv, vb3, 1, x1, vz);
#pragma unroll
        for (int k = 0; k < kSub; ++k) {
          if (!far[k]) continue;
          Scores xr;
          half_scores(kb, k / 2, xr);
          half_mask(tile_tok0 + 32 * (k / 2), xr);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
              for (int e = 0; e < 4; ++e) xr[rb][q2][e] = __builtin_fmaf(xr[rb][q2][e], c, -msub[rb]);
          const int ex = max(__builtin_amdgcn_frexp_expf(vfac[k]) - 1, -60);
          float vk[kSub];
#pragma unroll
          for (int k2 = 0; k2 < kSub; ++k2) vk[k2] = k2 == k ? __builtin_ldexpf(vfac[k], -ex) : 0.f;
          scale_o(__builtin_ldexpf(1.f, -ex));
          half_pv(f16pv, vb3, k / 2, xr, vk, false);
          scale_o(__builtin_ldexpf(1.f, ex));
        }
        return;
      }
    }
    half_pv(f16pv, vb3, 0, x0, vfac);
    half_pv(f16pv, vb3, 1, x1, vfac);
    __builtin_amdgcn_iglp_opt(1);
  };

  // ---- tile loop (every wave of the workgroup runs every tile: the LDS
  // buffers are shared, so the barriers must be reached by all of them).
  // f16pv: P . V in f16 (V converted on the way in for bf16 caches), else
  // with high and low bf16 weights.
  const int n_tiles = tok_end > tok_begin ? (tok_end - tok_begin + kTile - 1) / kTile : 0;
  auto run = [&](auto f16pv) __attribute__((always_inline)) {
    constexpr bool kViaRegs = decltype(f16pv)::value && kConvertV;
    const std::integral_constant<bool, kViaRegs> via_regs;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ref[rb] = kNegInf;
      msub[rb] = 0.f;
      lsum[rb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    VRegs vr;
    if (n_tiles > 0) {
      const bool tail = load_tile(via_regs, 0, tok_begin, vr);
      if constexpr (kViaRegs)
        store_v(0, tok_begin, vr);
      else if (tail)
        zero_tail(0, tok_begin);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int tok0 = tok_begin + t * kTile;
      const bool more = t + 1 < n_tiles;
      const bool tail = more && load_tile(via_regs, (t + 1) & 1, tok0 + kTile, vr);
      // a wave whose rows see none of this tile skips the arithmetic
      if (tok0 < wave_max_lim) compute_tile(f16pv, t & 1, tok0);
      if constexpr (kViaRegs) {
        if (more) store_v((t + 1) & 1, tok0 + kTile, vr);
      } else if (tail) {
        zero_tail((t + 1) & 1, tok0 + kTile);
      }
      __syncthreads();  // the next tile has landed (the compiler waits for it) and this one is done
    }
  };
  // 8-bit codes: the tile loop (with the per-sub-tile test for V factors far
  // below the running reference in the exact form)
  auto run_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      ref[rb] = kNegInf;
      msub[rb] = 0.f;
      lsum[rb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb) o[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    QRegs kr, vr;
    float ks = 0.f, vs = 0.f;
    if (n_tiles > 0) {
      load_tile_q(tok_begin, kr, vr, ks, vs);
      store_tile_q(0, tok_begin, kr, vr, ks, vs);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int tok0 = tok_begin + t * kTile;
      const bool more = t + 1 < n_tiles;
      if (more) load_tile_q(tok0 + kTile, kr, vr, ks, vs);
      if (tok0 < wave_max_lim) compute_tile(std::true_type(), t & 1, tok0);
      if (more) store_tile_q((t + 1) & 1, tok0 + kTile, kr, vr, ks, vs);
      __syncthreads();  // the next tile is in LDS and this one is done
    }
  };
  if constexpr (kQuant) {
    run_q();
  } else {
    run(std::true_type());
  }
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
    const bool bad = __builtin_amdgcn_ballot_w64(z != z) != 0;  // all lanes take part
    if (lane == 0) flags[wave] = bad;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) redo |= flags[w];
    if (redo) {  // workgroup-uniform, rare
      __syncthreads();  // every wave has read the flags before the loads reuse the buffers
      run(std::false_type());
    }
  }

  // ---- finish: normalize and write; row 4 g + e of the O layout takes its
  // sum and its reference from lane 4 g + e
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    lsum[rb] += shfl_xor(lsum[rb], 16);
    lsum[rb] += shfl_xor(lsum[rb], 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int src = (4 * g + e) << 2;
      const float le = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, lsum[rb])));
      const float re = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, ref[rb])));
      const int r_lin = wave_first + 16 * rb + 4 * g + e;
      if (r_lin >= p.rows_per_kvh) continue;
      const int i = div_by(r_lin, p.group_div);
      const int rid = (b * Sq + i) * Hq + kvh * G + (r_lin - i * G);
      const bool any = le > 0.f;  // no valid key: (0, -inf) instead of 0/0
      const float lse = any ? (re + log2f(le)) * kLn2 : kNegInf;
      // one division per row, a multiply per element (within 1.5 ulp of
      // dividing each element; the division sequence is ~10 instructions)
      const float inv = any ? (kQuant ? vref : 1.f) / le : 0.f;
      if (S == 1) {
        T* dst = static_cast<T*>(p.out) + static_cast<int64_t>(rid) * D;
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb) dst[16 * nb + li] = from_float<T>(o[rb][nb][e] * inv);
        if (li == 0 && p.lse != nullptr) p.lse[rid] = lse;
      } else {
        const int64_t prow = static_cast<int64_t>(rid) * S + split;
        float* dst = p.part_out + prow * D;
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb) dst[16 * nb + li] = o[rb][nb][e] * inv;
        if (li == 0) p.part_lse[prow] = lse;
      }
    }
  }
  return true;
}

// The exact form as a separate function: the compiler allocates its registers
// on their own, so its extra paths cost the common loop nothing.
// It reads the parameters through a pointer to the kernel's argument segment
// (a reference to the argument itself would make the kernel copy it to
// scratch memory and read it from there in the common loop too).
template <typename T, int D, int PS, int NW, int RB, typename KV>
__device__ __attribute__((noinline)) void prefill_body_exact(const AttnParams* p,
                                                             lds_char* smem3,
                                                             lds_float* sub_scale) {
  prefill_body<T, D, PS, NW, RB, KV, true>(*p, smem3, sub_scale);
}

// At D = 64 three workgroups of 4 waves share a compute unit (at most 170
// VGPRs per lane), at D = 128 two.
template <typename T, int D, int PS, int NW, int RB, typename KV = KvSame>
__global__ __launch_bounds__(NW * 64, (D == 64 ? 12 : 8) / NW) void attn_prefill_kernel(
    const AttnParams p) {
  __shared__ __attribute__((aligned(16))) char smem[prefill_tile_lds<D>()];
  __shared__ float sub_scale[KvTraits<KV>::quant ? 2 * 2 * 4 : 1];
  lds_char* smem3 = (lds_char*)(smem);
  lds_float* sub3 = (lds_float*)(sub_scale);
  if (!prefill_body<T, D, PS, NW, RB, KV, false>(p, smem3, sub3)) {
    if constexpr (KvTraits<KV>::quant) {
      // the kernel's only argument, at the start of its argument segment
      const AttnParams* args =
          (const AttnParams*)(const void*)__builtin_amdgcn_kernarg_segment_ptr();
      prefill_body_exact<T, D, PS, NW, RB, KV>(args, smem3, sub3);
    }
  }
}

}  // namespace pa
