/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention library (libpa.so).
 *
 * The library computes softmax(scale * Q K^T) V over a K/V cache that is
 * scattered in fixed-size pages and addressed through a per-sequence block
 * table, with grouped-query heads, ragged lengths, causal masking and
 * split-KV partials merged by a log-sum-exp combine.
 *
 * Sources of the operation (page title, section):
 *  - paged K/V as a lazy view over page addresses, dereferenced at tile
 *    lowering: rocMLIR "Paged Attention: migraphx & highlevel pipeline
 *    changes", Technical Details (rock.deref, rock.attention keyAddresses /
 *    valueAddresses);
 *  - the result is attention over the logical-order cache: rocMLIR "Paged
 *    Attention: rocmlir-gen changes", Technical Details, CPU Validation;
 *  - pages holding every kv head, ragged lengths, an unmapped id in the
 *    table's tail, caches past 2 GiB: rocm-libraries "one K/V resource per
 *    page on the gfx942 2D i64 path", Motivation and Coverage;
 *  - split ranges by ceiling division, empty splits, the -inf - (-inf) and
 *    0/0 guards, the f32 combine: rocMLIR "Fix split-kv attention masking and
 *    sweep RMS", Technical Details.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE memory owned by the caller.  The library
 *    allocates nothing and keeps no state between calls; it is thread-safe.
 *    (pa_decode_noalloc is the exception: it keeps its split partials in one
 *    static device array per GPU, shared by its calls on that GPU.)
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without waiting for it.
 *  - Every argument check runs on the host before anything is launched.  A
 *    failed check returns a negative pa_status and writes nothing.  A launch
 *    failure returns PA_EHIP.  No C++ exception crosses this interface.
 *  - q, k_cache and v_cache must be 16-byte aligned, block_table and
 *    seq_lens 4-byte aligned (else PA_EINVAL).
 *  - Tensors are dense and row-major unless a stride is given:
 *      q            [B, Sq, Hq, D]                 dtype
 *      k_cache      [num_pages, page_size, Hkv, D]  dtype (or kv_dtype codes)
 *      v_cache      [num_pages, page_size, Hkv, Dv] dtype (or kv_dtype codes)
 *      block_table  [B, W] int32, row stride block_table_stride (>= W)
 *      seq_lens     [B] int32
 *      out          [B, Sq, Hq, Dv]                dtype
 *      lse          [B, Sq, Hq] float32 natural-log LSE (may be NULL)
 *    Query head h reads kv head h / (Hq / Hkv).
 *  - Device-side preconditions (the caller's contract, not checked):
 *      0 <= seq_lens[b] <= W * page_size, and
 *      0 <= block_table[b][s] < num_pages for s < ceil(seq_lens[b] / page_size).
 *    Slots at or past ceil(seq_lens[b] / page_size) may hold anything (e.g.
 *    an unmapped id such as 0x7FFFFFFF): no page is ever read through them
 *    (a kernel may read such a slot's value ahead of the sequence length, but
 *    only inside the row's W slots, and then discards it).  Token slots of a
 *    last page past seq_lens[b] are never used, even if they hold NaN.
 *  - A row with no valid key (seq_lens[b] == 0, or a causal row placed before
 *    the first key) gets out = 0 and lse = -inf.
 *  - Page bases are formed as zero-extended page id times page bytes in
 *    64-bit arithmetic, so caches larger than 2 GiB (and 4 GiB) are read
 *    correctly.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k_cache, v_cache and out.  PA_I8 and PA_FP8_E4M3 name
 * 8-bit cache codes and are valid only as pa_shape.kv_dtype. */
typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_I8 = 3,       /* two's-complement int8 code                                  */
  PA_FP8_E4M3 = 4  /* OCP fp8 E4M3: exponent bias 7, subnormals, no infinity,
                      S.1111.111 is NaN                                          */
} pa_dtype;

/* Return codes. */
typedef enum pa_status {
  PA_OK = 0,
  PA_EINVAL = -1,       /* a null pointer, a non-positive size, Hq % Hkv != 0,
                           stride < W, a size overflow, a non-finite scale,
                           num_splits out of range, seq_q != 1 in pa_decode   */
  PA_EUNSUPPORTED = -2, /* valid but outside the compiled envelope            */
  PA_EWORKSPACE = -3,   /* workspace NULL or smaller than pa_workspace_bytes  */
  PA_EHIP = -4,         /* the HIP runtime refused a launch                   */
  PA_ESCRATCH = -5      /* pa_decode_noalloc: the split partials need more than
                           PA_NOALLOC_SCRATCH_BYTES                            */
} pa_status;

/* Problem shape shared by pa_decode, pa_prefill and pa_workspace_bytes. */
typedef struct pa_shape {
  int32_t dtype;              /* a pa_dtype                                     */
  int32_t batch;              /* B                                              */
  int32_t seq_q;              /* Sq: query rows per sequence (1 for decode)     */
  int32_t num_q_heads;        /* Hq                                             */
  int32_t num_kv_heads;       /* Hkv, divides Hq                                */
  int32_t head_dim_qk;        /* D                                              */
  int32_t head_dim_v;         /* Dv                                             */
  int32_t page_size;          /* tokens per page                                */
  int64_t num_pages;          /* physical pages per cache tensor (validation)   */
  int32_t max_pages_per_seq;  /* W: block-table width                           */
  int64_t block_table_stride; /* elements between block-table rows, >= W        */
  int32_t kv_dtype;           /* 0: k_cache and v_cache hold `dtype`; PA_I8 or
                                 PA_FP8_E4M3: they hold 8-bit codes, with the
                                 scales passed in pa_options                    */
} pa_shape;

/*
 * Supported envelope of the compiled kernels (else PA_EUNSUPPORTED):
 *   dtype F32, F16 or BF16; D == Dv in {32, 64, 128}; page_size in {16, 32};
 *   any group size Hq / Hkv >= 1; B <= 65535 and Hkv <= 65535.
 *   8-bit caches (kv_dtype PA_I8 or PA_FP8_E4M3): dtype F16 or BF16 and
 *   D == Dv in {64, 128}.
 *
 * Accuracy: against exact attention (8-bit codes times their scales taken as
 * the exact cache values), each output element is within 2e-3 + 2^-8 |x| for
 * F16/BF16 (the bound of rocm-libraries "one K/V resource per page on the
 * gfx942 2D i64 path", Coverage) and 1e-5 + 1e-5 |x| for F32; the float32
 * LSE and split partials within 1e-5 + 1e-5 |x| (partials of 16-bit problems
 * within the 16-bit bound).  Scores and the softmax run in float32; 16-bit
 * problems multiply on the matrix cores with the softmax weights kept to at
 * least 11 significant bits, for 8-bit caches whatever the spread of their
 * K and V scales.  Results are deterministic: the same inputs give the same
 * bits on every call.
 */

/*
 * pa_decode -- one new query token per sequence (Sq == 1) over its paged
 * cache: grouped-query decode with ragged lengths.  The split-KV form of the
 * decode step follows rocMLIR "Fix split-kv attention masking and sweep RMS"
 * (Technical Details) and the page-table loading follows rocm-libraries "one
 * K/V resource per page on the gfx942 2D i64 path" (Technical Details,
 * Changes): each page id is read once and turned into a 64-bit page base.
 *
 *  shape       problem shape; shape->seq_q must be 1.
 *  q, k_cache, v_cache, block_table, seq_lens, out: as in the table above.
 *  scale       multiplies q . k before the softmax; must be finite.
 *  causal      accepted for a uniform signature; with one query row per
 *              sequence, bottom-right causal masking keeps every key.
 *  num_splits  0 = pick automatically (see pa_resolve_num_splits); else the
 *              number S >= 1 of split-KV partitions of each sequence's pages.
 *              Split s covers pages [s*P, min((s+1)*P, n)) with
 *              n = ceil(seq_lens[b] / page_size) and P = ceil(n / S); splits
 *              past n are empty and contribute nothing.
 *  lse         optional [B, 1, Hq] float32 output.
 *  workspace   device scratch of at least pa_workspace_bytes(shape, S) bytes
 *              (NULL allowed when that is 0).  When S > 1 the partials are
 *              left in it: part_out [B*Sq*Hq, S, Dv] float32 at offset 0, then
 *              part_lse [B*Sq*Hq, S] float32 at the next 256-byte boundary
 *              (per split: output normalised by its own softmax sum, LSE in
 *              natural log; an empty split holds 0 and -inf).
 *  stream      hipStream_t or NULL.
 */
int pa_decode(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* seq_lens, float scale, int causal,
              int num_splits, void* out, float* lse, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * pa_prefill -- Sq >= 1 query rows per sequence, the last Sq positions of a
 * sequence of seq_lens[b] keys.  With causal != 0 the mask is bottom-right
 * aligned: row i sits at key position seq_lens[b] - Sq + i and sees keys up
 * to and including it.  Per-row validity follows rocMLIR "Fix split-kv
 * attention masking and sweep RMS" (Technical Details, host reference:
 * causal valid-split masking); the paged prefill shape follows rocMLIR
 * "Paged Attention: rocmlir-gen changes" (Example Usage).  Arguments and
 * workspace as for pa_decode; lse is [B, Sq, Hq].
 */
int pa_prefill(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens, float scale, int causal,
               int num_splits, void* out, float* lse, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * Optional inputs of pa_decode_ex and pa_prefill_ex.  A NULL pointer to this
 * struct, or one whose pointers are all NULL, gives exactly pa_decode /
 * pa_prefill (which therefore reject 8-bit caches).  The arrays are device
 * memory owned by the caller, 4-byte aligned (else PA_EINVAL); page_check
 * must not overlap any other argument.
 *
 *  prefix_offset  [B] int32 or NULL.  When given, row i of sequence b sits at
 *                 key position prefix_offset[b] + i and sees the keys
 *                 j <= prefix_offset[b] + i with j < seq_lens[b]
 *                 (prefix-causal masking, which is causal whatever `causal`
 *                 says).  Any int32 value is allowed: a row placed before key
 *                 0 sees nothing (out = 0, lse = -inf), a row at or past the
 *                 last key sees every key.  prefix_offset[b] = seq_lens[b] - Sq
 *                 is bottom-right causal masking.  Source: rocMLIR "Fix
 *                 split-kv attention masking and sweep RMS", Technical
 *                 Details (host reference: each row's effective key length
 *                 includes the prefix offset; prefix-causal counts as causal).
 *  page_check     [B + 1] int32 or NULL.  When given, a check pass (two small
 *                 kernels on `stream`) runs before the attention: sequence b
 *                 passes when 0 <= seq_lens[b] <= W * page_size and every id
 *                 in its slots [0, ceil(seq_lens[b] / page_size)) lies in
 *                 [0, num_pages).  A failing sequence is attended as empty
 *                 (its rows give out = 0 and lse = -inf, its splits 0 and
 *                 -inf) and none of its ids is ever dereferenced.  Afterwards
 *                 page_check[1 + b] holds the length attended (seq_lens[b],
 *                 or 0 for a failing sequence) and page_check[0] the smallest
 *                 failing b, or -1 when every sequence passes.  The device-side
 *                 preconditions above then reduce to readable seq_lens and
 *                 block-table slots [0, W) of each row.  Source: rocm-libraries
 *                 "one K/V resource per page on the gfx942 2D i64 path", Not
 *                 in this PR (page ids are bounded by slot index but not
 *                 checked against the cache's block count, which needs that
 *                 count as a kernel argument) and the review's LOW findings.
 *  k_scale,       [num_pages, Hkv] float32 each, required exactly when
 *  v_scale        shape->kv_dtype is PA_I8 or PA_FP8_E4M3 (else PA_EINVAL).
 *                 Element [p, t, h, d] of the K cache is
 *                 k_scale[p * Hkv + h] * value(code), value() decoding the
 *                 code as int8 or as OCP fp8 E4M3; likewise V.  The scales of
 *                 every page a sequence reads must be finite.  Queries, outputs
 *                 and arithmetic stay as for 16-bit caches: codes are decoded
 *                 exactly to the query type and the scales are applied in
 *                 float32 (to the scores, and to each tile's weighted V sum).
 *                 Sources: int8 paged attention, rocMLIR "Paged Attention:
 *                 rocmlir-gen changes" (file list, int8 e2e test); i8 split-KV
 *                 attention, rocMLIR "Fix split-kv attention masking and sweep
 *                 RMS" (Motivation); fp8 K/V loaders, rocm-libraries "one K/V
 *                 resource per page on the gfx942 2D i64 path" (review).  The
 *                 per-(page, kv head) scale and the OCP variant are this
 *                 library's choices.
 */
typedef struct pa_options {
  const int32_t* prefix_offset;
  int32_t* page_check;
  const float* k_scale;
  const float* v_scale;
} pa_options;

/* pa_decode with the optional inputs above; same arguments and results. */
int pa_decode_ex(const pa_shape* shape, const pa_options* options, const void* q,
                 const void* k_cache, const void* v_cache, const int32_t* block_table,
                 const int32_t* seq_lens, float scale, int causal, int num_splits, void* out,
                 float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* pa_prefill with the optional inputs above; same arguments and results.  With
 * prefix_offset, sequences may hold fewer than Sq real query rows (chunked or
 * variable-length prefill padded to Sq): rows past a sequence's own queries
 * are computed like the others and may be ignored by the caller. */
int pa_prefill_ex(const pa_shape* shape, const pa_options* options, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* seq_lens, float scale, int causal, int num_splits, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_combine -- log-sum-exp merge of split-KV partials, in float32 for every
 * storage type, cast to `dtype` once at the end (rocMLIR "Fix split-kv
 * attention masking and sweep RMS", Technical Details, host reference: f32
 * combine for narrow floats).  Per row: M = max_s lse_s; if M == -inf the
 * row is empty and gets out = 0, lse = -inf; else w_s = exp(lse_s - M),
 * out = sum_s w_s * o_s / sum_s w_s, lse = M + ln(sum_s w_s).
 *
 *  dtype       pa_dtype of out.
 *  rows        number of rows (> 0); num_splits S (> 0); head_dim_v Dv (> 0).
 *  part_out    [rows, S, Dv] float32.   part_lse [rows, S] float32.
 *  out         [rows, Dv] dtype.        lse      [rows] float32 or NULL.
 *  stream      hipStream_t (NULL = default stream); the call is asynchronous.
 *
 * Pointers are device memory owned by the caller, each aligned to its element
 * size (16-byte aligned partials with S <= 256 and Dv a multiple of 4, at
 * most 1024, take the faster one-workgroup-per-row kernel).  Returns PA_OK,
 * PA_EINVAL (bad dtype, a size <= 0, a NULL or misaligned pointer; nothing is
 * launched) or PA_EHIP (launch failure).
 */
int pa_combine(int32_t dtype, int32_t rows, int32_t num_splits, int32_t head_dim_v,
               const float* part_out, const float* part_lse, void* out, float* lse,
               void* stream);

/* Workspace bytes pa_decode / pa_prefill need for `num_splits` (0 = auto);
 * 0 when the resolved split count is 1 or the shape is invalid. */
size_t pa_workspace_bytes(const pa_shape* shape, int num_splits);

/* The split count a call with `num_splits` uses: `num_splits` itself when it
 * is > 0, else the automatic choice, which depends on the shape only (never
 * on device data), so it is known on the host without a synchronisation.
 * Negative pa_status for an invalid shape or num_splits. */
int pa_resolve_num_splits(const pa_shape* shape, int num_splits);

/*
 * pa_decode_noalloc -- pa_decode_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  It takes no workspace.  The split-KV partials (the only
 * scratch the path uses, S > 1) go to a static device array of
 * PA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * first call on that GPU until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine); on its first call on
 * a device it looks up that device's copy of the array.
 *
 *  options     as for pa_decode_ex, or NULL (then it is pa_decode).
 *  All other arguments, results and checks as for pa_decode_ex.  The device
 *  is the current one, which must be the device of `stream` and the tensors.
 *
 * Returns PA_ESCRATCH, before anything is launched, when the resolved split
 * count needs more partials than the array holds (pa_workspace_bytes(shape,
 * num_splits) > PA_NOALLOC_SCRATCH_BYTES; e.g. B * Hq * S * (Dv + 1) * 4
 * bytes at Sq = 1, so B = 256, Hq = 32, Dv = 128 allows S <= 3).  Calls on
 * one GPU share its array: calls that overlap in time on that GPU (on
 * different streams, or from several threads without ordering) race and may
 * return wrong results.  Calls ordered on one stream are safe; each call
 * writes every partial it later reads, so nothing has to be cleared between
 * calls.  The partials are not exposed.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int pa_decode_noalloc(const pa_shape* shape, const pa_options* options, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, float scale, int causal, int num_splits,
                      void* out, float* lse, void* stream);

/* Kernel families a call can take (pa_plan_info.kernel). */
typedef enum pa_kernel {
  PA_KERNEL_VALU = 0,             /* vector-ALU kernel (f32 caches)                     */
  PA_KERNEL_MFMA = 1,             /* matrix-core kernel, one 16-row block per wave      */
  PA_KERNEL_MFMA_TWO_BLOCKS = 2,  /* matrix-core kernel, two 16-row blocks per wave
                                     sharing each staged K/V tile                       */
  PA_KERNEL_SHARED_TILE = 3,      /* shared-tile kernel, one team of waves              */
  PA_KERNEL_SHARED_TILE_TEAMS = 4 /* shared-tile kernel, two teams in opposite phases   */
} pa_kernel;

/* Launch plan of a pa_decode / pa_prefill call (pa_describe_plan). */
typedef struct pa_plan_info {
  int32_t kernel;              /* a pa_kernel                                         */
  int32_t num_splits;          /* S the call uses (as pa_resolve_num_splits)          */
  int32_t rows_per_workgroup;  /* query rows of one kv head per workgroup             */
  int32_t row_groups;          /* ceil(Sq * Hq / Hkv / rows_per_workgroup)            */
  int32_t waves;               /* waves (64 lanes each) per workgroup                 */
  int32_t kv_heads_per_workgroup;
} pa_plan_info;

/* The plan a call with this shape and `num_splits` (0 = auto) takes, written
 * to *info.  Host-only: it depends on the shape alone, launches nothing and
 * touches no device memory.  Returns PA_OK, or a negative pa_status for an
 * invalid shape or num_splits, or a NULL info (then *info is not written).
 * Shape checks are those of pa_prefill (any seq_q). */
int pa_describe_plan(const pa_shape* shape, int num_splits, pa_plan_info* info);

/* Static, NUL-terminated description of a status code. */
const char* pa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
