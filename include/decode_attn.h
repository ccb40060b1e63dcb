/*
 * decode_attn.h - C ABI of the MI355X (gfx950) decode-phase paged attention library.
 *
 * What is computed. In the decode phase each sequence adds one query token that
 * attends over the keys and values cached for its earlier tokens (page "Eine
 * LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen", section 1.1). The cache
 * lives in fixed-size pages found through a per-sequence block table (swiftLLM README,
 * feature list: PagedAttention). Several query heads may share one KV head (xLLM README,
 * optimisation list: GQA). The cache is stored as fp16 or bf16 (the precisions the xLLM
 * README's quantisation list names), as per-row INT8 (same list), or as FP8 E4M3 with
 * per-row scales (FP8 cache quantisation is among the next steps in section 4 of the
 * C++/CUDA engine page). For sequence b and query head h, with G = n_q_heads / n_kv_heads
 * and g = h / G:
 *
 *     s_t = scale * <q[b,h,:], K_b[g,t,:]>        for t in [0, L_b)
 *     out[b,h,:] = sum_t softmax(s)_t * V_b[g,t,:]
 *     lse[b,h]   = ln sum_t exp(s_t)              (natural log; -inf when L_b = 0)
 *
 * The library reaches this with a single-pass online-normaliser softmax (xLLM README,
 * SoftMax operator) and cuts long caches into pieces whose partial (out, lse) are merged
 * by their log-sum-exp weights (swiftLLM feature list: PagedAttention v2 /
 * Flash-Decoding). Three plans cut the batch:
 *  - segment mode: a fixed grid of persistent workgroups, each taking whole
 *    (sequence, KV head) segments, longest sequences first (for batches of at most 256
 *    sequences; in index order beyond), its four wavefronts sharing the pages of each
 *    segment; no partial results;
 *  - stream mode: the (sequence, KV head, page) units of the whole batch are dealt out in
 *    equal contiguous runs to a fixed grid of persistent workgroups, one run per
 *    wavefront, so every wave streams the same number of pages whatever the length mix;
 *    segments cut between wavefronts are merged by a second kernel;
 *  - split mode: one workgroup per (page partition, KV head, sequence) with at least two
 *    partitions, merged by a second kernel; for a few very long caches.
 * Each only changes the order of rounding; out is the plain softmax result above.
 *
 * Precision: scores, the running max and sum, and all accumulators are fp32. With G >= 4
 * query heads per KV head both products of a page run on the matrix cores: the scores as
 * exact fp16 products (codes widened exactly; bf16 products for a BF16 cache) summed in
 * fp32, the weighted sum of V with each softmax weight rounded to fp16 (relative error at
 * most 2^-11), or for a BF16 cache split into two bf16 parts (at most 2^-16); the
 * normaliser adds the unrounded fp32 weights. With G <= 2 the weights stay fp32; there an
 * INT8 code enters as the exact fp16 value 1152 + x, and 1152 times the sum of the query
 * (per load) or of the weights (per segment) is taken off, which adds fp32 rounding of
 * about 2^-24 * 1152 * sqrt(L_b) of a value's row scale.
 *
 * Memory layout (all row-major and contiguous; all tensor pointers are DEVICE pointers
 * owned by the caller, for example torch tensors; the library never frees them):
 *
 *     q            fp16  [batch, n_q_heads, head_dim] (bf16 for a BF16 cache), 16-byte
 *                  aligned
 *     k_pages      fp16, bf16, int8 or FP8 E4M3 codes  [num_pages, n_kv_heads, block_size,
 *                  head_dim], 16-byte aligned
 *     v_pages      same type and shape as k_pages
 *     k_scale      fp32  [num_pages, n_kv_heads, block_size]   (INT8 and FP8 only, else
 *     v_scale      fp32  [num_pages, n_kv_heads, block_size]    NULL; 8-byte aligned)
 *     block_table  int32 [batch, max_blocks_per_seq]: entry (b, j) is the physical page
 *                  holding tokens j*block_size .. j*block_size+block_size-1 of sequence b.
 *                  Only entries j < ceil(L_b / block_size) are read; the rest may hold
 *                  anything (for example -1).
 *     seq_lens     int32 [batch]: L_b, with 0 <= L_b <= max_blocks_per_seq * block_size.
 *     out          fp32  [batch, n_q_heads, head_dim], 16-byte aligned; must not overlap
 *                  any input.
 *     lse_out      fp32  [batch, n_q_heads] or NULL.
 *
 * A (page, KV head) tile is block_size * head_dim contiguous elements (4 KiB in fp16 at
 * 16 x 128), so one page of one head is read with fully coalesced 16-byte loads. An INT8
 * row (token, KV head) has value int8 * scale with one fp32 scale per row, and an FP8 row
 * value e4m3(code) * scale the same way. BF16 is the upper half of an IEEE binary32. FP8
 * is E4M3 as the OCP 8-bit floating-point specification defines it: bias 7, subnormals at
 * exponent field 0, no infinities, S.1111.111 is NaN, largest magnitude 448. The slots of
 * a page past L_b are never used, whatever they hold (NaN included).
 *
 * Supported sizes: head_dim 128, block_size 16, G = n_q_heads / n_kv_heads in
 * {1, 2, 4, 8}, batch * max_blocks_per_seq * n_kv_heads < 2^31 and
 * num_pages * n_kv_heads < 2^32; stream mode also needs batch <= 4096 (the library's own
 * plan never picks it beyond that). Other values return
 * DECODE_ATTN_ERR_UNSUPPORTED.
 *
 * Calls are asynchronous: they validate arguments on the host, enqueue kernels on
 * `stream` and return. Nothing is synchronised and no device value is read back; the
 * caller's stream orders the work. The same inputs under the same plan give a
 * bitwise-identical out (no atomics; fixed reduction order).
 *
 * Bad device-side values never fault: a sequence whose L_b lies outside
 * [0, max_blocks_per_seq * block_size], or whose table holds a page id outside
 * [0, num_pages) among the entries it reads, gets NaN in its outputs instead, and no
 * memory is read through the bad entry.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point that returns int. */
typedef enum {
  DECODE_ATTN_OK = 0,
  DECODE_ATTN_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, Hq % Hkv != 0,
                                           scales given for FP16 or missing for INT8 */
  DECODE_ATTN_ERR_UNSUPPORTED = 2,      /* a size this build has no kernel for */
  DECODE_ATTN_ERR_WORKSPACE = 3,        /* workspace missing or too small */
  DECODE_ATTN_ERR_HIP = 4,              /* a HIP call or kernel launch failed */
  DECODE_ATTN_ERR_SCRATCH_LIMIT = 5     /* decode_attn_noalloc: the plan needs more workspace
                                           than DECODE_ATTN_STATIC_SCRATCH_BYTES */
} decode_attn_status;

/* Size of the device-resident workspace decode_attn_noalloc uses: 32 MiB per device. */
#define DECODE_ATTN_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* Storage type of k_pages / v_pages. */
typedef enum {
  DECODE_ATTN_KV_FP16 = 0,
  DECODE_ATTN_KV_INT8 = 1, /* per-row INT8 with fp32 row scales (xLLM README, quantisation) */
  DECODE_ATTN_KV_BF16 = 2, /* bf16 K/V and bf16 q (xLLM README, quantisation: FP16, BF16) */
  DECODE_ATTN_KV_FP8 = 3   /* OCP E4M3 codes with fp32 row scales; q fp16 (C++/CUDA engine
                              page, section 4: FP8 cache quantisation) */
} decode_attn_kv_dtype;

/* How a call cuts the batch into work (see the top of this file). */
typedef enum {
  DECODE_ATTN_MODE_STREAM = 0,
  DECODE_ATTN_MODE_SPLIT = 1,
  DECODE_ATTN_MODE_SEGMENT = 2
} decode_attn_mode;

/* A plan as decode_attn_plan reports it. */
typedef struct {
  int mode;               /* decode_attn_mode */
  int num_workgroups;     /* grid of the main kernel (256 threads per workgroup) */
  int num_splits;         /* partitions per (sequence, KV head): >= 2 in split mode, 1 in
                             segment mode, 0 in stream mode */
  int pages_per_split;    /* split mode: pages per partition; 0 otherwise */
  size_t workspace_bytes; /* device workspace decode_attn_ex needs for this plan */
} decode_attn_plan_t;

/*
 * Decode attention over a paged KV cache (the definition above).
 *
 * batch >= 0 (0 enqueues nothing and returns OK); max_blocks_per_seq >= 1;
 * num_pages >= 1 is the number of pages in each pool, used only to reject bad table
 * entries on the device; scale is the softmax scale (typically 1/sqrt(head_dim)).
 * The plan is the library's choice for the current device (decode_attn_plan with no
 * request), and the library uses a workspace it owns: one buffer per device, replaced by
 * a larger one (hipMalloc) when a call needs more. A replaced buffer is never freed: it
 * stays allocated until the process ends, so work already queued and HIP graphs captured
 * from earlier calls keep valid addresses. This entry point therefore may allocate (on
 * its first call for a larger shape; capture it in a HIP graph only after such a call),
 * and two calls that overlap on one device (different streams or host threads) must not
 * share that workspace; such callers use decode_attn_ex. Returns a decode_attn_status.
 */
int decode_attn(const void* q, const void* k_pages, const void* v_pages,
                const float* k_scale, const float* v_scale,
                const int32_t* block_table, const int32_t* seq_lens,
                int batch, int max_blocks_per_seq, int num_pages,
                int n_q_heads, int n_kv_heads, int head_dim, int block_size,
                int kv_dtype, float scale, float* out, hipStream_t stream);

/*
 * Planning (swiftLLM feature list: Flash-Decoding). The requests:
 *  - requested_splits == 1: segment mode, on requested_workgroups workgroups if that is
 *    > 0, else on as many as stay resident on num_cus compute units (never more than
 *    batch * n_kv_heads, and over caches of more than 64 pages no more than one per two
 *    pairs unless that is below num_cus);
 *  - requested_splits > 1 (requested_workgroups must be 0): split mode with that many page
 *    partitions per (sequence, KV head); the result may be smaller, namely
 *    ceil(max_blocks_per_seq / ceil(max_blocks_per_seq / requested_splits)), and a result
 *    of 1 is segment mode;
 *  - requested_workgroups > 0 alone: stream mode on that many workgroups;
 *  - both 0: the library's choice from the shapes, the format, G and num_cus. With fewer
 *    (sequence, KV head) pairs than compute units: segment mode for caches of at most 16
 *    pages, else split mode with num_cus / pairs partitions rounded to the nearest (segment
 *    mode when that is below 2). With more: segment mode when caches are at most 64 pages,
 *    when there are at least two pairs per compute unit, when the batch exceeds 4096
 *    sequences, or for every build but INT8 and FP8 with G <= 2; stream mode otherwise.
 * num_cus is the device's compute-unit count; 0 queries the current device (the only HIP
 * call, made only when the plan needs the count). kv_dtype is a decode_attn_kv_dtype (the
 * grid of segment mode depends on it). Fills *plan and returns a decode_attn_status.
 */
int decode_attn_plan(int batch, int max_blocks_per_seq, int n_q_heads, int n_kv_heads,
                     int block_size, int kv_dtype, int requested_workgroups,
                     int requested_splits, int num_cus, decode_attn_plan_t* plan);

/*
 * decode_attn with an explicit plan request and caller-owned workspace; never allocates.
 *
 * requested_workgroups and requested_splits as in decode_attn_plan (both 0 = the
 * library's choice for the current device). workspace: device memory of at least the
 * plan's workspace_bytes, 256-byte aligned; it may be NULL when that is 0 (segment mode
 * needs none). Its contents on entry do not matter and on return are unspecified; it must
 * not be in use by another call still running. lse_out (nullable, 4-byte aligned)
 * receives lse[b, h] as defined above. Every launch is a kernel (no memset, copy or
 * allocation), so the call can be captured in a HIP graph and replayed. Returns a
 * decode_attn_status.
 */
int decode_attn_ex(const void* q, const void* k_pages, const void* v_pages,
                   const float* k_scale, const float* v_scale,
                   const int32_t* block_table, const int32_t* seq_lens,
                   int batch, int max_blocks_per_seq, int num_pages,
                   int n_q_heads, int n_kv_heads, int head_dim, int block_size,
                   int kv_dtype, float scale, float* out, float* lse_out,
                   int requested_workgroups, int requested_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * decode_attn_ex for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, and harnesses that forbid hipMalloc. It takes the same arguments minus
 * the workspace and never allocates (no hipMalloc, hipFree or allocating library call):
 * the plan's workspace is a static device array of DECODE_ATTN_STATIC_SCRATCH_BYTES
 * (32 MiB) in the library's code object, one per device, held until the process ends. Its
 * device address is looked up (hipGetSymbolAddress) on the first call on each device, with
 * that device current. A plan whose workspace_bytes (see decode_attn_plan) exceeds the
 * limit returns DECODE_ATTN_ERR_SCRATCH_LIMIT before any HIP call; segment-mode plans need
 * none. Every call on one device shares that device's array and leaves its contents behind
 * (nothing in it has to start at zero: each call writes every entry it later reads), so
 * calls that overlap on one device (different streams or host threads) race and must be
 * serialised by the caller. Results are bitwise those of decode_attn_ex with the same
 * requests. Returns a decode_attn_status.
 */
int decode_attn_noalloc(const void* q, const void* k_pages, const void* v_pages,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        int batch, int max_blocks_per_seq, int num_pages,
                        int n_q_heads, int n_kv_heads, int head_dim, int block_size,
                        int kv_dtype, float scale, float* out, float* lse_out,
                        int requested_workgroups, int requested_splits, hipStream_t stream);

/*
 * Append a decode step's new key and value rows to the paged cache: every decode step
 * adds the new token's K and V before attending (page "Eine LLM-Inferenz-Engine von
 * Grund auf mit C++ und CUDA bauen", section 1.1), and token position p of sequence b
 * lives in page block_table[b, p / block_size], slot p % block_size (swiftLLM feature
 * list: PagedAttention).
 *
 *     k_new, v_new  fp16 [batch, n_kv_heads, head_dim] (bf16 for a BF16 cache), 16-byte
 *                   aligned: the new rows.
 *     positions     int32 [batch]: the new token's position p_b in sequence b (its
 *                   length before the step); p_b < 0 means no new token for b.
 *     block_table   as for decode_attn; entry (b, p_b / block_size) must name the page
 *                   that receives the row (the caller allocates pages).
 *     k_pages, v_pages (and k_scale, v_scale for INT8 and FP8) as for decode_attn, written in
 *                   place: row (b, g) goes to [page, g, p_b % block_size]. Nothing else
 *                   in the pools is touched.
 *
 * FP16 and BF16 pools store the row unchanged. INT8 pools (xLLM README, quantisation
 * list: per-row INT8) store symmetric codes: s = max_d |x_d| / 127 and
 * code_d = rint(x_d / s) (round half to even), both in fp32 with IEEE division, clamped
 * to [-127, 127]. FP8 pools (E4M3, section 4 of the C++/CUDA engine page) store
 * s = max_d |x_d| / 448 and code_d = the E4M3 code nearest to x_d / s (ties to the even
 * code; the sign of a zero is kept), with the same fp32 divisions. A row of zeros stores
 * s = 0 and codes 0. Rows must be finite.
 *
 * Bad device values never fault: a row whose position is at or past
 * max_blocks_per_seq * block_size, or whose table entry lies outside [0, num_pages), is
 * not written. Two sequences whose positions map to the same page slot race (the caller
 * must not do that). Asynchronous on `stream`; never allocates. Supported sizes: as for
 * decode_attn, plus batch * n_kv_heads < 2^31. Returns a decode_attn_status.
 */
int decode_attn_append(const void* k_new, const void* v_new, const int32_t* block_table,
                       const int32_t* positions, int batch, int max_blocks_per_seq,
                       int num_pages, int n_kv_heads, int head_dim, int block_size,
                       int kv_dtype, void* k_pages, void* v_pages, float* k_scale,
                       float* v_scale, hipStream_t stream);

/*
 * Chunked-prefill attention over the paged cache: several new tokens per sequence at once.
 * The prefill phase runs a prompt's tokens through the model and fills the cache (page
 * "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen", section 1.1; handling
 * several prompt tokens together with FlashAttention-style fused attention is among its
 * next steps, section 4), and swiftLLM's feature list piggybacks prefill chunks on decode
 * batches. Sequence b's chunk is its last C_b = q_start[b+1] - q_start[b] tokens, whose K
 * and V rows are already in the cache (L_b = seq_lens[b] counts them); chunk row i sits at
 * position p = L_b - C_b + i and attends causally to tokens 0 .. p:
 *
 *     out[q_start[b] + i, h, :] = sum_{t <= p} softmax_t(scale * <q[.., h, :], K_b[g,t,:]>) V_b[g,t,:]
 *
 * with g = h / G. A decode token is a chunk of one, so prefill chunks and decode tokens can
 * share a call.
 *
 *     q         [total_rows, n_q_heads, head_dim], 16-byte aligned: all chunks' rows; fp16,
 *               or bf16 for a BF16 cache (as for decode_attn)
 *     q_start   int32 [batch + 1]: 0 <= q_start[b] <= q_start[b+1] <= total_rows
 *     k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, num_pages, kv_dtype: as for
 *               decode_attn (row scales present iff INT8 or FP8)
 *     max_chunk an upper bound on C_b, used only to size the grid (total_rows is always
 *               safe); longer chunks are still computed in full
 *     out       fp32 [total_rows, n_q_heads, head_dim], 16-byte aligned; rows outside every
 *               chunk are not written
 *
 * Both products run on the matrix cores with fp32 accumulation. The scores take fp16 q and
 * K (bf16 for a BF16 cache); the weighted sum of V takes the softmax weights rounded to fp16
 * and V as fp16. BF16 V rows are rounded to fp16 on the way in, and INT8 and FP8 rows are
 * dequantised on the way in (code times the row's scale, rounded once to fp16), so those
 * values must lie within fp16's range (|value| < 65504); values below fp16's normal range
 * (2^-14) keep fp16's subnormal precision. Bad device values never
 * fault: a sequence whose q_start range leaves [0, total_rows] or is empty is skipped; one
 * whose chunk is longer than L_b, whose L_b exceeds the table, or whose table holds a page
 * id outside [0, num_pages) among its first ceil(L_b / block_size) entries gets NaN in all
 * its rows. Supported: head_dim 128, block_size 16, G in {1, 2, 4, 8}, batch * n_kv_heads
 * below 2^24. Asynchronous on `stream`; never allocates; capturable in a HIP graph. Returns
 * a decode_attn_status.
 */
int decode_attn_prefill(const void* q, const int32_t* q_start, const void* k_pages,
                        const void* v_pages, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens, int batch,
                        int total_rows, int max_blocks_per_seq, int num_pages, int n_q_heads,
                        int n_kv_heads, int head_dim, int block_size, int kv_dtype, int max_chunk,
                        float scale, float* out, hipStream_t stream);

/*
 * Reference reads for the HBM roofline; a measurement aid, not part of the attention path.
 * Decode attention streams the KV cache once per step and is bound by HBM bandwidth (xLLM
 * README, bottleneck analysis: attention score and output are memory-bound), so its
 * kernels are judged against the rate at which this GPU can read the same bytes. These
 * kernels read memory the way the decode kernels do, 16 bytes per lane, and fold the bits
 * into one value without other arithmetic:
 *
 *     kind 0  streaming read of `count` 16-byte words at `a` (nothing else used);
 *             depth = words per lane per step: 4, 8 or 16
 *     kind 1  tile gather: for every i < count, the 4 KiB tile tiles[i] of `a` and the
 *             one of `b` (tile t at byte offset 4096 t), as the decode kernels read the
 *             16-bit K and V tiles of one (page, KV head)
 *     kind 2  as kind 1 with 2 KiB tiles (offset 2048 t), plus the 64-byte records
 *             a_scale + 64 t and b_scale + 64 t: the codes and row scales of a 1-byte
 *             (INT8 or FP8) tile
 *
 *     For kinds 1 and 2, entries of tiles outside [0, num_tiles) are skipped; each wave
 *     takes an equal contiguous run of entries, and depth = entries in flight per wave:
 *     1, 2 or 4.
 *     nontemporal  1: loads carry the non-temporal hint (as the decode kernels'), 0: not
 *     grid         workgroups of 256 threads, 1 .. 65535
 *     sink         device uint32 [grid * 256]; a lane writes its fold there only if it
 *                  equals one fixed 32-bit value (never, for zero-filled memory)
 *
 * All pointers are device pointers: a and b 16-byte aligned, a_scale and b_scale 64-byte
 * aligned (kind 2 only; ignored otherwise), tiles 4-byte aligned. `a` holds at least
 * 16 count bytes (kind 0); a and b hold num_tiles tiles, a_scale and b_scale num_tiles
 * records (kinds 1, 2). Nothing is written but the sink. Asynchronous on `stream`; never
 * allocates. Returns DECODE_ATTN_ERR_INVALID_ARGUMENT for any other kind, depth,
 * nontemporal or grid, a null or misaligned pointer that the kind uses, or a negative
 * count or num_tiles.
 */
int decode_attn_hbm_reference(int kind, int depth, int nontemporal, const void* a,
                              const void* b, const void* a_scale, const void* b_scale,
                              const int32_t* tiles, long long count, long long num_tiles,
                              int grid, uint32_t* sink, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* decode_attn_status_string(int status);

/* Library ABI version: (major << 16) | minor. 6.0 adds the BF16 and FP8 formats;
   6.1 adds decode_attn_prefill; 6.2 gives it every storage format (row scale arguments);
   6.3 adds decode_attn_noalloc; 6.4 adds decode_attn_hbm_reference. */
int decode_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
