/*
 * decode_attn.h - C ABI of the MI355X (gfx950) decode-phase paged attention library.
 *
 * What is computed. In the decode phase each sequence adds one query token that
 * attends over the keys and values cached for its earlier tokens (page "Eine
 * LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen", section 1.1). The cache
 * lives in fixed-size pages found through a per-sequence block table (swiftLLM README,
 * feature list: PagedAttention). Several query heads may share one KV head (xLLM README,
 * optimisation list: GQA), and the cache may be stored as per-row INT8 (xLLM README,
 * quantisation list). For sequence b and query head h, with G = n_q_heads / n_kv_heads
 * and g = h / G:
 *
 *     s_t = scale * <q[b,h,:], K_b[g,t,:]>        for t in [0, L_b)
 *     out[b,h,:] = sum_t softmax(s)_t * V_b[g,t,:]
 *     lse[b,h]   = ln sum_t exp(s_t)              (natural log; -inf when L_b = 0)
 *
 * The library reaches this with a single-pass online-normaliser softmax (xLLM README,
 * SoftMax operator) and, for long caches, a split of each sequence into page-aligned
 * partitions whose partial (out, lse) are merged by their log-sum-exp weights
 * (swiftLLM feature list: PagedAttention v2 / Flash-Decoding). Both only change the
 * order of rounding; out is the plain softmax result above.
 *
 * Memory layout (all row-major and contiguous; all tensor pointers are DEVICE pointers
 * owned by the caller, for example torch tensors; the library never frees them):
 *
 *     q            fp16  [batch, n_q_heads, head_dim]
 *     k_pages      fp16 or int8  [num_pages, n_kv_heads, block_size, head_dim]
 *     v_pages      same type and shape as k_pages
 *     k_scale      fp32  [num_pages, n_kv_heads, block_size]   (INT8 only, else NULL)
 *     v_scale      fp32  [num_pages, n_kv_heads, block_size]   (INT8 only, else NULL)
 *     block_table  int32 [batch, max_blocks_per_seq]: entry (b, j) is the physical page
 *                  holding tokens j*block_size .. j*block_size+block_size-1 of sequence b.
 *                  Only entries j < ceil(L_b / block_size) are read; the rest may hold
 *                  anything (for example -1).
 *     seq_lens     int32 [batch]: L_b, with 0 <= L_b <= max_blocks_per_seq * block_size.
 *     out          fp32  [batch, n_q_heads, head_dim]; must not overlap any input.
 *     lse_out      fp32  [batch, n_q_heads] or NULL.
 *
 * A (page, KV head) tile is block_size * head_dim contiguous elements (4 KiB in fp16 at
 * 16 x 128), so one page of one head is read with fully coalesced 16-byte loads. An INT8
 * row (token, KV head) has value int8 * scale with one fp32 scale per row; the slots of
 * a page past L_b are never used, whatever they hold (NaN included).
 *
 * Supported sizes: head_dim 128, block_size 16, G = n_q_heads / n_kv_heads in
 * {1, 2, 4, 8}. Other values return DECODE_ATTN_ERR_UNSUPPORTED.
 *
 * Calls are asynchronous: they validate arguments on the host, enqueue kernels on
 * `stream` and return. Nothing is synchronised and no device value is read back; the
 * caller's stream orders the work. The same inputs with the same split count give a
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
  DECODE_ATTN_ERR_HIP = 4               /* a HIP call or kernel launch failed */
} decode_attn_status;

/* Storage type of k_pages / v_pages. */
typedef enum {
  DECODE_ATTN_KV_FP16 = 0,
  DECODE_ATTN_KV_INT8 = 1 /* per-row INT8 with fp32 row scales (xLLM README, quantisation) */
} decode_attn_kv_dtype;

/*
 * Decode attention over a paged KV cache (the definition above).
 *
 * batch >= 0 (0 enqueues nothing and returns OK); max_blocks_per_seq >= 1;
 * num_pages >= 1 is the number of pages in each pool, used only to reject bad table
 * entries on the device; scale is the softmax scale (typically 1/sqrt(head_dim)).
 * The split count is chosen by decode_attn_plan for the current device. When it is
 * above 1 the library uses a workspace it owns: one buffer per device, grown with
 * hipMalloc on demand and kept until the process ends. This entry point therefore may
 * allocate, and two calls that overlap on one device (different streams or host
 * threads) must not both need that workspace; such callers use decode_attn_ex.
 * Returns a decode_attn_status.
 */
int decode_attn(const void* q, const void* k_pages, const void* v_pages,
                const float* k_scale, const float* v_scale,
                const int32_t* block_table, const int32_t* seq_lens,
                int batch, int max_blocks_per_seq, int num_pages,
                int n_q_heads, int n_kv_heads, int head_dim, int block_size,
                int kv_dtype, float scale, float* out, hipStream_t stream);

/*
 * Split planning (swiftLLM feature list: Flash-Decoding). Each sequence's logical pages
 * [0, max_blocks_per_seq) are cut into *num_splits partitions of *pages_per_split pages;
 * one workgroup handles one (partition, KV head, sequence). requested_splits > 0 asks for
 * that many partitions (the result may be smaller: it is
 * ceil(max_blocks_per_seq / ceil(max_blocks_per_seq / requested_splits))); 0 lets the
 * library choose from the shape and num_cus (the device's compute-unit count; pass 0 to
 * query the current device, which is the only case that calls HIP). Pure host code
 * otherwise. Returns a decode_attn_status.
 */
int decode_attn_plan(int batch, int max_blocks_per_seq, int n_kv_heads, int block_size,
                     int requested_splits, int num_cus,
                     int* num_splits, int* pages_per_split);

/*
 * Bytes of workspace decode_attn_ex needs for a plan with num_splits partitions
 * (0 when num_splits <= 1). Pure host code; returns 0 for invalid sizes.
 */
size_t decode_attn_workspace_size(int batch, int n_q_heads, int head_dim, int num_splits);

/*
 * decode_attn with an explicit plan and caller-owned workspace; never allocates.
 *
 * requested_splits as in decode_attn_plan (0 = library's choice for the current
 * device). workspace: device memory of at least
 * decode_attn_workspace_size(batch, n_q_heads, head_dim, num_splits) bytes for the
 * resulting plan, 256-byte aligned; it may be NULL when the plan has one partition.
 * Its contents on entry do not matter and on return are unspecified; it must not be in
 * use by another call still running. lse_out (nullable) receives lse[b, h] as defined
 * above. Returns a decode_attn_status.
 */
int decode_attn_ex(const void* q, const void* k_pages, const void* v_pages,
                   const float* k_scale, const float* v_scale,
                   const int32_t* block_table, const int32_t* seq_lens,
                   int batch, int max_blocks_per_seq, int num_pages,
                   int n_q_heads, int n_kv_heads, int head_dim, int block_size,
                   int kv_dtype, float scale, float* out, float* lse_out,
                   int requested_splits, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* decode_attn_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int decode_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
