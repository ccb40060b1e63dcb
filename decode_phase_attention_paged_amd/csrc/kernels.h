// Internal interface between the host launcher (api.cpp) and the gfx950 kernels
// (kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace dattn {

constexpr int kHeadDim = 128;     // D: elements per (token, head) row
constexpr int kBlockSize = 16;    // bs: tokens per page
constexpr int kWaves = 4;         // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxBatch = 4096;   // sequences whose page counts one workgroup keeps in LDS
constexpr int kPieceSlots = 2;    // partial results a stream worker can leave

constexpr int kOrderMax = kThreads;  // batches up to this size run longest sequence first

// Storage format of the K/V pools (and, for kBF16, of q). kI8 and kFP8 carry one fp32 scale
// per (token, KV head) row.
enum class KvType { kF16 = 0, kI8 = 1, kBF16 = 2, kFP8 = 3 };
constexpr int kv_elem_bytes(KvType kv) { return kv == KvType::kF16 || kv == KvType::kBF16 ? 2 : 1; }
constexpr bool kv_scaled(KvType kv) { return kv == KvType::kI8 || kv == KvType::kFP8; }

// How the batch is cut into workgroups.
//  kStream:  a fixed grid of persistent workgroups; the (sequence, KV head, page) units of
//            the whole batch are dealt out in equal contiguous runs, one per wavefront.
//  kSplit:   one workgroup per (partition, KV head, sequence) with fixed-size page
//            partitions (at least two); for a few very long caches.
//  kSegment: a fixed grid of persistent workgroups, each taking whole (sequence, KV head)
//            segments, longest sequences first; no partial results.
enum class Mode { kStream = 0, kSplit = 1, kSegment = 2 };

constexpr int log2_group(int g) { return g == 1 ? 0 : g == 2 ? 1 : g == 4 ? 2 : 3; }

// Builds whose tile products run on the matrix cores: G >= 4, every format. Their work per
// tile does not depend on G, so their tuning is one entry per element width (index 0:
// 2-byte, 1: 1-byte); the vector-ALU builds (G <= 2) are tuned per width and log2 G.
constexpr bool use_mfma(KvType kv, int group) { return (void)kv, group >= 4; }
constexpr int width_index(KvType kv) { return kv_elem_bytes(kv) == 2 ? 0 : 1; }

// Waves per SIMD the segment-mode kernel is compiled for; the host sizes that mode's grid
// to the workgroups that stay resident at that occupancy.
constexpr int kSegWavesF16[2] = {1, 2};         // fp16 and BF16, G <= 2
constexpr int kSegWavesI8[2] = {3, 2};          // INT8 and FP8, G <= 2
constexpr int kSegWavesMf[2] = {1, 2};
constexpr int seg_waves(KvType kv, int group) {
  return use_mfma(kv, group)       ? kSegWavesMf[width_index(kv)]
         : kv_elem_bytes(kv) == 2 ? kSegWavesF16[log2_group(group)]
                                  : kSegWavesI8[log2_group(group)];
}
// Wavefronts of a segment-mode workgroup, which interleave the pages of its segment.
constexpr int kSegW = 4;
constexpr int kSegThreads = 64 * kSegW;
constexpr int seg_workgroups_per_cu(KvType kv, int group) {
  return 4 * seg_waves(kv, group) / kSegW > 0 ? 4 * seg_waves(kv, group) / kSegW : 1;
}

struct Args {
  const void* q;               // fp16 [B, Hq, D] (bf16 for a bf16 cache)
  const void* k_pages;         // fp16 | bf16 | int8 | fp8 e4m3 [NP, Hkv, bs, D]
  const void* v_pages;
  const float* k_scale;        // fp32 [NP, Hkv, bs] (int8 and fp8 only)
  const float* v_scale;
  const int32_t* block_table;  // int32 [B, MB]
  const int32_t* seq_lens;     // int32 [B]
  float* out;                  // fp32 [B, Hq, D]
  float* lse_out;              // fp32 [B, Hq] or null
  // Workspace. Stream mode: part_o [workers * kPieceSlots, G, D], part_lse [same rows]
  // (log2 units), pieces [workers, 4]. Split mode: part_o [B, Hq, S, D], part_lse [B, Hq, S].
  // Segment mode: none.
  float* part_o;
  float* part_lse;
  int32_t* pieces;
  int batch;
  int max_blocks;              // MB
  int num_pages;               // NP
  int n_q_heads;
  int n_kv_heads;
  int num_splits;              // split mode: S
  int pages_per_split;         // split mode: pages per partition
  float scale_log2;            // softmax scale * log2(e)
};

struct Plan {
  Mode mode;
  int num_workgroups;   // grid of the main kernel
  int num_splits;       // split mode only
  int pages_per_split;  // split mode only
};

// Bytes of workspace a plan needs.
size_t workspace_bytes(const Plan& plan, int batch, int n_q_heads, int n_kv_heads);
// Carve the workspace into the partial-result arrays of Args.
void bind_workspace(Args& a, const Plan& plan, void* workspace);

// Enqueue the main kernel and the merge of the partial results it leaves.
hipError_t launch(KvType kv, int group, const Args& a, const Plan& plan, hipStream_t stream);

// Workspace that lives in the code object, for calls that must not allocate: a static
// device array of kStaticScratchBytes per device. static_scratch gives the current
// device's copy (its address is looked up once per device and kept).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr);

// Appending a decode step's new K/V rows to the paged cache (append.hip).
struct AppendArgs {
  const void* k_new;           // fp16 [B, Hkv, D] (bf16 for a bf16 cache)
  const void* v_new;
  const int32_t* block_table;  // int32 [B, MB]
  const int32_t* positions;    // int32 [B]: token position of the new row, < 0 = none
  void* k_pages;               // fp16 | bf16 | int8 | fp8 e4m3 [NP, Hkv, bs, D]
  void* v_pages;
  float* k_scale;              // fp32 [NP, Hkv, bs] (int8 and fp8 only)
  float* v_scale;
  int batch;
  int max_blocks;              // MB
  int num_pages;               // NP
  int n_kv_heads;
};
hipError_t launch_append(KvType kv, const AppendArgs& a, hipStream_t stream);

// Chunked-prefill attention over the paged cache (prefill.hip).
struct PrefillArgs {
  const void* q;               // fp16 [T, Hq, D] (bf16 for a bf16 cache): every chunk's rows, stacked
  const int32_t* q_start;      // int32 [B + 1]: sequence b's rows are q_start[b] .. q_start[b+1]-1
  const void* k_pages;         // fp16 | bf16 | int8 | fp8 e4m3 [NP, Hkv, bs, D]
  const void* v_pages;
  const float* k_scale;        // fp32 [NP, Hkv, bs] (int8 and fp8 only)
  const float* v_scale;
  const int32_t* block_table;  // int32 [B, MB]
  const int32_t* seq_lens;     // int32 [B]: L_b, counting the chunk
  float* out;                  // fp32 [T, Hq, D]
  int batch;
  int total_rows;              // T
  int max_blocks;              // MB
  int num_pages;               // NP
  int n_kv_heads;
  float scale_log2;            // softmax scale * log2(e)
};
// max_chunk bounds C_b for sizing the grid only; longer chunks are still covered.
hipError_t launch_prefill(KvType kv, int group, const PrefillArgs& a, int max_chunk, hipStream_t stream);

// Reference reads for the HBM roofline (hbm_reference.hip); the host has checked every field.
struct HbmReferenceArgs {
  int kind;                    // 0: streaming read of a; 1: 4 KiB tile gather from a and
                               // b; 2: 2 KiB tile gather from a and b with 64-byte scale
                               // records from a_scale and b_scale
  int depth;                   // kind 0: 16-byte words per lane per step (4, 8, 16);
                               // kinds 1, 2: tile pairs in flight per wave (1, 2, 4)
  int nontemporal;             // 1: loads carry the non-temporal hint, as the decode kernels'
  int grid;                    // workgroups of 256 threads
  const void* a;
  const void* b;
  const void* a_scale;         // kind 2
  const void* b_scale;
  const int32_t* tiles;        // kinds 1, 2: tile indices
  uint64_t count;              // kind 0: 16-byte words; kinds 1, 2: entries of tiles
  uint64_t num_tiles;          // kinds 1, 2: tiles in each of a and b
  uint32_t* sink;              // uint32 [grid * 256]
};
hipError_t launch_hbm_reference(const HbmReferenceArgs& r, hipStream_t stream);

}  // namespace dattn
