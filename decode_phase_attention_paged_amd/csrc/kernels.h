// Internal interface between the host launcher (api.cpp) and the gfx950 kernels
// (kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace dattn {

constexpr int kHeadDim = 128;   // D: elements per (token, head) row
constexpr int kBlockSize = 16;  // bs: tokens per page
constexpr int kWaves = 4;       // wavefronts per split workgroup
constexpr int kSplitThreads = 64 * kWaves;
constexpr int kMergeThreads = 256;

enum class KvType { kF16 = 0, kI8 = 1 };

struct SplitArgs {
  const void* q;             // fp16 [B, Hq, D]
  const void* k_pages;       // fp16 | int8 [NP, Hkv, bs, D]
  const void* v_pages;
  const float* k_scale;      // fp32 [NP, Hkv, bs] (int8 only)
  const float* v_scale;
  const int32_t* block_table;  // int32 [B, MB]
  const int32_t* seq_lens;     // int32 [B]
  float* out;                // fp32 [B, Hq, D]          (num_splits == 1)
  float* lse_out;            // fp32 [B, Hq] or null      (num_splits == 1)
  float* part_o;             // fp32 [B, Hq, S, D]        (num_splits > 1)
  float* part_lse;           // fp32 [B, Hq, S], log2 units (num_splits > 1)
  int batch;
  int max_blocks;            // MB
  int num_pages;             // NP
  int n_q_heads;
  int n_kv_heads;
  int num_splits;            // S
  int pages_per_split;       // pages per partition
  float scale_log2;          // softmax scale * log2(e)
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* seq_lens;
  float* out;
  float* lse_out;
  int batch;
  int max_blocks;
  int n_q_heads;
  int num_splits;
  int pages_per_split;
};

// Enqueue the split kernel: one workgroup per (partition, KV head, sequence).
hipError_t launch_split(KvType kv, int group, const SplitArgs& a, hipStream_t stream);
// Enqueue the merge kernel: one workgroup per (sequence, query head).
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace dattn
