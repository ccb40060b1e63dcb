// C ABI of the decode-attention library: argument validation, split planning, workspace
// management and kernel launch order. Every check that can fail runs on the host before
// the first HIP call, so invalid arguments never reach a kernel.

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstdint>
#include <mutex>

#include "decode_attn.h"
#include "kernels.h"

namespace {

using dattn::kBlockSize;
using dattn::kHeadDim;

constexpr int kVersion = (1 << 16) | 0;
constexpr int kMaxDevices = 64;
// A workgroup streams at most this many pages when the library picks the split count:
// long caches are cut so that no single workgroup sets the kernel's tail.
constexpr int kAutoMaxPagesPerSplit = 64;
// Grow the split count until the grid holds this many workgroups per compute unit.
constexpr int kAutoWorkgroupsPerCu = 4;

constexpr size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

std::mutex g_mutex;
int g_cus[kMaxDevices];            // compute units per device, 0 = not queried yet
void* g_ws[kMaxDevices];           // library-owned workspace per device
size_t g_ws_bytes[kMaxDevices];

int current_device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DECODE_ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return DECODE_ATTN_ERR_HIP;
    g_cus[dev] = n;
  }
  *cus = g_cus[dev];
  return DECODE_ATTN_OK;
}

int plan_splits(int batch, int max_blocks, int n_kv_heads, int requested, int cus,
                int* num_splits, int* pages_per_split) {
  int s = 1;
  if (requested > 0) {
    s = requested < max_blocks ? requested : max_blocks;
  } else {
    s = (max_blocks + kAutoMaxPagesPerSplit - 1) / kAutoMaxPagesPerSplit;
    const long long items = static_cast<long long>(batch) * n_kv_heads;
    const long long target = static_cast<long long>(kAutoWorkgroupsPerCu) * cus;
    while (s < max_blocks && items * s < target) s = s * 2 < max_blocks ? s * 2 : max_blocks;
  }
  const int pps = (max_blocks + s - 1) / s;
  *pages_per_split = pps;
  *num_splits = (max_blocks + pps - 1) / pps;
  return DECODE_ATTN_OK;
}

size_t workspace_bytes(int batch, int n_q_heads, int head_dim, int num_splits) {
  if (batch <= 0 || n_q_heads <= 0 || head_dim <= 0 || num_splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(batch) * n_q_heads * num_splits;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Host-side argument checks shared by both entry points.
int validate(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
             const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
             int batch, int max_blocks, int num_pages, int n_q_heads, int n_kv_heads,
             int head_dim, int block_size, int kv_dtype, const float* out, int requested) {
  if (batch < 0 || max_blocks < 1 || num_pages < 1 || n_q_heads < 1 || n_kv_heads < 1 ||
      head_dim < 1 || block_size < 1 || requested < 0)
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (n_q_heads % n_kv_heads != 0) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (kv_dtype != DECODE_ATTN_KV_FP16 && kv_dtype != DECODE_ATTN_KV_INT8)
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  const bool int8 = kv_dtype == DECODE_ATTN_KV_INT8;
  if (int8 != (k_scale != nullptr) || int8 != (v_scale != nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (q == nullptr || k_pages == nullptr || v_pages == nullptr ||
                    block_table == nullptr || seq_lens == nullptr || out == nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 4) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(out, 4))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (head_dim != kHeadDim || block_size != kBlockSize) return DECODE_ATTN_ERR_UNSUPPORTED;
  const int group = n_q_heads / n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return DECODE_ATTN_ERR_UNSUPPORTED;
  // 32-bit index ranges used on the device.
  if (static_cast<long long>(max_blocks) * block_size > INT_MAX ||
      static_cast<long long>(batch) * max_blocks > INT_MAX ||
      static_cast<long long>(batch) * n_q_heads * head_dim > INT_MAX ||
      static_cast<long long>(batch) * n_q_heads > INT_MAX / 2)
    return DECODE_ATTN_ERR_UNSUPPORTED;
  return DECODE_ATTN_OK;
}

int run(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
        const float* v_scale, const int32_t* block_table, const int32_t* seq_lens, int batch,
        int max_blocks, int num_pages, int n_q_heads, int n_kv_heads, int kv_dtype,
        float scale, float* out, float* lse_out, int num_splits, int pages_per_split,
        void* workspace, hipStream_t stream) {
  (void)hipGetLastError();  // start from a clean error state
  dattn::SplitArgs sa{};
  sa.q = q;
  sa.k_pages = k_pages;
  sa.v_pages = v_pages;
  sa.k_scale = k_scale;
  sa.v_scale = v_scale;
  sa.block_table = block_table;
  sa.seq_lens = seq_lens;
  sa.out = out;
  sa.lse_out = lse_out;
  sa.batch = batch;
  sa.max_blocks = max_blocks;
  sa.num_pages = num_pages;
  sa.n_q_heads = n_q_heads;
  sa.n_kv_heads = n_kv_heads;
  sa.num_splits = num_splits;
  sa.pages_per_split = pages_per_split;
  sa.scale_log2 = scale * 1.4426950408889634f;
  if (num_splits > 1) {
    const size_t rows = static_cast<size_t>(batch) * n_q_heads * num_splits;
    sa.part_o = static_cast<float*>(workspace);
    sa.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           align256(rows * kHeadDim * sizeof(float)));
  }
  const dattn::KvType kv = kv_dtype == DECODE_ATTN_KV_INT8 ? dattn::KvType::kI8 : dattn::KvType::kF16;
  if (dattn::launch_split(kv, n_q_heads / n_kv_heads, sa, stream) != hipSuccess)
    return DECODE_ATTN_ERR_HIP;
  if (num_splits > 1) {
    dattn::MergeArgs ma{};
    ma.part_o = sa.part_o;
    ma.part_lse = sa.part_lse;
    ma.seq_lens = seq_lens;
    ma.out = out;
    ma.lse_out = lse_out;
    ma.batch = batch;
    ma.max_blocks = max_blocks;
    ma.n_q_heads = n_q_heads;
    ma.num_splits = num_splits;
    ma.pages_per_split = pages_per_split;
    if (dattn::launch_merge(ma, stream) != hipSuccess) return DECODE_ATTN_ERR_HIP;
  }
  return DECODE_ATTN_OK;
}

// Grid size check: one workgroup per (partition, KV head, sequence).
bool grid_fits(int batch, int n_kv_heads, int num_splits) {
  return static_cast<long long>(batch) * n_kv_heads * num_splits <= INT_MAX;
}

}  // namespace

extern "C" {

int decode_attn_plan(int batch, int max_blocks_per_seq, int n_kv_heads, int block_size,
                     int requested_splits, int num_cus, int* num_splits, int* pages_per_split) {
  if (num_splits == nullptr || pages_per_split == nullptr || batch < 0 || max_blocks_per_seq < 1 ||
      n_kv_heads < 1 || block_size < 1 || requested_splits < 0 || num_cus < 0)
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (requested_splits == 0 && num_cus == 0) {
    const int st = current_device_cus(&num_cus);
    if (st != DECODE_ATTN_OK) return st;
  }
  return plan_splits(batch, max_blocks_per_seq, n_kv_heads, requested_splits, num_cus, num_splits,
                     pages_per_split);
}

size_t decode_attn_workspace_size(int batch, int n_q_heads, int head_dim, int num_splits) {
  return workspace_bytes(batch, n_q_heads, head_dim, num_splits);
}

int decode_attn_ex(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                   const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                   int batch, int max_blocks_per_seq, int num_pages, int n_q_heads,
                   int n_kv_heads, int head_dim, int block_size, int kv_dtype, float scale,
                   float* out, float* lse_out, int requested_splits, void* workspace,
                   size_t workspace_size, hipStream_t stream) {
  int st = validate(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
                    max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, head_dim, block_size,
                    kv_dtype, out, requested_splits);
  if (st != DECODE_ATTN_OK) return st;
  if (!aligned(lse_out, 4)) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (batch == 0) return DECODE_ATTN_OK;
  int cus = 0;
  if (requested_splits == 0) {
    st = current_device_cus(&cus);
    if (st != DECODE_ATTN_OK) return st;
  }
  int splits = 1, pps = 1;
  plan_splits(batch, max_blocks_per_seq, n_kv_heads, requested_splits, cus, &splits, &pps);
  if (!grid_fits(batch, n_kv_heads, splits)) return DECODE_ATTN_ERR_UNSUPPORTED;
  if (splits > 1) {
    const size_t need = workspace_bytes(batch, n_q_heads, head_dim, splits);
    if (workspace == nullptr || workspace_size < need || !aligned(workspace, 256))
      return DECODE_ATTN_ERR_WORKSPACE;
  }
  return run(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
             max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, kv_dtype, scale, out, lse_out,
             splits, pps, workspace, stream);
}

int decode_attn(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                int batch, int max_blocks_per_seq, int num_pages, int n_q_heads, int n_kv_heads,
                int head_dim, int block_size, int kv_dtype, float scale, float* out,
                hipStream_t stream) {
  int st = validate(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
                    max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, head_dim, block_size,
                    kv_dtype, out, 0);
  if (st != DECODE_ATTN_OK) return st;
  if (batch == 0) return DECODE_ATTN_OK;
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != DECODE_ATTN_OK) return st;
  int splits = 1, pps = 1;
  plan_splits(batch, max_blocks_per_seq, n_kv_heads, 0, cus, &splits, &pps);
  if (!grid_fits(batch, n_kv_heads, splits)) return DECODE_ATTN_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (splits > 1) {
    const size_t need = workspace_bytes(batch, n_q_heads, head_dim, splits);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DECODE_ATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_ws_bytes[dev] < need) {
      if (g_ws[dev] != nullptr) {
        // Work already queued may still read the old buffer.
        if (hipDeviceSynchronize() != hipSuccess) return DECODE_ATTN_ERR_HIP;
        (void)hipFree(g_ws[dev]);
        g_ws[dev] = nullptr;
        g_ws_bytes[dev] = 0;
      }
      void* p = nullptr;
      if (hipMalloc(&p, need) != hipSuccess) return DECODE_ATTN_ERR_HIP;
      g_ws[dev] = p;
      g_ws_bytes[dev] = need;
    }
    ws = g_ws[dev];
  }
  return run(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
             max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, kv_dtype, scale, out, nullptr,
             splits, pps, ws, stream);
}

const char* decode_attn_status_string(int status) {
  switch (status) {
    case DECODE_ATTN_OK: return "DECODE_ATTN_OK";
    case DECODE_ATTN_ERR_INVALID_ARGUMENT: return "DECODE_ATTN_ERR_INVALID_ARGUMENT";
    case DECODE_ATTN_ERR_UNSUPPORTED: return "DECODE_ATTN_ERR_UNSUPPORTED";
    case DECODE_ATTN_ERR_WORKSPACE: return "DECODE_ATTN_ERR_WORKSPACE";
    case DECODE_ATTN_ERR_HIP: return "DECODE_ATTN_ERR_HIP";
    default: return "DECODE_ATTN_UNKNOWN_STATUS";
  }
}

int decode_attn_version(void) { return kVersion; }

}  // extern "C"
