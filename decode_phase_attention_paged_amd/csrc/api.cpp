// C ABI of the decode-attention library: argument validation, planning, workspace
// management and kernel launch. Every check that can fail runs on the host before the
// first HIP call, so invalid arguments never reach a kernel.

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cstdint>
#include <mutex>
#include <vector>

#include "decode_attn.h"
#include "kernels.h"

namespace {

using dattn::kBlockSize;
using dattn::kHeadDim;

constexpr int kVersion = (6 << 16) | 4;
constexpr int kMaxDevices = 64;
// Stream mode: persistent workgroups per compute unit when the library sizes the grid ...
constexpr int kStreamWorkgroupsPerCu = 2;
// ... but no more than one wavefront per this many units (pages x KV heads) the shapes
// allow, so that tiny batches do not launch idle waves.
constexpr long long kMinUnitsPerWave = 4;
// Split mode with several partitions is chosen when the batch has fewer (sequence, KV head)
// segments than compute units; it then aims at this many workgroups per compute unit.
constexpr int kSplitWorkgroupsPerCu = 1;
// Segment mode (no merge) is the library's choice when caches are at most this many pages
// (whole segments are then short enough to balance without cutting them) ...
constexpr int kShortCachePages = 64;
// ... or when there are at least this many segments per compute unit: over long caches the
// grid then shrinks (down to one workgroup per compute unit) so that every workgroup gets
// this many segments, longest first, which balances them ...
constexpr long long kMinSegmentsPerWorkgroup = 2;
// ... or when there are few segments but none longer than this many pages.
constexpr int kTinyCachePages = 16;

std::mutex g_mutex;
int g_cus[kMaxDevices];            // compute units per device, 0 = not queried yet
void* g_ws[kMaxDevices];           // library-owned workspace per device
size_t g_ws_bytes[kMaxDevices];
// Buffers a larger call superseded. They are never freed: work still queued, or a HIP
// graph captured from an earlier call, may read them at any later time.
std::vector<void*> g_ws_retired[kMaxDevices];

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

dattn::Plan split_plan(int batch, int max_blocks, int n_kv_heads, int splits) {
  dattn::Plan p{};
  p.mode = dattn::Mode::kSplit;
  if (splits > max_blocks) splits = max_blocks;
  p.pages_per_split = (max_blocks + splits - 1) / splits;
  p.num_splits = (max_blocks + p.pages_per_split - 1) / p.pages_per_split;
  p.num_workgroups = p.num_splits * n_kv_heads * batch;
  return p;
}

// Segment mode on `workgroups` persistent workgroups, or (0) as many as stay resident on
// `cus` compute units, but no more than there are segments, and over long caches no more
// than one per kMinSegmentsPerWorkgroup segments unless that is below one per compute unit.
dattn::Plan segment_plan(int batch, int max_blocks, int n_kv_heads, dattn::KvType kv, int group,
                         int workgroups, int cus) {
  dattn::Plan p{};
  p.mode = dattn::Mode::kSegment;
  p.num_splits = 1;
  const long long segments = static_cast<long long>(batch) * n_kv_heads;
  if (workgroups > 0) {
    p.num_workgroups = workgroups;
  } else {
    long long wgs = static_cast<long long>(dattn::seg_workgroups_per_cu(kv, group)) * cus;
    if (max_blocks > kShortCachePages) {
      const long long balanced = segments / kMinSegmentsPerWorkgroup;
      const long long cap = balanced > cus ? balanced : cus;
      if (wgs > cap) wgs = cap;
    }
    if (wgs > segments) wgs = segments;
    p.num_workgroups = wgs < 1 ? 1 : static_cast<int>(wgs);
  }
  return p;
}

// requested_splits == 1: segment mode (on requested_workgroups workgroups if > 0);
// requested_splits > 1: split mode; requested_workgroups > 0 alone: stream mode with that
// grid; both 0: the library's choice for a device with `cus` compute units.
dattn::Plan make_plan(int batch, int max_blocks, int n_kv_heads, dattn::KvType kv, int group,
                      int requested_workgroups, int requested_splits, int cus) {
  if (requested_splits == 1)
    return segment_plan(batch, max_blocks, n_kv_heads, kv, group, requested_workgroups, cus);
  if (requested_splits > 1) {
    dattn::Plan p = split_plan(batch, max_blocks, n_kv_heads, requested_splits);
    // A request rounded down to one partition is segment mode.
    return p.num_splits == 1 ? segment_plan(batch, max_blocks, n_kv_heads, kv, group, 0, cus) : p;
  }
  dattn::Plan p{};
  p.mode = dattn::Mode::kStream;
  if (requested_workgroups > 0) {
    p.num_workgroups = requested_workgroups;
    return p;
  }
  const long long segments = static_cast<long long>(batch) * n_kv_heads;
  // Segment mode needs a few segments per workgroup to balance whole segments, unless the
  // caches are short. Between one and two segments per compute unit only the 1-byte
  // vector-ALU builds (G <= 2) keep the balanced stream: the others measured 5-40 % faster
  // in segment mode (the stream's partial results and merge cost more than the imbalance
  // of whole segments), the 1-byte ones 30-45 % slower (too few waves to hide latency).
  const bool seg_balances = max_blocks <= kShortCachePages || segments >= kMinSegmentsPerWorkgroup * cus;
  const bool seg_preferred = dattn::use_mfma(kv, group) || dattn::kv_elem_bytes(kv) == 2;
  if (segments >= cus && (seg_balances || batch > dattn::kMaxBatch || seg_preferred))
    return segment_plan(batch, max_blocks, n_kv_heads, kv, group, 0, cus);
  // Few segments over caches of at most kTinyCachePages: each workgroup's run is a few
  // round trips long, so partitions would only add the merge kernel.
  if (segments < cus && max_blocks <= kTinyCachePages)
    return segment_plan(batch, max_blocks, n_kv_heads, kv, group, 0, cus);
  if (segments < cus) {
    // Partitions for about kSplitWorkgroupsPerCu workgroups per CU, rounded to the nearest
    // count; fewer than two (more than half as many segments as CUs) is segment mode, which
    // measured faster than two partitions' one and a half rounds of workgroups.
    const long long want = static_cast<long long>(kSplitWorkgroupsPerCu) * cus;
    const long long splits = segments > 0 ? (want + segments / 2) / segments : 1;
    if (splits < 2) return segment_plan(batch, max_blocks, n_kv_heads, kv, group, 0, cus);
    const dattn::Plan sp = split_plan(batch, max_blocks, n_kv_heads, static_cast<int>(splits));
    return sp.num_splits == 1 ? segment_plan(batch, max_blocks, n_kv_heads, kv, group, 0, cus) : sp;
  }
  const long long max_units = segments * max_blocks;
  long long wgs = static_cast<long long>(kStreamWorkgroupsPerCu) * cus;
  const long long cap = (max_units + kMinUnitsPerWave * dattn::kWaves - 1) /
                        (kMinUnitsPerWave * dattn::kWaves);
  if (wgs > cap) wgs = cap;
  p.num_workgroups = wgs < 1 ? 1 : static_cast<int>(wgs);
  return p;
}

// Whether make_plan reads the compute-unit count: every plan that ends in segment mode
// without an explicit grid, and the library's own choice.
bool plan_needs_cus(int max_blocks, int requested_workgroups, int requested_splits) {
  return requested_workgroups == 0 && (requested_splits <= 1 || max_blocks == 1);
}

bool known_kv(int kv_dtype) {
  return kv_dtype == DECODE_ATTN_KV_FP16 || kv_dtype == DECODE_ATTN_KV_INT8 ||
         kv_dtype == DECODE_ATTN_KV_BF16 || kv_dtype == DECODE_ATTN_KV_FP8;
}

// Formats whose rows carry an fp32 scale.
bool scaled_kv(int kv_dtype) {
  return kv_dtype == DECODE_ATTN_KV_INT8 || kv_dtype == DECODE_ATTN_KV_FP8;
}

dattn::KvType kv_of(int kv_dtype) {
  switch (kv_dtype) {
    case DECODE_ATTN_KV_INT8: return dattn::KvType::kI8;
    case DECODE_ATTN_KV_BF16: return dattn::KvType::kBF16;
    case DECODE_ATTN_KV_FP8: return dattn::KvType::kFP8;
    default: return dattn::KvType::kF16;
  }
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int validate_shapes(int batch, int max_blocks, int n_q_heads, int n_kv_heads, int block_size,
                    int requested_workgroups, int requested_splits) {
  if (batch < 0 || max_blocks < 1 || n_q_heads < 1 || n_kv_heads < 1 || block_size < 1 ||
      requested_workgroups < 0 || requested_splits < 0 ||
      (requested_workgroups > 0 && requested_splits > 1))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (n_q_heads % n_kv_heads != 0) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  return DECODE_ATTN_OK;
}

// Host-side argument checks shared by both entry points.
int validate(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
             const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
             int batch, int max_blocks, int num_pages, int n_q_heads, int n_kv_heads,
             int head_dim, int block_size, int kv_dtype, const float* out, const float* lse_out,
             int requested_workgroups, int requested_splits) {
  int st = validate_shapes(batch, max_blocks, n_q_heads, n_kv_heads, block_size,
                           requested_workgroups, requested_splits);
  if (st != DECODE_ATTN_OK) return st;
  if (num_pages < 1 || head_dim < 1) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!known_kv(kv_dtype)) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  const bool scaled = scaled_kv(kv_dtype);
  if (scaled != (k_scale != nullptr) || scaled != (v_scale != nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (q == nullptr || k_pages == nullptr || v_pages == nullptr ||
                    block_table == nullptr || seq_lens == nullptr || out == nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(k_scale, 8) || !aligned(v_scale, 8) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(out, 16) || !aligned(lse_out, 4))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (head_dim != kHeadDim || block_size != kBlockSize) return DECODE_ATTN_ERR_UNSUPPORTED;
  const int group = n_q_heads / n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return DECODE_ATTN_ERR_UNSUPPORTED;
  // 32-bit ranges used on the device: unit counts, tile indices, table and output offsets.
  if (static_cast<long long>(max_blocks) * block_size > INT_MAX ||
      static_cast<long long>(batch) * max_blocks * n_kv_heads > INT_MAX ||
      static_cast<long long>(num_pages) * n_kv_heads > UINT32_MAX ||
      static_cast<long long>(batch) * n_q_heads * head_dim > INT_MAX)
    return DECODE_ATTN_ERR_UNSUPPORTED;
  return DECODE_ATTN_OK;
}

// Checks that depend on the plan.
int validate_plan(const dattn::Plan& p, int batch) {
  if (p.mode == dattn::Mode::kStream && batch > dattn::kMaxBatch) return DECODE_ATTN_ERR_UNSUPPORTED;
  if (p.num_workgroups < 1 || p.num_workgroups > INT_MAX / dattn::kWaves)
    return DECODE_ATTN_ERR_UNSUPPORTED;
  if (p.mode == dattn::Mode::kSplit &&
      static_cast<long long>(batch) * p.num_splits > INT_MAX / 4)   // merge grid: batch * Hq
    return DECODE_ATTN_ERR_UNSUPPORTED;
  return DECODE_ATTN_OK;
}

int run(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
        const float* v_scale, const int32_t* block_table, const int32_t* seq_lens, int batch,
        int max_blocks, int num_pages, int n_q_heads, int n_kv_heads, int kv_dtype, float scale,
        float* out, float* lse_out, const dattn::Plan& plan, void* workspace, hipStream_t stream) {
  (void)hipGetLastError();  // start from a clean error state
  dattn::Args a{};
  a.q = q;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse_out = lse_out;
  a.batch = batch;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.num_splits = plan.num_splits;
  a.pages_per_split = plan.pages_per_split;
  a.scale_log2 = scale * 1.4426950408889634f;
  dattn::bind_workspace(a, plan, workspace);
  if (dattn::launch(kv_of(kv_dtype), n_q_heads / n_kv_heads, a, plan, stream) != hipSuccess)
    return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

void export_plan(const dattn::Plan& p, int batch, int n_q_heads, int n_kv_heads,
                 decode_attn_plan_t* out) {
  out->mode = p.mode == dattn::Mode::kStream  ? DECODE_ATTN_MODE_STREAM
              : p.mode == dattn::Mode::kSplit ? DECODE_ATTN_MODE_SPLIT
                                              : DECODE_ATTN_MODE_SEGMENT;
  out->num_workgroups = p.num_workgroups;
  out->num_splits = p.mode == dattn::Mode::kStream ? 0 : p.num_splits;
  out->pages_per_split = p.mode == dattn::Mode::kSplit ? p.pages_per_split : 0;
  out->workspace_bytes = dattn::workspace_bytes(p, batch, n_q_heads, n_kv_heads);
}

}  // namespace

extern "C" {

int decode_attn_plan(int batch, int max_blocks_per_seq, int n_q_heads, int n_kv_heads,
                     int block_size, int kv_dtype, int requested_workgroups,
                     int requested_splits, int num_cus, decode_attn_plan_t* plan) {
  if (plan == nullptr || num_cus < 0) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!known_kv(kv_dtype)) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  int st = validate_shapes(batch, max_blocks_per_seq, n_q_heads, n_kv_heads, block_size,
                           requested_workgroups, requested_splits);
  if (st != DECODE_ATTN_OK) return st;
  if (num_cus == 0 && plan_needs_cus(max_blocks_per_seq, requested_workgroups, requested_splits)) {
    st = current_device_cus(&num_cus);
    if (st != DECODE_ATTN_OK) return st;
  }
  const dattn::Plan p = make_plan(batch, max_blocks_per_seq, n_kv_heads, kv_of(kv_dtype),
                                  n_q_heads / n_kv_heads, requested_workgroups, requested_splits,
                                  num_cus);
  st = validate_plan(p, batch);
  if (st != DECODE_ATTN_OK) return st;
  export_plan(p, batch, n_q_heads, n_kv_heads, plan);
  return DECODE_ATTN_OK;
}

int decode_attn_ex(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                   const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                   int batch, int max_blocks_per_seq, int num_pages, int n_q_heads,
                   int n_kv_heads, int head_dim, int block_size, int kv_dtype, float scale,
                   float* out, float* lse_out, int requested_workgroups, int requested_splits,
                   void* workspace, size_t workspace_size, hipStream_t stream) {
  int st = validate(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
                    max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, head_dim, block_size,
                    kv_dtype, out, lse_out, requested_workgroups, requested_splits);
  if (st != DECODE_ATTN_OK) return st;
  if (batch == 0) return DECODE_ATTN_OK;
  int cus = 0;
  if (plan_needs_cus(max_blocks_per_seq, requested_workgroups, requested_splits)) {
    st = current_device_cus(&cus);
    if (st != DECODE_ATTN_OK) return st;
  }
  const dattn::Plan plan = make_plan(batch, max_blocks_per_seq, n_kv_heads, kv_of(kv_dtype),
                                     n_q_heads / n_kv_heads, requested_workgroups,
                                     requested_splits, cus);
  st = validate_plan(plan, batch);
  if (st != DECODE_ATTN_OK) return st;
  const size_t need = dattn::workspace_bytes(plan, batch, n_q_heads, n_kv_heads);
  if (need > 0 && (workspace == nullptr || workspace_size < need || !aligned(workspace, 256)))
    return DECODE_ATTN_ERR_WORKSPACE;
  return run(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
             max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, kv_dtype, scale, out, lse_out,
             plan, need > 0 ? workspace : nullptr, stream);
}

int decode_attn_noalloc(const void* q, const void* k_pages, const void* v_pages,
                        const float* k_scale, const float* v_scale, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int max_blocks_per_seq, int num_pages,
                        int n_q_heads, int n_kv_heads, int head_dim, int block_size, int kv_dtype,
                        float scale, float* out, float* lse_out, int requested_workgroups,
                        int requested_splits, hipStream_t stream) {
  int st = validate(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
                    max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, head_dim, block_size,
                    kv_dtype, out, lse_out, requested_workgroups, requested_splits);
  if (st != DECODE_ATTN_OK) return st;
  if (batch == 0) return DECODE_ATTN_OK;
  int cus = 0;
  if (plan_needs_cus(max_blocks_per_seq, requested_workgroups, requested_splits)) {
    st = current_device_cus(&cus);
    if (st != DECODE_ATTN_OK) return st;
  }
  const dattn::Plan plan = make_plan(batch, max_blocks_per_seq, n_kv_heads, kv_of(kv_dtype),
                                     n_q_heads / n_kv_heads, requested_workgroups,
                                     requested_splits, cus);
  st = validate_plan(plan, batch);
  if (st != DECODE_ATTN_OK) return st;
  const size_t need = dattn::workspace_bytes(plan, batch, n_q_heads, n_kv_heads);
  if (need > dattn::kStaticScratchBytes) return DECODE_ATTN_ERR_SCRATCH_LIMIT;
  // The device's static scratch array (its address is looked up on the first call that
  // gets here on each device); no allocation of any kind.
  void* ws = nullptr;
  if (dattn::static_scratch(&ws) != hipSuccess) return DECODE_ATTN_ERR_HIP;
  return run(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
             max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, kv_dtype, scale, out, lse_out,
             plan, need > 0 ? ws : nullptr, stream);
}

int decode_attn(const void* q, const void* k_pages, const void* v_pages, const float* k_scale,
                const float* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                int batch, int max_blocks_per_seq, int num_pages, int n_q_heads, int n_kv_heads,
                int head_dim, int block_size, int kv_dtype, float scale, float* out,
                hipStream_t stream) {
  int st = validate(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
                    max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, head_dim, block_size,
                    kv_dtype, out, nullptr, 0, 0);
  if (st != DECODE_ATTN_OK) return st;
  if (batch == 0) return DECODE_ATTN_OK;
  int cus = 0;
  st = current_device_cus(&cus);
  if (st != DECODE_ATTN_OK) return st;
  const dattn::Plan plan = make_plan(batch, max_blocks_per_seq, n_kv_heads, kv_of(kv_dtype),
                                     n_q_heads / n_kv_heads, 0, 0, cus);
  st = validate_plan(plan, batch);
  if (st != DECODE_ATTN_OK) return st;
  const size_t need = dattn::workspace_bytes(plan, batch, n_q_heads, n_kv_heads);
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DECODE_ATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_ws_bytes[dev] < need) {
      void* p = nullptr;
      if (hipMalloc(&p, need) != hipSuccess) return DECODE_ATTN_ERR_HIP;
      // The old buffer stays allocated: queued work and graphs captured from earlier
      // calls keep its address.
      if (g_ws[dev] != nullptr) g_ws_retired[dev].push_back(g_ws[dev]);
      g_ws[dev] = p;
      g_ws_bytes[dev] = need;
    }
    ws = g_ws[dev];
  }
  return run(q, k_pages, v_pages, k_scale, v_scale, block_table, seq_lens, batch,
             max_blocks_per_seq, num_pages, n_q_heads, n_kv_heads, kv_dtype, scale, out, nullptr,
             plan, ws, stream);
}

int decode_attn_append(const void* k_new, const void* v_new, const int32_t* block_table,
                       const int32_t* positions, int batch, int max_blocks_per_seq,
                       int num_pages, int n_kv_heads, int head_dim, int block_size,
                       int kv_dtype, void* k_pages, void* v_pages, float* k_scale,
                       float* v_scale, hipStream_t stream) {
  if (batch < 0 || max_blocks_per_seq < 1 || num_pages < 1 || n_kv_heads < 1 ||
      head_dim < 1 || block_size < 1)
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!known_kv(kv_dtype)) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  const bool scaled = scaled_kv(kv_dtype);
  if (scaled != (k_scale != nullptr) || scaled != (v_scale != nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (k_new == nullptr || v_new == nullptr || block_table == nullptr ||
                    positions == nullptr || k_pages == nullptr || v_pages == nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) ||
      !aligned(v_pages, 16) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(block_table, 4) || !aligned(positions, 4))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (head_dim != kHeadDim || block_size != kBlockSize) return DECODE_ATTN_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_blocks_per_seq) * block_size > INT_MAX ||
      static_cast<long long>(batch) * n_kv_heads > INT_MAX ||
      static_cast<long long>(batch) * max_blocks_per_seq > INT_MAX ||
      static_cast<long long>(num_pages) * n_kv_heads > UINT32_MAX)
    return DECODE_ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return DECODE_ATTN_OK;
  (void)hipGetLastError();  // start from a clean error state
  dattn::AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table;
  a.positions = positions;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.batch = batch;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.n_kv_heads = n_kv_heads;
  if (dattn::launch_append(kv_of(kv_dtype), a, stream) != hipSuccess) return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

int decode_attn_prefill(const void* q, const int32_t* q_start, const void* k_pages,
                        const void* v_pages, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens, int batch,
                        int total_rows, int max_blocks_per_seq, int num_pages, int n_q_heads,
                        int n_kv_heads, int head_dim, int block_size, int kv_dtype, int max_chunk,
                        float scale, float* out, hipStream_t stream) {
  int st = validate_shapes(batch, max_blocks_per_seq, n_q_heads, n_kv_heads, block_size, 0, 0);
  if (st != DECODE_ATTN_OK) return st;
  if (num_pages < 1 || head_dim < 1 || total_rows < 0 || max_chunk < 1)
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!known_kv(kv_dtype)) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  const bool scaled = scaled_kv(kv_dtype);
  if (scaled != (k_scale != nullptr) || scaled != (v_scale != nullptr))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (batch > 0 && (q_start == nullptr || block_table == nullptr || seq_lens == nullptr ||
                    k_pages == nullptr || v_pages == nullptr ||
                    (total_rows > 0 && (q == nullptr || out == nullptr))))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(q_start, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(out, 16))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (head_dim != kHeadDim || block_size != kBlockSize) return DECODE_ATTN_ERR_UNSUPPORTED;
  const int group = n_q_heads / n_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return DECODE_ATTN_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_blocks_per_seq) * block_size > INT_MAX ||
      static_cast<long long>(batch) * max_blocks_per_seq > INT_MAX ||
      static_cast<long long>(num_pages) * n_kv_heads > UINT32_MAX ||
      static_cast<long long>(max_chunk) * group > INT_MAX ||
      static_cast<long long>(batch) * n_kv_heads >= (1LL << 24))   // one-dimensional grid
    return DECODE_ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return DECODE_ATTN_OK;
  (void)hipGetLastError();  // start from a clean error state
  dattn::PrefillArgs a{};
  a.q = q;
  a.q_start = q_start;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.batch = batch;
  a.total_rows = total_rows;
  a.max_blocks = max_blocks_per_seq;
  a.num_pages = num_pages;
  a.n_kv_heads = n_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (dattn::launch_prefill(kv_of(kv_dtype), group, a, max_chunk, stream) != hipSuccess)
    return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

int decode_attn_hbm_reference(int kind, int depth, int nontemporal, const void* a,
                              const void* b, const void* a_scale, const void* b_scale,
                              const int32_t* tiles, long long count, long long num_tiles,
                              int grid, uint32_t* sink, hipStream_t stream) {
  if (kind < 0 || kind > 2) return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  const bool depth_ok = kind == 0 ? (depth == 4 || depth == 8 || depth == 16)
                                  : (depth == 1 || depth == 2 || depth == 4);
  if (!depth_ok || (nontemporal != 0 && nontemporal != 1) || grid < 1 || grid > 65535 ||
      count < 0 || num_tiles < 0 || a == nullptr || sink == nullptr || !aligned(a, 16))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (kind >= 1 && (b == nullptr || tiles == nullptr || !aligned(b, 16) || !aligned(tiles, 4)))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (kind == 2 && (a_scale == nullptr || b_scale == nullptr || !aligned(a_scale, 64) ||
                    !aligned(b_scale, 64)))
    return DECODE_ATTN_ERR_INVALID_ARGUMENT;
  if (count == 0) return DECODE_ATTN_OK;
  (void)hipGetLastError();  // start from a clean error state
  dattn::HbmReferenceArgs r{};
  r.kind = kind;
  r.depth = depth;
  r.nontemporal = nontemporal;
  r.grid = grid;
  r.a = a;
  r.b = b;
  r.a_scale = a_scale;
  r.b_scale = b_scale;
  r.tiles = tiles;
  r.count = static_cast<uint64_t>(count);
  r.num_tiles = static_cast<uint64_t>(num_tiles);
  r.sink = sink;
  if (dattn::launch_hbm_reference(r, stream) != hipSuccess) return DECODE_ATTN_ERR_HIP;
  return DECODE_ATTN_OK;
}

const char* decode_attn_status_string(int status) {
  switch (status) {
    case DECODE_ATTN_OK: return "DECODE_ATTN_OK";
    case DECODE_ATTN_ERR_INVALID_ARGUMENT: return "DECODE_ATTN_ERR_INVALID_ARGUMENT";
    case DECODE_ATTN_ERR_UNSUPPORTED: return "DECODE_ATTN_ERR_UNSUPPORTED";
    case DECODE_ATTN_ERR_WORKSPACE: return "DECODE_ATTN_ERR_WORKSPACE";
    case DECODE_ATTN_ERR_HIP: return "DECODE_ATTN_ERR_HIP";
    case DECODE_ATTN_ERR_SCRATCH_LIMIT: return "DECODE_ATTN_ERR_SCRATCH_LIMIT";
    default: return "DECODE_ATTN_UNKNOWN_STATUS";
  }
}

int decode_attn_version(void) { return kVersion; }

}  // extern "C"
