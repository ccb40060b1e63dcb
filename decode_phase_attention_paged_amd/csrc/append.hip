// gfx950 kernel that writes a decode step's new K/V rows into the paged cache.
//
// Every decode step adds the new token's key and value to the cache before attending
// (page "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen", section 1.1).
// Token position p of sequence b lives in page block_table[b, p / 16], slot p % 16
// (PagedAttention, swiftLLM feature list). FP16 and BF16 pools take the row as it is.
// INT8 pools (per-row INT8, xLLM README quantisation list) take symmetric max-abs codes
// with round-half-to-even, computed in fp32: s = max|x| / 127, code = rint(x / s), with IEEE
// division. FP8 pools (E4M3, the cache format named in section 4 of the C++/CUDA engine
// page) take s = max|x| / 448 and the nearest E4M3 code of x / s, ties to even, from the
// hardware conversion. Codes and scales are the same bits on every run; a row of zeros
// stores scale 0 and codes 0.
//
// One wavefront per two (sequence, KV head) rows: in each half of the wave, lanes 0..15
// carry the K row and lanes 16..31 the V row, 16 bytes of input each; the max of a
// quantised row runs as a DPP reduction inside its row of 16 lanes. The new rows are read
// before the position and table entry, so the two latencies overlap. Rows whose position
// is negative (no new token), at or past the table's reach, or whose page id is outside
// the pools are skipped: nothing is written for them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dattn {
namespace {

constexpr int kAppendWaves = 4;
constexpr int kAppendThreads = 64 * kAppendWaves;
constexpr int kRowLanes = kHeadDim * 2 / 16;   // lanes holding one fp16 row: 16

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i inside each group of 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i inside each row of 16

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Maximum over the 16 lanes of one DPP row; every lane of the row gets it.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}

// Eight fp16 values of one 16-byte chunk as fp32.
__device__ __forceinline__ void widen8(const u32x4& raw, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // Copy the element out first: a bit cast applied to raw[e] directly reads element 0.
    const uint32_t word = raw[e];
    const h2 pr = __builtin_bit_cast(h2, word);
    x[2 * e] = static_cast<float>(pr.x);
    x[2 * e + 1] = static_cast<float>(pr.y);
  }
}

template <KvType kKv>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const long long row =
      (static_cast<long long>(blockIdx.x) * kAppendWaves + wave) * 2 + (lane >> 5);
  const long long rows = static_cast<long long>(a.batch) * a.n_kv_heads;
  if (row >= rows) return;
  const bool is_v = (lane & 31) >= kRowLanes;
  const int chunk = lane % kRowLanes;   // 8 elements of the row
  const size_t src_row = static_cast<size_t>(row) * kHeadDim;
  const void* src = is_v ? a.v_new : a.k_new;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + src_row + chunk * 8);
  const int b = static_cast<int>(row / a.n_kv_heads);
  const int g = static_cast<int>(row - static_cast<long long>(b) * a.n_kv_heads);
  const int p = a.positions[b];
  if (p < 0 || p >= a.max_blocks * kBlockSize) return;
  const int phys = a.block_table[static_cast<size_t>(b) * a.max_blocks + p / kBlockSize];
  if (phys < 0 || phys >= a.num_pages) return;
  const size_t dst_row =
      (static_cast<size_t>(static_cast<uint32_t>(phys) * static_cast<uint32_t>(a.n_kv_heads) + g) *
           kBlockSize + p % kBlockSize);

  if constexpr (kv_elem_bytes(kKv) == 2) {
    uint16_t* dst = static_cast<uint16_t*>(is_v ? a.v_pages : a.k_pages);
    *reinterpret_cast<u32x4*>(dst + dst_row * kHeadDim + chunk * 8) = raw;
  } else {
    float x[8];
    widen8(raw, x);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
    m = row_max16(m);
    constexpr float kTop = kKv == KvType::kI8 ? 127.0f : 448.0f;   // largest code magnitude
    const float s = m / kTop;
    uint32_t packed[2] = {0u, 0u};
    if (m != 0.0f) {
      if constexpr (kKv == KvType::kI8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float c = fminf(fmaxf(__builtin_rintf(x[i] / s), -127.0f), 127.0f);
          packed[i / 4] |= (static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xFFu) << (8 * (i % 4));
        }
      } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w] / s, x[4 * w + 1] / s, 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2] / s, x[4 * w + 3] / s, word, true);
          packed[w] = static_cast<uint32_t>(word);
        }
      }
    }
    uint8_t* dst = static_cast<uint8_t*>(is_v ? a.v_pages : a.k_pages);
    *reinterpret_cast<uint2*>(dst + dst_row * kHeadDim + chunk * 8) = make_uint2(packed[0], packed[1]);
    if (chunk == 0) (is_v ? a.v_scale : a.k_scale)[dst_row] = s;
  }
}

}  // namespace

hipError_t launch_append(KvType kv, const AppendArgs& a, hipStream_t stream) {
  const long long rows = static_cast<long long>(a.batch) * a.n_kv_heads;
  const long long rows_per_block = 2LL * kAppendWaves;
  const unsigned grid = static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block);
  switch (kv) {
    case KvType::kF16:
      hipLaunchKernelGGL(append_kernel<KvType::kF16>, dim3(grid), dim3(kAppendThreads), 0, stream, a);
      break;
    case KvType::kI8:
      hipLaunchKernelGGL(append_kernel<KvType::kI8>, dim3(grid), dim3(kAppendThreads), 0, stream, a);
      break;
    case KvType::kBF16:
      hipLaunchKernelGGL(append_kernel<KvType::kBF16>, dim3(grid), dim3(kAppendThreads), 0, stream, a);
      break;
    case KvType::kFP8:
      hipLaunchKernelGGL(append_kernel<KvType::kFP8>, dim3(grid), dim3(kAppendThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace dattn
