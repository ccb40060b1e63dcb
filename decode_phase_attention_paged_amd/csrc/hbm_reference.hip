// gfx950 reference reads for the HBM roofline. They read memory the way the decode kernels
// do (16 bytes per lane; the (page, KV head) tiles of K and V gathered through an index
// list: 4 KiB for 16-bit formats, 2 KiB of codes plus a 64-byte row-scale record for the
// 1-byte ones) and do no arithmetic beyond folding the loaded bits into one value, so their
// rate is what this GPU delivers to that read pattern: the attainable part of the 8 TB/s
// peak that the decode kernels' roofline fraction is read against. A measurement aid, not
// part of the attention path.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dattn {
namespace {

constexpr int kRefThreads = 256;
constexpr int kRefWaves = kRefThreads / 64;
constexpr int kScaleBytes = 64;                  // one (page, KV head) row-scale record
// Folded bits equal to this value make a lane write its fold to the sink; that keeps every
// load live, and with zero-filled memory it never happens.
constexpr uint32_t kSinkKey = 0x9e3779b9u;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kNt>
__device__ __forceinline__ u32x4 ref_load(const char* p) {
  if constexpr (kNt) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  } else {
    return *reinterpret_cast<const u32x4*>(p);
  }
}

template <bool kNt>
__device__ __forceinline__ uint32_t ref_load_u32(const char* p) {
  if constexpr (kNt) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else {
    return *reinterpret_cast<const uint32_t*>(p);
  }
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Streaming read of `words` 16-byte words: each workgroup step reads kUnroll words per
// lane, consecutive lanes on consecutive words; steps are strided by the grid.
template <int kUnroll, bool kNt>
__global__ __launch_bounds__(kRefThreads) void ref_stream_kernel(const char* buf, uint64_t words,
                                                                 uint32_t* sink) {
  constexpr uint64_t kStep = static_cast<uint64_t>(kRefThreads) * kUnroll;
  uint32_t acc = 0;
  for (uint64_t base = blockIdx.x * kStep; base < words; base += gridDim.x * kStep) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t w = base + static_cast<uint64_t>(u) * kRefThreads + threadIdx.x;
      v[u] = w < words ? ref_load<kNt>(buf + w * 16) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  if (acc == kSinkKey) sink[blockIdx.x * kRefThreads + threadIdx.x] = acc;
}

// Tile gather: entry i of `tiles` names the K tile and the V tile to read (kTileBytes
// each), and with kScaled their row-scale records (kScaleBytes each, lanes reading dwords
// lane % 16 as the decode kernels' lanes read the scales of their rows). Each wave takes an
// equal contiguous run of entries and keeps kDepth entries' loads in flight; entries
// outside [0, num_tiles) are skipped.
template <int kTileBytes, int kDepth, bool kNt>
__global__ __launch_bounds__(kRefThreads) void ref_gather_kernel(const char* k, const char* v,
                                                                 const char* ks, const char* vs,
                                                                 const int32_t* tiles, uint64_t count,
                                                                 uint64_t num_tiles, uint32_t* sink) {
  constexpr bool kScaled = kTileBytes == 2048;
  constexpr int kTileLoads = kTileBytes / (64 * 16);
  const int lane = threadIdx.x & 63;
  const uint64_t wave = static_cast<uint64_t>(blockIdx.x) * kRefWaves +
                        __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const uint64_t waves = static_cast<uint64_t>(gridDim.x) * kRefWaves;
  const uint64_t u0 = wave * count / waves;
  const uint64_t u1 = (wave + 1) * count / waves;
  uint32_t acc = 0;
  for (uint64_t u = u0; u < u1; u += kDepth) {
    u32x4 r[kDepth][2 * kTileLoads];
    uint32_t sc[kDepth][2];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int32_t t = u + d < u1 ? __builtin_amdgcn_readfirstlane(tiles[u + d]) : -1;
      const bool ok = t >= 0 && static_cast<uint64_t>(t) < num_tiles;
      const uint64_t tile = static_cast<uint64_t>(ok ? t : 0);
      const uint64_t off = tile * kTileBytes + lane * 16;
#pragma unroll
      for (int i = 0; i < kTileLoads; ++i) {
        r[d][i] = ok ? ref_load<kNt>(k + off + i * 1024) : u32x4{0u, 0u, 0u, 0u};
        r[d][kTileLoads + i] = ok ? ref_load<kNt>(v + off + i * 1024) : u32x4{0u, 0u, 0u, 0u};
      }
      if constexpr (kScaled) {
        const uint64_t soff = tile * kScaleBytes + (lane & 15) * 4;
        sc[d][0] = ok ? ref_load_u32<kNt>(ks + soff) : 0u;
        sc[d][1] = ok ? ref_load_u32<kNt>(vs + soff) : 0u;
      }
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
#pragma unroll
      for (int i = 0; i < 2 * kTileLoads; ++i) acc ^= fold(r[d][i]);
      if constexpr (kScaled) acc ^= sc[d][0] ^ sc[d][1];
    }
  }
  if (acc == kSinkKey) sink[blockIdx.x * kRefThreads + threadIdx.x] = acc;
}

template <bool kNt>
hipError_t launch_stream(int unroll, const char* a, uint64_t words, int grid, uint32_t* sink,
                         hipStream_t stream) {
  switch (unroll) {
    case 4: hipLaunchKernelGGL((ref_stream_kernel<4, kNt>), dim3(grid), dim3(kRefThreads), 0, stream, a, words, sink); break;
    case 8: hipLaunchKernelGGL((ref_stream_kernel<8, kNt>), dim3(grid), dim3(kRefThreads), 0, stream, a, words, sink); break;
    case 16: hipLaunchKernelGGL((ref_stream_kernel<16, kNt>), dim3(grid), dim3(kRefThreads), 0, stream, a, words, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kTileBytes, bool kNt>
hipError_t launch_gather(const HbmReferenceArgs& r, hipStream_t stream) {
  const char* a = static_cast<const char*>(r.a);
  const char* b = static_cast<const char*>(r.b);
  const char* as = static_cast<const char*>(r.a_scale);
  const char* bs = static_cast<const char*>(r.b_scale);
  switch (r.depth) {
    case 1: hipLaunchKernelGGL((ref_gather_kernel<kTileBytes, 1, kNt>), dim3(r.grid), dim3(kRefThreads), 0, stream, a, b, as, bs, r.tiles, r.count, r.num_tiles, r.sink); break;
    case 2: hipLaunchKernelGGL((ref_gather_kernel<kTileBytes, 2, kNt>), dim3(r.grid), dim3(kRefThreads), 0, stream, a, b, as, bs, r.tiles, r.count, r.num_tiles, r.sink); break;
    case 4: hipLaunchKernelGGL((ref_gather_kernel<kTileBytes, 4, kNt>), dim3(r.grid), dim3(kRefThreads), 0, stream, a, b, as, bs, r.tiles, r.count, r.num_tiles, r.sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_hbm_reference(const HbmReferenceArgs& r, hipStream_t stream) {
  const char* a = static_cast<const char*>(r.a);
  if (r.kind == 0) {
    return r.nontemporal ? launch_stream<true>(r.depth, a, r.count, r.grid, r.sink, stream)
                         : launch_stream<false>(r.depth, a, r.count, r.grid, r.sink, stream);
  }
  if (r.kind == 1) {
    return r.nontemporal ? launch_gather<4096, true>(r, stream) : launch_gather<4096, false>(r, stream);
  }
  return r.nontemporal ? launch_gather<2048, true>(r, stream) : launch_gather<2048, false>(r, stream);
}

}  // namespace dattn
