// gfx950 (MI355X, CDNA4) kernels for decode-phase paged attention.
//
// Split kernel: one 256-thread workgroup per (partition, KV head, sequence). Each of its
// four wavefronts streams every fourth page of the partition straight from HBM into
// VGPRs with 16-byte loads (a (page, head) tile is one contiguous 4 KiB block in fp16,
// so one wave instruction reads 1 KiB of it with no gaps), scores the tile against all
// G query heads that share the KV head (GQA, xLLM README optimisation list), and folds
// the scores into a running max / running sum softmax (the online normaliser of the
// xLLM README SoftMax operator). Dot products over head_dim finish with DPP row
// reductions inside each 16-lane (fp16) or 8-lane (int8) token row, so no LDS and no
// atomics are used in the loop. Waves merge their states through LDS at the end in a
// fixed order. With one partition the workgroup writes the normalised output; with
// several it writes a partial (output, log-sum-exp) per partition, and the merge kernel
// combines them by their log-sum-exp weights (PagedAttention v2 / Flash-Decoding,
// swiftLLM feature list).
//
// The path is bound by HBM bandwidth: per token and KV head it reads 2 * 128 * 2 bytes
// (fp16) for 4 * G * 128 flops, far below the VALU or MFMA ridge point, so the kernel
// spends its effort on keeping enough loads in flight (two pages per wave, software
// pipelined) rather than on matrix cores.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dattn {
namespace {

constexpr int kWave = 64;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// Lane geometry. A lane owns one 16-byte chunk of one token row per load instruction:
// fp16 rows are 256 B = 16 lanes (4 rows per wave load, 4 loads per page), int8 rows are
// 128 B = 8 lanes (8 rows per wave load, 2 loads per page). Load i of a page covers bytes
// [i * 1024, i * 1024 + 1024) of the tile, lane l the 16 bytes at l * 16 within it.
template <KvType kKv>
struct Geo {
  static constexpr int kElem = kKv == KvType::kF16 ? 2 : 1;
  static constexpr int kChunk = 16 / kElem;                 // elements per lane per load
  static constexpr int kLanesPerRow = kHeadDim / kChunk;    // 16 | 8
  static constexpr int kRows = kWave / kLanesPerRow;        // token rows per load: 4 | 8
  static constexpr int kLoads = kBlockSize / kRows;         // loads per page tile: 4 | 2
  static constexpr int kLoadBytes = kRows * kHeadDim * kElem;   // 1024
  static constexpr int kTileBytes = kBlockSize * kHeadDim * kElem;
  static constexpr bool kScaled = kKv == KvType::kI8;
  static constexpr int kPairs = kChunk / 2;                 // fp16 pairs per lane per load
};

// ---------------------------------------------------------------------------------------
// Cross-lane helpers.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i inside each group of 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i inside each row of 16

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over the kLanes (8 or 16) consecutive lanes holding one token row. Each step adds
// a lane's value to its partner's in both lanes, and IEEE addition commutes, so every
// lane of the row ends with the bit-identical total.
template <int kLanes>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(kLanes == 8 || kLanes == 16, "row width");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (kLanes == 16) v += dpp<kDppMirror>(v);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }

// Four int8 values (one dword, lowest address in the low byte) to two exact fp16 pairs.
// Each byte is biased to x + 128 and placed as the low mantissa byte of 1024.0h, which
// gives the fp16 value 1152 + x exactly; subtracting 1152 leaves x exactly.
__device__ __forceinline__ void i8x4_to_h2(uint32_t w, h2& lo, h2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // u0, u1
  const uint32_t c = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // u2, u3
  const h2 bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  lo = as_h2(a) - bias;
  hi = as_h2(c) - bias;
}

template <KvType kKv>
__device__ __forceinline__ void unpack(const u32x4& raw, h2 (&x)[Geo<kKv>::kPairs]) {
  if constexpr (kKv == KvType::kF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = as_h2(raw[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) i8x4_to_h2(raw[e], x[2 * e], x[2 * e + 1]);
  }
}

// ---------------------------------------------------------------------------------------
// One page tile of K and V for one KV head, held in VGPRs.
template <KvType kKv>
struct Tile {
  using Gm = Geo<kKv>;
  u32x4 k[Gm::kLoads];
  u32x4 v[Gm::kLoads];
  float ks[Gm::kScaled ? Gm::kLoads : 1];
  float vs[Gm::kScaled ? Gm::kLoads : 1];
};

template <KvType kKv>
__device__ __forceinline__ void load_tile(Tile<kKv>& t, const SplitArgs& a, int phys, int g,
                                          int lane) {
  using Gm = Geo<kKv>;
  const size_t tile = static_cast<size_t>(phys) * a.n_kv_heads + g;
  const char* kb = static_cast<const char*>(a.k_pages) + tile * Gm::kTileBytes + lane * 16;
  const char* vb = static_cast<const char*>(a.v_pages) + tile * Gm::kTileBytes + lane * 16;
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) {
    t.k[i] = *reinterpret_cast<const u32x4*>(kb + i * Gm::kLoadBytes);
    t.v[i] = *reinterpret_cast<const u32x4*>(vb + i * Gm::kLoadBytes);
  }
  if constexpr (Gm::kScaled) {
    const int row = lane / Gm::kLanesPerRow;
    const float* ksb = a.k_scale + tile * kBlockSize + row;
    const float* vsb = a.v_scale + tile * kBlockSize + row;
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) {
      t.ks[i] = ksb[i * Gm::kRows];
      t.vs[i] = vsb[i * Gm::kRows];
    }
  }
}

// Per-lane softmax state for the G query heads of this KV head. All lanes of one token
// row see the same tokens and hold the same m and l; acc holds this lane's kChunk
// output columns. Scores are kept in log2 units (scale * log2 e folded in).
template <KvType kKv, int kGroup>
struct State {
  float m[kGroup];
  float l[kGroup];
  float acc[kGroup][Geo<kKv>::kChunk];
};

// Fold one page tile into the running state. With kMasked, tokens at or past `valid`
// inside the page contribute nothing, whatever their K, V or scale slots hold.
template <KvType kKv, int kGroup, bool kMasked>
__device__ __forceinline__ void consume_tile(Tile<kKv>& t, State<kKv, kGroup>& st,
                                             const h2 (&qh)[kGroup][Geo<kKv>::kPairs],
                                             float scale_log2, int row, int valid) {
  using Gm = Geo<kKv>;
  float s[kGroup][Gm::kLoads];
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) {
    h2 kx[Gm::kPairs];
    unpack<kKv>(t.k[i], kx);
    float f = scale_log2;
    if constexpr (Gm::kScaled) f *= t.ks[i];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < Gm::kPairs; ++e) d = __builtin_amdgcn_fdot2(kx[e], qh[h][e], d, false);
      s[h][i] = row_sum<Gm::kLanesPerRow>(d) * f;
    }
  }
  if constexpr (kMasked) {
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) {
      const bool ok = i * Gm::kRows + row < valid;
#pragma unroll
      for (int h = 0; h < kGroup; ++h) s[h][i] = ok ? s[h][i] : kNegInf;
      if (!ok) {
        t.v[i] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (Gm::kScaled) t.vs[i] = 0.0f;
      }
    }
  }
  float p[kGroup][Gm::kLoads];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    float mx = s[h][0];
#pragma unroll
    for (int i = 1; i < Gm::kLoads; ++i) mx = fmaxf(mx, s[h][i]);
    const float m_new = fmaxf(st.m[h], mx);
    const float base = m_new == kNegInf ? 0.0f : m_new;
    const float alpha = fast_exp2(st.m[h] - base);
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) {
      p[h][i] = fast_exp2(s[h][i] - base);
      sum += p[h][i];
    }
    st.l[h] = st.l[h] * alpha + sum;
#pragma unroll
    for (int j = 0; j < Gm::kChunk; ++j) st.acc[h][j] *= alpha;
    st.m[h] = m_new;
  }
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) {
    h2 vx[Gm::kPairs];
    unpack<kKv>(t.v[i], vx);
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float pw = p[h][i];
      if constexpr (Gm::kScaled) pw *= t.vs[i];
#pragma unroll
      for (int e = 0; e < Gm::kPairs; ++e) {
        st.acc[h][2 * e] = fmaf(pw, static_cast<float>(vx[e].x), st.acc[h][2 * e]);
        st.acc[h][2 * e + 1] = fmaf(pw, static_cast<float>(vx[e].y), st.acc[h][2 * e + 1]);
      }
    }
  }
}

// Merge the (m, l, acc) of the lane `off` away into this lane's, for every head.
template <KvType kKv, int kGroup>
__device__ __forceinline__ void merge_lanes(State<kKv, kGroup>& st, int off) {
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    const float mo = __shfl_xor(st.m[h], off);
    const float lo = __shfl_xor(st.l[h], off);
    const float mm = fmaxf(st.m[h], mo);
    const float base = mm == kNegInf ? 0.0f : mm;
    const float wa = fast_exp2(st.m[h] - base);
    const float wb = fast_exp2(mo - base);
    st.l[h] = st.l[h] * wa + lo * wb;
#pragma unroll
    for (int j = 0; j < Geo<kKv>::kChunk; ++j) {
      const float ao = __shfl_xor(st.acc[h][j], off);
      st.acc[h][j] = st.acc[h][j] * wa + ao * wb;
    }
    st.m[h] = mm;
  }
}

template <KvType kKv, int kGroup>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(SplitArgs a) {
  using Gm = Geo<kKv>;
  __shared__ float sm_acc[kWaves][kGroup][kHeadDim];
  __shared__ float sm_m[kWaves][kGroup];
  __shared__ float sm_l[kWaves][kGroup];
  __shared__ int sm_bad[kWaves];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row = lane / Gm::kLanesPerRow;
  const int col = lane % Gm::kLanesPerRow;

  int wg = blockIdx.x;
  const int split = wg % a.num_splits;
  wg /= a.num_splits;
  const int g = wg % a.n_kv_heads;
  const int b = wg / a.n_kv_heads;

  const int seq_len = a.seq_lens[b];
  const bool bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockSize;
  const int nb = bad_len ? 0 : (seq_len + kBlockSize - 1) / kBlockSize;
  const int j0 = split * a.pages_per_split;
  const int j1 = min(j0 + a.pages_per_split, nb);
  // A partition with no tokens is never read by the merge; with a single partition the
  // workgroup still runs to write zeros (empty cache) or NaN (bad length).
  if (a.num_splits > 1 && j0 >= j1) return;

  const int group_base = g * kGroup;
  h2 qh[kGroup][Gm::kPairs];
  {
    const _Float16* qb = static_cast<const _Float16*>(a.q) +
                         (static_cast<size_t>(b) * a.n_q_heads + group_base) * kHeadDim +
                         col * Gm::kChunk;
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
#pragma unroll
      for (int c = 0; c < Gm::kChunk / 8; ++c) {
        const u32x4 raw = *reinterpret_cast<const u32x4*>(qb + h * kHeadDim + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) qh[h][c * 4 + e] = as_h2(raw[e]);
      }
    }
  }

  State<kKv, kGroup> st;
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < Gm::kChunk; ++j) st.acc[h][j] = 0.0f;
  }

  bool bad = bad_len;
  const int npages = j1 - j0;
  const int n_mine = npages > wave ? (npages - wave + kWaves - 1) / kWaves : 0;
  const int32_t* bt = a.block_table + static_cast<size_t>(b) * a.max_blocks + j0 + wave;
  for (int k0 = 0; k0 < n_mine && !bad; k0 += kWave) {
    const int cnt = min(kWave, n_mine - k0);
    // One table entry per lane for the next (up to) 64 pages of this wave; every entry
    // is range-checked before any page is touched.
    const int phys = lane < cnt ? bt[static_cast<size_t>(k0 + lane) * kWaves] : 0;
    if (__any(lane < cnt && static_cast<unsigned>(phys) >= static_cast<unsigned>(a.num_pages))) {
      bad = true;
      break;
    }
    const int j_last = j0 + wave + (k0 + cnt - 1) * kWaves;
    const int valid_last = min(kBlockSize, seq_len - j_last * kBlockSize);

    Tile<kKv> ta, tb;
    load_tile<kKv>(ta, a, __builtin_amdgcn_readlane(phys, 0), g, lane);
    int k = 0;
    for (; k + 2 < cnt; k += 2) {
      load_tile<kKv>(tb, a, __builtin_amdgcn_readlane(phys, k + 1), g, lane);
      consume_tile<kKv, kGroup, false>(ta, st, qh, a.scale_log2, row, kBlockSize);
      load_tile<kKv>(ta, a, __builtin_amdgcn_readlane(phys, k + 2), g, lane);
      consume_tile<kKv, kGroup, false>(tb, st, qh, a.scale_log2, row, kBlockSize);
    }
    if (cnt - k == 2) {
      load_tile<kKv>(tb, a, __builtin_amdgcn_readlane(phys, k + 1), g, lane);
      consume_tile<kKv, kGroup, false>(ta, st, qh, a.scale_log2, row, kBlockSize);
      consume_tile<kKv, kGroup, true>(tb, st, qh, a.scale_log2, row, valid_last);
    } else {
      consume_tile<kKv, kGroup, true>(ta, st, qh, a.scale_log2, row, valid_last);
    }
  }

  // Rows of this wave saw disjoint tokens: merge them so every lane holds the wave's
  // state for its columns.
#pragma unroll
  for (int off = Gm::kLanesPerRow; off < kWave; off <<= 1) merge_lanes<kKv, kGroup>(st, off);

  if (row == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h)
#pragma unroll
      for (int j = 0; j < Gm::kChunk; ++j) sm_acc[wave][h][col * Gm::kChunk + j] = st.acc[h][j];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      sm_m[wave][h] = st.m[h];
      sm_l[wave][h] = st.l[h];
    }
    sm_bad[wave] = bad ? 1 : 0;
  }
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_bad |= sm_bad[w] != 0;
  const float nan = __builtin_nanf("");
  for (int o = threadIdx.x; o < kGroup * kHeadDim; o += kSplitThreads) {
    const int h = o / kHeadDim;
    const int d = o % kHeadDim;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm_m[w][h]);
    const float base = mm == kNegInf ? 0.0f : mm;
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(sm_m[w][h] - base);
      num += e * sm_acc[w][h][d];
      den += e * sm_l[w][h];
    }
    const float val = any_bad ? nan : (den > 0.0f ? num / den : 0.0f);
    const float lse2 = any_bad ? nan : (den > 0.0f ? mm + __log2f(den) : kNegInf);
    const size_t qrow = static_cast<size_t>(b) * a.n_q_heads + group_base + h;
    if (a.num_splits == 1) {
      a.out[qrow * kHeadDim + d] = val;
      if (a.lse_out != nullptr && d == 0) a.lse_out[qrow] = lse2 * kLn2;
    } else {
      const size_t slot = qrow * a.num_splits + split;
      a.part_o[slot * kHeadDim + d] = val;
      if (d == 0) a.part_lse[slot] = lse2;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Merge kernel: one workgroup per (sequence, query head). Partition s holds the
// normalised partial output o_s and lse_s (log2 units) over its tokens; the result is
// sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M) with M = max_s lse_s, summed in a fixed
// order. Only partitions that hold tokens of the sequence are read.

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

constexpr int kMergeWaves = kMergeThreads / kWave;
constexpr int kMergeParts = kMergeThreads / kHeadDim;   // partition subsets summed apart

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  __shared__ float sm_red[kMergeWaves];
  __shared__ int sm_nan[kMergeWaves];
  __shared__ float sm_part[kMergeParts][kHeadDim];

  const int qrow = blockIdx.x;   // b * Hq + h
  const int b = qrow / a.n_q_heads;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  const int seq_len = a.seq_lens[b];
  const bool bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockSize;
  const int nb = bad_len ? 0 : (seq_len + kBlockSize - 1) / kBlockSize;
  const int ns = (nb + a.pages_per_split - 1) / a.pages_per_split;
  const float* lse = a.part_lse + static_cast<size_t>(qrow) * a.num_splits;
  const float* po = a.part_o + static_cast<size_t>(qrow) * a.num_splits * kHeadDim;

  // M = max_s lse_s, and whether any partition reported NaN (a bad page).
  float mx = kNegInf;
  int has_nan = 0;
  for (int s = tid; s < ns; s += kMergeThreads) {
    const float v = lse[s];
    has_nan |= v != v;
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  has_nan = __any(has_nan) ? 1 : 0;
  if (lane == 0) {
    sm_red[wave] = mx;
    sm_nan[wave] = has_nan;
  }
  __syncthreads();
  mx = sm_red[0];
  has_nan = sm_nan[0];
#pragma unroll
  for (int w = 1; w < kMergeWaves; ++w) {
    mx = fmaxf(mx, sm_red[w]);
    has_nan |= sm_nan[w];
  }
  const float base = mx == kNegInf ? 0.0f : mx;
  __syncthreads();

  // Denominator sum_s 2^(lse_s - M), reduced in a fixed tree order.
  float den = 0.0f;
  for (int s = tid; s < ns; s += kMergeThreads) den += fast_exp2(lse[s] - base);
  den = wave_sum(den);
  if (lane == 0) sm_red[wave] = den;
  __syncthreads();
  den = 0.0f;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) den += sm_red[w];

  // Numerator: thread (part, d) sums partitions part, part + kMergeParts, ...
  const int d = tid % kHeadDim;
  const int part = tid / kHeadDim;
  float num = 0.0f;
#pragma unroll 4
  for (int s = part; s < ns; s += kMergeParts)
    num += fast_exp2(lse[s] - base) * po[static_cast<size_t>(s) * kHeadDim + d];
  sm_part[part][d] = num;
  __syncthreads();
  if (part == 0) {
    float total = 0.0f;
#pragma unroll
    for (int p = 0; p < kMergeParts; ++p) total += sm_part[p][d];
    const bool poisoned = bad_len || has_nan;
    const float nan = __builtin_nanf("");
    a.out[static_cast<size_t>(qrow) * kHeadDim + d] =
        poisoned ? nan : (den > 0.0f ? total / den : 0.0f);
    if (a.lse_out != nullptr && d == 0)
      a.lse_out[qrow] = poisoned ? nan : (den > 0.0f ? (mx + __log2f(den)) * kLn2 : kNegInf);
  }
}

template <KvType kKv, int kGroup>
hipError_t launch_split_t(const SplitArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.num_splits) * a.n_kv_heads * a.batch;
  hipLaunchKernelGGL((split_kernel<kKv, kGroup>), dim3(grid), dim3(kSplitThreads), 0, stream, a);
  return hipGetLastError();
}

template <KvType kKv>
hipError_t launch_split_kv(int group, const SplitArgs& a, hipStream_t stream) {
  switch (group) {
    case 1: return launch_split_t<kKv, 1>(a, stream);
    case 2: return launch_split_t<kKv, 2>(a, stream);
    case 4: return launch_split_t<kKv, 4>(a, stream);
    case 8: return launch_split_t<kKv, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_split(KvType kv, int group, const SplitArgs& a, hipStream_t stream) {
  return kv == KvType::kF16 ? launch_split_kv<KvType::kF16>(group, a, stream)
                            : launch_split_kv<KvType::kI8>(group, a, stream);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.batch) * a.n_q_heads;
  hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dattn
