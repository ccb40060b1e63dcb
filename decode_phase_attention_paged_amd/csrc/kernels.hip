// gfx950 (MI355X, CDNA4) kernels for decode-phase paged attention.
//
// A unit is one (sequence b, KV head g, logical page j): the 16 tokens of one KV head in
// one page, i.e. one K tile and one V tile (4 KiB each in fp16). A segment is the run of
// units of one (b, g) pair. Every kernel here streams units from HBM straight into VGPRs
// with 16-byte non-temporal loads, keeps several units in flight per wave, and scores each
// tile against all G query heads sharing the KV head (GQA, xLLM README optimisation list),
// folding the scores into a running max / running sum softmax (the online normaliser of
// the xLLM README SoftMax operator). Two tile consumes exist: with G <= 2 the vector ALU
// (dot products finished with DPP reductions inside each token row of 16 lanes for 16-bit
// formats, 8 for 1-byte ones); with G >= 4 the matrix cores, the G heads as the N columns
// of 16x16 MFMA tiles for both the scores and the weighted sum. Where a segment is cut
// between workers, the pieces leave partial (output, log-sum-exp) pairs that a second
// kernel merges by their log-sum-exp weights in a fixed order (PagedAttention v2 /
// Flash-Decoding, swiftLLM feature list). No atomics anywhere, so a given plan gives
// bitwise-identical results.
//
// Three ways of cutting the batch into work:
//  * segment mode: a fixed grid of persistent workgroups takes whole segments, longest
//    sequences first; a workgroup's four waves share each segment's pages and merge their
//    states in LDS, so nothing is cut and no second kernel runs. Used for most batches.
//  * stream mode: a fixed grid of persistent workgroups; units are numbered b-major, then
//    g, then j, and wavefront w of W takes units [w T / W, (w + 1) T / W) of the T units.
//    Every wave streams the same number of pages whatever the mix of lengths. The
//    library's choice only for 1-byte caches with G <= 2 and one to two segments per
//    compute unit over long caches.
//  * split mode: one workgroup per (page partition, g, b), its four waves interleaving the
//    partition's pages and merging in LDS. Used for fewer segments than compute units over
//    long caches.
//
// The path is bound by HBM bandwidth: per token and KV head it reads 2 * 128 * 2 bytes
// (fp16) for 4 * G * 128 flops, far below the VALU or MFMA ridge point, so the design
// spends its effort on keeping loads in flight; the matrix cores take the tile products
// only where G made the vector ALU work per byte large enough to matter. The only vector
// memory operations inside the streaming loops are the tile loads: page ids come through
// scalar loads (or LDS) and query rows from LDS, so the compiler can wait for exactly the
// oldest tile and leave the newer ones in flight.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "kernels.h"

namespace dattn {
namespace {

constexpr int kWave = 64;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kQLdsBytes = 16384;   // query rows a stream workgroup stages in LDS
constexpr int kSplitTable = 1024;   // table entries a split workgroup stages in LDS at a time

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// Lane geometry. A lane owns one chunk of one token row per load instruction.
// fp16: a row is 256 B = 16 lanes of 16 B; load i of a tile covers tokens 4i .. 4i+3, i.e.
//       the contiguous bytes [1024 i, 1024 i + 1024), lane l at byte 16 l.
// int8: a row is 128 B = 8 lanes of 16 B; lane row r covers tokens 2r and 2r + 1 (loads 0
//       and 1) so that its two row scales are one 8-byte load.
// bf16 takes the fp16 geometry and fp8 the int8 one. These are the vector-ALU builds (G <= 2);
// G >= 4 runs on the matrix cores with its own layout (below).
template <KvType kKv, int kGroup>
struct Geo {
  static constexpr int kElem = kv_elem_bytes(kKv);
  static constexpr int kLoadBytes = 16;                     // bytes per lane per load
  static constexpr int kWords = kLoadBytes / 4;
  static constexpr int kChunk = kLoadBytes / kElem;         // elements per lane per load
  static constexpr int kLanesPerRow = kHeadDim / kChunk;    // 16 | 8
  static constexpr int kRows = kWave / kLanesPerRow;        // lane rows: 4 | 8
  static constexpr int kLoads = kBlockSize / kRows;         // loads per tile: 4 | 2
  static constexpr int kRowBytes = kHeadDim * kElem;
  static constexpr int kTileBytes = kBlockSize * kRowBytes;
  static constexpr bool kScaled = kv_scaled(kKv);
  static constexpr int kPairs = kChunk / 2;                 // element pairs per lane per load
  using Load = u32x4;

  __device__ static int token(int row, int i) {
    if constexpr (kElem == 2) return i * kRows + row;
    else return kLoads * row + i;
  }
  __device__ static int offset(int lane, int i) {
    if constexpr (kElem == 2) return i * 1024 + lane * 16;
    else return token(lane / kLanesPerRow, i) * kRowBytes + (lane % kLanesPerRow) * kLoadBytes;
  }
};

// Tuning per kernel: units kept in flight per wave, and the waves per SIMD the kernel is
// compiled for (which caps its VGPRs at 512 / waves). Vector-ALU builds (G <= 2) are
// indexed by log2 G; the matrix-core builds (G >= 4) by element width (0: 2-byte, 1: 1-byte).
constexpr int kStreamDepthF16[2] = {4, 4};
constexpr int kStreamDepthI8[2] = {6, 4};
constexpr int kStreamDepthMf[2] = {3, 3};
constexpr int kStreamWavesF16[2] = {2, 2};
constexpr int kStreamWavesI8[2] = {2, 2};
constexpr int kStreamWavesMf[2] = {2, 1};
// Split mode runs a few long partitions per sequence, about one workgroup per CU, so each
// wave keeps many tiles in flight.
constexpr int kSplitDepthF16[2] = {4, 4};
constexpr int kSplitDepthI8[2] = {6, 4};
constexpr int kSplitDepthMf[2] = {3, 3};
constexpr int kSplitWavesF16[2] = {1, 1};
constexpr int kSplitWavesI8[2] = {1, 1};
constexpr int kSplitWavesMf[2] = {1, 1};
// Segment mode (waves per SIMD in kSegWaves*, kernels.h, which the host plan also reads).
// Shallow rings (one or two units in flight per wave) measured faster than deep ones: with
// about 16 MB of tiles in flight over the chip, more only lengthens the memory queue.
constexpr int kSegDepthF16[2] = {2, 2};
constexpr int kSegDepthI8[2] = {1, 3};
constexpr int kSegDepthMf[2] = {2, 2};

template <KvType kKv, int kGroup>
constexpr int pick(const int (&f16)[2], const int (&i8)[2], const int (&mf)[2]) {
  return use_mfma(kKv, kGroup)       ? mf[width_index(kKv)]
         : kv_elem_bytes(kKv) == 2 ? f16[log2_group(kGroup)]
                                   : i8[log2_group(kGroup)];
}
template <KvType kKv, int kGroup>
constexpr int stream_depth() { return pick<kKv, kGroup>(kStreamDepthF16, kStreamDepthI8, kStreamDepthMf); }
template <KvType kKv, int kGroup>
constexpr int stream_waves() { return pick<kKv, kGroup>(kStreamWavesF16, kStreamWavesI8, kStreamWavesMf); }
template <KvType kKv, int kGroup>
constexpr int split_depth() { return pick<kKv, kGroup>(kSplitDepthF16, kSplitDepthI8, kSplitDepthMf); }
template <KvType kKv, int kGroup>
constexpr int split_waves() { return pick<kKv, kGroup>(kSplitWavesF16, kSplitWavesI8, kSplitWavesMf); }
template <KvType kKv, int kGroup>
constexpr int seg_depth() { return pick<kKv, kGroup>(kSegDepthF16, kSegDepthI8, kSegDepthMf); }

// ---------------------------------------------------------------------------------------
// Cross-lane and conversion helpers.
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

// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one lane of each 16-lane row)
// on the VALU: v_permlane16_swap of a value with itself leaves rows (0, 0, 2, 2) in one
// result and (1, 1, 3, 3) in the other, v_permlane32_swap the halves (lo, lo) and (hi, hi).
// Every lane of the four ends with the same bits. (A shuffle through ds_bpermute would wait
// on the LDS queue, behind the operand reads in flight.) The two results are copied out
// before any bit cast: a bit cast of an element of the returned pair read element 0.
__device__ __forceinline__ float max_across_rows(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float m = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t w = __builtin_bit_cast(uint32_t, m);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}
__device__ __forceinline__ float sum_across_rows(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float s = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const uint32_t w = __builtin_bit_cast(uint32_t, s);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}


__device__ __forceinline__ h2 as_h2(uint32_t w) { return __builtin_bit_cast(h2, w); }
__device__ __forceinline__ bf2 as_bf2(uint32_t w) { return __builtin_bit_cast(bf2, w); }

// The two bf16 values of a dword as exact fp32: a bf16 is the upper half of an fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

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

// The same four int8 values as 1152 + x, exactly, without the subtraction: the vector-ALU
// consume takes 1152 times the sum of what it multiplies out once per load (scores) or
// once per segment (outputs) instead of once per pair.
constexpr float kI8Bias = 1152.0f;
__device__ __forceinline__ void i8x4_to_h2_biased(uint32_t w, h2& lo, h2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));  // 1152 + x0, 1152 + x1
  hi = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));  // 1152 + x2, 1152 + x3
}

// Four E4M3 codes (one dword, lowest address in the low byte) to two fp16 pairs. Every
// finite E4M3 value is exact in fp16 (magnitudes 2^-9 .. 448), and the hardware conversion
// (unit scale) maps the NaN codes to NaN.
__device__ __forceinline__ void fp8x4_to_h2(uint32_t w, h2& lo, h2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

// A load's elements as exact fp16 pairs (fp16, int8 and fp8 storage; bf16 values are not
// all fp16 values and take their own path). INT8 elements come out as 1152 + x.
template <KvType kKv, int kGroup>
__device__ __forceinline__ void unpack(const typename Geo<kKv, kGroup>::Load& raw,
                                       h2 (&x)[Geo<kKv, kGroup>::kPairs]) {
  static_assert(kKv != KvType::kBF16, "bf16 is not unpacked to fp16");
  constexpr int kWords = Geo<kKv, kGroup>::kWords;
  if constexpr (kKv == KvType::kF16) {
#pragma unroll
    for (int e = 0; e < kWords; ++e) x[e] = as_h2(raw[e]);
  } else if constexpr (kKv == KvType::kI8) {
#pragma unroll
    for (int e = 0; e < kWords; ++e) i8x4_to_h2_biased(raw[e], x[2 * e], x[2 * e + 1]);
  } else {
#pragma unroll
    for (int e = 0; e < kWords; ++e) fp8x4_to_h2(raw[e], x[2 * e], x[2 * e + 1]);
  }
}

// q . k over this lane's elements of one load, accumulated in fp32 onto d. The query pairs
// hold the query's raw 16-bit patterns: fp16 for every format but bf16, whose q is bf16.
// For INT8 this is q . (k + 1152); the caller takes off 1152 times the sum of the q pairs.
template <KvType kKv, int kGroup>
__device__ __forceinline__ float dot_row(const typename Geo<kKv, kGroup>::Load& raw,
                                         const h2 (&q)[Geo<kKv, kGroup>::kPairs]) {
  float d = 0.0f;
  if constexpr (kKv == KvType::kBF16) {
#pragma unroll
    for (int e = 0; e < Geo<kKv, kGroup>::kPairs; ++e) {
      const uint32_t word = raw[e];
      d = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(word), __builtin_bit_cast(bf2, q[e]), d, false);
    }
  } else {
    h2 kx[Geo<kKv, kGroup>::kPairs];
    unpack<kKv, kGroup>(raw, kx);
#pragma unroll
    for (int e = 0; e < Geo<kKv, kGroup>::kPairs; ++e) d = __builtin_amdgcn_fdot2(kx[e], q[e], d, false);
  }
  return d;
}

// acc[j] += w * v[j] over this lane's elements of one load (for INT8, w * (v[j] + 1152): the
// state keeps the sum of the weights and takes 1152 times it off when the outputs leave).
template <KvType kKv, int kGroup>
__device__ __forceinline__ void axpy_row(const typename Geo<kKv, kGroup>::Load& raw, float w,
                                         float (&acc)[Geo<kKv, kGroup>::kChunk]) {
  if constexpr (kKv == KvType::kBF16) {
#pragma unroll
    for (int e = 0; e < Geo<kKv, kGroup>::kPairs; ++e) {
      const uint32_t word = raw[e];
      acc[2 * e] = fmaf(w, bf16_lo(word), acc[2 * e]);
      acc[2 * e + 1] = fmaf(w, bf16_hi(word), acc[2 * e + 1]);
    }
  } else {
    h2 vx[Geo<kKv, kGroup>::kPairs];
    unpack<kKv, kGroup>(raw, vx);
#pragma unroll
    for (int e = 0; e < Geo<kKv, kGroup>::kPairs; ++e) {
      acc[2 * e] = fmaf(w, static_cast<float>(vx[e].x), acc[2 * e]);
      acc[2 * e + 1] = fmaf(w, static_cast<float>(vx[e].y), acc[2 * e + 1]);
    }
  }
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ uint32_t lds_scalar(const uint32_t* p) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(*p)));
}

// Read-only scalar load (constant address space: through the scalar cache, counted apart
// from the vector loads in flight).
__device__ __forceinline__ int32_t scalar_load(const int32_t* base, size_t idx) {
  typedef const __attribute__((address_space(4))) int32_t* ConstPtr;
  return ((ConstPtr)(base))[idx];
}

// ---------------------------------------------------------------------------------------
// One page tile of K and V for one KV head, held in VGPRs.
template <KvType kKv, int kGroup>
struct Tile {
  using Gm = Geo<kKv, kGroup>;
  typename Gm::Load k[Gm::kLoads];
  typename Gm::Load v[Gm::kLoads];
  float ks[Gm::kScaled ? Gm::kLoads : 1];   // row scale of the token of load i
  float vs[Gm::kScaled ? Gm::kLoads : 1];
};

// Cache tiles are read once per step, so their loads carry the non-temporal hint: a random
// 4 KiB tile gather streams about 12 % faster from HBM with it than without (6.6-6.7 against
// 5.9-6.0 TB/s on MI355X, measured with the reference reads of hbm_reference.hip), and a
// plain streaming read 6.7-7.1 against 5.8-6.3 TB/s.
template <typename T>
__device__ __forceinline__ T stream_load(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// A ring slot with no unit left keeps loading, so that every wait on the ring stays an
// exact vmcnt count, but it loads a tile it has already read with this many valid tokens:
// every lane then reads the tile's first row, one or two cache lines. Re-reading whole tiles
// instead cost HBM traffic: non-temporal lines are not kept in L2 for a second read (one
// extra tile per wave per slot, 3-4 % of the bytes of a step).
constexpr int kIdleValid = 1;

// Tile index = phys * Hkv + g. A unit whose page id failed the range check reads tile 0
// instead (its output is NaN whatever is read), so every load targets a valid tile.
// `valid` is the number of the page's tokens inside the sequence. On a partly filled last
// page (0 < valid < 16) the lanes of rows at or past `valid` load the last valid row
// instead: their addresses fall in cache lines the wave reads anyway, so rows the softmax
// masks out cost no HBM traffic. Other values (full pages, and units that only re-read an
// earlier tile) load the whole tile with immediate offsets.
template <KvType kKv, int kGroup>
__device__ __forceinline__ void load_tile(Tile<kKv, kGroup>& t, const Args& a, uint32_t tile_index,
                                          int lane, int valid) {
  using Gm = Geo<kKv, kGroup>;
  using L = typename Gm::Load;
  const size_t base = static_cast<size_t>(tile_index) * Gm::kTileBytes;
  const char* kb = static_cast<const char*>(a.k_pages) + base;
  const char* vb = static_cast<const char*>(a.v_pages) + base;
  if (valid <= 0 || valid >= kBlockSize) {
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) {
      t.k[i] = stream_load<L>(kb + Gm::offset(lane, i));
      t.v[i] = stream_load<L>(vb + Gm::offset(lane, i));
    }
  } else {
    const int row = lane / Gm::kLanesPerRow;
    const int in_row = (lane % Gm::kLanesPerRow) * Gm::kLoadBytes;
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) {
      const int off = min(Gm::token(row, i), valid - 1) * Gm::kRowBytes + in_row;
      t.k[i] = stream_load<L>(kb + off);
      t.v[i] = stream_load<L>(vb + off);
    }
  }
  if constexpr (Gm::kScaled) {
    // The lane row's tokens are consecutive, so their row scales are one load.
    typedef float Scales __attribute__((ext_vector_type(Gm::kLoads)));
    const size_t srow = static_cast<size_t>(tile_index) * kBlockSize + Gm::token(lane / Gm::kLanesPerRow, 0);
    const Scales ks = stream_load<Scales>(a.k_scale + srow);
    const Scales vs = stream_load<Scales>(a.v_scale + srow);
#pragma unroll
    for (int i = 0; i < Gm::kLoads; ++i) {
      t.ks[i] = ks[i];
      t.vs[i] = vs[i];
    }
  }
}

// Per-lane softmax state for the G query heads of one KV head. All lanes of one token row
// see the same tokens and hold the same m and l; acc holds this lane's kChunk output
// columns. Scores are kept in log2 units (scale * log2 e folded in).
template <KvType kKv, int kGroup>
struct State {
  float m[kGroup];
  float l[kGroup];
  float acc[kGroup][Geo<kKv, kGroup>::kChunk];
  float wsum[kGroup];   // INT8: sum of the weights folded into acc (rescaled and merged alike)
};

template <KvType kKv, int kGroup>
__device__ __forceinline__ void reset(State<kKv, kGroup>& st) {
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    st.m[h] = kNegInf;
    st.l[h] = 0.0f;
    st.wsum[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < Geo<kKv, kGroup>::kChunk; ++j) st.acc[h][j] = 0.0f;
  }
}

// The outputs of an INT8 state without the 1152 offset of its values (once per segment).
template <KvType kKv, int kGroup>
__device__ __forceinline__ void unbias(State<kKv, kGroup>& st) {
  if constexpr (kKv == KvType::kI8) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
#pragma unroll
      for (int j = 0; j < Geo<kKv, kGroup>::kChunk; ++j)
        st.acc[h][j] = fmaf(-kI8Bias, st.wsum[h], st.acc[h][j]);
      st.wsum[h] = 0.0f;
    }
  }
}

// Query rows of one segment: this lane's kChunk columns of each of the G heads.
template <KvType kKv, int kGroup>
using QRegs = h2[kGroup][Geo<kKv, kGroup>::kPairs];

// Fold one page tile into the running state. With kMasked, tokens at or past `valid`
// inside the page contribute nothing, whatever their K, V or scale slots hold. The tile is
// only read: masking works on copies.
template <KvType kKv, int kGroup, bool kMasked>
__device__ __forceinline__ void consume_tile(const Tile<kKv, kGroup>& t, State<kKv, kGroup>& st,
                                             const QRegs<kKv, kGroup>& qh,
                                             const float (&qsum)[kGroup], float scale_log2,
                                             int row, int valid) {
  using Gm = Geo<kKv, kGroup>;
  bool ok[Gm::kLoads];
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) ok[i] = !kMasked || Gm::token(row, i) < valid;
  float s[kGroup][Gm::kLoads];
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) {
    float f = scale_log2;
    if constexpr (Gm::kScaled) f *= t.ks[i];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float d = dot_row<kKv, kGroup>(t.k[i], qh[h]);
      if constexpr (kKv == KvType::kI8) d = fmaf(-kI8Bias, qsum[h], d);
      const float sc = row_sum<Gm::kLanesPerRow>(d) * f;
      s[h][i] = ok[i] ? sc : kNegInf;
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
    if constexpr (kKv == KvType::kI8) st.wsum[h] *= alpha;
    st.m[h] = m_new;
  }
#pragma unroll
  for (int i = 0; i < Gm::kLoads; ++i) {
    typename Gm::Load raw = t.v[i];
    if constexpr (kMasked) raw = ok[i] ? raw : typename Gm::Load(0u);
    float vscale = 1.0f;
    if constexpr (Gm::kScaled) vscale = ok[i] ? t.vs[i] : 0.0f;
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float pw = p[h][i];
      if constexpr (Gm::kScaled) pw *= vscale;
      axpy_row<kKv, kGroup>(raw, pw, st.acc[h]);
      if constexpr (kKv == KvType::kI8) st.wsum[h] += pw;
    }
  }
}

template <KvType kKv, int kGroup>
__device__ __forceinline__ void consume(const Tile<kKv, kGroup>& t, State<kKv, kGroup>& st,
                                        const QRegs<kKv, kGroup>& qh, const float (&qsum)[kGroup],
                                        float scale_log2, int row, int valid) {
  if (valid == kBlockSize) consume_tile<kKv, kGroup, false>(t, st, qh, qsum, scale_log2, row, kBlockSize);
  else consume_tile<kKv, kGroup, true>(t, st, qh, qsum, scale_log2, row, valid);
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
    if constexpr (kKv == KvType::kI8) st.wsum[h] = st.wsum[h] * wa + __shfl_xor(st.wsum[h], off) * wb;
#pragma unroll
    for (int j = 0; j < Geo<kKv, kGroup>::kChunk; ++j) {
      const float ao = __shfl_xor(st.acc[h][j], off);
      st.acc[h][j] = st.acc[h][j] * wa + ao * wb;
    }
    st.m[h] = mm;
  }
}

// Rows of a wave saw disjoint tokens: merge them so every lane holds the wave's state for
// its columns.
template <KvType kKv, int kGroup>
__device__ __forceinline__ void merge_rows(State<kKv, kGroup>& st) {
#pragma unroll
  for (int off = Geo<kKv, kGroup>::kLanesPerRow; off < kWave; off <<= 1) merge_lanes<kKv, kGroup>(st, off);
}

// ---------------------------------------------------------------------------------------
// Matrix-core tile consume, for G >= 4 over fp16, INT8 and FP8 caches. With G query heads
// per KV head the vector-ALU consume grows with G (every head repeats the dot products, the
// softmax and the weighted sum), and at G = 4 it kept the SIMDs 59 % busy with one wave
// each (rocprofv3 VALU counters). Here both products of a tile run on the matrix cores,
// with the G heads as the N columns of a 16x16 tile (columns G .. 15 hold zero queries):
//   S^T[token][head]  = K[token][:] . Q[head][:]     v_mfma_f32_16x16x32_f16, 4 steps of 32 d
//   O^T[d][head]     += V^T[d][token] P^T[token][head]   v_mfma_f32_16x16x16f16, 8 blocks of d
// Operand layouts (lane l, q = l / 16): the 16x16x32 A operand holds A[l % 16][slot 8q + e],
// B holds B[slot 8q + e][l % 16], and D holds D[4q + e][l % 16]; the 16x16x16 ones hold
// 4 k slots per lane, A[l % 16][4q + e] and B[4q + e][l % 16]. A contraction is correct for
// any assignment of the k values to slots that A and B share, and an output row may stand
// for any d as long as the writer knows which:
//  * scores: lane (q, t) holds 32 d of K[token t] and step s takes d = k_dim(q, s) + e for
//    slot 8q + e; the query operand uses the same map. For fp16 the lane's four 16-byte
//    loads sit at row bytes 64s + 16q, so that the four lanes of a row read one contiguous
//    64-byte run per load instruction (16 rows x 64 bytes, the fewest cache lines a load
//    can touch when lane l % 16 is the token); a 1-byte row is 128 bytes and the lane reads
//    its 32-byte quarter q;
//  * the score output leaves lane (q, n) with tokens 4q .. 4q + 3 of head n, which is the
//    B operand (P^T) of the weighted sum as it stands, so the softmax weights never move;
//  * weighted sum: lane (q, m) loads V[token 4q + j][d in [8m, 8m + 8)] for j < 4 (whole
//    rows per load instruction), so output row m of block b stands for d = 8m + b, and the
//    A operand of block b is element b of the four loaded rows, gathered with byte permutes.
//    Lane (q, n) then ends with O[head n][d] for d = 32q + 8e + b: a contiguous 32-float run.
// The softmax runs per head column: the tile max over 16 tokens is two cross-lane steps,
// and the running max moves only when a tile exceeds it by more than kLazyRescale (log2
// units), so most tiles skip the rescale and the weights, rounded to fp16 for the matrix
// cores, stay below 2^8. INT8 and FP8 codes are widened exactly to fp16 (as in the vector
// path); a row's K scale multiplies its score and its V scale its weight. BF16 caches run
// the bf16 shapes (v_mfma_f32_16x16x32_bf16, v_mfma_f32_16x16x16_bf16): the scores take
// bf16 q and K (exact products, as in the vector path), and each weight enters the weighted
// sum as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi), in two products, since one
// bf16 weight would carry errors up to 2^-8 of a value (the two parts keep 2^-16).
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b4 __attribute__((ext_vector_type(4)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLazyRescale = 8.0f;

template <KvType kKv>
struct MGeo {
  static constexpr int kElem = kv_elem_bytes(kKv);
  static constexpr int kRowBytes = kHeadDim * kElem;
  static constexpr int kTileBytes = kBlockSize * kRowBytes;
  static constexpr int kKLoads = 32 * kElem / 16;   // 16-byte K loads per lane: 4 | 2
  using VLoad = typename std::conditional<kElem == 2, u32x4, u32x2>::type;
  static constexpr bool kScaled = kv_scaled(kKv);
  // Row byte offset of K load i of lane group q, and the first d of score step s there.
  __device__ static constexpr int k_offset(int q, int i) { return kElem == 2 ? 64 * i + 16 * q : 32 * q + 16 * i; }
  __device__ static constexpr int k_dim(int q, int s) { return kElem == 2 ? 32 * s + 8 * q : 32 * q + 8 * s; }
};

template <KvType kKv>
struct MTile {
  u32x4 k[MGeo<kKv>::kKLoads];
  typename MGeo<kKv>::VLoad v[4];
  f4 ks, vs;   // row scales of tokens 4q .. 4q + 3 (1-byte formats)
};

struct MState {
  float m;     // running max of head l % 16 (log2 units), the same in its four lanes
  float l;     // this lane's share of the running sum
  f4 o[8];     // O[head l % 16][32q + 8e + b] in o[b][e]
};

struct MQ {
  h8 s[4];     // Q[head l % 16][k_dim(q, s) ..  + 7] for score step s (zero past G)
};

__device__ __forceinline__ void mreset(MState& st) {
  st.m = kNegInf;
  st.l = 0.0f;
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] = f4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Same tile index and partial-page rule as load_tile: rows at or past `valid` re-read the
// last valid row.
template <KvType kKv>
__device__ __forceinline__ void mload_tile(MTile<kKv>& t, const Args& a, uint32_t tile_index,
                                           int lane, int valid) {
  using Gm = MGeo<kKv>;
  using VL = typename Gm::VLoad;
  const size_t base = static_cast<size_t>(tile_index) * Gm::kTileBytes;
  const char* kb = static_cast<const char*>(a.k_pages) + base;
  const char* vb = static_cast<const char*>(a.v_pages) + base;
  const int q = lane >> 4;
  const int c = lane & 15;
  const bool clamp = valid > 0 && valid < kBlockSize;
  const int tk = clamp ? min(c, valid - 1) : c;
  const char* krow = kb + tk * Gm::kRowBytes;
#pragma unroll
  for (int i = 0; i < Gm::kKLoads; ++i) t.k[i] = stream_load<u32x4>(krow + Gm::k_offset(q, i));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tv = clamp ? min(4 * q + j, valid - 1) : 4 * q + j;
    t.v[j] = stream_load<VL>(vb + tv * Gm::kRowBytes + c * 8 * Gm::kElem);
  }
  if constexpr (Gm::kScaled) {
    const size_t srow = static_cast<size_t>(tile_index) * kBlockSize + 4 * q;
    t.ks = stream_load<f4>(a.k_scale + srow);
    t.vs = stream_load<f4>(a.v_scale + srow);
  }
}

// Eight K values of score step s as an fp16 operand (the raw bf16 bits for a BF16 cache).
template <KvType kKv>
__device__ __forceinline__ h8 mk_operand(const MTile<kKv>& t, int s) {
  if constexpr (kv_elem_bytes(kKv) == 2) {
    return __builtin_bit_cast(h8, t.k[s]);
  } else {
    const u32x4 w = t.k[s >> 1];
    h2 x[4];
    const uint32_t w0 = (s & 1) ? w[2] : w[0];
    const uint32_t w1 = (s & 1) ? w[3] : w[1];
    if constexpr (kKv == KvType::kI8) {
      i8x4_to_h2(w0, x[0], x[1]);
      i8x4_to_h2(w1, x[2], x[3]);
    } else {
      fp8x4_to_h2(w0, x[0], x[1]);
      fp8x4_to_h2(w1, x[2], x[3]);
    }
    return h8{x[0].x, x[0].y, x[1].x, x[1].y, x[2].x, x[2].y, x[3].x, x[3].y};
  }
}

// The four V rows of the lane as 16-bit words (word w of row j holds d = 8m + 2w, 8m + 2w + 1):
// fp16, or the raw bf16 of a BF16 cache.
template <KvType kKv>
__device__ __forceinline__ void mv_words(const MTile<kKv>& t, u32x4 (&v)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kv_elem_bytes(kKv) == 2) {
      v[j] = t.v[j];
    } else {
      h2 x[4];
      if constexpr (kKv == KvType::kI8) {
        i8x4_to_h2(t.v[j][0], x[0], x[1]);
        i8x4_to_h2(t.v[j][1], x[2], x[3]);
      } else {
        fp8x4_to_h2(t.v[j][0], x[0], x[1]);
        fp8x4_to_h2(t.v[j][1], x[2], x[3]);
      }
      v[j] = u32x4{__builtin_bit_cast(uint32_t, x[0]), __builtin_bit_cast(uint32_t, x[1]),
                   __builtin_bit_cast(uint32_t, x[2]), __builtin_bit_cast(uint32_t, x[3])};
    }
  }
}

template <KvType kKv, bool kMasked>
__device__ __forceinline__ void mconsume_tile(const MTile<kKv>& t, MState& st, const MQ& qm,
                                              float scale_log2, int lane, int valid) {
  const int q = lane >> 4;
  f4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (kKv == KvType::kBF16)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, mk_operand<kKv>(t, s)),
                                                  __builtin_bit_cast(b8, qm.s[s]), sc, 0, 0, 0);
    else
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(mk_operand<kKv>(t, s), qm.s[s], sc, 0, 0, 0);
  }
  float sv[4];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float f = scale_log2;
    if constexpr (MGeo<kKv>::kScaled) f *= t.ks[j];
    sv[j] = sc[j] * f;
    if constexpr (kMasked) sv[j] = 4 * q + j < valid ? sv[j] : kNegInf;
    mx = fmaxf(mx, sv[j]);
  }
  mx = max_across_rows(mx);
  const bool grow = mx > st.m + kLazyRescale;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = grow ? mx : st.m;
    const float alpha = grow ? fast_exp2(st.m - m_new) : 1.0f;
    st.l *= alpha;
#pragma unroll
    for (int b = 0; b < 8; ++b) st.o[b] *= alpha;
    st.m = m_new;
  }
  const float base = st.m == kNegInf ? 0.0f : st.m;
  float pf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float p = fast_exp2(sv[j] - base);
    st.l += p;
    if constexpr (MGeo<kKv>::kScaled) {
      const bool ok = !kMasked || 4 * q + j < valid;
      p *= ok ? t.vs[j] : 0.0f;
    }
    pf[j] = p;
  }
  h4 pw;     // fp16 weights; for BF16, the two bf16 parts
  b4 pw_hi, pw_lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kKv == KvType::kBF16) {
      pw_hi[j] = static_cast<__bf16>(pf[j]);
      pw_lo[j] = static_cast<__bf16>(pf[j] - static_cast<float>(pw_hi[j]));
    } else {
      pw[j] = static_cast<_Float16>(pf[j]);
    }
  }
  u32x4 v[4];
  mv_words<kKv>(t, v);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    // Element b of the four rows: rows 0, 1 into the first word and rows 2, 3 into the
    // second (low halves for even b, high halves for odd b).
    const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(v[1][b >> 1], v[0][b >> 1], sel);
    const uint32_t hi = __builtin_amdgcn_perm(v[3][b >> 1], v[2][b >> 1], sel);
    if constexpr (kKv == KvType::kBF16) {
      const b4 va = __builtin_bit_cast(b4, u32x2{lo, hi});
      st.o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pw_hi, st.o[b], 0, 0, 0);
      st.o[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pw_lo, st.o[b], 0, 0, 0);
    } else {
      const h4 va = __builtin_bit_cast(h4, u32x2{lo, hi});
      st.o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pw, st.o[b], 0, 0, 0);
    }
  }
}

template <KvType kKv>
__device__ __forceinline__ void mconsume(const MTile<kKv>& t, MState& st, const MQ& qm,
                                         float scale_log2, int lane, int valid) {
  if (valid == kBlockSize) mconsume_tile<kKv, false>(t, st, qm, scale_log2, lane, kBlockSize);
  else mconsume_tile<kKv, true>(t, st, qm, scale_log2, lane, valid);
}

// The query operand from a segment's query rows, G x D fp16 laid out head-major at `rows`
// (global memory or LDS): for step s lane (q, n) takes head n's d from k_dim(q, s), zero
// past G.
template <KvType kKv, int kGroup>
__device__ __forceinline__ void mload_q(MQ& qm, const u32x4* rows, int lane) {
  const int q = lane >> 4;
  const int n = lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (n < kGroup) w = rows[(n * kHeadDim + MGeo<kKv>::k_dim(q, s)) / 8];
    qm.s[s] = __builtin_bit_cast(h8, w);
  }
}

// The wave's state for the merge across waves: per head n < G its running max, its sum (the
// four lanes of column n added) and its 128 unnormalised outputs.
template <int kGroup>
__device__ __forceinline__ void mpublish(const MState& st, float* acc, float* m, float* l, int lane) {
  const int q = lane >> 4;
  const int n = lane & 15;
  const float sum = sum_across_rows(st.l);
  if (n < kGroup) {
    float* o = acc + n * kHeadDim + 32 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<float4*>(o + 8 * e) = make_float4(st.o[0][e], st.o[1][e], st.o[2][e], st.o[3][e]);
      *reinterpret_cast<float4*>(o + 8 * e + 4) = make_float4(st.o[4][e], st.o[5][e], st.o[6][e], st.o[7][e]);
    }
    if (q == 0) {
      m[n] = st.m;
      l[n] = sum;
    }
  }
}

__device__ __forceinline__ void store_chunk(float* dst, const float* src, int n) {
  for (int j = 0; j < n; j += 4)
    *reinterpret_cast<float4*>(dst + j) = make_float4(src[j], src[j + 1], src[j + 2], src[j + 3]);
}

// The tile consume a (G, format) build takes in every mode: the matrix cores for G >= 4, the
// vector ALU otherwise.
template <KvType kKv, int kGroup>
struct Path {
  static constexpr bool kMf = use_mfma(kKv, kGroup);
  using Gm = Geo<kKv, kGroup>;
  struct QV {
    QRegs<kKv, kGroup> v;
    float sum[kGroup];   // INT8: this lane's sum of each head's q elements
  };
  using TileT = typename std::conditional<kMf, MTile<kKv>, Tile<kKv, kGroup>>::type;
  using StateT = typename std::conditional<kMf, MState, State<kKv, kGroup>>::type;
  using QT = typename std::conditional<kMf, MQ, QV>::type;

  __device__ __forceinline__ static void reset_state(StateT& st) {
    if constexpr (kMf) mreset(st);
    else reset(st);
  }
  __device__ __forceinline__ static void load(TileT& t, const Args& a, uint32_t tile_index,
                                              int lane, int valid) {
    if constexpr (kMf) mload_tile<kKv>(t, a, tile_index, lane, valid);
    else load_tile<kKv, kGroup>(t, a, tile_index, lane, valid);
  }
  __device__ __forceinline__ static void consume_unit(const TileT& t, StateT& st, const QT& q,
                                                      float scale_log2, int lane, int valid) {
    if constexpr (kMf) mconsume<kKv>(t, st, q, scale_log2, lane, valid);
    else consume<kKv, kGroup>(t, st, q.v, q.sum, scale_log2, lane / Gm::kLanesPerRow, valid);
  }
  // Query operand of a segment whose G query rows (head-major, fp16 or bf16) are at `rows`.
  __device__ __forceinline__ static void load_q(QT& q, const u32x4* rows, int lane) {
    if constexpr (kMf) {
      mload_q<kKv, kGroup>(q, rows, lane);
    } else {
      const int col = lane % Gm::kLanesPerRow;
#pragma unroll
      for (int h = 0; h < kGroup; ++h)
#pragma unroll
        for (int c = 0; c < Gm::kChunk / 8; ++c) {
          const u32x4 raw = rows[(h * kHeadDim * 2 + (col * Gm::kChunk + c * 8) * 2) / 16];
#pragma unroll
          for (int e = 0; e < 4; ++e) q.v[h][c * 4 + e] = as_h2(raw[e]);
        }
      if constexpr (kKv == KvType::kI8) {
#pragma unroll
        for (int h = 0; h < kGroup; ++h) {
          float sum = 0.0f;
#pragma unroll
          for (int e = 0; e < Gm::kPairs; ++e)
            sum += static_cast<float>(q.v[h][e].x) + static_cast<float>(q.v[h][e].y);
          q.sum[h] = sum;
        }
      }
    }
  }
  // The wave's state for the merge across waves: per head its running max (log2 units),
  // sum and 128 unnormalised outputs, at m[h], l[h] and acc[h * 128 ..].
  __device__ __forceinline__ static void publish(StateT& st, float* acc, float* m, float* l,
                                                 int lane) {
    if constexpr (kMf) {
      mpublish<kGroup>(st, acc, m, l, lane);
    } else {
      merge_rows<kKv, kGroup>(st);
      unbias<kKv, kGroup>(st);
      const int row = lane / Gm::kLanesPerRow;
      const int col = lane % Gm::kLanesPerRow;
      if (row == 0) {
#pragma unroll
        for (int h = 0; h < kGroup; ++h)
#pragma unroll
          for (int j = 0; j < Gm::kChunk; ++j) acc[h * kHeadDim + col * Gm::kChunk + j] = st.acc[h][j];
      }
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < kGroup; ++h) {
          m[h] = st.m[h];
          l[h] = st.l[h];
        }
      }
    }
  }
  // The normalised result of the state: o[h * 128 + d] = acc / l and, unless lse is null,
  // lse[h] = (m + log2 l) * lse_mul; NaN everywhere for a bad segment.
  __device__ __forceinline__ static void store_normalised(StateT& st, float* o, float* lse,
                                                          float lse_mul, bool bad, int lane) {
    const float nan = __builtin_nanf("");
    if constexpr (kMf) {
      const int q = lane >> 4;
      const int n = lane & 15;
      const float sum = sum_across_rows(st.l);
      if (n < kGroup) {
        const float inv = 1.0f / sum;
        float* row = o + n * kHeadDim + 32 * q;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float4 lo = make_float4(st.o[0][e], st.o[1][e], st.o[2][e], st.o[3][e]);
          float4 hi = make_float4(st.o[4][e], st.o[5][e], st.o[6][e], st.o[7][e]);
          lo = bad ? make_float4(nan, nan, nan, nan) : make_float4(lo.x * inv, lo.y * inv, lo.z * inv, lo.w * inv);
          hi = bad ? make_float4(nan, nan, nan, nan) : make_float4(hi.x * inv, hi.y * inv, hi.z * inv, hi.w * inv);
          *reinterpret_cast<float4*>(row + 8 * e) = lo;
          *reinterpret_cast<float4*>(row + 8 * e + 4) = hi;
        }
        if (q == 0 && lse != nullptr) lse[n] = bad ? nan : (st.m + __log2f(sum)) * lse_mul;
      }
    } else {
      merge_rows<kKv, kGroup>(st);
      unbias<kKv, kGroup>(st);
      const int row = lane / Gm::kLanesPerRow;
      const int col = lane % Gm::kLanesPerRow;
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        const float inv = 1.0f / st.l[h];
        float v[Gm::kChunk];
#pragma unroll
        for (int j = 0; j < Gm::kChunk; ++j) v[j] = bad ? nan : st.acc[h][j] * inv;
        if (row == 0) store_chunk(o + h * kHeadDim + col * Gm::kChunk, v, Gm::kChunk);
        if (lane == 0 && lse != nullptr) lse[h] = bad ? nan : (st.m[h] + __log2f(st.l[h])) * lse_mul;
      }
    }
  }
};

// ---------------------------------------------------------------------------------------
// Stream mode. Per sequence the workgroup keeps in LDS its first unit (s_pre) and its
// page count and last-page fill (s_seq). A wave walks its run with a scalar cursor.
constexpr uint32_t kFillShift = 24;   // s_seq[b] = pages | (tokens in the last page << 24)

struct Cursor {
  uint32_t b, g, j;   // sequence, KV head, logical page
  uint32_t nb;        // pages of sequence b
  uint32_t fill;      // tokens in its last page (1..16)
};

// One unit as the streaming loop needs it, all in scalar registers.
struct Rec {
  uint32_t tile;   // phys * Hkv + g (0 when the page id failed the range check)
  uint32_t lin;    // b * Hkv + g: the segment's query rows and output rows start at lin * G
  uint32_t j, nb;
  int valid;       // tokens of the page inside the sequence
  bool ok;         // page id in range
};

// First unit of worker w, for T units over W workers.
__device__ __forceinline__ uint32_t unit_begin(uint32_t w, uint32_t total, uint32_t workers) {
  return static_cast<uint32_t>(static_cast<uint64_t>(w) * total / workers);
}

// Largest b in [0, batch) with pre[b] <= u, given pre[batch] > u (empty sequences have
// pre[b] == pre[b + 1] and are skipped).
__device__ __forceinline__ int find_seq(const uint32_t* pre, int batch, uint32_t u) {
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (lds_scalar(pre + mid) <= u) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ void load_seq(Cursor& c, const uint32_t* s_seq) {
  const uint32_t v = lds_scalar(s_seq + c.b);
  c.nb = v & ((1u << kFillShift) - 1);
  c.fill = v >> kFillShift;
}

__device__ __forceinline__ Cursor cursor_at(const uint32_t* s_pre, const uint32_t* s_seq, int batch,
                                            uint32_t u) {
  Cursor c;
  c.b = static_cast<uint32_t>(find_seq(s_pre, batch, u));
  load_seq(c, s_seq);
  const uint32_t r = u - lds_scalar(s_pre + c.b);
  c.g = r / c.nb;
  c.j = r - c.g * c.nb;
  return c;
}

// Move to the next unit; the caller guarantees there is one.
__device__ __forceinline__ void advance(Cursor& c, const uint32_t* s_pre, const uint32_t* s_seq,
                                        uint32_t hkv) {
  if (++c.j < c.nb) return;
  c.j = 0;
  if (++c.g < hkv) return;
  c.g = 0;
  do {
    ++c.b;
  } while (lds_scalar(s_pre + c.b + 1) == lds_scalar(s_pre + c.b));
  load_seq(c, s_seq);
}

__device__ __forceinline__ Rec make_rec(const Cursor& c, int32_t phys, const Args& a, uint32_t hkv) {
  Rec r;
  r.ok = static_cast<unsigned>(phys) < static_cast<unsigned>(a.num_pages);
  r.tile = r.ok ? static_cast<uint32_t>(phys) * hkv + c.g : 0u;
  r.lin = c.b * hkv + c.g;
  r.j = c.j;
  r.nb = c.nb;
  r.valid = c.j + 1 == c.nb ? static_cast<int>(c.fill) : kBlockSize;
  return r;
}

// End of this worker's piece of the segment with rows lin: merge the lane rows, then either
// write the normalised output (the whole segment was here) or leave the piece in a slot
// for the merge kernel, recording where all the pieces are if this is the first one.
template <KvType kKv, int kGroup>
__device__ __forceinline__ void finish_piece(const Args& a, typename Path<kKv, kGroup>::StateT& st,
                                             uint32_t lin, bool seg_first, bool seg_whole,
                                             bool seg_bad, bool last_page, uint32_t seg_end,
                                             uint32_t worker, uint32_t workers,
                                             uint32_t total_units, int lane, int32_t (&record)[4]) {
  const bool complete = last_page && seg_whole;
  const int slot = static_cast<int>(worker) * kPieceSlots + (seg_first ? 0 : 1);
  // A whole segment goes to the output (lse in natural-log units), a piece to its slot.
  const size_t qrow = static_cast<size_t>(lin) * kGroup;
  const size_t prow = static_cast<size_t>(slot) * kGroup;
  float* o = complete ? a.out + qrow * kHeadDim : a.part_o + prow * kHeadDim;
  float* lse = complete ? (a.lse_out != nullptr ? a.lse_out + qrow : nullptr) : a.part_lse + prow;
  Path<kKv, kGroup>::store_normalised(st, o, lse, complete ? kLn2 : 1.0f, seg_bad, lane);
  if (!complete && seg_whole) {
    // First piece of a segment that continues into later workers; its last piece is in
    // the last worker w' with unit_begin(w') <= seg_end - 1, i.e. w' = ceil(seg_end W / T) - 1.
    const uint32_t last_worker = static_cast<uint32_t>(
        (static_cast<uint64_t>(seg_end) * workers + total_units - 1) / total_units - 1);
    record[0] = static_cast<int32_t>(lin);
    record[1] = static_cast<int32_t>(last_worker - worker + 1);
    record[2] = slot;
  }
}

// One wave's run of units [unit_begin(worker), unit_begin(worker + 1)).
template <KvType kKv, int kGroup, bool kQInLds, int kDepth>
__device__ __forceinline__ void run_worker(const Args& a, const uint32_t* s_pre,
                                           const uint32_t* s_seq, const u32x4* s_q, uint32_t q_lin0,
                                           uint32_t worker, uint32_t workers, uint32_t total_units,
                                           int lane) {
  using P = Path<kKv, kGroup>;
  constexpr int kQRowBytes = kGroup * kHeadDim * 2;
  const uint32_t hkv = static_cast<uint32_t>(a.n_kv_heads);
  const uint32_t u0 = unit_begin(worker, total_units, workers);
  const uint32_t n = unit_begin(worker + 1, total_units, workers) - u0;
  int32_t record[4] = {0, 0, 0, 0};   // lin, piece count, first slot, unused

  if (n == 0) {
    // A worker with no units can still sit between two pieces of a cut segment (when
    // there are fewer units than workers): leave a piece of weight zero in its slot.
    for (int h = 0; h < kGroup; ++h) {
      const size_t prow = static_cast<size_t>(worker) * kPieceSlots * kGroup + h;
      *reinterpret_cast<float2*>(a.part_o + prow * kHeadDim + 2 * lane) = make_float2(0.0f, 0.0f);
      if (lane == 0) a.part_lse[prow] = kNegInf;
    }
  } else {
    Cursor cur = cursor_at(s_pre, s_seq, a.batch, u0);
    int32_t phys_next = scalar_load(a.block_table, static_cast<size_t>(cur.b) * a.max_blocks + cur.j);
    uint32_t taken = 0;   // units whose record has left the cursor
    // Record of the cursor's unit; then move the cursor on and start the scalar load of
    // the next page id, which has a whole step to arrive.
    auto take = [&]() -> Rec {
      const Rec r = make_rec(cur, phys_next, a, hkv);
      if (++taken < n) {
        advance(cur, s_pre, s_seq, hkv);
        phys_next = scalar_load(a.block_table, static_cast<size_t>(cur.b) * a.max_blocks + cur.j);
      }
      return r;
    };

    Rec rec[kDepth];
    typename P::TileT tiles[kDepth];
    static_for<0, kDepth>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if constexpr (d == 0) {
        rec[0] = take();
      } else if (static_cast<uint32_t>(d) < n) {
        rec[d] = take();
      } else {
        rec[d] = rec[d - 1];
        rec[d].valid = kIdleValid;
      }
      P::load(tiles[d], a, rec[d].tile, lane, rec[d].valid);
    });

    typename P::StateT st;
    P::reset_state(st);
    typename P::QT qh;
    uint32_t seg_lin = 0;
    bool seg_first = true;      // the segment is this worker's first
    bool seg_whole = false;     // the segment started inside this worker (at page 0)
    bool seg_bad = false;

    auto process = [&](uint32_t k, const Rec& r, const typename P::TileT& t) {
      if (k == 0 || r.j == 0) {   // a segment starts: fetch its query rows
        seg_first = k == 0;
        seg_whole = r.j == 0;
        seg_lin = r.lin;
        seg_bad = false;
        if constexpr (kQInLds)
          P::load_q(qh, s_q + (r.lin - q_lin0) * (kQRowBytes / 16), lane);
        else
          P::load_q(qh, static_cast<const u32x4*>(a.q) + static_cast<size_t>(r.lin) * (kQRowBytes / 16), lane);
      }
      seg_bad |= !r.ok;
      P::consume_unit(t, st, qh, a.scale_log2, lane, r.valid);
      const bool last_page = r.j + 1 == r.nb;
      if (last_page || k + 1 == n) {
        finish_piece<kKv, kGroup>(a, st, seg_lin, seg_first, seg_whole, seg_bad, last_page,
                                  u0 + k - r.j + r.nb, worker, workers, total_units, lane, record);
        P::reset_state(st);
      }
    };

    // Steady state: consume the oldest unit, refill its slot kDepth units ahead. Past the
    // end of the run a slot re-reads the first row of its own tile (kIdleValid).
    uint32_t k0 = 0;
    for (; k0 + kDepth <= n; k0 += kDepth) {
      static_for<0, kDepth>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        const uint32_t k = k0 + d;
        process(k, rec[d], tiles[d]);
        if (k + kDepth < n) rec[d] = take();
        else rec[d].valid = kIdleValid;
        P::load(tiles[d], a, rec[d].tile, lane, rec[d].valid);
      });
    }
    static_for<0, kDepth>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (k0 + d < n) process(k0 + d, rec[d], tiles[d]);
    });
  }
  if (lane == 0) {
    int32_t* p = a.pieces + static_cast<size_t>(worker) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = record[i];
  }
}

template <KvType kKv, int kGroup>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(stream_waves<kKv, kGroup>(), stream_waves<kKv, kGroup>())))
void stream_kernel(Args a) {
  __shared__ uint32_t s_pre[kMaxBatch + 1];   // s_pre[b]: first unit of sequence b
  __shared__ uint32_t s_seq[kMaxBatch];       // pages | last-page fill << 24
  __shared__ uint32_t s_part[kWaves];
  __shared__ u32x4 s_q[kQLdsBytes / 16];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // The wave index is the same for all 64 lanes; reading it through an SGPR lets the
  // compiler keep everything derived from it (the unit run, loop bounds) scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int batch = a.batch;
  const uint32_t hkv = static_cast<uint32_t>(a.n_kv_heads);

  // 1. Exclusive scan of units per sequence (Hkv * pages; 0 for an empty or invalid
  //    length), 256 sequences per pass.
  uint32_t carry = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    uint32_t units = 0;
    if (b < batch) {
      const int len = a.seq_lens[b];
      uint32_t seq = 0;
      if (len > 0 && len <= a.max_blocks * kBlockSize) {
        const uint32_t nb = static_cast<uint32_t>((len + kBlockSize - 1) / kBlockSize);
        units = nb * hkv;
        seq = nb | (static_cast<uint32_t>(len - static_cast<int>(nb - 1) * kBlockSize) << kFillShift);
      }
      s_seq[b] = seq;
    }
    uint32_t x = units;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) s_part[wave] = x;
    __syncthreads();
    uint32_t before = carry, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) before += s_part[w];
      total += s_part[w];
    }
    if (b < batch) s_pre[b + 1] = before + x;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  const uint32_t total_units = s_pre[batch];

  // 2. Sequences with no units: zeros for an empty cache, NaN for an invalid length.
  if (blockIdx.x == 0) {
    for (int b = tid; b < batch; b += kThreads) {
      if (s_pre[b + 1] != s_pre[b]) continue;
      const bool bad = a.seq_lens[b] != 0;
      const float val = bad ? __builtin_nanf("") : 0.0f;
      float* o = a.out + static_cast<size_t>(b) * a.n_q_heads * kHeadDim;
      for (int i = 0; i < a.n_q_heads * kHeadDim; ++i) o[i] = val;
      if (a.lse_out != nullptr)
        for (int h = 0; h < a.n_q_heads; ++h)
          a.lse_out[static_cast<size_t>(b) * a.n_q_heads + h] = bad ? val : kNegInf;
    }
  }

  // 3. Stage the query rows of every segment this workgroup touches in LDS, if they fit.
  //    Segments in unit order are (b, g) pairs in b-major order, which is also the order of
  //    q in memory ([B, Hkv, G, D]), so they are one contiguous slice.
  const uint32_t workers = gridDim.x * kWaves;
  const uint32_t wg_u0 = unit_begin(blockIdx.x * kWaves, total_units, workers);
  const uint32_t wg_u1 = unit_begin((blockIdx.x + 1) * kWaves, total_units, workers);
  constexpr int kQRowBytes = kGroup * kHeadDim * 2;
  uint32_t q_lin0 = 0;
  bool q_in_lds = false;
  if (wg_u1 > wg_u0) {
    const Cursor c0 = cursor_at(s_pre, s_seq, batch, wg_u0);
    const Cursor c1 = cursor_at(s_pre, s_seq, batch, wg_u1 - 1);
    q_lin0 = c0.b * hkv + c0.g;
    const uint32_t bytes = (c1.b * hkv + c1.g - q_lin0 + 1) * kQRowBytes;
    q_in_lds = bytes <= static_cast<uint32_t>(kQLdsBytes);
    if (q_in_lds) {
      const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.q) +
                                                        static_cast<size_t>(q_lin0) * kQRowBytes);
      for (uint32_t i = tid; i < bytes / 16; i += kThreads) s_q[i] = src[i];
    }
  }
  __syncthreads();

  // 4. This wave's run of units. The query rows come from LDS when the workgroup's slice
  //    fit, else straight from global memory; the two loops are separate so that the fast
  //    one never waits on a global query load.
  const uint32_t worker = blockIdx.x * kWaves + wave;
  constexpr int kDepth = stream_depth<kKv, kGroup>();
  if (q_in_lds)
    run_worker<kKv, kGroup, true, kDepth>(a, s_pre, s_seq, s_q, q_lin0, worker, workers,
                                          total_units, lane);
  else
    run_worker<kKv, kGroup, false, kDepth>(a, s_pre, s_seq, s_q, q_lin0, worker, workers,
                                           total_units, lane);
}

// Stream-mode merge: one wave per worker; a worker that recorded a cut segment combines
// its pieces, piece p living in slot (p == 0 ? first_slot : (worker + p) * kPieceSlots),
// as sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M) with M = max_p lse_p, in piece order.
template <int kGroup>
__global__ __launch_bounds__(kThreads) void piece_merge_kernel(Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint32_t worker = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int32_t* rec = a.pieces + static_cast<size_t>(worker) * 4;
  const int count = scalar_load(rec, 1);
  if (count <= 0) return;
  const uint32_t lin = static_cast<uint32_t>(scalar_load(rec, 0));
  const int first_slot = scalar_load(rec, 2);
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    float mx = kNegInf;
    bool poisoned = false;
    for (int p = 0; p < count; ++p) {
      const int slot = p == 0 ? first_slot : static_cast<int>(worker + p) * kPieceSlots;
      const float v = a.part_lse[static_cast<size_t>(slot) * kGroup + h];
      poisoned |= v != v;
      mx = fmaxf(mx, v);
    }
    float den = 0.0f, n0 = 0.0f, n1 = 0.0f;
    for (int p = 0; p < count; ++p) {
      const int slot = p == 0 ? first_slot : static_cast<int>(worker + p) * kPieceSlots;
      const size_t prow = static_cast<size_t>(slot) * kGroup + h;
      const float wgt = fast_exp2(a.part_lse[prow] - mx);
      const float2 o = *reinterpret_cast<const float2*>(a.part_o + prow * kHeadDim + 2 * lane);
      den += wgt;
      n0 += wgt * o.x;
      n1 += wgt * o.y;
    }
    const size_t qrow = static_cast<size_t>(lin) * kGroup + h;
    const float inv = 1.0f / den;
    *reinterpret_cast<float2*>(a.out + qrow * kHeadDim + 2 * lane) =
        poisoned ? make_float2(nan, nan) : make_float2(n0 * inv, n1 * inv);
    if (lane == 0 && a.lse_out != nullptr) a.lse_out[qrow] = poisoned ? nan : (mx + __log2f(den)) * kLn2;
  }
}

// ---------------------------------------------------------------------------------------
// Segment mode: a fixed grid of P persistent workgroups, each taking whole segments (all
// pages of one (sequence, KV head) pair). Segments are listed rank-major, then by KV head,
// where rank orders the sequences by decreasing length when the batch has at most
// kOrderMax of them (ties by index; every workgroup ranks the lengths itself, the same
// way) and by index otherwise. The list is dealt out in a snake: in round r workgroup w
// takes position r P + w, or r P + P - 1 - w when r is odd, so the longest segments start
// first and each workgroup's total stays close to the mean. The four waves of a workgroup
// interleave the pages of its current segment; each wave keeps one pipeline of tile loads
// running across segment boundaries. At the end of every segment the waves merge their
// states through LDS after one barrier; the barrier waits for LDS traffic only, so the
// tile loads already issued for the next segments stay in flight.
constexpr int kSegQBytes = 16384;   // query rows of the segments staged in LDS at a time

struct SegInfo {
  uint32_t b, g;
  int len;       // tokens, as passed
  uint32_t nb;   // pages; 0 for an empty cache or an invalid length
  bool bad;      // invalid length
};

struct SegList {
  uint32_t w, P, n, hkv;
  int max_tokens;
  bool ordered, lens_in_lds;
  const uint32_t* order;      // LDS: sequence of each rank
  const uint32_t* lens;       // LDS: lengths, when lens_in_lds
  const int32_t* seq_lens;    // global

  // Position in the list of this workgroup's k-th segment.
  __device__ __forceinline__ uint32_t index(uint32_t k) const {
    return k * P + ((k & 1u) != 0u ? P - 1u - w : w);
  }
  // Sequence and KV head of the k-th segment; with kUniform the caller guarantees k is the
  // same in all lanes and the lookups go through scalar registers.
  template <bool kUniform>
  __device__ __forceinline__ void head_of(uint32_t k, uint32_t& b, uint32_t& g) const {
    const uint32_t i = index(k);
    uint32_t rank = i / hkv;
    // The division runs on the vector unit; bring a uniform result back to a scalar
    // register so that the loads it addresses stay scalar.
    if constexpr (kUniform) rank = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(rank)));
    g = i - rank * hkv;
    if (!ordered) b = rank;
    else if constexpr (kUniform) b = lds_scalar(order + rank);
    else b = order[rank];
  }
  __device__ __forceinline__ SegInfo info(uint32_t k) const {
    SegInfo s;
    head_of<true>(k, s.b, s.g);
    s.len = lens_in_lds ? static_cast<int>(lds_scalar(lens + s.b)) : scalar_load(seq_lens, s.b);
    s.bad = s.len < 0 || s.len > max_tokens;
    s.nb = s.bad ? 0u : static_cast<uint32_t>((s.len + kBlockSize - 1) / kBlockSize);
    return s;
  }
};

// Workgroups are dispatched to the 8 XCDs round robin (workgroup w runs on XCD w mod 8),
// and each XCD has its own L2. The snake deal gives list positions 2m and 2m + 1 (the same
// sequence, KV heads 2j and 2j + 1) to the logical workgroups of one pair {2i, 2i + 1}. This
// map from a launched workgroup to its logical index places both of a pair on one XCD
// (launched workgroups 16c + x and 16c + 8 + x), so the 128-byte lines that hold two heads'
// row scales (64 bytes each) are fetched from HBM once and then hit in that XCD's L2.
// A grid that is not a multiple of 16 keeps the plain order in its last partial block.
constexpr bool kPairHeadsOnXcd = true;
__device__ __forceinline__ uint32_t logical_workgroup(uint32_t w, uint32_t grid) {
  if (!kPairHeadsOnXcd || w >= (grid & ~15u)) return w;
  const uint32_t j = w & 15u;
  return (w & ~15u) + 2u * (j & 7u) + (j >> 3);
}

// One unit of a wave's run, all in scalar registers.
struct SegRec {
  uint32_t tile;   // phys * Hkv + g (0 when the page id failed the range check)
  uint32_t k;      // segment index in the workgroup's list; n once the run is over
  int valid;       // tokens of the page inside the sequence
  bool ok;         // page id in range
  bool live;       // false past the end of the run (the slot re-reads an earlier tile)
};

template <KvType kKv, int kGroup>
__global__ __launch_bounds__(kSegThreads)
__attribute__((amdgpu_waves_per_eu(seg_waves(kKv, kGroup), seg_waves(kKv, kGroup))))
void seg_kernel(Args a) {
  using P = Path<kKv, kGroup>;
  constexpr int kDepth = seg_depth<kKv, kGroup>();
  constexpr uint32_t kQRow16 = kGroup * kHeadDim * 2 / 16;   // 16-byte words per segment's queries
  constexpr uint32_t kChunk = kSegQBytes / (kQRow16 * 16);  // segments per staged chunk
  __shared__ uint32_t s_len[kOrderMax];
  __shared__ int4 s_key[kOrderMax / 4];
  __shared__ uint32_t s_order[kOrderMax];
  __shared__ u32x4 s_q[kSegQBytes / 16];
  __shared__ float sm_acc[2][kSegW][kGroup][kHeadDim];
  __shared__ float sm_m[2][kSegW][kGroup];
  __shared__ float sm_l[2][kSegW][kGroup];
  __shared__ int sm_bad[2][kSegW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int batch = a.batch;
  const uint32_t hkv = static_cast<uint32_t>(a.n_kv_heads);
  const uint32_t mb = static_cast<uint32_t>(a.max_blocks);

  SegList L;
  L.w = logical_workgroup(blockIdx.x, gridDim.x);
  L.P = gridDim.x;
  L.hkv = hkv;
  L.max_tokens = a.max_blocks * kBlockSize;
  L.ordered = batch <= kOrderMax;
  L.lens_in_lds = L.ordered;   // else lengths come through scalar loads
  L.order = s_order;
  L.lens = s_len;
  L.seq_lens = a.seq_lens;
  {
    const uint32_t total = static_cast<uint32_t>(batch) * hkv;
    const uint32_t full = total / L.P;
    const uint32_t rem = total - full * L.P;
    const uint32_t last = (full & 1u) != 0u ? L.P - 1u - L.w : L.w;
    L.n = full + (last < rem ? 1u : 0u);
  }

  // 1. When ordering, lengths into LDS and the rank of each sequence by decreasing length
  //    (empty and invalid lengths count as 0, so they come last). In index order nothing
  //    has to be read before the first loads below: lengths come through scalar loads.
  if (L.ordered) {
    // The order is by decreasing length, ties by index, with lengths clamped to 2^24 - 1
    // (longer caches tie). Length and index fold into one unsigned key,
    // (length << 8) | (255 - index), so that the rank is one comparison per sequence; the
    // pads past the batch are 0, below every real key.
    uint32_t key = 0;
    if (tid < batch) {
      const int len = a.seq_lens[tid];
      s_len[tid] = static_cast<uint32_t>(len);
      const uint32_t valid = len > 0 && len <= L.max_tokens ? static_cast<uint32_t>(len) : 0u;
      key = (min(valid, (1u << 24) - 1u) << 8) | static_cast<uint32_t>(kOrderMax - 1 - tid);
    }
    if (tid < kOrderMax) reinterpret_cast<uint32_t*>(s_key)[tid] = key;
    __syncthreads();
    if (tid < batch) {
      uint32_t rank = 0;
      for (int u4 = 0; u4 < (batch + 3) / 4; ++u4) {
        const u32x4 k = reinterpret_cast<const u32x4*>(s_key)[u4];
        rank += static_cast<uint32_t>(k[0] > key) + static_cast<uint32_t>(k[1] > key) +
                static_cast<uint32_t>(k[2] > key) + static_cast<uint32_t>(k[3] > key);
      }
      s_order[rank] = static_cast<uint32_t>(tid);
    }
    __syncthreads();
  }
  if (L.n == 0) return;   // more workgroups than segments (same for the whole workgroup)

  // 2. Query rows of segments [k0, k0 + kChunk) go to LDS: each thread loads at most
  //    kQPerThread 16-byte words of them into registers, then stores them.
  constexpr int kQPerThread = (kSegQBytes / 16 + kSegThreads - 1) / kSegThreads;
  const u32x4* q16 = static_cast<const u32x4*>(a.q);
  u32x4 qbuf[kQPerThread];
  auto stage_load = [&](uint32_t k0) __attribute__((always_inline)) {
    const uint32_t words = min(kChunk, L.n - k0) * kQRow16;
#pragma unroll
    for (int i = 0; i < kQPerThread; ++i) {
      const uint32_t idx = static_cast<uint32_t>(tid + i * kSegThreads);
      if (idx < words) {
        const uint32_t t = idx / kQRow16;
        uint32_t b, g;
        L.head_of<false>(k0 + t, b, g);
        qbuf[i] = q16[static_cast<size_t>(b * hkv + g) * kQRow16 + (idx - t * kQRow16)];
      }
    }
  };
  auto stage_store = [&](uint32_t k0) __attribute__((always_inline)) {
    const uint32_t words = min(kChunk, L.n - k0) * kQRow16;
#pragma unroll
    for (int i = 0; i < kQPerThread; ++i) {
      const uint32_t idx = static_cast<uint32_t>(tid + i * kSegThreads);
      if (idx < words) s_q[idx] = qbuf[i];
    }
  };
  auto stage = [&](uint32_t k0) __attribute__((always_inline)) {
    stage_load(k0);
    stage_store(k0);
  };

  typename P::QT qh;
  auto load_q = [&](uint32_t k) __attribute__((always_inline)) {
    P::load_q(qh, s_q + (k % kChunk) * kQRow16, lane);
  };

  // 3. This wave's cursor: segment k, page j (j = wave, wave + 4, ...), skipping segments
  //    too short to give this wave a page.
  uint32_t ck = 0, cj = 0, cnb = 0, cb = 0, cg = 0;
  int clen = 0;
  auto seek = [&]() __attribute__((always_inline)) {
    for (; ck < L.n; ++ck) {
      const SegInfo s = L.info(ck);
      if (static_cast<uint32_t>(wave) < s.nb) {
        cj = static_cast<uint32_t>(wave);
        cnb = s.nb;
        cb = s.b;
        cg = s.g;
        clen = s.len;
        return;
      }
    }
  };
  // The first segment's length and this wave's first page id in it are loaded together
  // (the page id speculatively: table entries below max_blocks are always in bounds), and
  // its query rows go straight to registers, ahead of the first tile loads.
  int32_t phys_next = 0;
  {
    uint32_t b0, g0;
    L.head_of<true>(0, b0, g0);
    const int32_t first_page =
        static_cast<uint32_t>(wave) < mb ? scalar_load(a.block_table, static_cast<size_t>(b0) * mb + wave) : 0;
    P::load_q(qh, q16 + static_cast<size_t>(b0 * hkv + g0) * kQRow16, lane);
    seek();
    if (ck < L.n)
      phys_next = ck == 0 ? first_page : scalar_load(a.block_table, static_cast<size_t>(cb) * mb + cj);
  }
  uint32_t last_tile = 0;
  auto take = [&]() __attribute__((always_inline)) -> SegRec {
    SegRec r;
    if (ck >= L.n) {
      r.live = false;
      r.ok = true;
      r.k = L.n;
      r.tile = last_tile;
      r.valid = kIdleValid;
      return r;
    }
    r.live = true;
    r.ok = static_cast<unsigned>(phys_next) < static_cast<unsigned>(a.num_pages);
    r.tile = r.ok ? static_cast<uint32_t>(phys_next) * hkv + cg : 0u;
    r.k = ck;
    r.valid = cj + 1 == cnb ? clen - static_cast<int>(cnb - 1) * kBlockSize : kBlockSize;
    last_tile = r.tile;
    cj += kSegW;
    if (cj >= cnb) {
      ++ck;
      seek();
    }
    if (ck < L.n) phys_next = scalar_load(a.block_table, static_cast<size_t>(cb) * a.max_blocks + cj);
    return r;
  };

  SegRec rec[kDepth];
  typename P::TileT tiles[kDepth];
  static_for<0, kDepth>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    rec[d] = take();
    P::load(tiles[d], a, rec[d].tile, lane, rec[d].valid);
  });
  // The first chunk of query rows goes to LDS only now, behind the first tile loads: the
  // first segment's rows are already on their way to registers.
  stage_load(0);
  stage_store(0);   // read only after the barrier of the first segment's end

  typename P::StateT st;
  P::reset_state(st);
  bool seg_bad = false;
  uint32_t cur = 0;   // segment whose state st holds

  // End of segment k for this wave: publish the wave's state, meet the other waves, merge
  // the four states into the output, and stage the next chunk of query rows when k + 1
  // starts one. Every wave calls this exactly once per segment, in order, so the barriers
  // pair up.
  auto finish = [&](uint32_t k) __attribute__((always_inline)) {
    const uint32_t slot = k & 1u;
    P::publish(st, &sm_acc[slot][wave][0][0], &sm_m[slot][wave][0], &sm_l[slot][wave][0], lane);
    if (lane == 0) sm_bad[slot][wave] = seg_bad ? 1 : 0;
    __syncthreads();
    const SegInfo s = L.info(k);
    bool any_bad = s.bad;
#pragma unroll
    for (int w = 0; w < kSegW; ++w) any_bad |= sm_bad[slot][w] != 0;
    const uint32_t lin = s.b * hkv + s.g;
    const float nan = __builtin_nanf("");
    for (int o = tid; o < kGroup * kHeadDim; o += kSegThreads) {
      const int h = o / kHeadDim;
      const int d = o % kHeadDim;
      float mm = kNegInf;
#pragma unroll
      for (int w = 0; w < kSegW; ++w) mm = fmaxf(mm, sm_m[slot][w][h]);
      const float base = mm == kNegInf ? 0.0f : mm;
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int w = 0; w < kSegW; ++w) {
        const float e = fast_exp2(sm_m[slot][w][h] - base);
        num += e * sm_acc[slot][w][h][d];
        den += e * sm_l[slot][w][h];
      }
      const size_t qrow = static_cast<size_t>(lin) * kGroup + h;
      a.out[qrow * kHeadDim + d] = any_bad ? nan : (den > 0.0f ? num / den : 0.0f);
      if (a.lse_out != nullptr && d == 0)
        a.lse_out[qrow] = any_bad ? nan : (den > 0.0f ? (mm + __log2f(den)) * kLn2 : kNegInf);
    }
    if (k + 1 < L.n && (k + 1) % kChunk == 0) {
      stage(k + 1);
      __syncthreads();
    }
  };
  auto next_segment = [&]() __attribute__((always_inline)) {
    finish(cur);
    ++cur;
    P::reset_state(st);
    seg_bad = false;
    if (cur < L.n) load_q(cur);
  };

  // Consume the oldest unit, refill its slot kDepth units ahead. Past the end of the run a
  // slot re-reads the first row of the last tile (kIdleValid).
  while (rec[0].live) {
    static_for<0, kDepth>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (rec[d].live) {
        while (cur < rec[d].k) next_segment();
        seg_bad |= !rec[d].ok;
        P::consume_unit(tiles[d], st, qh, a.scale_log2, lane, rec[d].valid);
      }
      rec[d] = take();
      P::load(tiles[d], a, rec[d].tile, lane, rec[d].valid);
    });
  }
  while (cur < L.n) next_segment();
}

// ---------------------------------------------------------------------------------------
// Split mode: one workgroup per (partition s, KV head g, sequence b), S >= 2; wave w
// streams pages j0 + w, j0 + w + 4, ... of the partition, then the four waves merge
// through LDS into a partial result per (b, query head, s) for split_merge_kernel.
template <KvType kKv, int kGroup>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(split_waves<kKv, kGroup>(), split_waves<kKv, kGroup>())))
void split_kernel(Args a) {
  using P = Path<kKv, kGroup>;
  constexpr int kDepth = split_depth<kKv, kGroup>();
  __shared__ float sm_acc[kWaves][kGroup][kHeadDim];
  __shared__ float sm_m[kWaves][kGroup];
  __shared__ float sm_l[kWaves][kGroup];
  __shared__ int sm_bad[kWaves];
  __shared__ int32_t s_tab[kSplitTable];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  int wg = blockIdx.x;
  const int split = wg % a.num_splits;
  wg /= a.num_splits;
  const int g = wg % a.n_kv_heads;
  const int b = wg / a.n_kv_heads;
  const uint32_t hkv = static_cast<uint32_t>(a.n_kv_heads);

  const int seq_len = scalar_load(a.seq_lens, b);
  const bool bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockSize;
  const int nb = bad_len ? 0 : (seq_len + kBlockSize - 1) / kBlockSize;
  const int j0 = split * a.pages_per_split;
  const int j1 = min(j0 + a.pages_per_split, nb);
  // A partition with no tokens is never read by the merge.
  if (j0 >= j1) return;

  const uint32_t lin = static_cast<uint32_t>(b) * hkv + g;
  typename P::QT qh;
  P::load_q(qh, static_cast<const u32x4*>(a.q) + static_cast<size_t>(lin) * kGroup * kHeadDim * 2 / 16, lane);

  typename P::StateT st;
  P::reset_state(st);
  bool bad = bad_len;
  // The partition's table entries go through LDS, kSplitTable pages at a time, so the
  // streaming loop reads page ids with short LDS loads instead of scalar global loads.
  const size_t row0 = static_cast<size_t>(b) * a.max_blocks;
  for (int c0 = j0; c0 < j1; c0 += kSplitTable) {
    const int c1 = min(c0 + kSplitTable, j1);
    __syncthreads();   // the previous chunk's entries are no longer read
    for (int i = threadIdx.x; i < c1 - c0; i += kThreads) s_tab[i] = a.block_table[row0 + c0 + i];
    __syncthreads();
    const int npages = c1 - c0;
    const uint32_t n = npages > wave ? static_cast<uint32_t>((npages - wave + kWaves - 1) / kWaves) : 0u;
    if (n == 0) continue;
    // Page k of this wave in the chunk is c0 + wave + 4k.
    uint32_t taken = 0;
    auto take = [&]() -> Rec {
      Rec r;
      const int i = wave + static_cast<int>(taken) * kWaves;
      const int32_t phys = static_cast<int32_t>(lds_scalar(reinterpret_cast<const uint32_t*>(s_tab) + i));
      r.ok = static_cast<unsigned>(phys) < static_cast<unsigned>(a.num_pages);
      r.tile = r.ok ? static_cast<uint32_t>(phys) * hkv + g : 0u;
      r.valid = min(kBlockSize, seq_len - (c0 + i) * kBlockSize);
      ++taken;
      return r;
    };
    Rec rec[kDepth];
    typename P::TileT tiles[kDepth];
    static_for<0, kDepth>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if constexpr (d == 0) {
        rec[0] = take();
      } else if (static_cast<uint32_t>(d) < n) {
        rec[d] = take();
      } else {
        rec[d] = rec[d - 1];
        rec[d].valid = kIdleValid;
      }
      P::load(tiles[d], a, rec[d].tile, lane, rec[d].valid);
    });
    uint32_t k0 = 0;
    for (; k0 + kDepth <= n; k0 += kDepth) {
      static_for<0, kDepth>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        bad |= !rec[d].ok;
        P::consume_unit(tiles[d], st, qh, a.scale_log2, lane, rec[d].valid);
        if (k0 + d + kDepth < n) rec[d] = take();
        else rec[d].valid = kIdleValid;
        P::load(tiles[d], a, rec[d].tile, lane, rec[d].valid);
      });
    }
    static_for<0, kDepth>([&](auto dc) {
      constexpr int d = decltype(dc)::value;
      if (k0 + d < n) {
        bad |= !rec[d].ok;
        P::consume_unit(tiles[d], st, qh, a.scale_log2, lane, rec[d].valid);
      }
    });
  }
  P::publish(st, &sm_acc[wave][0][0], &sm_m[wave][0], &sm_l[wave][0], lane);
  if (lane == 0) sm_bad[wave] = bad ? 1 : 0;
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any_bad |= sm_bad[w] != 0;
  const float nan = __builtin_nanf("");
  for (int o = threadIdx.x; o < kGroup * kHeadDim; o += kThreads) {
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
    const size_t slot = (static_cast<size_t>(lin) * kGroup + h) * a.num_splits + split;
    a.part_o[slot * kHeadDim + d] = val;
    if (d == 0) a.part_lse[slot] = lse2;
  }
}

// Split-mode merge: one workgroup per (sequence, query head) over the partitions that hold
// tokens of the sequence: sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s,
// reduced in a fixed order.
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

constexpr int kMergeParts = kThreads / kHeadDim;   // partition subsets summed apart

__global__ __launch_bounds__(kThreads) void split_merge_kernel(Args a) {
  __shared__ float sm_red[kWaves];
  __shared__ int sm_nan[kWaves];
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

  float mx = kNegInf;
  int has_nan = 0;
  for (int s = tid; s < ns; s += kThreads) {
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
  for (int w = 1; w < kWaves; ++w) {
    mx = fmaxf(mx, sm_red[w]);
    has_nan |= sm_nan[w];
  }
  const float base = mx == kNegInf ? 0.0f : mx;
  __syncthreads();

  float den = 0.0f;
  for (int s = tid; s < ns; s += kThreads) den += fast_exp2(lse[s] - base);
  den = wave_sum(den);
  if (lane == 0) sm_red[wave] = den;
  __syncthreads();
  den = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) den += sm_red[w];

  const int d = tid % kHeadDim;
  const int part = tid / kHeadDim;
  float num = 0.0f;
#pragma unroll 8
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

// ---------------------------------------------------------------------------------------
template <KvType kKv, int kGroup>
hipError_t launch_t(const Args& a, const Plan& plan, hipStream_t stream) {
  if (plan.mode == Mode::kStream) {
    hipLaunchKernelGGL((stream_kernel<kKv, kGroup>), dim3(plan.num_workgroups), dim3(kThreads), 0,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((piece_merge_kernel<kGroup>), dim3(plan.num_workgroups), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (plan.mode == Mode::kSegment) {
    hipLaunchKernelGGL((seg_kernel<kKv, kGroup>), dim3(plan.num_workgroups), dim3(kSegThreads),
                       0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((split_kernel<kKv, kGroup>), dim3(plan.num_workgroups), dim3(kThreads), 0,
                     stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(split_merge_kernel, dim3(a.batch * a.n_q_heads), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <KvType kKv>
hipError_t launch_kv(int group, const Args& a, const Plan& plan, hipStream_t stream) {
  switch (group) {
    case 1: return launch_t<kKv, 1>(a, plan, stream);
    case 2: return launch_t<kKv, 2>(a, plan, stream);
    case 4: return launch_t<kKv, 4>(a, plan, stream);
    case 8: return launch_t<kKv, 8>(a, plan, stream);
    default: return hipErrorInvalidValue;
  }
}

constexpr size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace

// The no-allocation entry point's workspace: one array per device, alive until the process
// ends. Host code never passes `scratch` itself to a kernel (on the host it is only a
// stand-in for the symbol); it passes the device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices];   // device address of `scratch`, per device
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t workspace_bytes(const Plan& plan, int batch, int n_q_heads, int n_kv_heads) {
  const size_t group = static_cast<size_t>(n_q_heads / n_kv_heads);
  if (plan.mode == Mode::kStream) {
    const size_t workers = static_cast<size_t>(plan.num_workgroups) * kWaves;
    const size_t rows = workers * kPieceSlots * group;
    return align256(rows * kHeadDim * sizeof(float)) + align256(rows * sizeof(float)) +
           align256(workers * 4 * sizeof(int32_t));
  }
  if (plan.mode == Mode::kSegment) return 0;
  const size_t rows = static_cast<size_t>(batch) * n_q_heads * plan.num_splits;
  return align256(rows * kHeadDim * sizeof(float)) + align256(rows * sizeof(float));
}

void bind_workspace(Args& a, const Plan& plan, void* workspace) {
  a.part_o = a.part_lse = nullptr;
  a.pieces = nullptr;
  if (workspace == nullptr || plan.mode == Mode::kSegment) return;
  const size_t group = static_cast<size_t>(a.n_q_heads / a.n_kv_heads);
  char* p = static_cast<char*>(workspace);
  if (plan.mode == Mode::kStream) {
    const size_t workers = static_cast<size_t>(plan.num_workgroups) * kWaves;
    const size_t rows = workers * kPieceSlots * group;
    a.part_o = reinterpret_cast<float*>(p);
    p += align256(rows * kHeadDim * sizeof(float));
    a.part_lse = reinterpret_cast<float*>(p);
    p += align256(rows * sizeof(float));
    a.pieces = reinterpret_cast<int32_t*>(p);
  } else {
    const size_t rows = static_cast<size_t>(a.batch) * a.n_q_heads * plan.num_splits;
    a.part_o = reinterpret_cast<float*>(p);
    p += align256(rows * kHeadDim * sizeof(float));
    a.part_lse = reinterpret_cast<float*>(p);
  }
}

hipError_t launch(KvType kv, int group, const Args& a, const Plan& plan, hipStream_t stream) {
  switch (kv) {
    case KvType::kF16: return launch_kv<KvType::kF16>(group, a, plan, stream);
    case KvType::kI8: return launch_kv<KvType::kI8>(group, a, plan, stream);
    case KvType::kBF16: return launch_kv<KvType::kBF16>(group, a, plan, stream);
    case KvType::kFP8: return launch_kv<KvType::kFP8>(group, a, plan, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dattn
