// gfx950 kernel for chunked-prefill attention over the paged cache, on the matrix cores.
//
// The prefill phase runs several prompt tokens through the model at once and fills the KV
// cache (page "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen", sections 1.1
// and 4, which also names FlashAttention-style fusion as the way to do it); swiftLLM's
// feature list serves such chunks piggybacked on decode batches. Sequence b's chunk is its
// last C_b cached tokens (their K/V already appended), so chunk row i sits at position
// p = L_b - C_b + i and attends to tokens 0 .. p. A decode token is a chunk of one.
//
// Unlike decode, this is a dense contraction: each K/V page is used by every chunk row of
// the (sequence, KV head), G * C_b query rows. A workgroup owns 128 rows (4 waves x 2
// groups of 16) of one (sequence, KV head) and walks the cache in tiles of 64 tokens (four
// pages), staged once in LDS: K as [token][d], V transposed to [d][token]. Both products run
// on gfx950's double-rate v_mfma_f32_16x16x32_f16 (fp16 in, fp32 accumulate), transposed
// so that each lane keeps one query row throughout:
//   S^T[token][row] = K[token][:] . Q[row][:]      A = K tile (LDS), B = Q^T (VGPRs)
//   O^T[d][row]    += V^T[d][token] P^T[token][row] A = V^T tile (LDS), B = P^T (VGPRs)
// The first product leaves lane l with tokens of row l % 16, which is exactly the layout the
// second one takes P^T in, and its result O^T keeps row l % 16 in lane l, so the online-
// normaliser rescale (fp32, log2 units) is a per-lane multiply with no cross-lane traffic.
//
// Storage formats: fp16 K/V with fp16 q on the fp16 matrix cores. bf16 K/V with bf16 q: the
// scores on the bf16 ones (v_mfma_f32_16x16x32_bf16, exact products), while V is rounded to
// fp16 when staged, so that the weights of P V keep fp16's 11-bit precision (bf16 weights
// would carry errors up to 2^-9 of a value). Per-row INT8 and FP8 E4M3 K/V are dequantised
// while staged (code times its row's fp32 scale, rounded once to fp16) and then take the
// fp16 path with fp16 q.
//
// 16x16x32 operand layout (lane l, q = l / 16, item e): A[l % 16][slot 8q + e] for e < 8,
// B[slot 8q + e][l % 16], D[4q + e][l % 16] for e < 4. A and B share the slot order, so a
// contraction is correct for any assignment of the 32 k values to slots, provided A and B
// use the same one; the P V product assigns slot 8q + e to tile token 32c + 4q + e (e < 4)
// and 32c + 16 + 4q + (e - 4) (e >= 4), which is how the first product's output falls.

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "kernels.h"

namespace dattn {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRowGroups = 2;                         // 16-row groups per wave
constexpr int kRowsPerWave = 16 * kRowGroups;
constexpr int kRowsPerBlock = kRowsPerWave * kPfWaves;
constexpr int kTileTok = 64;                          // tokens staged per step
constexpr int kPagesPerTile = kTileTok / kBlockSize;
constexpr int kKStride = kHeadDim * 2 + 16;           // LDS bytes per K token row (padded)
constexpr int kVtStride = kTileTok * 2 + 8;           // LDS bytes per V^T d row (padded)
constexpr float kNegInfPf = -__builtin_huge_valf();
constexpr int kOrderMaxPf = kPfThreads;              // batches ranked longest-first in-kernel
constexpr int kXcds = 8;                              // gfx950 dies; workgroup i runs on die i % 8
// The running max only moves when a tile's max exceeds it by more than this (log2 units),
// so the weights stay below 2^8 (exact to fp16's precision) and most tiles skip the rescale.
constexpr float kLazyRescale = 8.0f;

static_assert(kPagesPerTile * kBlockSize == kTileTok, "tiles are whole pages");
static_assert(kTileTok * kHeadDim * 2 == kPfThreads * 4 * 16, "four 16-byte K loads per thread");

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one lane of each 16-lane row)
// on the VALU: v_permlane16_swap of a value with itself leaves rows (0, 0, 2, 2) in one
// result and (1, 1, 3, 3) in the other, v_permlane32_swap the halves (lo, lo) and (hi, hi).
// Every lane of the four ends with the same bits. (A shuffle through ds_bpermute would wait
// on the LDS queue, behind the operand reads in flight.) The two results are copied out
// before any bit cast: a bit cast of an element of the returned pair read element 0.
__device__ __forceinline__ float max_across_rows_pf(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float m = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t w = __builtin_bit_cast(uint32_t, m);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}
__device__ __forceinline__ float sum_across_rows_pf(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float s = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const uint32_t w = __builtin_bit_cast(uint32_t, s);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}


// Read-only load through the scalar cache (constant address space), for values every lane
// of the workgroup shares.
__device__ __forceinline__ int32_t scalar_load_pf(const int32_t* base, int idx) {
  typedef const __attribute__((address_space(4))) int32_t* ConstPtr;
  return ((ConstPtr)(base))[idx];
}

// Byte offset of V^T[d][token] in the staged tile: rows of kVtStride bytes; the 4-token
// granules of rows with bit 4 of d set are XOR-swizzled by 4 granules, so that the staging
// writes (16 lanes: four token granules x four d chunks) and the operand reads (16 lanes:
// sixteen consecutive d) both fall on distinct banks.
__device__ __forceinline__ int vt_offset(int d, int granule) {
  return d * kVtStride + 8 * (granule ^ (4 * ((d >> 4) & 1)));
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma32(b8 a, b8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const h2 r = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, r);
}

// Operand type of the score product: bf16 for a bf16 cache, fp16 for every other format.
// The P V product is fp16 for every format.
template <KvType kKv> struct PfOperand { typedef h8 V8; };
template <> struct PfOperand<KvType::kBF16> { typedef b8 V8; };

// Two bf16 values (one dword, the lower one first) rounded to an fp16 pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u));
}


// Eight stored 1-byte codes (lowest address first) times the row's scale, as eight fp16
// values: INT8 codes exactly through fp32 (the sign bit flipped makes them unsigned bytes
// u = x + 128, and x s = u s - 128 s in one fma), E4M3 codes exactly to fp16 by the hardware
// conversion (unit scale), then times s in fp32; each product is rounded once to fp16.
template <KvType kKv>
__device__ __forceinline__ u32x4 dequant8(u32x2 w, float sc) {
  u32x4 r;
  if constexpr (kKv == KvType::kI8) {
    const float bias = -128.0f * sc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t u = w[h] ^ 0x80808080u;
      const float x0 = __builtin_fmaf(static_cast<float>(u & 0xffu), sc, bias);
      const float x1 = __builtin_fmaf(static_cast<float>((u >> 8) & 0xffu), sc, bias);
      const float x2 = __builtin_fmaf(static_cast<float>((u >> 16) & 0xffu), sc, bias);
      const float x3 = __builtin_fmaf(static_cast<float>(u >> 24), sc, bias);
      r[2 * h] = pack_f16(x0, x1);
      r[2 * h + 1] = pack_f16(x2, x3);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.0f, false);
      const h2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[h], 1.0f, true);
      r[2 * h] = pack_f16(static_cast<float>(lo.x) * sc, static_cast<float>(lo.y) * sc);
      r[2 * h + 1] = pack_f16(static_cast<float>(hi.x) * sc, static_cast<float>(hi.y) * sc);
    }
  }
  return r;
}

// One workgroup: query-row block mb of (sequence b, KV head g), looping over further blocks
// `nx` apart. The grid is one-dimensional, nx * Hkv * B workgroups. Work order: for batches
// of up to 256 sequences the (sequence, KV head) pairs are taken longest sequence first
// (every workgroup ranks the lengths itself, ties by index), and each pair's row blocks
// last rows first, since later rows see more of the cache. When the pair count is a
// multiple of the die count, all row blocks of a pair run on one die, so its K/V pages are
// fetched into that die's L2 once.
template <KvType kKv, int kGroup>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a, int nx) {
  constexpr bool kCodes = kv_scaled(kKv);                      // 1-byte codes + row scales
  constexpr int kRowBytes = kHeadDim * kv_elem_bytes(kKv);     // one stored (token, head) row
  constexpr int kPageB = kBlockSize * kRowBytes;               // one stored (page, head) tile
  using V8 = typename PfOperand<kKv>::V8;
  __shared__ __attribute__((aligned(16))) unsigned char s_k[kTileTok * kKStride];
  __shared__ __attribute__((aligned(16))) unsigned char s_vt[kHeadDim * kVtStride];
  __shared__ int s_len[kOrderMaxPf];
  __shared__ int s_bad;
  __shared__ int s_pick;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int hq = a.n_kv_heads * kGroup;
  const int pairs = a.batch * a.n_kv_heads;

  const int id = blockIdx.x;
  int pair, mbx;
  if (pairs % kXcds == 0) {
    const int k = id / kXcds;
    pair = id % kXcds + kXcds * (k / nx);
    mbx = k % nx;
  } else {
    pair = id / nx;
    mbx = id % nx;
  }
  mbx = nx - 1 - mbx;
  const int g = pair % a.n_kv_heads;
  const int rank = pair / a.n_kv_heads;
  int b = rank;
  if (a.batch <= kOrderMaxPf) {
    const int my = tid < a.batch ? a.seq_lens[tid] : 0;
    s_len[tid] = my;
    __syncthreads();
    if (tid < a.batch) {
      int r = 0;
      for (int t = 0; t < a.batch; ++t) {
        const int o = s_len[t];
        r += (o > my) | ((o == my) & (t < tid));
      }
      if (r == rank) s_pick = tid;
    }
    __syncthreads();
    b = s_pick;
  }

  const int L = a.seq_lens[b];
  const int r0 = a.q_start[b];
  const int r1 = a.q_start[b + 1];
  const int C = r1 - r0;
  // Rows outside [0, T) are never touched; a chunk longer than its sequence, or a length
  // beyond the table, makes the sequence's rows NaN.
  if (r0 < 0 || r1 > a.total_rows || C <= 0) return;
  const bool bad_len = C > L || L > a.max_blocks * kBlockSize;
  const int nb = bad_len ? 0 : (L + kBlockSize - 1) / kBlockSize;
  const int32_t* table = a.block_table + static_cast<size_t>(b) * a.max_blocks;

  // Every page id of the sequence must be in range, else all its rows are NaN.
  if (tid == 0) s_bad = bad_len ? 1 : 0;
  __syncthreads();
  for (int j = tid; j < nb; j += kPfThreads) {
    if (static_cast<unsigned>(table[j]) >= static_cast<unsigned>(a.num_pages)) s_bad = 1;
  }
  __syncthreads();
  const bool bad = s_bad != 0;

  const int rows_total = C * kGroup;
  // Scores are scaled by ssc >= FLT_MIN (a zero scale gives the same weights as the
  // smallest normal one), so a masked -inf score stays -inf through the fma.
  const float ssc = fmaxf(fabsf(a.scale_log2), __FLT_MIN__);
  const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  const u32x4 qflip = u32x4{qsign, qsign, qsign, qsign};
  const int col = lane & 15;        // this lane's query row within a 16-row group
  const int quad = lane >> 4;       // which k slots (and output rows of D) the lane holds

  // Staging roles. K: 16-byte chunk sc of tile tokens st + 16 i (i = 0..3), slot st of the
  // tile's page i. V: wave w stages the tile's page w; lane (vs, vc) moves 16-byte chunk vc
  // (d = 8 vc .. 8 vc + 7) of the page's tokens 4 vs .. 4 vs + 3.
  const int sc = tid & 15;
  const int st = tid >> 4;
  const int vs = lane & 3;
  const int vc = lane >> 2;
  const char* kbase = static_cast<const char*>(a.k_pages) + static_cast<size_t>(g) * kPageB;
  const char* vbase = static_cast<const char*>(a.v_pages) + static_cast<size_t>(g) * kPageB;
  const size_t page_stride = static_cast<size_t>(a.n_kv_heads) * kPageB;
  const size_t scale_stride = static_cast<size_t>(a.n_kv_heads) * kBlockSize;   // floats per page

  for (int mb = mbx; mb * kRowsPerBlock < rows_total; mb += nx) {
    const int wrow0 = mb * kRowsPerBlock + wave * kRowsPerWave;
    // ---- this wave's rows: row r = chunk token r / G, head r % G; lane holds row col of
    // each group. Q^T as the B operand: Q[row][32 kb + 8 quad + e].
    // A negative scale is applied as |scale| to -q (exact), so that the largest score is the
    // largest product and the scale folds into one fma per score.
    V8 qb[kRowGroups][4];
    int pos[kRowGroups];        // last visible token of the lane's row (-1: none)
    int diag_from[kRowGroups];  // last visible token of the group's first row
#pragma unroll
    for (int grp = 0; grp < kRowGroups; ++grp) {
      const int row = wrow0 + 16 * grp + col;
      const bool live = row < rows_total;
      const int tok = live ? row / kGroup : 0;
      const int h = live ? row % kGroup : 0;
      pos[grp] = live && !bad ? L - C + tok : -1;
      const int first = wrow0 + 16 * grp;
      diag_from[grp] = first < rows_total ? L - C + first / kGroup : INT_MAX;
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(r0 + tok) * hq + g * kGroup + h) * kHeadDim + 8 * quad;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (live) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 32 * kb);
          qb[grp][kb] = __builtin_bit_cast(V8, w ^ qflip);
        } else {
          qb[grp][kb] = __builtin_bit_cast(V8, u32x4{0u, 0u, 0u, 0u});
        }
      }
    }
    // Tiles this block reads (up to its last row's position), and the last position of
    // this wave's rows (tiles past it need no arithmetic from this wave).
    const int last_row = min(rows_total, (mb + 1) * kRowsPerBlock) - 1;
    const int last_pos = bad ? -1 : L - C + last_row / kGroup;
    const int tiles = (last_pos + kTileTok) / kTileTok;
    const int wave_last_row = min(rows_total, wrow0 + kRowsPerWave) - 1;
    const int wave_last_pos = (bad || wave_last_row < wrow0) ? -1 : L - C + wave_last_row / kGroup;

    float m[kRowGroups], l[kRowGroups];           // running max (log2 units) and this lane's sum
    f4 o[kRowGroups][8];                          // O^T[16 db + 4 quad + e][row col]
#pragma unroll
    for (int grp = 0; grp < kRowGroups; ++grp) {
      m[grp] = kNegInfPf;
      l[grp] = 0.0f;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[grp][db] = f4{0.f, 0.f, 0.f, 0.f};
    }

    // Loads of tile j into registers. Tokens at or past L_b load the last valid row instead
    // (its cache lines are fetched anyway): their slots may hold anything, NaN included.
    // Their scores are masked, and their V rows are staged as zeros, since a zero weight
    // times NaN would still be NaN in P V.
    // 2-byte formats load straight into kr/vr; 1-byte formats load codes and row scales
    // into kc/vcode/ksc/vsc, dequantised into kr/vr when the tile is staged.
    u32x4 kr[4], vr[4];
    u32x2 kc[4], vcode[4];
    float ksc[4], vsc[4];
    // Page ids of tile j's four pages: uniform, through the scalar cache (clamped to the
    // last page, so every index is valid for any j once nb > 0).
    auto page_ids = [&](int j, int* phys) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kPagesPerTile; ++i) phys[i] = scalar_load_pf(table, min(kPagesPerTile * j + i, nb - 1));
    };
    auto fetch = [&](int j, const int* phys) __attribute__((always_inline)) {
      const int last_slot = (L - 1) % kBlockSize;
#pragma unroll
      for (int i = 0; i < kPagesPerTile; ++i) {
        const int t = (kPagesPerTile * j + i) * kBlockSize + st;
        const int slot = t < L ? st : last_slot;
        // SGPR page base plus an unsigned 32-bit lane offset (the scalar-base load form).
        const char* page = kbase + phys[i] * page_stride;
        if constexpr (kCodes) {
          const uint32_t off = static_cast<uint32_t>(slot * kRowBytes + sc * 8);
          kc[i] = *reinterpret_cast<const u32x2*>(page + off);
          const float* srow = a.k_scale + phys[i] * scale_stride + g * kBlockSize;   // uniform
          ksc[i] = srow[static_cast<uint32_t>(slot)];
        } else {
          const uint32_t off = static_cast<uint32_t>(slot * kRowBytes + sc * 16);
          kr[i] = *reinterpret_cast<const u32x4*>(page + off);
        }
      }
      const int vphys = wave == 0 ? phys[0] : wave == 1 ? phys[1] : wave == 2 ? phys[2] : phys[3];
      const char* vpage = vbase + vphys * page_stride;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = kTileTok * j + kBlockSize * wave + 4 * vs + e;
        const int slot = t < L ? 4 * vs + e : last_slot;
        if constexpr (kCodes) {
          const uint32_t off = static_cast<uint32_t>(slot * kRowBytes + vc * 8);
          vcode[e] = *reinterpret_cast<const u32x2*>(vpage + off);
          const float* srow = a.v_scale + vphys * scale_stride + g * kBlockSize;    // uniform per wave
          vsc[e] = srow[static_cast<uint32_t>(slot)];
        } else {
          const uint32_t off = static_cast<uint32_t>(slot * kRowBytes + vc * 16);
          vr[e] = *reinterpret_cast<const u32x4*>(vpage + off);
        }
      }
      if (kTileTok * (j + 1) > L) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (kTileTok * j + kBlockSize * wave + 4 * vs + e >= L) {
            if constexpr (kCodes) {
              vcode[e] = u32x2{0u, 0u};
            } else {
              vr[e] = u32x4{0u, 0u, 0u, 0u};
            }
          }
        }
      }
    };
    if (tiles > 0) {
      int phys[kPagesPerTile];
      page_ids(0, phys);
      fetch(0, phys);
    }
    for (int j = 0; j < tiles; ++j) {
      __syncthreads();   // the previous tile is no longer read
      // The next tile's page ids are requested before the staging, so their latency
      // overlaps it instead of delaying the tile loads below.
      int next[kPagesPerTile];
      page_ids(j + 1, next);
      if constexpr (kCodes) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kr[i] = dequant8<kKv>(kc[i], ksc[i]);
          vr[i] = dequant8<kKv>(vcode[i], vsc[i]);
        }
      } else if constexpr (kKv == KvType::kBF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int x = 0; x < 4; ++x) vr[i][x] = bf16x2_to_f16x2(vr[i][x]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(s_k + (st + 16 * i) * kKStride + sc * 16) = kr[i];
      // V^T[8 vc + x][tile tokens 16 w + 4 vs .. + 3]: element x of each of the four rows.
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int w = x >> 1;
        uint32_t lo, hi;
        // One byte permute per dword: the (x & 1) halves of rows 0 and 1 (and 2 and 3).
        const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
        lo = __builtin_amdgcn_perm(vr[1][w], vr[0][w], sel);
        hi = __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel);
        *reinterpret_cast<u32x2*>(s_vt + vt_offset(8 * vc + x, 4 * wave + vs)) = u32x2{lo, hi};
      }
      // Keep the page-id loads above the barrier (they are used only past it).
      asm volatile("" ::"s"(next[0]), "s"(next[1]), "s"(next[2]), "s"(next[3]));
      __syncthreads();
      if (j + 1 < tiles) fetch(j + 1, next);
      if (kTileTok * j > wave_last_pos) continue;   // every row of this wave ends earlier

      // S^T for the tile's four 16-token subtiles, both row groups; each K operand is read
      // once from LDS and used for both groups.
      f4 s[kRowGroups][4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        s[0][sb] = f4{0.f, 0.f, 0.f, 0.f};
        s[1][sb] = f4{0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (!kCodes) {
        // d-slice major: the four subtiles' operands of one 32-wide d slice are read together
        // and feed eight independent products.
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          V8 ka[4];
#pragma unroll
          for (int sb = 0; sb < 4; ++sb)
            ka[sb] = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(
                s_k + (16 * sb + col) * kKStride + (32 * kb + 8 * quad) * 2));
#pragma unroll
          for (int sb = 0; sb < 4; ++sb) {
            s[0][sb] = mfma32(ka[sb], qb[0][kb], s[0][sb]);
            s[1][sb] = mfma32(ka[sb], qb[1][kb], s[1][sb]);
          }
        }
      } else {
        // Subtile major, one operand live at a time: the 1-byte formats keep their codes
        // and row scales in registers too, and four live operands would spill.
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const V8 ka = __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(
                s_k + (16 * sb + col) * kKStride + (32 * kb + 8 * quad) * 2));
            s[0][sb] = mfma32(ka, qb[0][kb], s[0][sb]);
            s[1][sb] = mfma32(ka, qb[1][kb], s[1][sb]);
          }
        }
      }
      // Online softmax per row: lane holds S[row col][tile token 16 sb + 4 quad + e]. Only
      // tiles that reach past a group's first row's last visible token need the causal mask.
      // The reference max m moves only when a row's tile max exceeds it by more than
      // kLazyRescale (then O and l are rescaled); otherwise the weights exp2(s ssc - m) stay
      // below 2^kLazyRescale. The final normalisation divides both by the same sum, so the
      // result is the softmax whatever reference is used.
      h8 pb[kRowGroups][2];
#pragma unroll
      for (int grp = 0; grp < kRowGroups; ++grp) {
        if (kTileTok * j + kTileTok - 1 > diag_from[grp]) {
          const int lim = pos[grp] - (kTileTok * j + 4 * quad);
#pragma unroll
          for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (16 * sb + e > lim) s[grp][sb][e] = kNegInfPf;
          }
        }
        float mx = kNegInfPf;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[grp][sb][e]);
        }
        mx = max_across_rows_pf(mx);
        mx *= ssc;
        const bool grow = mx > m[grp] + kLazyRescale;
        if (__ballot(grow)) {
          const float m_new = grow ? mx : m[grp];
          const float alpha = grow ? exp2_fast(m[grp] - m_new) : 1.0f;
          l[grp] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) o[grp][db] *= alpha;
          m[grp] = m_new;
        }
        const float mu = m[grp] == kNegInfPf ? 0.0f : m[grp];
        float sum = 0.0f;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = exp2_fast(__builtin_fmaf(s[grp][sb][e], ssc, -mu));
            sum += p;
            pb[grp][sb >> 1][4 * (sb & 1) + e] = static_cast<_Float16>(p);
          }
        }
        l[grp] += sum;
      }
      // O^T += V^T P^T over the tile's two 32-token halves, half-major: consecutive
      // products update different accumulators.
      // The two 4-token granules of an operand are 32 bytes apart, in either order (the
      // swizzle swaps them on odd d blocks). Each granule of each half is read through a
      // base address of its own that the compiler cannot relate to the others, so that
      // every read lands in its place in the operand rather than in a paired read whose
      // halves would then be moved.
      uint32_t vt_base[2][2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t o = static_cast<uint32_t>(vt_offset(col, quad) + 64 * (k >> 1) + 32 * (k & 1));
        if (k > 0) asm volatile("" : "+v"(o));
        vt_base[k >> 1][k & 1] = o;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          const uint32_t off = 16 * db * kVtStride;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(s_vt + vt_base[c][db & 1] + off);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(s_vt + vt_base[c][(db & 1) ^ 1] + off);
          const h8 va = __builtin_bit_cast(h8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          o[0][db] = mfma32(va, pb[0][c], o[0][db]);
          o[1][db] = mfma32(va, pb[1][c], o[1][db]);
        }
      }
    }

    // Normalise and store: lane holds O[row col][d = 16 db + 4 quad + e], four consecutive d.
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int grp = 0; grp < kRowGroups; ++grp) {
      const float lt = sum_across_rows_pf(l[grp]);
      const int row = wrow0 + 16 * grp + col;
      if (row >= rows_total) continue;
      const float inv = 1.0f / lt;
      float* dst = a.out + (static_cast<size_t>(r0 + row / kGroup) * hq + g * kGroup + row % kGroup) * kHeadDim +
                   4 * quad;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f4 v = bad ? f4{nan, nan, nan, nan} : o[grp][db] * inv;
        *reinterpret_cast<f4*>(dst + 16 * db) = v;
      }
    }
  }
}

template <KvType kKv>
hipError_t launch_prefill_kv(int group, const PrefillArgs& a, dim3 grid, int nx, hipStream_t stream) {
  switch (group) {
    case 1: hipLaunchKernelGGL((prefill_kernel<kKv, 1>), grid, dim3(kPfThreads), 0, stream, a, nx); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<kKv, 2>), grid, dim3(kPfThreads), 0, stream, a, nx); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<kKv, 4>), grid, dim3(kPfThreads), 0, stream, a, nx); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<kKv, 8>), grid, dim3(kPfThreads), 0, stream, a, nx); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(KvType kv, int group, const PrefillArgs& a, int max_chunk, hipStream_t stream) {
  // nx row blocks per (sequence, KV head); workgroups loop over the rest of a longer chunk.
  // The grid stays below 2^24 workgroups (2^32 work-items).
  const long long pairs = static_cast<long long>(a.batch) * a.n_kv_heads;
  const long long want = (static_cast<long long>(max_chunk) * group + kRowsPerBlock - 1) / kRowsPerBlock;
  const long long cap = ((1LL << 24) - 1) / pairs;
  const long long nx = want < 1 ? 1 : (want > cap ? cap : want);
  if (nx < 1) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(nx * pairs));
  const int nxi = static_cast<int>(nx);
  switch (kv) {
    case KvType::kF16: return launch_prefill_kv<KvType::kF16>(group, a, grid, nxi, stream);
    case KvType::kBF16: return launch_prefill_kv<KvType::kBF16>(group, a, grid, nxi, stream);
    case KvType::kI8: return launch_prefill_kv<KvType::kI8>(group, a, grid, nxi, stream);
    case KvType::kFP8: return launch_prefill_kv<KvType::kFP8>(group, a, grid, nxi, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dattn
