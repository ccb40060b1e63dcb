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
// the (sequence, KV head), G * C_b query rows, so the page tiles are staged once in LDS and
// both products run on MFMA (v_mfma_f32_16x16x16_f16, fp32 accumulate):
//   S^T[token][row] = K[token][:] . Q[row][:]   (A = K tile from LDS, B = Q^T in VGPRs)
//   O[row][d]      += P[row][token] V[token][d]  (A = P as fp16, straight from S^T's layout;
//                                                B = V tile read as columns from LDS)
// with the online-normaliser softmax per row in between (fp32, log2 units). Rows are
// (chunk token, query head of the group) pairs, 16 per wavefront, 64 per workgroup.
//
// 16x16x16 MFMA operand layout (lane l, k = 4 * (l / 16) + e for e = 0..3):
//   A: A[l % 16][k];  B: B[k][l % 16];  D: D[4 * (l / 16) + e][l % 16].

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dattn {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerBlock = kRowsPerWave * kPfWaves;
constexpr int kTileStride = kHeadDim * 2 + 16;   // LDS bytes per token row (padded: no bank clash)
constexpr float kNegInfPf = -__builtin_huge_valf();

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// One workgroup: query-row block mb of (sequence b, KV head g), looping over further blocks
// gridDim.x apart.
template <int kGroup>
__global__ __launch_bounds__(kPfThreads) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char s_k[kBlockSize * kTileStride];
  __shared__ __attribute__((aligned(16))) unsigned char s_v[kBlockSize * kTileStride];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int hq = a.n_kv_heads * kGroup;

  const int L = a.seq_lens[b];
  const int r0 = a.q_start[b];
  const int r1 = a.q_start[b + 1];
  const int C = r1 - r0;
  // Rows outside [0, T) are never touched; a chunk longer than its sequence, or a length
  // beyond the table, makes the sequence's rows NaN.
  if (r0 < 0 || r1 > a.total_rows || C <= 0) return;
  const bool bad_len = C > L || L > a.max_blocks * kBlockSize;
  const int nb = bad_len ? 0 : (L + kBlockSize - 1) / kBlockSize;

  // Every page id of the sequence must be in range, else all its rows are NaN.
  if (tid == 0) s_bad = bad_len ? 1 : 0;
  __syncthreads();
  for (int j = tid; j < nb; j += kPfThreads) {
    const int phys = a.block_table[static_cast<size_t>(b) * a.max_blocks + j];
    if (static_cast<unsigned>(phys) >= static_cast<unsigned>(a.num_pages)) s_bad = 1;
  }
  __syncthreads();
  const bool bad = s_bad != 0;

  const int rows_total = C * kGroup;
  const int col = lane & 15;        // this lane's row in S^T / the B operand
  const int quad = lane >> 4;       // which 4 of the 16 k-indices this lane holds

  for (int mb = blockIdx.x; mb * kRowsPerBlock < rows_total; mb += gridDim.x) {
    // ---- this wave's 16 rows: row r = chunk token r / G, head r % G
    const int row = mb * kRowsPerBlock + wave * kRowsPerWave + col;
    const bool live = row < rows_total;
    const int tok = live ? row / kGroup : 0;
    const int h = live ? row % kGroup : 0;
    const int pos = live && !bad ? L - C + tok : -1;      // last visible token of the row
    const size_t q_off = (static_cast<size_t>(r0 + tok) * hq + g * kGroup + h) * kHeadDim;
    // Q^T as the B operand: lane holds Q[row][16 kb + 4 quad + e], kb = 0..7.
    h4 qb[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      if (live) {
        const uint2 w = *reinterpret_cast<const uint2*>(
            static_cast<const _Float16*>(a.q) + q_off + 16 * kb + 4 * quad);
        qb[kb] = __builtin_bit_cast(h4, w);
      } else {
        qb[kb] = h4{0, 0, 0, 0};
      }
    }
    // Last page any row of this block reads.
    const int last_row = min(rows_total, (mb + 1) * kRowsPerBlock) - 1;
    const int last_pos = bad ? -1 : L - C + last_row / kGroup;
    const int pages = bad ? 0 : last_pos / kBlockSize + 1;

    float m = kNegInfPf, l = 0.0f;                // softmax state of row `col`
    f4 o[8];                                      // O[4 quad + e][16 db + col]
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f4{0.f, 0.f, 0.f, 0.f};

    // Staging: thread t moves 16 bytes of each tile: token t / 16, bytes 16 (t % 16). Slots
    // past L_b in the last page are stored as zeros (they may hold anything, NaN included,
    // and a zero weight times NaN would still be NaN in P V); their loads re-read the last
    // valid row, whose cache lines are fetched anyway.
    const int st_tok = tid >> 4;
    const int st_col = (tid & 15) * 16;
    auto fetch = [&](int j, u32x4& kr, u32x4& vr) __attribute__((always_inline)) {
      const int phys = a.block_table[static_cast<size_t>(b) * a.max_blocks + j];
      const size_t base = (static_cast<size_t>(phys) * a.n_kv_heads + g) * (kBlockSize * kHeadDim * 2);
      const int valid = L - j * kBlockSize;          // >= 1 for every page read
      const int tok = min(st_tok, valid - 1);
      kr = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k_pages) + base + tok * 256 + st_col);
      vr = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_pages) + base + tok * 256 + st_col);
      if (st_tok >= valid) kr = vr = u32x4{0u, 0u, 0u, 0u};
    };
    u32x4 kr, vr;
    if (pages > 0) fetch(0, kr, vr);
    for (int j = 0; j < pages; ++j) {
      __syncthreads();   // the previous page is no longer read
      *reinterpret_cast<u32x4*>(s_k + st_tok * kTileStride + st_col) = kr;
      *reinterpret_cast<u32x4*>(s_v + st_tok * kTileStride + st_col) = vr;
      __syncthreads();
      if (j + 1 < pages) fetch(j + 1, kr, vr);

      // S^T = K Q^T over d = 128 in 8 steps of 16.
      f4 s = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const uint2 w = *reinterpret_cast<const uint2*>(s_k + col * kTileStride + (16 * kb + 4 * quad) * 2);
        s = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, w), qb[kb], s, 0, 0, 0);
      }
      // Lane holds S[row col][token 16 j + 4 quad + e]. Online softmax for row `col`.
      float sv[4];
      float mx = kNegInfPf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = j * kBlockSize + 4 * quad + e;
        sv[e] = t <= pos ? s[e] * a.scale_log2 : kNegInfPf;
        mx = fmaxf(mx, sv[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float base = m_new == kNegInfPf ? 0.0f : m_new;
      const float alpha = exp2_fast(m - base);
      float p[4], sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = exp2_fast(sv[e] - base);
        sum += p[e];
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      l = l * alpha + sum;
      m = m_new;
      // Rescale O: its rows are 4 quad + e, whose alpha sits in lane 4 quad + e.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __shfl(alpha, 4 * quad + e);
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][e] *= ae;
      }
      // O += P V: P[row col][token 4 quad + e] is already the A operand's layout.
      const h4 pa = h4{static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1]),
                       static_cast<_Float16>(p[2]), static_cast<_Float16>(p[3])};
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        h4 vb;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vb[e] = *reinterpret_cast<const _Float16*>(s_v + (4 * quad + e) * kTileStride + (16 * db + col) * 2);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, o[db], 0, 0, 0);
      }
    }

    // Normalise and store: lane holds O[row 4 quad + e][d = 16 db + col].
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = mb * kRowsPerBlock + wave * kRowsPerWave + 4 * quad + e;
      const float le = __shfl(l, 4 * quad + e);
      if (r >= rows_total) continue;
      const int rt = r / kGroup;
      const int rh = r % kGroup;
      float* dst = a.out + (static_cast<size_t>(r0 + rt) * hq + g * kGroup + rh) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 8; ++db) dst[16 * db + col] = bad ? nan : o[db][e] / le;
    }
  }
}

}  // namespace

hipError_t launch_prefill(int group, const PrefillArgs& a, int max_chunk, hipStream_t stream) {
  const long long blocks = (static_cast<long long>(max_chunk) * group + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid(static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 65535 ? 65535 : blocks)),
                  static_cast<unsigned>(a.n_kv_heads), static_cast<unsigned>(a.batch));
  switch (group) {
    case 1: hipLaunchKernelGGL(prefill_kernel<1>, grid, dim3(kPfThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(kPfThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(kPfThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL(prefill_kernel<8>, grid, dim3(kPfThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dattn
