// Group-scaled int8 GEMM on the CDNA4 matrix cores (gfx950): the consumer of
// the two quantised layouts the fused SwiGLU pass writes.
//
//   C[m, n] = sum_g sA[m, g] * sB[n / Bb, g] * sum_{k in group g} A[m, k] * B[n, k]
//
// A [M, K] and B [N, K] are int8 row-major (C = A . B^T), groups are G = 128,
// 64 or 32 wide along K (K a multiple of G), sA is fp32 [M, K/G], sB fp32
// [ceil(N/Bb), K/G] with Bb = 1 (one scale per row, as y_s_t) or 128 (one per
// 128-row block, a weight's layout).
// The fusion bullet of the page "kernelgen-challenge-9-task3-silu-quant"
// names the two quantisations (K-group for [d_gate, d_up] along channels,
// M-group for y^T along tokens); each is a group split of the contraction
// axis of the GEMM that reads it:
//   dgrad:  dX[T, D]  = grad_input_q[T, 2H] . Wt[D, 2H]^T      (K = 2H)
//   wgrad:  dW[D, H]  = go_q_t[D, T] . y_q_t[H, T]^T           (K = T)
//
// Arithmetic: each group's dot product is an exact int32 from
// v_mfma_i32_32x32x32_i8 (|sum| <= 128 * 127 * 127 < 2^21); it is converted
// to fp32 (exact) and accumulated as acc = fma(float(I), sA * sB, acc), group
// by group in ascending order.  The result is C in fp32 or rounded once to
// bf16 (nearest, ties to even).
//
// Kernel: 256 threads (4 waves in a 2 x 2 grid) per 128 x 128 tile of C, and
// two workgroups per CU, so that one's loads and promotion overlap the other's
// MFMAs.  Each wave owns 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  Per group,
// the A and B tiles (128 x 128 bytes each) and their scales are staged in LDS,
// double buffered: the next group is loaded into registers while the matrix
// cores work on this one.  Tiles are handed out in groups of 4 tile-rows, and
// each XCD takes a contiguous range of that order, so that the workgroups
// resident on one XCD share A and B tiles in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "siluquant.h"

namespace {

constexpr int kBK = 128;                  // the K step: one group
constexpr int kWavesM = 2, kWavesN = 2;   // wave grid of a workgroup
constexpr int kBM = 64 * kWavesM, kBN = 64 * kWavesN;  // tile of C: 128 x 128
constexpr int kGemmThreads = 64 * kWavesM * kWavesN;   // 256
constexpr int kGroupM = 4;                // tile-rows per raster group (2, 6, 8, 16, 32 measured slower)
constexpr int kStageBytes = (kBM + kBN) * kBK;         // A and B tiles of one group
constexpr int kChunksPerThread = kStageBytes / 16 / kGemmThreads;  // 16-byte chunks staged per thread
constexpr int kAChunks = kBM * kBK / 16;  // chunk ids below this are A's, the rest B's
static_assert(kStageBytes % (16 * kGemmThreads) == 0, "whole chunks per thread");
static_assert(kAChunks % kGemmThreads == 0, "a thread's chunks are all A or all B per step");
static_assert(kBM + kBN <= kGemmThreads, "one scale per thread");

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// LDS layout of a tile: rows of 128 bytes, whose eight 16-byte chunks are
// stored at positions XOR-permuted by the row.  Staging writes (eight lanes
// per row, one chunk each) and MFMA operand reads (32 consecutive rows, one
// chunk each) then both fall on distinct banks, for 32 or 64 banks.  Byte
// offset of logical chunk c (0..7) of row r:
__device__ __forceinline__ int lds_at(int r, int c) { return r * kBK + 16 * (c ^ ((r ^ (r >> 3)) & 7)); }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One stage (128 of K) in flight: kChunksPerThread 16-byte chunks and the
// thread's scale of each of the stage's kSub groups.
template <int kSub>
struct Stage {
  i32x4 v[kChunksPerThread];
  float sc[kSub], sb[kSub];
};

// kBlockScale: B's scale rows cover 128 rows (constant over a wave's 64
// columns).  kG: the group size along K (128, 64 or 32); a stage of 128 of K
// holds kSub = 128 / kG groups, each promoted on its own.
template <bool kBf16Out, bool kBlockScale, int kG>
__global__ __launch_bounds__(kGemmThreads, 2) void i8_gemm_kernel(const int8_t* __restrict__ A,
                                                                  const float* __restrict__ sA,
                                                                  const int8_t* __restrict__ B,
                                                                  const float* __restrict__ sB, void* __restrict__ C,
                                                                  int64_t M, int64_t N, int64_t K, int b_rows,
                                                                  int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(16))) char s_tile[2][kStageBytes];
  constexpr int kSub = kBK / kG, kStepsPerGroup = 4 / kSub;  // MFMA k-steps (32 of K) per group
  __shared__ __attribute__((aligned(16))) float s_scale[2][kSub][kBM + kBN];

  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= tiles_m * tiles_n) return;
  // grouped raster: kGroupM tile-rows, column by column
  const int per_group = kGroupM * tiles_n;
  const int first_m = (tile / per_group) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in_group = tile - (tile / per_group) * per_group;
  const int tm = first_m + in_group % gsz, tn = in_group / gsz;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave / kWavesN) * 64, wn = (wave % kWavesN) * 64;  // the wave's 64 x 64 corner
  // K is a multiple of kG; with kG < 128 the last stage may hold fewer than
  // kSub groups, and its chunks past K read as zeros (see load_stage).
  const int stages = (int)((K + kBK - 1) / kBK), groups = (int)(K / kG);

  // Rows past M or N read as zeros: the buffer's record count ends at the last row.
  const int a_rows = M - m0 < kBM ? (int)(M - m0) : kBM;
  const int b_rows_here = N - n0 < kBN ? (int)(N - n0) : kBN;
  const __amdgpu_buffer_rsrc_t ra = rsrc(A + m0 * K, (int64_t)a_rows * K);
  const __amdgpu_buffer_rsrc_t rb = rsrc(B + n0 * K, (int64_t)b_rows_here * K);
  // this thread's scale: A rows for tid < kBM, then B rows
  const bool sc_is_a = tid < kBM;
  const int sc_row = sc_is_a ? tid : tid - kBM;
  const bool sc_live = tid < kBM + kBN && (sc_is_a ? sc_row < a_rows : sc_row < b_rows_here);
  const float* sc_ptr = sc_is_a ? sA + (m0 + sc_row) * groups : sB + ((n0 + sc_row) / b_rows) * groups;
  // with block scales one B scale covers the whole tile (n0 is a multiple of
  // 128): it is folded into the A scales when they are staged
  const float* sb_blk = sB + (n0 / kBN) * groups;

  // Chunk i of this thread is row (tid >> 3) + d of A or of B (d a multiple
  // of 32), 16-byte chunk tid & 7: one byte offset per thread, the row step in
  // the scalar offset.  In LDS, row r + d (r < 32 or d a multiple of 64) has
  // the swizzle of row r XOR (d / 8) mod 8, so the store offsets are the
  // thread's offset XOR a constant plus a constant.
  constexpr int kAPer = kAChunks / kGemmThreads;  // A chunks per thread
  const int g_off = (tid >> 3) * (int)K + 16 * (tid & 7);
  // In a last stage that K ends inside (a multiple of 32 bytes), the chunks
  // past K take an offset past the record count and read as zeros; so do
  // their groups' scales, which do not exist.
  const int k_last = (stages - 1) * kBK;
  const int g_off_last = 16 * (tid & 7) < K - k_last ? g_off : (int)0x80000000;
  const int l_off = lds_at(tid >> 3, tid & 7);
  auto load_stage = [&](int g, Stage<kSub>& st) {
    const int k0 = g * kBK;
    const int off = g == stages - 1 ? g_off_last : g_off;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int row_step = (i < kAPer ? i : i - kAPer) * (kGemmThreads / 8);
      st.v[i] = __builtin_bit_cast(
          i32x4, __builtin_amdgcn_raw_buffer_load_b128(i < kAPer ? ra : rb, off, k0 + row_step * (int)K, 0));
    }
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const bool live = g * kSub + j < groups;
      st.sc[j] = sc_live && live ? sc_ptr[g * kSub + j] : 0.0f;
      if constexpr (kBlockScale) st.sb[j] = live ? sb_blk[g * kSub + j] : 0.0f;
    }
  };
  auto store_stage = [&](int buf, const Stage<kSub>& st) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int row_step = (i < kAPer ? i : i - kAPer) * (kGemmThreads / 8);
      *reinterpret_cast<i32x4*>(&s_tile[buf][(i < kAPer ? 0 : kBM * kBK) + row_step * kBK +
                                            (l_off ^ (16 * ((row_step >> 3) & 7)))]) = st.v[i];
    }
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      float sc = st.sc[j];
      if constexpr (kBlockScale) sc = sc_is_a ? sc * st.sb[j] : 0.0f;
      if (tid < kBM + kBN) s_scale[buf][j][tid] = sc;
    }
  };

  float acc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  // This lane's operand rows are wm + 32 i + lrow (A) and wn + 32 j + lrow
  // (B); k-step s reads logical chunk 2 s + lhalf.  Since wm and wn are
  // multiples of 64 and lrow < 32, the swizzled chunk position of block i is
  // that of block 0 with bit 2 flipped, and k-step s flips bits 1-2 by s: the
  // offset of (i, s) is the (0, 0) offset XOR 32 s XOR 64 i, plus 4096 i.
  const int a_base = lds_at(wm + lrow, lhalf);
  const int b_base = kBM * kBK + lds_at(wn + lrow, lhalf);
  auto off = [](int base, int blk, int s) { return (base ^ (32 * s) ^ (64 * blk)) + 32 * kBK * blk; };

  // One group from LDS buffer buf: 4 k-steps of 2 x 2 MFMAs into exact int32
  // sums, then acc += float(I) * (sA[m] * sB[n]).  The lane's rows are
  // 8 q + 4 lhalf + e (q = r / 4, e = r % 4) of each 32-row block, its column
  // lrow of each 32-column block.  With block scales the staged A scale
  // already holds the product.
  auto compute = [&](int buf) {
    const char* t = s_tile[buf];
    // With several groups per stage the loop over them stays rolled, so that
    // one group's int32 sums are promoted before the next group's MFMAs start
    // (unrolled, the scheduler overlaps them and runs out of registers).
#pragma unroll 1
    for (int j = 0; j < kSub; ++j) {
      i32x16 I[2][2];
#pragma unroll
      for (int s = j * kStepsPerGroup; s < (j + 1) * kStepsPerGroup; ++s) {
        i32x4 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const i32x4*>(t + off(a_base, i, s));
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) fb[jj] = *reinterpret_cast<const i32x4*>(t + off(b_base, jj, s));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            I[i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[jj],
                                                             s == j * kStepsPerGroup ? (i32x16){} : I[i][jj], 0, 0, 0);
      }
      const float* scl = s_scale[buf][j];
      float sb[2];
      if constexpr (!kBlockScale) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) sb[jj] = scl[kBM + wn + 32 * jj + lrow];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 sa = *reinterpret_cast<const float4*>(&scl[wm + 32 * i + 8 * q + 4 * lhalf]);
          const float sav[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const float sc = kBlockScale ? sav[e] : sav[e] * sb[jj];
              acc[i][jj][r] = __builtin_fmaf((float)I[i][jj][r], sc, acc[i][jj][r]);
            }
          }
        }
      }
    }
  };

  // The next group's operands are loaded into registers while this group is
  // computed from LDS, then written to the other LDS buffer.
  Stage<kSub> st;
  if (stages > 0) {
    load_stage(0, st);
    store_stage(0, st);
  }
  __syncthreads();
  // The fence keeps the LDS writes (which wait for the loads) after the whole
  // group's compute, so that the loads have that long to arrive.
  auto group_step = [&](int g, int buf) {
    if (g + 1 < stages) load_stage(g + 1, st);
    compute(buf);
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < stages) store_stage(buf ^ 1, st);
    __syncthreads();
  };
  for (int g = 0; g < stages; ++g) group_step(g, g & 1);

  // epilogue: row m0 + wm + 32 i + 8 q + 4 lhalf + e, column n0 + wn + 32 j + lrow
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn + 32 * j + lrow;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (m < M) {
          if constexpr (kBf16Out)
            static_cast<uint16_t*>(C)[m * N + n] = bf16_rne(acc[i][j][r]);
          else
            static_cast<float*>(C)[m * N + n] = acc[i][j][r];
        }
      }
    }
}

bool spans_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int i8_gemm_group_scaled(const int8_t* A, const float* sA, const int8_t* B,
                                                                const float* sB, void* C, int64_t M, int64_t N,
                                                                int64_t K, int64_t group, int64_t b_rows_per_scale,
                                                                int c_dtype, hipStream_t stream) {
  if (group != 32 && group != 64 && group != 128) return SILUQUANT_ERR_BAD_GROUP;
  if (M < 0 || N < 0 || K < 0 || K % group != 0 || (b_rows_per_scale != 1 && b_rows_per_scale != kBN) ||
      (c_dtype != SILUQUANT_GEMM_OUT_F32 && c_dtype != SILUQUANT_GEMM_OUT_BF16))
    return SILUQUANT_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return SILUQUANT_OK;
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  // int tile indices; a tile's rows of A or B (at most 256 x K bytes) must fit
  // a buffer resource's 31-bit record count
  if (tiles_m * tiles_n > (int64_t(1) << 30) || K > (int64_t(1) << 22)) return SILUQUANT_ERR_BAD_SHAPE;
  if (!C || (K > 0 && (!A || !sA || !B || !sB))) return SILUQUANT_ERR_NULL_PTR;
  auto mis = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (mis(A, 16) || mis(B, 16) || mis(sA, 4) || mis(sB, 4) || mis(C, c_dtype == SILUQUANT_GEMM_OUT_F32 ? 4 : 2))
    return SILUQUANT_ERR_MISALIGNED;
  const int64_t groups = K / group;
  const int64_t c_bytes = M * N * (c_dtype == SILUQUANT_GEMM_OUT_F32 ? 4 : 2);
  const void* in[4] = {A, sA, B, sB};
  const int64_t in_bytes[4] = {M * K, 4 * M * groups, N * K, 4 * ((N + b_rows_per_scale - 1) / b_rows_per_scale) * groups};
  for (int i = 0; i < 4; ++i)
    if (in[i] && spans_overlap(in[i], in_bytes[i], C, c_bytes)) return SILUQUANT_ERR_OVERLAP;

  const int tiles = (int)(tiles_m * tiles_n);
  const int per_xcd = (tiles + 7) / 8;
  const dim3 grid(8 * per_xcd), block(kGemmThreads);
  hipStream_t s = stream;
  const bool bf16 = c_dtype == SILUQUANT_GEMM_OUT_BF16, blk = b_rows_per_scale == kBN;
  using KernelFn = void (*)(const int8_t*, const float*, const int8_t*, const float*, void*, int64_t, int64_t, int64_t,
                            int, int, int, int);
  auto pick = [&](auto g_tag) -> KernelFn {
    constexpr int kG = decltype(g_tag)::value;
    return bf16 ? (blk ? i8_gemm_kernel<true, true, kG> : i8_gemm_kernel<true, false, kG>)
                : (blk ? i8_gemm_kernel<false, true, kG> : i8_gemm_kernel<false, false, kG>);
  };
  const KernelFn kernel = group == 128 ? pick(std::integral_constant<int, 128>{})
                          : group == 64 ? pick(std::integral_constant<int, 64>{})
                                        : pick(std::integral_constant<int, 32>{});
  hipLaunchKernelGGL(kernel, grid, block, 0, s, A, sA, B, sB, C, M, N, K, (int)b_rows_per_scale, (int)tiles_m,
                     (int)tiles_n, per_xcd);
  if (hipGetLastError() != hipSuccess) return SILUQUANT_ERR_LAUNCH_FAILED;
  return SILUQUANT_OK;
}

}  // extern "C"
