// Group-scaled int8 GEMM on the CDNA4 matrix cores (gfx950): the consumer of
// the two quantised layouts the fused SwiGLU pass writes.
//
//   C[m, n] = sum_g sA[m, g] * sB[n / Bb, g] * sum_{k in group g} A[m, k] * B[n, k]
//
// A [M, K] and B [N, K] are int8 row-major (C = A . B^T), groups are 128 wide
// along K, sA is fp32 [M, K/128], sB fp32 [ceil(N/Bb), K/128] with Bb = 1 (one
// scale per row, as y_s_t) or 128 (one per 128-row block, a weight's layout).
// The fusion bullet of the page "kernelgen-challenge-9-task3-silu-quant"
// names the two quantisations (K-group for [d_gate, d_up] along channels,
// M-group for y^T along tokens); each is a group-128 split of the contraction
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
// Kernel: 256 threads (4 waves in a 2 x 2 grid) per 128 x 128 tile of C; each
// wave owns 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  Per group the A and B
// tiles (128 x 128 bytes each) and their 256 scales are staged in LDS, double
// buffered: the global loads of group g + 1 are in flight while the matrix
// cores work on group g.  LDS rows are 128 bytes of 16-byte chunks stored at a
// position XOR-swizzled by the row, so that both the staging writes and the
// MFMA operand reads (32 rows, one chunk each) hit distinct banks.  Tiles are
// handed out in groups of 8 tile-rows, and each XCD takes a contiguous range
// of that order, so that the workgroups resident on one XCD share A and B
// tiles in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "siluquant.h"

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 128;  // tile of C and the K step (one group)
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;                    // tile-rows per raster group
constexpr int kStageBytes = (kBM + kBN) * kBK;  // A and B tiles of one group

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Byte offset of logical 16-byte chunk c of row r inside a 128-byte-row tile.
__device__ __forceinline__ int swz(int r, int c) { return r * kBK + 16 * (c ^ ((r ^ (r >> 3)) & 7)); }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool kBf16Out>
__global__ __launch_bounds__(kGemmThreads, 2) void i8_gemm_kernel(const int8_t* __restrict__ A,
                                                                  const float* __restrict__ sA,
                                                                  const int8_t* __restrict__ B,
                                                                  const float* __restrict__ sB, void* __restrict__ C,
                                                                  int64_t M, int64_t N, int64_t K, int b_rows,
                                                                  int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(16))) char s_tile[2][kStageBytes];
  __shared__ __attribute__((aligned(16))) float s_scale[2][kBM + kBN];

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
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;  // the wave's 64 x 64 corner
  const int groups = (int)(K / kBK);

  // Staging: 16-byte chunk ids tid + 256 i, i = 0..3, for each of A and B.
  const int64_t a_rows_left = M - m0, b_rows_left = N - n0;
  auto load_stage = [&](int g, u32x4 (&ra)[4], u32x4 (&rb)[4], float& sc) {
    const int64_t k0 = (int64_t)g * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kGemmThreads * i, r = id >> 3, c = id & 7;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      ra[i] = r < a_rows_left ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A + (m0 + r) * K + k0 + 16 * c))
                              : zero;
      rb[i] = r < b_rows_left ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(B + (n0 + r) * K + k0 + 16 * c))
                              : zero;
    }
    if (tid < kBM)
      sc = tid < a_rows_left ? sA[(m0 + tid) * groups + g] : 0.0f;
    else
      sc = tid - kBM < b_rows_left ? sB[((n0 + tid - kBM) / b_rows) * groups + g] : 0.0f;
  };
  auto store_stage = [&](int buf, const u32x4 (&ra)[4], const u32x4 (&rb)[4], float sc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + kGemmThreads * i, r = id >> 3, c = id & 7;
      *reinterpret_cast<u32x4*>(&s_tile[buf][swz(r, c)]) = ra[i];
      *reinterpret_cast<u32x4*>(&s_tile[buf][kBM * kBK + swz(r, c)]) = rb[i];
    }
    s_scale[buf][tid] = sc;
  };

  float acc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 ra[4], rb[4];
  float sc = 0.0f;
  if (groups > 0) {
    load_stage(0, ra, rb, sc);
    store_stage(0, ra, rb, sc);
  }
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int g = 0; g < groups; ++g) {
    const int buf = g & 1;
    if (g + 1 < groups) load_stage(g + 1, ra, rb, sc);

    const char* ta = s_tile[buf];
    const char* tb = s_tile[buf] + kBM * kBK;
    i32x16 I[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) I[i][j] = (i32x16){};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + lhalf;
      i32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const i32x4*>(ta + swz(wm + 32 * i + lrow, c));
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const i32x4*>(tb + swz(wn + 32 * j + lrow, c));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) I[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], I[i][j], 0, 0, 0);
    }
    // promotion: acc += float(I) * (sA[m] * sB[n]); the lane's rows are
    // 8 q + 4 lhalf + e (q = r / 4, e = r % 4) of each 32-row block, its
    // column lrow of each 32-column block
    float sb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sb[j] = s_scale[buf][kBM + wn + 32 * j + lrow];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 sa = *reinterpret_cast<const float4*>(&s_scale[buf][wm + 32 * i + 8 * q + 4 * lhalf]);
        const float sav[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int r = 4 * q + e;
            acc[i][j][r] = __builtin_fmaf((float)I[i][j][r], sav[e] * sb[j], acc[i][j][r]);
          }
      }
    }
    if (g + 1 < groups) {
      store_stage(buf ^ 1, ra, rb, sc);
    }
    __syncthreads();
  }

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
                                                                int c_dtype, void* stream) {
  if (group != kBK) return SILUQUANT_ERR_BAD_GROUP;
  if (M < 0 || N < 0 || K < 0 || K % kBK != 0 || (b_rows_per_scale != 1 && b_rows_per_scale != kBN) ||
      (c_dtype != SILUQUANT_GEMM_OUT_F32 && c_dtype != SILUQUANT_GEMM_OUT_BF16))
    return SILUQUANT_ERR_BAD_SHAPE;
  if (M == 0 || N == 0) return SILUQUANT_OK;
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  // int tile indices; 32-bit K per row is ample, but row offsets are int64
  if (tiles_m * tiles_n > (int64_t(1) << 30) || K > (int64_t(1) << 30)) return SILUQUANT_ERR_BAD_SHAPE;
  if (!C || (K > 0 && (!A || !sA || !B || !sB))) return SILUQUANT_ERR_NULL_PTR;
  auto mis = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
  if (mis(A, 16) || mis(B, 16) || mis(sA, 4) || mis(sB, 4) || mis(C, c_dtype == SILUQUANT_GEMM_OUT_F32 ? 4 : 2))
    return SILUQUANT_ERR_MISALIGNED;
  const int64_t groups = K / kBK;
  const int64_t c_bytes = M * N * (c_dtype == SILUQUANT_GEMM_OUT_F32 ? 4 : 2);
  const void* in[4] = {A, sA, B, sB};
  const int64_t in_bytes[4] = {M * K, 4 * M * groups, N * K, 4 * ((N + b_rows_per_scale - 1) / b_rows_per_scale) * groups};
  for (int i = 0; i < 4; ++i)
    if (in[i] && spans_overlap(in[i], in_bytes[i], C, c_bytes)) return SILUQUANT_ERR_OVERLAP;

  const int tiles = (int)(tiles_m * tiles_n);
  const int per_xcd = (tiles + 7) / 8;
  const dim3 grid(8 * per_xcd), block(kGemmThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c_dtype == SILUQUANT_GEMM_OUT_BF16)
    hipLaunchKernelGGL(i8_gemm_kernel<true>, grid, block, 0, s, A, sA, B, sB, C, M, N, K, (int)b_rows_per_scale,
                       (int)tiles_m, (int)tiles_n, per_xcd);
  else
    hipLaunchKernelGGL(i8_gemm_kernel<false>, grid, block, 0, s, A, sA, B, sB, C, M, N, K, (int)b_rows_per_scale,
                       (int)tiles_m, (int)tiles_n, per_xcd);
  if (hipGetLastError() != hipSuccess) return SILUQUANT_ERR_LAUNCH_FAILED;
  return SILUQUANT_OK;
}

}  // extern "C"
