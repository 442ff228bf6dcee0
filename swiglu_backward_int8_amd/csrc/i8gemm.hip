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
// MFMAs.  Each wave owns 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.  Per stage of
// 128 along K, the A and B tiles (128 x 128 bytes each) and the scales of the
// stage's groups go from memory straight into LDS (buffer loads with the lds
// flag: no staging registers, no LDS write instructions), double buffered:
// the next stage is in flight while the matrix cores work on this one.  Tiles
// are handed out in groups of 4 tile-rows, and each XCD takes a contiguous
// range of that order, so that the workgroups resident on one XCD share A and
// B tiles in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "siluquant.h"

namespace {

constexpr int kBK = 128;                  // the K stage
constexpr int kWavesM = 2, kWavesN = 2;   // wave grid of a workgroup
constexpr int kBM = 64 * kWavesM, kBN = 64 * kWavesN;  // tile of C: 128 x 128
constexpr int kGemmThreads = 64 * kWavesM * kWavesN;   // 256
constexpr int kWaves = kGemmThreads / 64;
constexpr int kGroupM = 4;                // tile-rows per raster group (2, 6, 8, 16, 32 measured slower)
constexpr int kOpBytes = kBM * kBK;       // one operand's stage: 16 KB
constexpr int kStageBytes = 2 * kOpBytes; // A, then B
constexpr int kRowsPerLoad = 8;           // a wave-wide 16-byte-per-lane load covers 8 rows of 128 bytes
constexpr int kLoadsPerWave = kBM / kRowsPerLoad / kWaves;  // per operand and stage: 4
static_assert(kBM == kBN && kBM + kBN == kGemmThreads, "one scale per thread; A and B share row offsets");

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// LDS layout of a tile: rows of 128 bytes, whose eight 16-byte chunks are
// stored at positions XOR-permuted by the row.  MFMA operand reads (32
// consecutive rows, one chunk each) then fall on distinct banks, for 32 or 64
// banks.  Logical chunk c of row r sits at physical chunk c ^ swz(r):
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Buffer resource words: base, 32-bit record count (loads at or past it read
// as zeros), raw addressing.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (i32x4){(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xFFFF, (int)bytes, 0x00020000};
}

// Loads into LDS: each lane reads 16 (or 4) bytes at voffset + soffset of the
// buffer (voffset is range-checked against the record count) and the wave
// writes them, lane by lane, to consecutive LDS bytes from address lds (M0)
// on.  They are written as asm so that the compiler, which cannot tell which
// LDS bytes they write, does not wait for all of them before every LDS read;
// the kernel waits for them itself (wait_vm_all) before the barrier that
// publishes a stage.  The instructions have no register result.  A load that
// takes its LDS address from M0 needs one wait state after M0 is written; the
// compiler writes M0 right before the asm and does not look inside it, so the
// asm starts with an s_nop.
__device__ __forceinline__ void lds_load16(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void lds_load4(i32x4 rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// kBlockScale: B's scale rows cover 128 rows (one scale per tile and group).
// kG: the group size along K (128, 64 or 32); a stage holds kSub = 128 / kG
// groups, each promoted on its own.
template <bool kBf16Out, bool kBlockScale, int kG>
__global__ __launch_bounds__(kGemmThreads, 2) void i8_gemm_kernel(const int8_t* __restrict__ A,
                                                                  const float* __restrict__ sA,
                                                                  const int8_t* __restrict__ B,
                                                                  const float* __restrict__ sB, void* __restrict__ C,
                                                                  int64_t M, int64_t N, int64_t K, int tiles_m,
                                                                  int tiles_n, int per_xcd) {
  constexpr int kSub = kBK / kG, kStepsPerGroup = kG / 32;  // MFMA k-steps (32 of K) per group
  __shared__ __attribute__((aligned(16))) char s_tile[2][kStageBytes];
  // scales of the stage's groups: [buffer][group in stage][A rows, then B rows]
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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / kWavesN) * 64, wn = (wave % kWavesN) * 64;  // the wave's 64 x 64 corner
  // K is a multiple of kG; with kG < 128 the last stage may hold fewer than
  // kSub groups, and its chunks past K read as zeros.
  const int stages = (int)((K + kBK - 1) / kBK), groups = (int)(K / kG);

  // Rows past M or N read as zeros: the record count ends at the tile's last
  // row, and every row offset is in the range-checked lane offset.
  const int a_rows = M - m0 < kBM ? (int)(M - m0) : kBM;
  const int b_rows_here = N - n0 < kBN ? (int)(N - n0) : kBN;
  const i32x4 ra = rsrc_words(A + m0 * K, (int64_t)a_rows * K);
  const i32x4 rb = rsrc_words(B + n0 * K, (int64_t)b_rows_here * K);
  // Scales: waves 0-1 load the tile's A rows, waves 2-3 its B rows (with
  // block scales, the tile's one B scale into every B slot).
  const bool sc_a = wave < 2;
  const i32x4 rsc = sc_a ? rsrc_words(sA + m0 * groups, (int64_t)a_rows * groups * 4)
                    : kBlockScale ? rsrc_words(sB + (n0 / kBN) * groups, (int64_t)groups * 4)
                                  : rsrc_words(sB + n0 * groups, (int64_t)b_rows_here * groups * 4);
  const uint32_t sc_voff = (!sc_a && kBlockScale) ? 0u : (uint32_t)((64 * (wave & 1) + lane) * groups * 4);

  // Load j of this wave per operand covers rows R0 = 8 (4 w + j) + [0, 8):
  // lane L writes LDS row R0 + L / 8 at physical chunk L % 8, so it reads
  // logical chunk (L % 8) ^ swz(row) of that row.
  uint32_t voff[kLoadsPerWave], voff_last[kLoadsPerWave];
  const int k_last = (stages - 1) * kBK;
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) {
    const int R = kRowsPerLoad * (kLoadsPerWave * wave + j) + (lane >> 3);
    const int c = (lane & 7) ^ swz(R);
    voff[j] = (uint32_t)(R * K + 16 * c);
    // in a last stage that K ends inside (a multiple of 32 bytes), chunks
    // past K read as zeros
    voff_last[j] = 16 * c < K - k_last ? voff[j] : 0x80000000u;
  }
  const uint32_t lds_tile = (uint32_t)reinterpret_cast<uintptr_t>(&s_tile[0][0]);
  const uint32_t lds_scale = (uint32_t)reinterpret_cast<uintptr_t>(&s_scale[0][0][0]);

  // Stage s into buffer s % 2: the scales of its groups, then the A and B rows.
  auto issue = [&](int s) {
    const int buf = s & 1;
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const int g = s * kSub + u;
      if (g < groups)
        lds_load4(rsc, lds_scale + 4 * ((buf * kSub + u) * (kBM + kBN) + 64 * wave), sc_voff, (uint32_t)(4 * g));
    }
    const bool last = s == stages - 1;
    const uint32_t k0 = (uint32_t)(s * kBK);
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const uint32_t at = lds_tile + buf * kStageBytes + kRowsPerLoad * (kLoadsPerWave * wave + j) * kBK;
      lds_load16(ra, at, last ? voff_last[j] : voff[j], k0);
      lds_load16(rb, at + kOpBytes, last ? voff_last[j] : voff[j], k0);
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
  const int a_base = (wm + lrow) * kBK + 16 * (lhalf ^ swz(wm + lrow));
  const int b_base = kOpBytes + (wn + lrow) * kBK + 16 * (lhalf ^ swz(wn + lrow));
  auto off = [](int base, int blk, int s) { return (base ^ (32 * s) ^ (64 * blk)) + 32 * kBK * blk; };

  // One stage from LDS buffer buf: per group, its k-steps of 2 x 2 MFMAs into
  // exact int32 sums, then acc += float(I) * (sA[m] * sB[n]).  The lane's
  // rows are 8 q + 4 lhalf + e (q = r / 4, e = r % 4) of each 32-row block,
  // its column lrow of each 32-column block.
  auto compute = [&](int s) {
    const int buf = s & 1;
    const char* t = s_tile[buf];
    // With several groups per stage the loop over them stays rolled, so that
    // one group's int32 sums are promoted before the next group's MFMAs start
    // (unrolled, the scheduler overlaps them and runs out of registers).
#pragma unroll 1
    for (int j = 0; j < kSub; ++j) {
      if (s * kSub + j >= groups) break;  // a last stage that K ends inside
      i32x16 I[2][2];
#pragma unroll
      for (int ks = j * kStepsPerGroup; ks < (j + 1) * kStepsPerGroup; ++ks) {
        i32x4 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const i32x4*>(t + off(a_base, i, ks));
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) fb[jj] = *reinterpret_cast<const i32x4*>(t + off(b_base, jj, ks));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            I[i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[jj],
                                                             ks == j * kStepsPerGroup ? (i32x16){} : I[i][jj], 0, 0, 0);
      }
      const float* scl = s_scale[buf][j];
      float sb[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) sb[jj] = kBlockScale ? scl[kBM] : scl[kBM + wn + 32 * jj + lrow];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 sa = *reinterpret_cast<const float4*>(&scl[wm + 32 * i + 8 * q + 4 * lhalf]);
          const float sav[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q + e;
            const float sc0 = sav[e] * sb[0];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const float sc = kBlockScale ? sc0 : sav[e] * sb[jj];
              acc[i][jj][r] = __builtin_fmaf((float)I[i][jj][r], sc, acc[i][jj][r]);
            }
          }
        }
      }
    }
  };

  // Stage s: wait for this thread's loads of it, then the barrier publishes
  // them to every wave and tells that every wave is done with the other
  // buffer, into which stage s + 1 then goes while s is computed.
  if (stages > 0) issue(0);
  for (int s = 0; s < stages; ++s) {
    wait_vm_all();
    __syncthreads();
    if (s + 1 < stages) issue(s + 1);
    compute(s);
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
                            int, int, int);
  auto pick = [&](auto g_tag) -> KernelFn {
    constexpr int kG = decltype(g_tag)::value;
    return bf16 ? (blk ? i8_gemm_kernel<true, true, kG> : i8_gemm_kernel<true, false, kG>)
                : (blk ? i8_gemm_kernel<false, true, kG> : i8_gemm_kernel<false, false, kG>);
  };
  const KernelFn kernel = group == 128 ? pick(std::integral_constant<int, 128>{})
                          : group == 64 ? pick(std::integral_constant<int, 64>{})
                                        : pick(std::integral_constant<int, 32>{});
  hipLaunchKernelGGL(kernel, grid, block, 0, s, A, sA, B, sB, C, M, N, K, (int)tiles_m, (int)tiles_n, per_xcd);
  if (hipGetLastError() != hipSuccess) return SILUQUANT_ERR_LAUNCH_FAILED;
  return SILUQUANT_OK;
}

}  // extern "C"
