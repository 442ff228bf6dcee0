// libsiluquant: fused SwiGLU forward recompute + backward + two-axis int8
// quantisation for gfx950 (MI355X).
//
// Operation: the page "kernelgen-challenge-9-task3-silu-quant" (githubhelp.com),
// entry-point listing and output bullets; its design-constraint list asks for
// 128 x 128 tiles (both group axes are 128 long), one fused pass, a bf16 round
// trip before quantising, and a multiply by a precomputed inverse scale.  The
// arithmetic contract is spelled out in include/siluquant.h.
//
// Design (one kernel, one pass over HBM):
//   * one 512-thread workgroup per 128-token x 128-channel tile; every group of
//     both quantisation axes lies inside one tile, so no workgroup ever waits on
//     another;
//   * lane (q, p) = (tid / 16, tid % 16) owns tokens 4q..4q+3 and channels
//     8p..8p+7: each of its 12 loads is 16 bytes and a wave's load covers four
//     whole 256-byte row segments;
//   * sigmoid comes from a 31 KB table in LDS indexed by the bf16 bits of the
//     gate.  Gates are bf16, so only 7,223 inputs give a sigmoid outside
//     {0, 1/2, 1}; the table holds every magnitude between the ranges where it
//     saturates, and clamping the index reproduces the saturated values.  The
//     table is built once per device with fp64 exp rounded to fp32, which makes
//     the sigmoid bit-exact rather than within an ulp;
//   * group maxima: each lane reduces inside its registers, writes partial
//     maxima to LDS, and one thread per group (384 groups per tile) finishes
//     the reduction and computes scale and inverse with IEEE division;
//   * grad_input_q is stored straight from registers (a wave writes four whole
//     128-byte row segments); y_q_t goes through an XOR-swizzled LDS transpose
//     so that it, too, leaves in whole 128-byte rows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "siluquant.h"

namespace {

constexpr int kGroup = 128;
constexpr int kTile = 128;
constexpr int kThreads = 512;

// Sigmoid table: entry k of half `sign` holds s(g) for the bf16 gate with bits
// (sign << 15) | (kSigM0 + k).  Every magnitude at or below kSigM0 gives
// s == 1/2 for both signs, and every magnitude at or above kSigM0 + kSigL - 1
// gives s == 1 (g > 0) or s == 0 (g < 0), so clamping k covers all bf16 gates.
constexpr uint32_t kSigM0 = 0x3380;  // 2^-24
constexpr int kSigL = 3892;          // up to 0x42B3 (-89.5 .. past the s == 0 edge at -89)
constexpr int kSigEntries = 2 * kSigL;
static_assert(kSigEntries % 4 == 0, "table copied in 16-byte pieces");

__device__ float g_sigma_tab[kSigEntries];

// LDS layout (floats).  The table stays live through the elementwise phase;
// the partial maxima and the transpose buffer follow it.
constexpr int kRowPartStride = 2 * kTile + 4;  // 260: rows of 16-byte writes spread over banks
constexpr int kRowPartFloats = 16 * kRowPartStride;
constexpr int kColPartFloats = 32 * kTile;
constexpr int kInvFloats = 3 * kTile;  // 256 row groups + 128 column groups
constexpr int kYqtBytes = kTile * kTile;
static_assert(kYqtBytes <= kRowPartFloats * 4, "transpose buffer reuses the row partials");

constexpr int kLdsFloats = kSigEntries + kRowPartFloats + kColPartFloats + kInvFloats;

__global__ void build_sigma_table_kernel() {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= kSigEntries) return;
  uint32_t sign = i >= kSigL ? 1u : 0u;
  uint32_t mag = kSigM0 + (uint32_t)(i - (int)sign * kSigL);
  float g = __uint_as_float(((sign << 15) | mag) << 16);
  float e = (float)exp(-(double)g);
  float den = 1.0f + e;
  g_sigma_tab[i] = 1.0f / den;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to the nearest bf16 (ties to even) and return it widened to fp32.
__device__ __forceinline__ float round_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u = u + 0x7fffu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xffff0000u);
}

__device__ __forceinline__ int sigma_index(uint32_t b16) {
  int k = (int)(b16 & 0x7fffu) - (int)kSigM0;
  k = min(max(k, 0), kSigL - 1);
  return k + (int)(b16 >> 15) * kSigL;
}

// One (t, h) position: gate g (bits gb), up u, grad_y d -> bf16-rounded
// y, d_gate, d_up.  Operation order is fixed; no contraction (-ffp-contract=off).
__device__ __forceinline__ void pair(const float* __restrict__ tab, uint32_t gb, float g, float u, float d,
                                     float& y, float& dg, float& du) {
  float s = tab[sigma_index(gb)];
  float silu = g * s;
  float yv = silu * u;
  float a = d * u;
  float b = a * s;
  float c = 1.0f - s;
  float k = g * c;
  float m = 1.0f + k;
  float dgv = b * m;
  float duv = d * silu;
  y = round_bf16(yv);
  dg = round_bf16(dgv);
  du = round_bf16(duv);
}

__device__ __forceinline__ float amax2(float a, float b) { return fmaxf(fabsf(a), fabsf(b)); }

// Quantise one value: the low byte of the returned word is the int8 code.
// Adding 1.5 * 2^23 moves |t| <= 128 into the range where fp32 spacing is 1,
// so the add itself rounds to the nearest integer, ties to even, and the
// integer sits in the low mantissa bits in two's complement.  With a finite
// inverse scale |v * inv| stays below 127.5, so no clamp is needed; kSafe adds
// the clamp and the v == 0 rule for groups whose inverse overflowed.
template <bool kSafe>
__device__ __forceinline__ uint32_t code_word(float v, float inv) {
  float t = v * inv;
  if (kSafe) t = (v == 0.0f) ? 0.0f : fminf(fmaxf(t, -127.0f), 127.0f);
  return __float_as_uint(t + 12582912.0f);
}

// Low bytes of four words -> one word, b0 in the lowest byte.
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  uint32_t a = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  uint32_t b = __builtin_amdgcn_perm(b2, a, 0x0c040100u);
  return (b3 << 24) | b;
}

__device__ __forceinline__ float group_scale(float amax) { return amax == 0.0f ? 1.0f : amax / 127.0f; }

template <bool kSafe>
__device__ __forceinline__ void quantise_tile(const float (&Y)[4][8], const float (&DG)[4][8],
                                              const float (&DU)[4][8], const float4 inv_dg, const float4 inv_du,
                                              const float4 inv_y0, const float4 inv_y1, int8_t* __restrict__ gq_row0,
                                              int64_t two_h, int64_t H, uint32_t* __restrict__ yqt_words, int p,
                                              int q) {
  const float idg[4] = {inv_dg.x, inv_dg.y, inv_dg.z, inv_dg.w};
  const float idu[4] = {inv_du.x, inv_du.y, inv_du.z, inv_du.w};
  const float iy[8] = {inv_y0.x, inv_y0.y, inv_y0.z, inv_y0.w, inv_y1.x, inv_y1.y, inv_y1.z, inv_y1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[8], v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      w[j] = code_word<kSafe>(DG[i][j], idg[i]);
      v[j] = code_word<kSafe>(DU[i][j], idu[i]);
    }
    uint2 cg = make_uint2(pack4(w[0], w[1], w[2], w[3]), pack4(w[4], w[5], w[6], w[7]));
    uint2 cu = make_uint2(pack4(v[0], v[1], v[2], v[3]), pack4(v[4], v[5], v[6], v[7]));
    int8_t* row = gq_row0 + (int64_t)i * two_h;
    *reinterpret_cast<uint2*>(row) = cg;
    *reinterpret_cast<uint2*>(row + H) = cu;
  }
  // y codes, transposed: channel 8p + j gets tokens 4q..4q+3 as one word.
  // Word q of transposed row h is stored at position q ^ (4 * ((h >> 3) & 7)),
  // which spreads a wave's 64 writes evenly over the 32 banks and keeps every
  // aligned group of four words (16 tokens) contiguous for the read-back.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t word = pack4(code_word<kSafe>(Y[0][j], iy[j]), code_word<kSafe>(Y[1][j], iy[j]),
                          code_word<kSafe>(Y[2][j], iy[j]), code_word<kSafe>(Y[3][j], iy[j]));
    int h = 8 * p + j;
    yqt_words[h * 32 + (q ^ ((p & 7) << 2))] = word;
  }
}

__global__ __launch_bounds__(kThreads) void silu_quant_bwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ grad_y, int8_t* __restrict__ grad_input_q,
    float* __restrict__ grad_input_s, int8_t* __restrict__ y_q_t, float* __restrict__ y_s_t, int64_t T, int64_t H,
    int tiles_h) {
  __shared__ __align__(16) float lds[kLdsFloats];
  float* s_tab = lds;
  float* s_rowpart = lds + kSigEntries;
  float* s_colpart = s_rowpart + kRowPartFloats;
  float* s_inv = s_colpart + kColPartFloats;
  uint32_t* s_yqt = reinterpret_cast<uint32_t*>(s_rowpart);

  const int tid = threadIdx.x;
  const int p = tid & 15;
  const int q = tid >> 4;
  const int tile = blockIdx.x;
  const int tb = tile / tiles_h;
  const int hb = tile - tb * tiles_h;
  const int64_t t0 = (int64_t)tb * kTile;
  const int64_t h0 = (int64_t)hb * kTile;
  const int64_t two_h = 2 * H;

  // Inputs: 4 rows x (gate, up, grad_y) x 8 channels, 16 bytes each.
  uint4 gin[4], uin[4], din[4];
  {
    const uint16_t* xr = x + (t0 + 4 * q) * two_h + h0 + 8 * p;
    const uint16_t* dr = grad_y + (t0 + 4 * q) * H + h0 + 8 * p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gin[i] = *reinterpret_cast<const uint4*>(xr + i * two_h);
      uin[i] = *reinterpret_cast<const uint4*>(xr + i * two_h + H);
      din[i] = *reinterpret_cast<const uint4*>(dr + i * H);
    }
  }
  // Sigmoid table into LDS.
  {
    const float4* src = reinterpret_cast<const float4*>(g_sigma_tab);
    float4* dst = reinterpret_cast<float4*>(s_tab);
    for (int i = tid; i < kSigEntries / 4; i += kThreads) dst[i] = src[i];
  }
  __syncthreads();

  float Y[4][8], DG[4][8], DU[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t gw[4] = {gin[i].x, gin[i].y, gin[i].z, gin[i].w};
    const uint32_t uw[4] = {uin[i].x, uin[i].y, uin[i].z, uin[i].w};
    const uint32_t dw[4] = {din[i].x, din[i].y, din[i].z, din[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pair(s_tab, gw[k] & 0xffffu, bf16_lo(gw[k]), bf16_lo(uw[k]), bf16_lo(dw[k]), Y[i][2 * k], DG[i][2 * k],
           DU[i][2 * k]);
      pair(s_tab, gw[k] >> 16, bf16_hi(gw[k]), bf16_hi(uw[k]), bf16_hi(dw[k]), Y[i][2 * k + 1],
           DG[i][2 * k + 1], DU[i][2 * k + 1]);
    }
  }

  // Partial maxima.  Row groups: lane (q, p) covers 8 channels of rows 4q..4q+3.
  // Column groups: the lane covers 4 tokens of channels 8p..8p+7.
  {
    float rg[4], ru[4], cm[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = amax2(DG[i][0], DG[i][1]), b = amax2(DU[i][0], DU[i][1]);
#pragma unroll
      for (int j = 2; j < 8; ++j) {
        a = fmaxf(a, fabsf(DG[i][j]));
        b = fmaxf(b, fabsf(DU[i][j]));
      }
      rg[i] = a;
      ru[i] = b;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cm[j] = fmaxf(amax2(Y[0][j], Y[1][j]), amax2(Y[2][j], Y[3][j]));
    }
    float4* rp = reinterpret_cast<float4*>(s_rowpart + p * kRowPartStride + 4 * q);
    rp[0] = make_float4(rg[0], rg[1], rg[2], rg[3]);
    rp[kTile / 4] = make_float4(ru[0], ru[1], ru[2], ru[3]);
    // column partials: [q][half][4p + jj] for channel 8p + 4*half + jj
    float4* cp = reinterpret_cast<float4*>(s_colpart + q * kTile + 4 * p);
    cp[0] = make_float4(cm[0], cm[1], cm[2], cm[3]);
    cp[16] = make_float4(cm[4], cm[5], cm[6], cm[7]);
  }
  __syncthreads();

  // One thread per group: finish the maximum, compute scale and inverse.
  if (tid < 2 * kTile) {
    const int g = tid;  // g < 128: d_gate of row g; else d_up of row g - 128
    float m = 0.0f;
#pragma unroll
    for (int pp = 0; pp < 16; ++pp) m = fmaxf(m, s_rowpart[pp * kRowPartStride + g]);
    float scale = group_scale(m);
    s_inv[g] = 1.0f / scale;
    const int r = g & (kTile - 1);
    const int64_t row_groups = two_h / kGroup;
    const int64_t col = (g >> 7) * (H / kGroup) + hb;
    grad_input_s[(t0 + r) * row_groups + col] = scale;
  } else if (tid < 3 * kTile) {
    const int c = tid - 2 * kTile;  // channel within the tile
    const int idx = ((c >> 2) & 1) * 64 + (c >> 3) * 4 + (c & 3);
    float m = 0.0f;
#pragma unroll
    for (int qq = 0; qq < 32; ++qq) m = fmaxf(m, s_colpart[qq * kTile + idx]);
    float scale = group_scale(m);
    s_inv[2 * kTile + c] = 1.0f / scale;
    y_s_t[(h0 + c) * (T / kGroup) + tb] = scale;
  }
  __syncthreads();

  {
    const float4 inv_dg = *reinterpret_cast<const float4*>(s_inv + 4 * q);
    const float4 inv_du = *reinterpret_cast<const float4*>(s_inv + kTile + 4 * q);
    const float4 inv_y0 = *reinterpret_cast<const float4*>(s_inv + 2 * kTile + 8 * p);
    const float4 inv_y1 = *reinterpret_cast<const float4*>(s_inv + 2 * kTile + 8 * p + 4);
    // An inverse scale overflows only for a group whose maximum is below
    // 127 * 2^-128; such a group needs the clamp and the v == 0 rule.
    const float big = fmaxf(fmaxf(fmaxf(inv_dg.x, inv_dg.y), fmaxf(inv_dg.z, inv_dg.w)),
                            fmaxf(fmaxf(inv_du.x, inv_du.y), fmaxf(inv_du.z, inv_du.w)));
    const float bigy = fmaxf(fmaxf(fmaxf(inv_y0.x, inv_y0.y), fmaxf(inv_y0.z, inv_y0.w)),
                             fmaxf(fmaxf(inv_y1.x, inv_y1.y), fmaxf(inv_y1.z, inv_y1.w)));
    int8_t* gq_row0 = grad_input_q + (t0 + 4 * q) * two_h + h0 + 8 * p;
    if (__builtin_expect(fmaxf(big, bigy) == __builtin_huge_valf(), 0)) {
      quantise_tile<true>(Y, DG, DU, inv_dg, inv_du, inv_y0, inv_y1, gq_row0, two_h, H, s_yqt, p, q);
    } else {
      quantise_tile<false>(Y, DG, DU, inv_dg, inv_du, inv_y0, inv_y1, gq_row0, two_h, H, s_yqt, p, q);
    }
  }
  __syncthreads();

  // Transposed codes out: 128 rows of y_q_t x 128 tokens, 16 bytes per thread
  // per step; eight neighbouring threads write one whole 128-byte row segment.
#pragma unroll
  for (int step = 0; step < 2; ++step) {
    const int id = tid + step * kThreads;
    const int h = id >> 3;
    const int chunk = id & 7;
    const int phys = chunk ^ ((h >> 3) & 7);
    const uint4 v = *reinterpret_cast<const uint4*>(s_yqt + h * 32 + phys * 4);
    *reinterpret_cast<uint4*>(y_q_t + (h0 + h) * T + t0 + 16 * chunk) = v;
  }
}

// Diagnostics: the fused kernel's own sigmoid lookup and elementwise helpers,
// run on their own so tests can compare them bit for bit.
__global__ void eval_sigmoid_kernel(const uint16_t* __restrict__ gate, float* __restrict__ s, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  s[i] = g_sigma_tab[sigma_index(gate[i])];
}

__global__ void eval_intermediates_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ grad_y,
                                          uint16_t* __restrict__ y_out, uint16_t* __restrict__ dgdu_out,
                                          int64_t T, int64_t H) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * H) return;
  int64_t t = i / H, h = i - t * H;
  uint32_t gb = x[t * 2 * H + h];
  float g = __uint_as_float(gb << 16);
  float u = __uint_as_float((uint32_t)x[t * 2 * H + H + h] << 16);
  float d = __uint_as_float((uint32_t)grad_y[i] << 16);
  float y, dg, du;
  pair(g_sigma_tab, gb, g, u, d, y, dg, du);
  y_out[i] = (uint16_t)(__float_as_uint(y) >> 16);
  dgdu_out[t * 2 * H + h] = (uint16_t)(__float_as_uint(dg) >> 16);
  dgdu_out[t * 2 * H + H + h] = (uint16_t)(__float_as_uint(du) >> 16);
}

constexpr int kMaxDevices = 64;
std::atomic<bool> g_table_ready[kMaxDevices];
std::mutex g_table_mutex;

int ensure_table(int* device_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SILUQUANT_ERR_DEVICE;
  *device_out = dev;
  if (g_table_ready[dev].load(std::memory_order_acquire)) return SILUQUANT_OK;
  std::lock_guard<std::mutex> lock(g_table_mutex);
  if (g_table_ready[dev].load(std::memory_order_relaxed)) return SILUQUANT_OK;
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return SILUQUANT_ERR_DEVICE;
  hipLaunchKernelGGL(build_sigma_table_kernel, dim3((kSigEntries + 255) / 256), dim3(256), 0, s);
  hipError_t e1 = hipGetLastError();
  hipError_t e2 = hipStreamSynchronize(s);
  hipError_t e3 = hipStreamDestroy(s);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess) return SILUQUANT_ERR_DEVICE;
  g_table_ready[dev].store(true, std::memory_order_release);
  return SILUQUANT_OK;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int64_t siluquant_algorithmic_bytes(int64_t T, int64_t H, int64_t group) {
  if (T < 0 || H < 0 || group != kGroup) return -1;
  const int64_t pairs = T * H;
  // x (4) + grad_y (2) in; grad_input_q (2) + y_q_t (1) out, per pair;
  // plus one fp32 scale per 128 codes on each axis.
  return 9 * pairs + 4 * (2 * pairs / kGroup) + 4 * (pairs / kGroup);
}

__attribute__((visibility("default"))) const char* siluquant_strerror(int status) {
  switch (status) {
    case SILUQUANT_OK: return "ok";
    case SILUQUANT_ERR_NULL_PTR: return "a buffer pointer is NULL";
    case SILUQUANT_ERR_BAD_SHAPE: return "T and H must be non-negative multiples of 128";
    case SILUQUANT_ERR_BAD_GROUP: return "group must be 128";
    case SILUQUANT_ERR_MISALIGNED: return "x, grad_y, grad_input_q, y_q_t need 16-byte and scales 4-byte alignment";
    case SILUQUANT_ERR_OVERLAP: return "buffers overlap";
    case SILUQUANT_ERR_DEVICE: return "HIP runtime error (device query or sigmoid table build)";
    case SILUQUANT_ERR_LAUNCH_FAILED: return "kernel launch failed";
    default: return "unknown status";
  }
}

__attribute__((visibility("default"))) int siluquant_prepare(void) {
  int dev = 0;
  return ensure_table(&dev);
}

__attribute__((visibility("default"))) int silu_dot_fwd_bwd_quant_fuse(const void* x, const void* grad_y,
                                                                       int8_t* grad_input_q, float* grad_input_s,
                                                                       int8_t* y_q_t, float* y_s_t, int64_t T,
                                                                       int64_t H, int64_t group, void* stream) {
  if (group != kGroup) return SILUQUANT_ERR_BAD_GROUP;
  if (T < 0 || H < 0 || T % kTile != 0 || H % kTile != 0) return SILUQUANT_ERR_BAD_SHAPE;
  if (T == 0 || H == 0) return SILUQUANT_OK;
  // Tile indices are int and byte offsets int64: bound both.
  if (T > (int64_t(1) << 40) / H || (T / kTile) * (H / kTile) > 0x7fffffff) return SILUQUANT_ERR_BAD_SHAPE;
  if (!x || !grad_y || !grad_input_q || !grad_input_s || !y_q_t || !y_s_t) return SILUQUANT_ERR_NULL_PTR;
  auto mis16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; };
  auto mis4 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) != 0; };
  if (mis16(x) || mis16(grad_y) || mis16(grad_input_q) || mis16(y_q_t) || mis4(grad_input_s) || mis4(y_s_t))
    return SILUQUANT_ERR_MISALIGNED;
  const int64_t pairs = T * H;
  const void* bufs[6] = {x, grad_y, grad_input_q, grad_input_s, y_q_t, y_s_t};
  const int64_t sizes[6] = {4 * pairs, 2 * pairs, 2 * pairs, 4 * (2 * pairs / kGroup), pairs, 4 * (pairs / kGroup)};
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlaps(bufs[i], sizes[i], bufs[j], sizes[j])) return SILUQUANT_ERR_OVERLAP;

  int dev = 0;
  int rc = ensure_table(&dev);
  if (rc != SILUQUANT_OK) return rc;

  const int tiles_h = (int)(H / kTile);
  const int tiles = (int)(T / kTile) * tiles_h;
  hipLaunchKernelGGL(silu_quant_bwd_kernel, dim3(tiles), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(grad_y), grad_input_q,
                     grad_input_s, y_q_t, y_s_t, T, H, tiles_h);
  if (hipGetLastError() != hipSuccess) return SILUQUANT_ERR_LAUNCH_FAILED;
  return SILUQUANT_OK;
}

__attribute__((visibility("default"))) int siluquant_eval_sigmoid(const void* gate, float* s, int64_t n,
                                                                  void* stream) {
  if (n < 0) return SILUQUANT_ERR_BAD_SHAPE;
  if (n == 0) return SILUQUANT_OK;
  if (!gate || !s) return SILUQUANT_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(gate) & 1u) || (reinterpret_cast<uintptr_t>(s) & 3u))
    return SILUQUANT_ERR_MISALIGNED;
  if (overlaps(gate, 2 * n, s, 4 * n)) return SILUQUANT_ERR_OVERLAP;
  if (n > (int64_t(1) << 40)) return SILUQUANT_ERR_BAD_SHAPE;
  int dev = 0;
  int rc = ensure_table(&dev);
  if (rc != SILUQUANT_OK) return rc;
  hipLaunchKernelGGL(eval_sigmoid_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(gate), s, n);
  return hipGetLastError() == hipSuccess ? SILUQUANT_OK : SILUQUANT_ERR_LAUNCH_FAILED;
}

__attribute__((visibility("default"))) int siluquant_eval_intermediates(const void* x, const void* grad_y,
                                                                        void* y_bf16, void* dgdu_bf16, int64_t T,
                                                                        int64_t H, void* stream) {
  if (T < 0 || H < 0) return SILUQUANT_ERR_BAD_SHAPE;
  if (T == 0 || H == 0) return SILUQUANT_OK;
  if (T > (int64_t(1) << 40) / H) return SILUQUANT_ERR_BAD_SHAPE;
  if (!x || !grad_y || !y_bf16 || !dgdu_bf16) return SILUQUANT_ERR_NULL_PTR;
  auto mis2 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 1u) != 0; };
  if (mis2(x) || mis2(grad_y) || mis2(y_bf16) || mis2(dgdu_bf16)) return SILUQUANT_ERR_MISALIGNED;
  const int64_t pairs = T * H;
  const void* bufs[4] = {x, grad_y, y_bf16, dgdu_bf16};
  const int64_t sizes[4] = {4 * pairs, 2 * pairs, 2 * pairs, 4 * pairs};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(bufs[i], sizes[i], bufs[j], sizes[j])) return SILUQUANT_ERR_OVERLAP;
  int dev = 0;
  int rc = ensure_table(&dev);
  if (rc != SILUQUANT_OK) return rc;
  hipLaunchKernelGGL(eval_intermediates_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(grad_y), static_cast<uint16_t*>(y_bf16),
                     static_cast<uint16_t*>(dgdu_bf16), T, H);
  return hipGetLastError() == hipSuccess ? SILUQUANT_OK : SILUQUANT_ERR_LAUNCH_FAILED;
}

}  // extern "C"
