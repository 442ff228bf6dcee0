/*
 * libsiluquant -- fused SwiGLU forward recompute, SwiGLU backward and
 * two-axis int8 quantisation for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the page "kernelgen-challenge-9-task3-silu-quant"
 * (githubhelp.com) defines: its entry-point listing gives the name and the
 * argument order, its two output bullets give the outputs, and its list of
 * design constraints gives the 128 x 128 tiling, the bf16 round trip before
 * quantising and the multiplication by a precomputed inverse scale.
 *
 * Plain C ABI: pointers and sizes only.  Device pointers are HIP device (or
 * managed) memory on the current HIP device; `stream` is a hipStream_t (NULL =
 * the null stream).  The library allocates nothing, keeps no state between
 * calls and never waits on a stream: every call checks its arguments, asks
 * the runtime for the current device's compute-unit count, enqueues its
 * kernels and returns, so a call may be captured into a HIP graph, the first
 * call of a process included.
 */
#ifndef SILUQUANT_H
#define SILUQUANT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle, declared as the runtime declares it so
 * that this header needs no HIP header (repeating the typedef is allowed). */
typedef struct ihipStream_t* hipStream_t;

/* Status codes.  Every argument check runs on the host before any HIP call,
 * so a call that returns one of the first five codes has touched neither the
 * device nor any buffer. */
enum siluquant_status {
  SILUQUANT_OK = 0,
  SILUQUANT_ERR_NULL_PTR = 1,      /* a buffer pointer is NULL while T*H > 0 */
  SILUQUANT_ERR_BAD_SHAPE = 2,     /* T < 0, H < 0, too large, H not a multiple of 32 (q8_1 blocks)
                                      or K not a multiple of the group (GEMM) */
  SILUQUANT_ERR_BAD_GROUP = 3,     /* a group size the entry point does not take */
  SILUQUANT_ERR_MISALIGNED = 4,    /* x, grad_y, grad_input_q, y_q_t not 16-byte aligned,
                                      or a scale buffer not 4-byte aligned */
  SILUQUANT_ERR_OVERLAP = 5,       /* two buffers share bytes */
  SILUQUANT_ERR_DEVICE = 6,        /* a HIP runtime call failed (no current device, or the
                                      device query failed) */
  SILUQUANT_ERR_LAUNCH_FAILED = 7, /* the kernel launch reported an error */
};

/*
 * silu_dot_fwd_bwd_quant_fuse -- one fused pass.
 *
 * Inputs (read only):
 *   x       bf16 [T, 2H] row-major; columns [0, H) are gate, [H, 2H) are up.
 *   grad_y  bf16 [T, H]  row-major; the gradient of y = silu(gate) * up.
 * Outputs (fully overwritten; every element written):
 *   grad_input_q  int8 [T, 2H]       [d_gate | d_up] quantised per row, in groups of
 *                                    128 consecutive positions of the 2H-long row
 *                                    (the last group of a row has the 2H % 128
 *                                    positions that remain);
 *   grad_input_s  fp32 [T, ceil(2H/128)]  one scale per such group;
 *   y_q_t         int8 [H, T]        y transposed, quantised in groups of 128
 *                                    consecutive tokens along each row (the last
 *                                    group of a T that is not a multiple of 128
 *                                    has the T % 128 tokens that remain);
 *   y_s_t         fp32 [H, ceil(T/128)]  one scale per such group.
 * Arithmetic: fp32 throughout, no fused multiply-add.  s = 1 / (1 + exp(-g)) with
 * exp(-g) correctly rounded to fp32; y = (g*s)*u;
 * d_gate = ((d*u)*s) * (1 + g*(1 - s)); d_up = d*(g*s); each rounded to bf16
 * (nearest, ties to even) before quantising.  Per group: amax over the bf16
 * values, scale = amax/127 (1.0 when amax == 0), inv = 1/scale (fp32),
 * p = v*inv (one fp32 multiplication), q = clamp(rne(p), -127, 127) (nearest
 * integer, ties to even), with q = 0 for v == 0.
 *   -128 is never produced.  Inputs must be finite and keep y, d_gate and d_up
 *   finite.
 * Group size: `group` is 128 (the page's default), 64 or 32; the scale tensors
 *   are then grad_input_s fp32 [T, ceil(2H/group)] and y_s_t fp32
 *   [H, ceil(T/group)].  When H is not a multiple of `group`, the group at
 *   row position group * floor(H/group) holds the last H % group channels of
 *   d_gate and the first channels of d_up.  Any other group returns
 *   SILUQUANT_ERR_BAD_GROUP.
 * Sizes: any T >= 0 and H >= 0 (T == 0 or H == 0 is a no-op that returns
 *   SILUQUANT_OK), T <= 2^23, H <= 2^22.  y_q_t is written with 16-byte
 *   stores when T % 16 == 0; other T work, with narrower stores.  The results
 *   do not depend on the kernel that runs: H a multiple of `group` takes the
 *   tiled kernel; other multiples of 8 above 128 a tiled kernel that walks
 *   runs of channel blocks and hands each block's d_up to the shifted d_up
 *   groups (below 128, two work items per tile); H not a multiple of 8 (rows
 *   then start off 16 bytes) a tiled kernel over 128-position tiles of the
 *   2H-long row [d_gate | d_up] that loads aligned 16-byte pieces and shifts
 *   them across lanes (slower: d_up is computed in tiles of its own).
 * Ownership: the caller allocates and owns every buffer; the library keeps no
 *   pointer after the call returns.  Buffers must not overlap.
 * Asynchrony: the work is enqueued on `stream` and the call returns without
 *   waiting; outputs are valid once the stream reaches this point.  The
 *   kernels' 31 KB sigmoid table is constant data of the library's code
 *   object, so no call builds, allocates or waits for anything.
 * Returns a siluquant_status code.
 */
int silu_dot_fwd_bwd_quant_fuse(const void* x, const void* grad_y, int8_t* grad_input_q, float* grad_input_s,
                                int8_t* y_q_t, float* y_s_t, int64_t T, int64_t H, int64_t group,
                                hipStream_t stream);

/*
 * silu_dot_fwd_bwd_quant_fuse_fp8 -- the same pass with FP8 codes.
 *
 * The pages name an fp8 quantise kernel among the benchmarked ops (the AstrAI
 * commit page, csrc/bench, its list of added benchmarks) without fixing its
 * format; the format here is OCP FP8 E4M3 (the OCP 8-bit floating point
 * specification: bias 7, no infinities, largest finite 448, subnormals
 * k * 2^-9), which gfx950 converts to in hardware.
 *
 * Arguments, layouts, sizes, ownership, asynchrony and status codes are those
 * of silu_dot_fwd_bwd_quant_fuse; the recomputation of y and of the gradients
 * and the bf16 round trip are identical.  Only the code format differs:
 *   grad_input_q  uint8 [T, 2H] E4M3 bit patterns, per-row 128-channel groups;
 *   y_q_t         uint8 [H, T]  E4M3 bit patterns, 128-token groups;
 *   scale = amax/448 (fp32 division; 1.0 when amax == 0), inv = 1/scale (fp32);
 *   code = E4M3(v * inv) where v * inv is the fp32 product and the conversion
 *   rounds to nearest, ties to even; magnitudes above 448 (only reachable when
 *   inv overflows to infinity for a group of subnormal scale) saturate to
 *   +-448 (0x7E / 0xFE); a zero v gives the zero of its own sign (0x00 / 0x80).
 *   NaN codes (0x7F, 0xFF) are never produced.
 */
int silu_dot_fwd_bwd_quant_fuse_fp8(const void* x, const void* grad_y, void* grad_input_q, float* grad_input_s,
                                    void* y_q_t, float* y_s_t, int64_t T, int64_t H, int64_t group, hipStream_t stream);

/*
 * silu_fwd_quant -- forward SwiGLU with row-wise int8 group quantisation.
 *
 * The fused launch shape of kquant_swiglu_q8_1_rows on the page "kquant_mmq.rs"
 * (docs.atlascybernetics.ai): y = bf16((silu(gate) * up) * w[t]) rounded once to
 * bf16 (nearest, ties to even), then quantised per row in groups of `group`
 * (128, 64 or 32) contiguous channels exactly as above (scale = amax/127, 1.0 for an all-zero
 * group; q = clamp(rne(v * inv)), v == 0 -> 0).  With no row weight, y is the
 * same bf16 value the backward pass recomputes.  The page's `limit` argument
 * has no stated meaning and is not provided.
 *
 *   x           bf16 [T, 2H] as above (read only; 16-byte aligned)
 *   row_weight  fp32 [T], or NULL for weight 1 (4-byte aligned)
 *   y_q         int8 [T, H]       codes (16-byte aligned)
 *   y_s         fp32 [T, ceil(H/group)] one scale per group (4-byte aligned)
 *   y_bf16      bf16 [T, H] the rounded y, or NULL (16-byte aligned)
 * Sizes: any T >= 0 (T <= 2^31), any H >= 0 (H <= 2^22); the last group of a
 *   row has the H % group channels that remain when H is not a multiple of
 *   the group.  H not a multiple of 8 (rows off 16 bytes) loads aligned
 *   pieces and shifts them across lanes, and is slower; long rows of that
 *   kind go a token row x 512 channels per wave.
 * Same ownership, asynchrony and error conventions as above.
 */
int silu_fwd_quant(const void* x, const float* row_weight, int8_t* y_q, float* y_s, void* y_bf16, int64_t T,
                   int64_t H, int64_t group, hipStream_t stream);

/*
 * silu_fwd_quant_q8_1 -- the forward quantiser in the page's q8_1 block layout.
 *
 * The page "kquant_mmq.rs" (docs.atlascybernetics.ai) writes the fused
 * swiglu rows as block_q8_1: per 32 channels, 32 int8 codes and a half2
 * (d, sum), 36 bytes.  y is computed and quantised exactly as silu_fwd_quant
 * with group 32; the block holds, in this order (the page gives the content
 * and size, not the order):
 *   bytes 0-1   d    the group's fp32 scale (amax/127, 1.0 for an all-zero
 *                    group) rounded to IEEE binary16 (nearest, ties to even)
 *   bytes 2-3   sum  fl32(scale * sum of the 32 codes) rounded to binary16:
 *                    the block's values as its codes give them
 *   bytes 4-35  the 32 codes, channel order
 * both halves little-endian.  d overflows to infinity for scales past 65504
 * (|y| above about 8.3e6) and is 0 below 2^-25: the format's range.
 *
 *   x           bf16 [T, 2H] as above (read only; 16-byte aligned)
 *   row_weight  fp32 [T], or NULL for weight 1 (4-byte aligned)
 *   y_q8        uint8 [T, (H/32) * 36] the blocks (4-byte aligned)
 * Sizes: any T >= 0 (T <= 2^28), H a multiple of 32 (H <= 2^22).
 * Same ownership, asynchrony and error conventions as above.
 */
int silu_fwd_quant_q8_1(const void* x, const float* row_weight, void* y_q8, int64_t T, int64_t H, hipStream_t stream);

/*
 * kquant_swiglu_q8_1_rows -- the same forward quantiser in the argument shape
 * of the page's fused launch.
 *
 * The page "kquant_mmq.rs" (docs.atlascybernetics.ai) documents
 * kquant_swiglu_q8_1_rows: separate gate and up inputs, an optional weight
 * per row, and two outputs, h = bf16(swiglu(gate, up) * w[row]) and the
 * block_q8_1 blocks of h, byte-identical to the swiglu launch followed by the
 * q8_1 launch.  Here h and the blocks are exactly those of silu_fwd_quant_q8_1
 * (with y_bf16) on x = [gate | up]:
 *   gate, up  bf16 [rows, inter] row-major (read only; 16-byte aligned; they
 *             may share memory with each other)
 *   w         fp32 [rows], or NULL for weight 1 (4-byte aligned)
 *   h_bf16    bf16 [rows, inter] the rounded h, or NULL (16-byte aligned)
 *   out_q8    uint8 [rows, (inter/32) * 36] the blocks (4-byte aligned)
 * Sizes: any rows >= 0 (rows <= 2^28), inter a multiple of 32 (the page's
 *   check), inter <= 2^22.  The page's `limit` argument has no stated meaning
 *   and is not provided.  Outputs must not overlap any other buffer.
 * Same ownership, asynchrony and error conventions as above.
 */
int kquant_swiglu_q8_1_rows(const void* gate, const void* up, const float* w, void* h_bf16, void* out_q8,
                            int64_t rows, int64_t inter, hipStream_t stream);

/*
 * i8_gemm_group_scaled -- the consumer of the two quantised layouts.
 *
 * The fusion bullet of the page "kernelgen-challenge-9-task3-silu-quant"
 * names the K-group and M-group quantisations: groups of 128 along the
 * contraction axis of the GEMM that reads each product.  This is that GEMM, on
 * the matrix cores (v_mfma_i32_32x32x32_i8):
 *   C[m, n] = sum_g sA[m, g] * sB[n / Bb, g] * sum_{k in group g} A[m, k] * B[n, k]
 *   A  int8 [M, K] row-major (16-byte aligned), sA fp32 [M, K/group];
 *   B  int8 [N, K] row-major (16-byte aligned), sB fp32 [ceil(N/Bb), K/group];
 *   Bb = b_rows_per_scale: 1 (a scale per row of B and group, as y_s_t) or 128
 *        (one per 128 x 128 block of B, a pre-quantised weight);
 *   C  [M, N] row-major, fp32 (c_dtype SILUQUANT_GEMM_OUT_F32, 4-byte aligned)
 *      or bf16 (SILUQUANT_GEMM_OUT_BF16, 2-byte aligned), fully overwritten.
 * Uses: dgrad dX[T, D] = grad_input_q[T, 2H] . Wt[D, 2H]^T (sA = grad_input_s,
 *   Wt the gate/up weight transposed and quantised in 128 x 128 blocks, Bb =
 *   128); wgrad dW[D, H] = go_q_t[D, T] . y_q_t[H, T]^T (sB = y_s_t, Bb = 1).
 * Arithmetic: each group's integer dot is exact (int32); the groups are
 *   accumulated in ascending order as acc = fma(float(dot), sA * sB, acc) in
 *   fp32; bf16 output rounds that once (nearest, ties to even).
 * Group: `group` is 128, 64 or 32 (the pass's group sizes); sA is then
 *   [M, K/group] and sB [ceil(N/Bb), K/group].
 * Sizes: any M, N >= 0 (M == 0 or N == 0 is a no-op), K >= 0 a multiple of
 *   the group (K == 0 writes zeros), K <= 2^22.  Same ownership, asynchrony and status conventions
 *   as above; C must not overlap an input.
 */
enum siluquant_gemm_out { SILUQUANT_GEMM_OUT_F32 = 0, SILUQUANT_GEMM_OUT_BF16 = 1 };
int i8_gemm_group_scaled(const int8_t* A, const float* sA, const int8_t* B, const float* sB, void* C, int64_t M,
                         int64_t N, int64_t K, int64_t group, int64_t b_rows_per_scale, int c_dtype, hipStream_t stream);

/* Optional: makes the HIP runtime load the library's kernels on the current
 * device now, which it otherwise does at the first launch.  No entry point
 * needs it first.  Enqueues nothing, allocates nothing itself; safe to call
 * repeatedly and from several threads.  SILUQUANT_ERR_DEVICE if there is no
 * usable current device. */
int siluquant_prepare(void);

/* Static text for a status code (never NULL). */
const char* siluquant_strerror(int status);

/* Bytes the pass must move per call: reads 6*T*H (x, grad_y), writes 3*T*H
 * int8 codes plus 4*(T*ceil(2H/group) + H*ceil(T/group)) bytes of scales.
 * Host-only arithmetic; returns -1 for negative sizes or a group other than
 * 32, 64 or 128. */
int64_t siluquant_algorithmic_bytes(int64_t T, int64_t H, int64_t group);

/* Diagnostics.  They run the fused kernel's own device helpers on their own so
 * that tests can compare intermediate values bit for bit; the pass itself
 * never needs them.
 *
 * siluquant_eval_sigmoid: s[i] = sigmoid of the bf16 gate gate[i] exactly as the
 *   fused kernel evaluates it.  gate: bf16 [n] (2-byte aligned), s: fp32 [n]
 *   (4-byte aligned), both device memory.  Enqueued on `stream`.
 * siluquant_eval_intermediates: the bf16 values the fused kernel quantises:
 *   y_bf16 [T, H] = bf16(y) and dgdu_bf16 [T, 2H] = [bf16(d_gate) | bf16(d_up)],
 *   from x [T, 2H] and grad_y [T, H] as above; any T, H >= 0; 2-byte aligned
 *   device buffers that must not overlap.  Enqueued on `stream`.
 * Both return siluquant_status codes with the same meanings as above. */
int siluquant_eval_sigmoid(const void* gate, float* s, int64_t n, hipStream_t stream);
int siluquant_eval_intermediates(const void* x, const void* grad_y, void* y_bf16, void* dgdu_bf16, int64_t T,
                                 int64_t H, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SILUQUANT_H */
