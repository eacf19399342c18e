/*
 * iqblock.h -- C ABI of the integer-only operators around the attention in a
 * vision-transformer block, for AMD MI355X (gfx950): ShiftGELU (between the
 * two MLP projections) and I-LayerNorm (before the attention and the MLP).
 *
 * Passages that define the operations: I-ViT: Integer-only Quantization for
 * Efficient Vision Transformer Inference (mer.run summary), sec. 3.4
 * "Integer-only GELU: ShiftGELU" and sec. 3.5 "Integer-only LayerNorm:
 * I-LayerNorm"; sec. 3.3 for the shift-based exponential and the IntDiv both
 * reuse; sec. 3.2 for the dyadic requantisation (b * y) >> c of the results;
 * sec. 3.1 for where the operators sit in the block.  ">>" is the arithmetic
 * (floor) shift, every division a floor division.
 *
 * Both operators take a row-major int8 tensor x [rows][cols] and return an
 * int8 tensor of the same shape; each row is independent.
 *
 * ShiftGELU, input scale 1 / i0:
 *   Ip   = x + (x >> 1) + (x >> 3) + (x >> 4)               (1.702 ~ 1.1011b)
 *   Imax = max(0, max over the row of Ip)
 *   E(D) = ((i0 + ((-r) >> 1)) << n) >> q   with -(D + (D >> 1) - (D >> 4))
 *          = q * i0 + r, 0 <= r < i0                         (for D <= 0)
 *   e1   = E(Ip - Imax), e2 = E(-Imax)
 *   sig  = e1 = 0 ? 0 : min((floor(2^M / (e1 + e2)) * e1) >> (M - k_out + 1),
 *                           2^(k_out - 1) - 1)
 *   out  = clip((b * (x * sig)) >> c, -127, 127)
 * The maximum is clamped at 0 so that both exponents are non-positive; e1 = 0
 * gives sig = 0 without a division (e1 + e2 may be 0 when E(-Imax)
 * underflows).
 *
 * I-LayerNorm, gamma int8 [cols] and beta int32 [cols]:
 *   mean = floor(sum x / cols),  var = floor(sum (x - mean)^2 / cols)
 *   sd   = ten steps I <- (I + floor(var / I)) >> 1 from I = 2^floor(bits(var)/2)
 *          (bits = bit length), sd = 1 where that gives 0 (var = 0)
 *   nrm  = ((x - mean) * floor(2^M / sd)) >> (M - F)     (F fraction bits)
 *   out  = clip((b * (nrm * gamma + beta)) >> c, -127, 127)
 */
#ifndef IQBLOCK_H
#define IQBLOCK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes are those of iqattn.h (IQATTN_OK, IQATTN_E_*). */

/* ---------------------------------------------------------------- ShiftGELU
 * Ranges (checked by iqgelu_create: IQATTN_E_SHAPE for rows/cols,
 * IQATTN_E_INVAL otherwise):
 *   rows >= 0 (0 makes iqgelu_forward a no-op); 16 <= cols <= 16384, a
 *   multiple of 16; rows * cols <= 2^31 - 1;
 *   1 <= i0 <= 32768; 0 <= exp_frac_bits (n) <= 30; 2 <= k_out <= 8;
 *   k_out - 1 <= intdiv_m (M) <= 40; 1 <= b <= 2^31 - 1; 0 <= c <= 62.   */
typedef struct iqgelu_params {
  int32_t rows, cols;
  int32_t i0, exp_frac_bits, intdiv_m, k_out;
  int32_t b, c;
} iqgelu_params;

typedef struct iqgelu_ctx iqgelu_ctx;

/* Validate *p and build the operator on the current HIP device: allocates a
 * 32 KiB device table of the outputs for every (clamped row maximum, x) pair
 * and fills it with a kernel.  Synchronous.  *out is NULL on error
 * (IQATTN_E_ALLOC, IQATTN_E_LAUNCH, IQATTN_E_DEVICE besides the range codes). */
int iqgelu_create(const iqgelu_params* p, iqgelu_ctx** out);

/* Enqueue out = ShiftGELU(x) on `hip_stream` (a hipStream_t; NULL = null
 * stream).  x and out: caller-owned int8 device tensors [rows][cols],
 * 16-byte aligned, not overlapping.  Asynchronous, allocates nothing.
 * IQATTN_E_NULL / IQATTN_E_ALIGN for bad pointers, IQATTN_E_LAUNCH when the
 * launch fails.                                                              */
int iqgelu_forward(iqgelu_ctx* ctx, const int8_t* x, int8_t* out, void* hip_stream);

/* Free the device table and the context (NULL accepted).  The caller makes
 * sure no enqueued forward still runs.                                       */
int iqgelu_destroy(iqgelu_ctx* ctx);

/* ---------------------------------------------------------------- I-LayerNorm
 * Ranges (checked by iqlayernorm_create):
 *   rows >= 0; 16 <= cols <= 16384, a multiple of 16; rows * cols <= 2^31 - 1;
 *   0 <= norm_frac_bits (F) <= 8; F <= intdiv_m (M) <= 22;
 *   1 <= b <= 2^31 - 1; 0 <= c <= 62.  gamma and beta take any int8 / int32
 *   values.                                                                  */
typedef struct iqlayernorm_params {
  int32_t rows, cols;
  int32_t norm_frac_bits, intdiv_m;
  int32_t b, c;
} iqlayernorm_params;

typedef struct iqlayernorm_ctx iqlayernorm_ctx;

/* Validate *p for the current HIP device.  Allocates only the host context. */
int iqlayernorm_create(const iqlayernorm_params* p, iqlayernorm_ctx** out);

/* Enqueue out = I-LayerNorm(x; gamma, beta) on `hip_stream`.  x, out int8
 * [rows][cols], gamma int8 [cols], beta int32 [cols]: caller-owned device
 * tensors, 16-byte aligned, out overlapping none of the inputs.
 * Asynchronous, allocates nothing.  Error codes as iqgelu_forward.           */
int iqlayernorm_forward(iqlayernorm_ctx* ctx, const int8_t* x, const int8_t* gamma,
                        const int32_t* beta, int8_t* out, void* hip_stream);

/* Free the context (NULL accepted).                                          */
int iqlayernorm_destroy(iqlayernorm_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif
