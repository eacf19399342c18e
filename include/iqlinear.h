/*
 * iqlinear.h -- C ABI of the integer-only int8 linear layer (the projections
 * around the attention core) for AMD MI355X (gfx950).
 *
 * One call computes, for int8 activations X [rows][in] and int8 weights
 * W [out][in] (the row-major layout of a linear layer's weight matrix):
 *   acc[m][n] = sum_k X[m][k] * W[n][k]                 int32
 *   Y[m][n]   = clip((b * acc[m][n]) >> c, -127, 127)    int8
 * with one dyadic pair (b, c) per output tensor.  There is no bias term.
 *
 * Passage that defines the operation: I-ViT: Integer-only Quantization for
 * Efficient Vision Transformer Inference (mer.run summary), sec. 3.2 "Dyadic
 * Arithmetic for Linear Operations" -- the integer product of the quantised
 * operands followed by DN(S_X S_W / S_Y) = b / 2^c and (b * acc) >> c;
 * sec. 3.1 gives the MSA projections Q = X W_Q, K = X W_K, V = X W_V and the
 * output projection.  Trio-ViT (cloud.tencent.com article), requantisation
 * module, Eq. 12: b and c are positive integers.  ">>" is the arithmetic
 * (floor) shift.
 *
 * Output layouts:
 *   IQLINEAR_PLAIN      Y is [rows][out] row-major (out0; out1, out2 unused).
 *   IQLINEAR_QKV_HEADS  rows = batch * seq_len tokens (row m = token t of
 *                       image bidx, m = bidx * seq_len + t); out = 3 * heads
 *                       * head_dim; output column n = which * (heads *
 *                       head_dim) + h * head_dim + i goes to tensor `which`
 *                       (0 = Q -> out0, 1 = K -> out1, 2 = V -> out2) at
 *                       [bidx][h][t][i], the [B, H, N, d] layout that
 *                       iqattn_forward takes; (b[which], c[which]) requantise it.
 */
#ifndef IQLINEAR_H
#define IQLINEAR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IQLINEAR_PLAIN      0
#define IQLINEAR_QKV_HEADS  1

/* Parameters (checked by iqlinear_create; IQATTN_E_INVAL / IQATTN_E_SHAPE of
 * iqattn.h otherwise):
 *   rows >= 0 (0 makes iqlinear_forward a no-op);
 *   in_features >= 64 and a multiple of 64; out_features >= 16 and a
 *   multiple of 16;
 *   1 <= b[i] <= 2^31 - 1, 0 <= c[i] <= 62 for the pairs in use (one for
 *   PLAIN, three for QKV_HEADS);
 *   QKV_HEADS: batch, seq_len, heads >= 1, head_dim a multiple of 4,
 *   rows == batch * seq_len, out_features == 3 * heads * head_dim, and
 *   heads * head_dim a multiple of 16.                                       */
typedef struct iqlinear_params {
  int32_t rows, in_features, out_features;
  int32_t layout;                 /* IQLINEAR_PLAIN or IQLINEAR_QKV_HEADS     */
  int32_t batch, seq_len, heads, head_dim; /* QKV_HEADS only                  */
  int32_t b[3], c[3];             /* dyadic pairs per output tensor           */
} iqlinear_params;

typedef struct iqlinear_ctx iqlinear_ctx;

/* Validate *p and pick the kernel for the current HIP device.  Synchronous;
 * allocates the context and its device tile table (8 bytes per output tile of
 * 256 x 256, 256 x 128 or 128 x 128).  *out is NULL on error.                */
int iqlinear_create(const iqlinear_params* p, iqlinear_ctx** out);

/* Enqueue Y = requant(X W^T) on `hip_stream` (a hipStream_t; NULL = null
 * stream).  x [rows][in] and w [out][in] are caller-owned int8 device
 * tensors; out0 (and out1, out2 for QKV_HEADS) are caller-owned int8 device
 * outputs that do not overlap the inputs.  All pointers 16-byte aligned.
 * Asynchronous, allocates nothing.  IQATTN_E_NULL / IQATTN_E_ALIGN for bad
 * pointers, IQATTN_E_LAUNCH when the launch fails.  The kernel's waves wait
 * for each other only at workgroup barriers (no polled waits), so a launch
 * that starts runs to completion.  Launches of one context may overlap.     */
int iqlinear_forward(iqlinear_ctx* ctx, const int8_t* x, const int8_t* w, int8_t* out0,
                     int8_t* out1, int8_t* out2, void* hip_stream);

/* Free the context (NULL accepted).                                          */
int iqlinear_destroy(iqlinear_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif
