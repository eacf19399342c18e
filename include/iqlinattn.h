/*
 * iqlinattn.h -- C ABI of the softmax-free integer linear attention (ReLU
 * global attention) for AMD MI355X (gfx950).
 *
 * Passages that define the operation: Trio-ViT (cloud.tencent.com article),
 * sec. III "Structure of EfficientViT", Eq. 4 (ReLU(Q) (sum_j ReLU(K_j)^T V_j)
 * over ReLU(Q) (sum_j ReLU(K_j)^T)); sec. V "Distinct Computational Pattern of
 * Attention" (the five steps: the token sums i and ii, the products iii and
 * iv, the division v); sec. IV "Log2 Quantization for Divisors in MSAs",
 * Eq. 11 (the divisor's log2 by a leading-one detector plus the next bit,
 * division replaced by a shift).  I-ViT (mer.run summary) sec. 3.2 for the
 * dyadic requantisation (b * x) >> c.  ">>" is the arithmetic (floor) shift.
 *
 * For int8 Q, K, V [batch][heads][seq_len][head_dim], per head, with
 * Qr = max(Q, 0) and Kr = max(K, 0):
 *   KV[a][b] = sum_j Kr[j][a] V[j][b],  ks[a] = sum_j Kr[j][a]          int32
 *   KVq = clip((kv_b KV) >> kv_c, -127, 127),  ksq = clip((ks_b ks) >> ks_c,
 *         -127, 127)                                                   int8
 *   num[i][b] = sum_a Qr[i][a] KVq[a][b],  den[i] = sum_a Qr[i][a] ksq[a]
 *   L[i] = index of the leading one of den[i] plus the bit below it (0 when
 *          den[i] = 0, where every num[i][b] is 0 too)
 *   out[i][b] = clip((out_b num[i][b]) >> (out_c + L[i]), -127, 127)
 * (out_b, out_c) carry the output scale and the constant log2 of the
 * divisor's scale, which is known before the call.
 */
#ifndef IQLINATTN_H
#define IQLINATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes are those of iqattn.h (IQATTN_OK, IQATTN_E_*).
 *
 * Ranges (checked by iqlinattn_create: IQATTN_E_SHAPE for the shape,
 * IQATTN_E_INVAL for the pairs):
 *   batch >= 0 (0 makes forward a no-op); heads >= 1; 1 <= seq_len <= 65536;
 *   head_dim 16, 32 or 64; batch * heads * seq_len * head_dim <= 2^31 - 1;
 *   1 <= kv_b, ks_b, out_b <= 2^31 - 1; 0 <= kv_c, ks_c, out_c <= 62.       */
typedef struct iqlinattn_params {
  int32_t batch, heads, seq_len, head_dim;
  int32_t kv_b, kv_c, ks_b, ks_c, out_b, out_c;
} iqlinattn_params;

typedef struct iqlinattn_ctx iqlinattn_ctx;

/* Validate *p for the current HIP device.  Allocates only the host context. */
int iqlinattn_create(const iqlinattn_params* p, iqlinattn_ctx** out);

/* Enqueue the attention on `hip_stream` (a hipStream_t; NULL = null stream):
 * one workgroup per head.  q, k, v, out: caller-owned contiguous int8 device
 * tensors [batch][heads][seq_len][head_dim], 16-byte aligned, out overlapping
 * none of the inputs.  Asynchronous, allocates nothing.  IQATTN_E_NULL /
 * IQATTN_E_ALIGN for bad pointers, IQATTN_E_LAUNCH when the launch fails.   */
int iqlinattn_forward(iqlinattn_ctx* ctx, const int8_t* q, const int8_t* k, const int8_t* v,
                      int8_t* out, void* hip_stream);

/* Free the context (NULL accepted).                                          */
int iqlinattn_destroy(iqlinattn_ctx* ctx);

#ifdef __cplusplus
}
#endif
#endif
