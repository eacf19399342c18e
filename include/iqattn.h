/*
 * iqattn.h -- C ABI of the integer-only int8 multi-head self-attention core
 * for AMD MI355X (gfx950).
 *
 * One call computes, for every head (b, h) of int8 Q, K, V tensors:
 *   acc  = Q K^T in int32                                     (1)
 *   acc += relative-position bias            (windowed attention only)
 *   L    = clip((qk_b * acc) >> qk_c, -127, 127)              (2)
 *   P    = Shiftmax(L)  -> k_out-bit probabilities            (3)
 *        | LIS(L)       -> lis_bits-bit log2 codes
 *   o    = P V in int32 | sum_j V_j << (F - code_j)           (4)
 *   Out  = clip((pv_b * o) >> pv_c, -127, 127)                (5)
 * The logits never leave the chip: one fused kernel launch per call.
 *
 * Passages that define the operations:
 *   (1), (2)  I-ViT: Integer-only Quantization for Efficient Vision
 *             Transformer Inference (mer.run summary), sec. 3.2 "Dyadic
 *             Arithmetic for Linear Operations": integer product of the
 *             quantised operands, then DN(S_Q S_K / S_A) = b / 2^c and
 *             I_A = (b * (I_Q * I_K^T)) >> c.  Trio-ViT (cloud.tencent.com
 *             article), requantisation module, Eq. 12: b and c are positive
 *             integers.  1/sqrt(d) of sec. 3.1 is folded into (qk_b, qk_c).
 *   (3)       I-ViT sec. 3.3 "Integer-only Softmax: Shiftmax": row max
 *             subtraction, log2 e ~ 1.0111b by shifts, 2^x = linear piece
 *             shifted right by the integer part, integer sum and IntDiv with
 *             constant M to k_out-bit outputs of scale 1/2^(k_out-1).
 *             Log-Int-Softmax: FQ-ViT: Post-Training Quantization for Fully
 *             Quantized Vision Transformer (IJCAI 2022 record), abstract:
 *             4-bit log2 attention and the BitShift operator; the integer
 *             log2 rounds by a leading-one detector plus the next bit
 *             (Trio-ViT sec. IV "Log2 Quantization for Divisors in MSAs",
 *             Eq. 11).
 *   bias      Swin Transformer abstract (aixpaper list): attention inside
 *             non-overlapping local windows; the (2w-1)^2 relative table is
 *             indexed by (dr + w - 1) * (2w - 1) + (dc + w - 1).
 *   (4), (5)  I-ViT sec. 3.1 MSA formula with every MatMul dyadic (sec. 3.2).
 *
 * Integer conventions: ">>" is the arithmetic (floor) shift; the exponential
 * keeps exp_frac_bits extra fraction bits before its shift by the integer
 * part; P is clamped to 2^(k_out-1) - 1; LIS keeps F = 2^lis_bits - 1
 * fraction bits and maps a zero probability to code F.
 */
#ifndef IQATTN_H
#define IQATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes (every entry point returns 0 or one of these). */
#define IQATTN_OK             0
#define IQATTN_E_INVAL       -1  /* a parameter is out of its documented range   */
#define IQATTN_E_SHAPE       -2  /* B, H, N, d or window not supported            */
#define IQATTN_E_ALLOC       -3  /* device allocation failed in iqattn_create      */
#define IQATTN_E_LAUNCH      -4  /* a HIP call or kernel launch failed             */
#define IQATTN_E_NULL        -5  /* a required pointer is NULL                     */
#define IQATTN_E_ALIGN       -6  /* a tensor pointer is not 16-byte aligned        */
#define IQATTN_E_DEVICE      -7  /* no usable gfx950 device is current             */
#define IQATTN_E_INCOMPLETE  -8  /* a kernel's bounded wait gave up: some output
                                    rows of a launch were not written          */
#define IQATTN_E_TOOBIG      -9  /* iqattn_forward_noalloc: the windowed bias does
                                    not fit its static device memory            */

#define IQATTN_SHIFTMAX 0
#define IQATTN_LIS      1

/* P.V engines of the Log-Int-Softmax variant (identical results):
 * VALU: sum_j V_j << (F - code_j) with one shift-add per (query, key, feature),
 *       the BitShift operator of FQ-ViT's abstract;
 * MFMA: the same sum as two int8 matrix products over the bit planes of the
 *       weights 2^(F - code).                                                  */
#define IQATTN_LIS_VALU 0
#define IQATTN_LIS_MFMA 1

/* Layouts of the output tensor:
 * HEADS:  [batch][heads][seq_len][head_dim], the layout of Q, K and V;
 * TOKENS: [batch][seq_len][heads][head_dim], i.e. rows of heads * head_dim
 *         features per token: the [tokens][features] input of the output
 *         projection, with no transpose in between.                          */
#define IQATTN_OUT_HEADS  0
#define IQATTN_OUT_TOKENS 1

#define IQATTN_MAX_SEQ 1024      /* largest N (up to 640 keys the row stays in
                                    registers; longer rows take three passes over
                                    LDS-resident K)                                */

/* Parameters of one attention shape.  All values are plain integers.
 * Ranges (checked by iqattn_create, which returns IQATTN_E_INVAL or
 * IQATTN_E_SHAPE otherwise):
 *   batch >= 0 (0 makes iqattn_forward a no-op), heads >= 1,
 *   1 <= seq_len <= IQATTN_MAX_SEQ, head_dim in {32, 64};
 *   1 <= qk_b, pv_b <= 2^31 - 1;  0 <= qk_c, pv_c <= 62;
 *   1 <= i0, 0 <= exp_frac_bits, i0 * 2^exp_frac_bits <= 2^22;
 *   2 <= k_out <= 8;  k_out - 1 <= intdiv_m <= 31;
 *   variant IQATTN_SHIFTMAX or IQATTN_LIS; for LIS 1 <= lis_bits <= 4,
 *   intdiv_m >= 2^lis_bits - 1 and lis_engine IQATTN_LIS_VALU or
 *   IQATTN_LIS_MFMA (ignored for Shiftmax);
 *   rel_bias == NULL and window == 0, or rel_bias != NULL, window >= 1,
 *   seq_len == window * window and |rel_bias[.]| <= 2^30;
 *   out_layout IQATTN_OUT_HEADS or IQATTN_OUT_TOKENS; for OUT_TOKENS
 *   heads * seq_len * head_dim <= 2^31 - 1 (one head's output rows are
 *   addressed with 32-bit offsets).                                       */
typedef struct iqattn_params {
  int32_t batch, heads, seq_len, head_dim;
  int32_t qk_b, qk_c;        /* dyadic pair of Q.K^T -> int8 logits            */
  int32_t pv_b, pv_c;        /* dyadic pair of P.V -> int8 output              */
  int32_t i0;                /* integer 1.0 at the logit scale (S_logit = 1/i0) */
  int32_t exp_frac_bits;     /* extra fraction bits of the integer 2^x         */
  int32_t intdiv_m;          /* M of IntDiv                                     */
  int32_t k_out;             /* Shiftmax output bits                            */
  int32_t variant;           /* IQATTN_SHIFTMAX or IQATTN_LIS                   */
  int32_t lis_bits;          /* LIS code bits                                   */
  int32_t lis_engine;        /* IQATTN_LIS_VALU or IQATTN_LIS_MFMA               */
  int32_t window;            /* w when rel_bias != NULL, else 0                 */
  int32_t out_layout;        /* IQATTN_OUT_HEADS or IQATTN_OUT_TOKENS           */
  const int32_t* rel_bias;   /* HOST pointer, [heads][(2w-1)^2] int32, or NULL;
                                copied by iqattn_create                         */
} iqattn_params;

typedef struct iqattn_ctx iqattn_ctx;

/* Validate *p, then, on the current HIP device, allocate and fill the
 * context's device constants (exponential table, expanded bias) and its
 * status word (see iqattn_check), and pick the kernel.  Synchronous.  On success *out owns a context that the caller frees
 * with iqattn_destroy; on error *out is set to NULL and nothing leaks.
 * Parameter checks happen before any HIP call.                              */
int iqattn_create(const iqattn_params* p, iqattn_ctx** out);

/* Enqueue the fused attention on `hip_stream` (a hipStream_t; NULL = the
 * null stream) of the device the context was created on.  q, k, v (inputs)
 * are caller-owned device pointers to contiguous [batch][heads][seq_len]
 * [head_dim] int8 tensors and out (output) to a contiguous int8 tensor of the
 * same size in the context's out_layout, all 16-byte aligned; out must not
 * overlap the inputs.  Asynchronous: no allocation, no host
 * synchronisation.  Returns IQATTN_E_NULL / IQATTN_E_ALIGN for bad pointers
 * (checked before launch) and IQATTN_E_LAUNCH when the launch fails; out is
 * undefined after an error.  A context may be used by several streams at once. */
int iqattn_forward(iqattn_ctx* ctx, const int8_t* q, const int8_t* k,
                   const int8_t* v, int8_t* out, void* hip_stream);

/* Completion check of the launches enqueued so far.  The kernels' work
 * queues wait for data with bounded polls; a wave whose poll gives up (only
 * a broken invariant or a test's spin limit can cause it) leaves its output
 * rows unwritten and records the event in a status word owned by the context
 * (set with a device atomic).  iqattn_check synchronises `hip_stream`, reads
 * and clears that word, and returns IQATTN_OK, IQATTN_E_INCOMPLETE (some
 * output of a launch since the last check is missing) or IQATTN_E_LAUNCH.
 * The word is shared by every stream that uses the context.                 */
int iqattn_check(iqattn_ctx* ctx, void* hip_stream);

/* Diagnostic hook for tests of the failure path: every bounded poll of this
 * context's later launches gives up after `polls` polls (>= 1; the default
 * is 4194304, about 0.1 s per wait).  A small value makes waves give up
 * while their data is still on the way: the kernels then exit normally and
 * iqattn_check reports IQATTN_E_INCOMPLETE.  Returns IQATTN_E_INVAL for
 * polls < 1.                                                                  */
int iqattn_set_spin_limit(iqattn_ctx* ctx, int32_t polls);

/* Free the context's device memory.  NULL is accepted (returns 0).  The
 * caller must make sure no forward using ctx is still running.              */
int iqattn_destroy(iqattn_ctx* ctx);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * attention of *p in one call that allocates nothing -- no context, no
 * hipMalloc / hipFree, no allocating library routine.  It enqueues on
 * `hip_stream` a set-up kernel (exponential table, cleared status word), the
 * bias expansion when p->rel_bias is set, and the fused kernel of
 * iqattn_forward; the results are byte-identical to iqattn_create +
 * iqattn_forward with the same parameters.  q, k, v, out as for
 * iqattn_forward; p->rel_bias (host memory) is read during the call only.
 * The device memory it uses is a static array of the library (about 260 KB
 * per GPU, kept until the process ends) that every call on that GPU shares:
 * calls that overlap in time on one GPU race (serialise them on one stream).
 * Limit: p->heads * (2 window - 1)^2 <= 960 and p->heads * 16 ceil(N/16) *
 * 16 ceil(N/16) * 4 <= 262144 bytes when rel_bias is set (IQATTN_E_TOOBIG
 * otherwise, checked before any HIP call, like the ranges of iqattn_create).
 * There is no completion check for these calls (the status word is cleared by
 * each call).  Returns as iqattn_create and iqattn_forward.                 */
int iqattn_forward_noalloc(const iqattn_params* p, const int8_t* q, const int8_t* k,
                           const int8_t* v, int8_t* out, void* hip_stream);

/* Static text for an error code (for IQATTN_E_LAUNCH: the last HIP error
 * seen by this thread).                                                      */
const char* iqattn_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif
