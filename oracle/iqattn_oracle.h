/*
 * iqattn_oracle.h -- CPU oracle of the integer-only attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  This oracle exists to check the HIP path.  Only
 * the test-suite, the smoke check and the CPU-baseline leg of the benchmark
 * may load it; the product library never includes, links or calls it, and it
 * shares no code, header, table or helper with the product.
 *
 * What it computes (all integers, every step in the order of the pages):
 *   I-ViT: Integer-only Quantization for Efficient Vision Transformer
 *   Inference (mer.run summary of the paper):
 *     sec. 3.2 "Dyadic Arithmetic for Linear Operations":  Q.K^T in integers,
 *       then the dyadic requantisation (b * acc) >> c to int8 logits;
 *     sec. 3.3 "Integer-only Softmax: Shiftmax":  subtract the row max,
 *       multiply by log2(e) as x + (x>>1) - (x>>4), split into an integer
 *       power q and a remainder r, 2^x by a linear piece and a right shift,
 *       integer row sum, IntDiv to k_out-bit probabilities;
 *     sec. 3.1 "Overview":  Attn = Softmax(Q K^T / sqrt(d)) V, uniform
 *       symmetric quantiser (int8 range +-127).
 *   FQ-ViT: Post-Training Quantization for Fully Quantized Vision Transformer
 *   (IJCAI 2022 record), abstract:  Log-Int-Softmax, attention map quantised
 *     to 4-bit log2 codes, P.V by the BitShift operator.
 *   Trio-ViT (cloud.tencent.com article), sec. IV "Log2 Quantization for
 *     Divisors in MSAs" (Eq. 11):  integer log2 by a leading-one detector
 *     plus the next lower bit;  sec. V, requantisation module (Eq. 12):
 *     b and c positive integers.
 *
 *   I-ViT sec. 3.4 "Integer-only GELU: ShiftGELU" and sec. 3.5 "Integer-only
 *     LayerNorm: I-LayerNorm" for the two element-wise/row-wise operators
 *     around the attention (orc_shiftgelu, orc_ilayernorm).
 *   Trio-ViT (cloud.tencent.com article), sec. III "Structure of EfficientViT"
 *     Eq. 4, sec. IV "Log2 Quantization for Divisors in MSAs" Eq. 11 and
 *     sec. V "Distinct Computational Pattern of Attention" (steps i-v) for the
 *     softmax-free linear attention (orc_linattn).
 *
 * Readings taken where the pages are silent, garbled or ambiguous are listed
 * next to the code that takes them (R1..R22, G1..G3, L1..L4 in the comments of
 * the .c file; LA1..LA6 for the linear attention).
 * Parity unpinned: the readings themselves (I0 = 1/S_logit, the extra exponent
 * fraction bits n, M, the clamp of P at 2^(k_out-1)-1, floor requantisation,
 * bias added to the int32 accumulator, the midpoint of the log2 rounding, the
 * Q15 LIS accumulation) are choices; no number printed on the pages fixes
 * them.  The tests pin the implementation of each choice and the whole
 * pipeline against float64 softmax.
 */
#ifndef IQATTN_ORACLE_H
#define IQATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, heads, seq_len, head_dim;
  int32_t qk_b, qk_c;         /* dyadic pair of the Q.K^T requantisation     */
  int32_t pv_b, pv_c;         /* dyadic pair of the P.V requantisation       */
  int32_t i0;                 /* integer 1.0 at the logit scale (S = 1/i0)   */
  int32_t exp_frac_bits;      /* n: extra fraction bits of the integer 2^x   */
  int32_t intdiv_m;           /* M of IntDiv                                 */
  int32_t k_out;              /* Shiftmax output bits                        */
  int32_t variant;            /* 0 = Shiftmax, 1 = Log-Int-Softmax           */
  int32_t lis_bits;           /* LIS code bits                               */
  int32_t window;             /* w > 0: relative bias table present, N = w*w */
  const int32_t* rel_bias;    /* [heads][(2w-1)^2], or NULL                  */
} orc_params;

/* Optional per-head dumps of the intermediates, for heads [begin, end) in
 * the flattened (b * heads + h) order.  Any pointer may be NULL.             */
typedef struct {
  int64_t* acc;     /* [nh][N][N]  Q.K^T (+ bias)                    */
  int32_t* logit;   /* [nh][N][N]  int8 logits L                     */
  int64_t* expv;    /* [nh][N][N]  integer exponentials e            */
  int64_t* rowsum;  /* [nh][N]     row sums s                        */
  int64_t* prob;    /* [nh][N][N]  P (Shiftmax) or Ph (LIS)          */
  int32_t* code;    /* [nh][N][N]  LIS codes                         */
  int64_t* pv;      /* [nh][N][d]  P.V accumulator o                 */
} orc_dump;

int orc_check_params(const orc_params* p);

/* Full pipeline for heads [head_begin, head_end).  q, k, v, out are whole
 * [B, H, N, d] int8 tensors (row-major); out is written for those heads only.
 * Returns 0, or a negative value for invalid parameters.                      */
int orc_forward(const orc_params* p, const int8_t* q, const int8_t* k,
                const int8_t* v, int8_t* out, int64_t head_begin,
                int64_t head_end, const orc_dump* dump);

/* Integer-only linear layer (I-ViT sec. 3.2 applied to a projection):
 *   out[m][n] = clip(floor(b * sum_k x[m][k] * w[n][k] / 2^c), -127, 127)
 * for rows [row_begin, row_end); x is [rows][in] and w is [out][in] int8,
 * row-major; out is [rows][out] (only the given rows are written).  No bias
 * term: the pages give the dyadic product alone.  Returns 0, or -1 for
 * out-of-range arguments.                                                    */
int orc_linear(const int8_t* x, const int8_t* w, int64_t rows, int64_t in_features,
               int64_t out_features, int32_t b, int32_t c, int8_t* out, int64_t row_begin,
               int64_t row_end);

/* ShiftGELU (I-ViT sec. 3.4) on x [rows][cols] int8 at scale 1/i0:
 *   Ip   = x + (x >> 1) + (x >> 3) + (x >> 4)        1.702 ~ 1.1011b
 *   Imax = max(0, max over the row of Ip)            (G1)
 *   e1   = shift_exp(Ip - Imax), e2 = shift_exp(-Imax)   (Shiftmax's 2^x)
 *   sig  = min((floor(2^M / (e1 + e2)) * e1) >> (M - (k_out - 1)),
 *              2^(k_out - 1) - 1), 0 when e1 = 0     (G2, R9)
 *   out  = clip((b * (x * sig)) >> c, -127, 127)     (G3)
 * Rows [row_begin, row_end) are written; dump, when not NULL, receives
 * (Ip, e1, e2, sig) per element [rows][cols][4].  Returns 0 or -1 (bad
 * arguments).                                                                */
int orc_shiftgelu(const int8_t* x, int64_t rows, int64_t cols, int32_t i0, int32_t exp_frac_bits,
                  int32_t intdiv_m, int32_t k_out, int32_t b, int32_t c, int8_t* out,
                  int64_t row_begin, int64_t row_end, int64_t* dump);

/* Integer square root of I-LayerNorm (I-ViT sec. 3.5): ten iterations of
 * I <- (I + floor(v / I)) >> 1 from I = 2^floor(bits(v) / 2), bits(v) the
 * bit length of v; v = 0 gives 0.                                            */
int64_t orc_isqrt10(int64_t v);

/* I-LayerNorm (I-ViT sec. 3.5) on x [rows][cols] int8 with per-column gamma
 * (int8) and beta (int32):
 *   mean = floor(sum x / cols); xc = x - mean                 (L1)
 *   var  = floor(sum xc^2 / cols); sd = isqrt10(var), 0 -> 1   (L2)
 *   n    = (xc * floor(2^M / sd)) >> (M - F)                   (L3)
 *   out  = clip((b * (n * gamma + beta)) >> c, -127, 127)      (L4)
 * Rows [row_begin, row_end) are written; stat_dump, when not NULL, receives
 * (mean, var, sd, floor(2^M / sd)) per row [rows][4].  Returns 0 or -1.      */
int orc_ilayernorm(const int8_t* x, const int8_t* gamma, const int32_t* beta, int64_t rows,
                   int64_t cols, int32_t norm_frac_bits, int32_t intdiv_m, int32_t b, int32_t c,
                   int8_t* out, int64_t row_begin, int64_t row_end, int64_t* stat_dump);

/* Softmax-free integer linear attention (Trio-ViT, cloud.tencent.com article:
 * EfficientViT's ReLU global attention, Eq. 4; log2 quantisation of the
 * divisor, Eq. 11, with the leading-one detector and shift division) on one
 * batch of int8 Q, K, V [batch][heads][seq_len][head_dim]:
 *   Qr = max(Q, 0), Kr = max(K, 0)                                  (LA1)
 *   KV[a][b] = sum_j Kr[j][a] V[j][b],  ks[a] = sum_j Kr[j][a]        int64
 *   KVq = clip((kv_b KV) >> kv_c, -127, 127), ksq = clip((ks_b ks) >> ks_c,
 *         -127, 127)                                                (LA2)
 *   num[i][b] = sum_a Qr[i][a] KVq[a][b],  den[i] = sum_a Qr[i][a] ksq[a]
 *   L[i] = ilog2r(den[i]) (0 when den[i] = 0)                       (LA3, LA5)
 *   out[i][b] = clip((out_b num[i][b]) >> (out_c + L[i]), -127, 127)  (LA4)
 * Heads [head_begin, head_end) of the flattened batch * heads are written;
 * dump, when not NULL, receives per head (KVq [d][d], ksq [d]) as int64
 * [heads][d * d + d].  Returns 0, or -1 for out-of-range arguments.          */
typedef struct orc_linattn_params {
  int64_t batch, heads, seq_len, head_dim;
  int32_t kv_b, kv_c, ks_b, ks_c, out_b, out_c;
} orc_linattn_params;

int orc_linattn(const orc_linattn_params* p, const int8_t* q, const int8_t* k, const int8_t* v,
                int8_t* out, int64_t head_begin, int64_t head_end, int64_t* dump);

/* Steps exposed one at a time for the tests. */
int32_t orc_requant(int64_t x, int32_t b, int32_t c);
void    orc_requant_array(const int64_t* x, int64_t n, int32_t b, int32_t c,
                          int32_t* out);
int64_t orc_shift_exp(int32_t delta, int32_t i0, int32_t n);
int32_t orc_ilog2r(int64_t x);
/* Shiftmax / LIS on one row of int8 logits (steps after the requantisation). */
int orc_softmax_row(const orc_params* p, const int32_t* logits, int32_t n,
                    int64_t* e_out, int64_t* s_out, int64_t* prob_out,
                    int32_t* code_out);

#ifdef __cplusplus
}
#endif
#endif
