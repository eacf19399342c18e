/*
 * iqattn_oracle.c -- plain, slow, single-threaded CPU oracle of the
 * integer-only multi-head self-attention core (Shiftmax and Log-Int-Softmax).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline of the benchmark to check the HIP path.  Shares no code with it.
 *
 * Every quantity is an exact integer.  ">>" on the pages is read as floor
 * division by a power of two for both signs (R4), written here with an
 * explicit floor_div so that no C shift of a negative value is involved.
 * Intermediates are int64, far from overflow for the validated ranges.
 *
 * Readings (where the pages are silent, garbled or ambiguous):
 *  R1  I0 is the integer that represents 1.0 at the logit scale, S_logit = 1/I0
 *      (I-ViT sec. 3.3 uses I0 in the linear 2^x piece without defining it).
 *  R2  The exponent split printed as "(2 - q)" is read as "-q".
 *  R3  q = floor(-p / I0) and r = -p - q*I0 in [0, I0), so S*p = -q + S*(-r).
 *  R4  ">>" is the arithmetic (floor) shift, also on negative values.
 *  R5  The integer exponential keeps n extra fraction bits: the mantissa
 *      ((-r) >> 1) + I0 is shifted left by n before the right shift by q.
 *  R6  A right shift by q >= the word width yields the mathematical floor (0).
 *  R7  The IntDiv sum runs over the N keys of the row.
 *  R8  M is a parameter (30 in every workload here).
 *  R9  P is clamped to 2^(k_out-1) - 1 (it reaches 2^(k_out-1) only when one
 *      key holds the whole row), so it stays a signed k_out-bit value.
 *  R10 Requantisation is floor((b*x) / 2^c): the literal ">>", no rounding.
 *  R11 b*x is formed in 64 bits.
 *  R12 int8 results saturate to the symmetric range [-127, 127].
 *  R13 1/sqrt(d) is folded into (qk_b, qk_c); nothing applies it separately.
 *  R15 A relative-position bias is added to the int32 accumulator before the
 *      requantisation; token t sits at row t / w, column t % w of its window.
 *  R16 LIS reuses the Shiftmax exponential and IntDiv up to the probability.
 *  R17 log2 rounding: leading-one index plus the next lower bit (rounds up
 *      from 1.5 * 2^k).
 *  R18 The LIS probability is kept with F = 2^lis_bits - 1 fraction bits.
 *  R19 Ph = 0 maps to code F (the smallest representable weight 2^-F).
 *  R20 LIS P.V accumulates V_j * 2^(F - code_j) exactly (Q-F fixed point).
 *  R22 Keys beyond N do not exist: they take no part in max, sum or P.V.
 */
#include "iqattn_oracle.h"

#include <stdlib.h>

/* Floor of a / b for b > 0 and any sign of a. */
static int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b; /* C division truncates toward zero */
  if ((a % b) != 0 && a < 0) q -= 1;
  return q;
}

static int64_t pow2(int64_t k) { return (int64_t)1 << k; } /* 0 <= k <= 62 */

static int64_t clip64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

int orc_check_params(const orc_params* p) {
  if (!p) return -1;
  if (p->batch < 0 || p->heads < 1 || p->seq_len < 1 || p->seq_len > 65536) return -2;
  if (p->head_dim < 1 || p->head_dim > 4096) return -2;
  if (p->qk_b < 1 || p->qk_c < 0 || p->qk_c > 62) return -1;
  if (p->pv_b < 1 || p->pv_c < 0 || p->pv_c > 62) return -1;
  if (p->i0 < 1 || p->exp_frac_bits < 0 || p->exp_frac_bits > 30) return -1;
  if (p->k_out < 2 || p->k_out > 31) return -1;
  if (p->intdiv_m < p->k_out - 1 || p->intdiv_m > 62) return -1;
  if (p->variant != 0 && p->variant != 1) return -1;
  if (p->variant == 1) {
    if (p->lis_bits < 1 || p->lis_bits > 4) return -1;
    if (p->intdiv_m < (1 << p->lis_bits) - 1) return -1;
  }
  if (p->window < 0) return -1;
  if (p->window > 0 && (p->rel_bias == 0 || p->window * p->window != p->seq_len)) return -1;
  return 0;
}

/* Dyadic requantisation (I-ViT sec. 3.2; Trio-ViT Eq. 12):
 * I_out = (b * acc) >> c with DN(S_in S_w / S_out) = b / 2^c, then the
 * symmetric int8 clip (R10, R11, R12). */
int32_t orc_requant(int64_t x, int32_t b, int32_t c) {
  return (int32_t)clip64(floor_div((int64_t)b * x, pow2(c)), -127, 127);
}

void orc_requant_array(const int64_t* x, int64_t n, int32_t b, int32_t c, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_requant(x[i], b, c);
}

/* Shiftmax exponential (I-ViT sec. 3.3) of delta = L - L_max <= 0:
 *   I_p   = delta + (delta >> 1) - (delta >> 4)        (log2 e ~ 1.0111b)
 *   -I_p  = q * I0 + r,  0 <= r < I0                   (R2, R3)
 *   2^(S*(-r)) ~ S * (((-r) >> 1) + I0)                (2^z ~ z/2 + 1 on (-1, 0])
 *   e     = ((((-r) >> 1) + I0) << n) >> q              (R5, R6)           */
int64_t orc_shift_exp(int32_t delta, int32_t i0, int32_t n) {
  int64_t d = delta;
  int64_t ip = d + floor_div(d, 2) - floor_div(d, 16);
  int64_t neg_p = -ip;
  int64_t q = floor_div(neg_p, i0);
  int64_t r = neg_p - q * i0;
  int64_t mant = (int64_t)i0 + floor_div(-r, 2);
  if (q >= 62) return 0;
  return floor_div(mant * pow2(n), pow2(q));
}

/* Integer log2 with rounding by a leading-one detector (Trio-ViT sec. IV,
 * Eq. 11): the index i of the first non-zero bit plus the value of bit i-1
 * (R17).  Defined for x >= 1; returns -1 otherwise. */
int32_t orc_ilog2r(int64_t x) {
  if (x < 1) return -1;
  int32_t i = 0;
  while (i < 62 && (x >> (i + 1)) != 0) ++i;
  int32_t next = (i >= 1) ? (int32_t)((x >> (i - 1)) & 1) : 0;
  return i + next;
}

/* Shiftmax (I-ViT sec. 3.3) or Log-Int-Softmax (FQ-ViT) on one row of int8
 * logits.  prob_out receives P (Shiftmax) or Ph (LIS); code_out the LIS
 * codes.  Any output may be NULL except prob_out/code_out as the variant
 * needs them. */
int orc_softmax_row(const orc_params* p, const int32_t* logits, int32_t n,
                    int64_t* e_out, int64_t* s_out, int64_t* prob_out,
                    int32_t* code_out) {
  if (n < 1) return -2;
  int64_t* e = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  if (!e) return -3;
  /* integer row max, I_delta = I_x - I_max */
  int32_t mx = logits[0];
  for (int32_t j = 1; j < n; ++j)
    if (logits[j] > mx) mx = logits[j];
  /* exponentials and their integer sum (R7) */
  int64_t s = 0;
  for (int32_t j = 0; j < n; ++j) {
    e[j] = orc_shift_exp(logits[j] - mx, p->i0, p->exp_frac_bits);
    s += e[j];
  }
  /* IntDiv: floor(2^M / sum) -- s >= e(0) = I0 * 2^n >= 1 */
  int64_t f = floor_div(pow2(p->intdiv_m), s);
  if (p->variant == 0) {
    int64_t sh = p->intdiv_m - (p->k_out - 1);
    int64_t pmax = pow2(p->k_out - 1) - 1; /* R9 */
    for (int32_t j = 0; j < n; ++j) {
      int64_t pj = floor_div(f * e[j], pow2(sh));
      if (pj > pmax) pj = pmax;
      if (prob_out) prob_out[j] = pj;
    }
  } else {
    int64_t F = pow2(p->lis_bits) - 1; /* R18 */
    for (int32_t j = 0; j < n; ++j) {
      int64_t ph = floor_div(f * e[j], pow2(p->intdiv_m - F));
      int32_t code = (ph == 0) ? (int32_t)F                               /* R19 */
                                : (int32_t)clip64(F - orc_ilog2r(ph), 0, F); /* R17 */
      if (prob_out) prob_out[j] = ph;
      if (code_out) code_out[j] = code;
    }
  }
  if (e_out)
    for (int32_t j = 0; j < n; ++j) e_out[j] = e[j];
  if (s_out) *s_out = s;
  free(e);
  return 0;
}

/* Relative-position bias index of query token ti and key token tj in a w x w
 * window (R15): (dr + w - 1) * (2w - 1) + (dc + w - 1). */
static int64_t rel_index(int32_t ti, int32_t tj, int32_t w) {
  int32_t dr = ti / w - tj / w;
  int32_t dc = ti % w - tj % w;
  return (int64_t)(dr + w - 1) * (2 * w - 1) + (dc + w - 1);
}

int orc_forward(const orc_params* p, const int8_t* q, const int8_t* k,
                const int8_t* v, int8_t* out, int64_t head_begin,
                int64_t head_end, const orc_dump* dump) {
  int rc = orc_check_params(p);
  if (rc) return rc;
  const int64_t N = p->seq_len, d = p->head_dim, H = p->heads;
  const int64_t total = (int64_t)p->batch * H;
  if (head_begin < 0 || head_end > total || head_begin > head_end) return -2;
  const int64_t span = (2 * (int64_t)p->window - 1) * (2 * (int64_t)p->window - 1);
  const int64_t F = pow2(p->lis_bits) - 1;

  int32_t* lrow = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int64_t* erow = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  int64_t* prow = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  int32_t* crow = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
  int64_t* wrow = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  if (!lrow || !erow || !prow || !crow || !wrow) {
    free(lrow); free(erow); free(prow); free(crow); free(wrow);
    return -3;
  }

  for (int64_t u = head_begin; u < head_end; ++u) {
    const int64_t h = u % H;
    const int64_t base = u * N * d;
    const int64_t du = u - head_begin; /* index into the dumps */
    for (int64_t i = 0; i < N; ++i) {
      /* Q.K^T in integers and the dyadic requantisation (I-ViT sec. 3.2) */
      for (int64_t j = 0; j < N; ++j) {
        int64_t acc = 0;
        for (int64_t t = 0; t < d; ++t)
          acc += (int64_t)q[base + i * d + t] * (int64_t)k[base + j * d + t];
        if (p->window > 0)
          acc += p->rel_bias[h * span + rel_index((int32_t)i, (int32_t)j, p->window)];
        lrow[j] = orc_requant(acc, p->qk_b, p->qk_c);
        if (dump && dump->acc) dump->acc[(du * N + i) * N + j] = acc;
        if (dump && dump->logit) dump->logit[(du * N + i) * N + j] = lrow[j];
      }
      /* Shiftmax or Log-Int-Softmax on the row (I-ViT sec. 3.3; FQ-ViT) */
      int64_t s = 0;
      rc = orc_softmax_row(p, lrow, (int32_t)N, erow, &s, prow, crow);
      if (rc) break;
      for (int64_t j = 0; j < N; ++j)
        wrow[j] = (p->variant == 0) ? prow[j] : pow2(F - crow[j]); /* R20 */
      if (dump) {
        for (int64_t j = 0; j < N; ++j) {
          if (dump->expv) dump->expv[(du * N + i) * N + j] = erow[j];
          if (dump->prob) dump->prob[(du * N + i) * N + j] = prow[j];
          if (dump->code) dump->code[(du * N + i) * N + j] = (p->variant == 1) ? crow[j] : 0;
        }
        if (dump->rowsum) dump->rowsum[du * N + i] = s;
      }
      /* P.V in integers and the final dyadic requantisation */
      for (int64_t t = 0; t < d; ++t) {
        int64_t o = 0;
        for (int64_t j = 0; j < N; ++j) o += wrow[j] * (int64_t)v[base + j * d + t];
        if (dump && dump->pv) dump->pv[(du * N + i) * d + t] = o;
        out[base + i * d + t] = (int8_t)orc_requant(o, p->pv_b, p->pv_c);
      }
    }
    if (rc) break;
  }
  free(lrow); free(erow); free(prow); free(crow); free(wrow);
  return rc;
}

/* Linear layer: integer product over the input features, then the same dyadic
 * requantisation as the attention's (R10, R11, R12).  Plain loops, int64. */
int orc_linear(const int8_t* x, const int8_t* w, int64_t rows, int64_t in_features,
               int64_t out_features, int32_t b, int32_t c, int8_t* out, int64_t row_begin,
               int64_t row_end) {
  if (rows < 0 || in_features < 1 || out_features < 1 || b < 1 || c < 0 || c > 62 ||
      row_begin < 0 || row_end > rows || row_begin > row_end)
    return -1;
  for (int64_t m = row_begin; m < row_end; ++m)
    for (int64_t n = 0; n < out_features; ++n) {
      int64_t acc = 0;
      for (int64_t k = 0; k < in_features; ++k)
        acc += (int64_t)x[m * in_features + k] * (int64_t)w[n * in_features + k];
      out[m * out_features + n] = (int8_t)orc_requant(acc, b, c);
    }
  return 0;
}

/* ---------------------------------------------------------------- ShiftGELU
 * G1  The max is taken over the row (the last axis, as the softmax's), and
 *     clamped at 0 so that both exponents, Ip - Imax and -Imax, are <= 0: the
 *     shift-based 2^x of sec. 3.3 is defined for non-positive arguments only.
 * G2  sigma = e1 / (e1 + e2) by the IntDiv of sec. 3.3 with k_out output bits;
 *     sigma reaches 2^(k_out - 1) only when e2 = 0 and is clamped below it (R9).
 *     A zero numerator (e1 = 0: Ip far below Imax) gives sigma = 0; the
 *     division is then not taken, since e1 + e2 can be 0 as well when Imax is
 *     large enough that 2^x of -Imax underflows.
 * G3  The product x * sigma is requantised to int8 by a dyadic pair (sec. 3.2),
 *     as every integer operator's output is.                                 */
int orc_shiftgelu(const int8_t* x, int64_t rows, int64_t cols, int32_t i0, int32_t exp_frac_bits,
                  int32_t intdiv_m, int32_t k_out, int32_t b, int32_t c, int8_t* out,
                  int64_t row_begin, int64_t row_end, int64_t* dump) {
  if (rows < 0 || cols < 1 || i0 < 1 || i0 > 32768 || exp_frac_bits < 0 || exp_frac_bits > 30 ||
      k_out < 2 || k_out > 8 ||
      intdiv_m < k_out - 1 || intdiv_m > 40 || b < 1 || c < 0 || c > 62 || row_begin < 0 ||
      row_end > rows || row_begin > row_end)
    return -1;
  int64_t* ip = (int64_t*)malloc((size_t)cols * sizeof(int64_t));
  if (!ip) return -1;
  const int64_t pmax = pow2(k_out - 1) - 1;
  for (int64_t m = row_begin; m < row_end; ++m) {
    int64_t imax = 0; /* G1: clamped at 0 */
    for (int64_t j = 0; j < cols; ++j) {
      const int64_t v = x[m * cols + j];
      ip[j] = v + floor_div(v, 2) + floor_div(v, 8) + floor_div(v, 16); /* 1.1011b */
      if (ip[j] > imax) imax = ip[j];
    }
    for (int64_t j = 0; j < cols; ++j) {
      const int64_t e1 = orc_shift_exp((int32_t)(ip[j] - imax), i0, exp_frac_bits);
      const int64_t e2 = orc_shift_exp((int32_t)(-imax), i0, exp_frac_bits);
      int64_t sig = 0; /* G2: e1 = 0 gives 0 */
      if (e1 > 0) {
        const int64_t f = floor_div(pow2(intdiv_m), e1 + e2);
        sig = floor_div(f * e1, pow2(intdiv_m - (k_out - 1)));
        if (sig > pmax) sig = pmax;
      }
      if (dump) {
        int64_t* dj = dump + (m * cols + j) * 4;
        dj[0] = ip[j];
        dj[1] = e1;
        dj[2] = e2;
        dj[3] = sig;
      }
      out[m * cols + j] = (int8_t)orc_requant((int64_t)x[m * cols + j] * sig, b, c); /* G3 */
    }
  }
  free(ip);
  return 0;
}

/* ---------------------------------------------------------------- I-LayerNorm */
static int64_t bit_length(int64_t v) {
  int64_t n = 0;
  while (v > 0) { ++n; v >>= 1; }
  return n;
}

int64_t orc_isqrt10(int64_t v) {
  if (v <= 0) return 0;
  int64_t r = pow2(bit_length(v) / 2);
  for (int it = 0; it < 10; ++it) r = floor_div(r + floor_div(v, r), 2);
  return r;
}

/* L1  mean = floor(sum / cols) (integer division rounding down).
 * L2  var = floor(sum of squared deviations / cols); the square root by the
 *     page's ten fixed Newton steps; a zero deviation (constant row) takes
 *     sd = 1 so that the division is defined (every n is then 0).
 * L3  The division by sd is the IntDiv of sec. 3.3 with constant M: n keeps
 *     F fraction bits, n = (xc * floor(2^M / sd)) >> (M - F).
 * L4  gamma is int8, beta int32 at the scale of n * gamma; the affine result
 *     is requantised to int8 by a dyadic pair (sec. 3.2).                    */
int orc_ilayernorm(const int8_t* x, const int8_t* gamma, const int32_t* beta, int64_t rows,
                   int64_t cols, int32_t norm_frac_bits, int32_t intdiv_m, int32_t b, int32_t c,
                   int8_t* out, int64_t row_begin, int64_t row_end, int64_t* stat_dump) {
  if (rows < 0 || cols < 1 || norm_frac_bits < 0 || intdiv_m < norm_frac_bits ||
      intdiv_m > 40 || b < 1 || c < 0 || c > 62 || row_begin < 0 || row_end > rows ||
      row_begin > row_end)
    return -1;
  for (int64_t m = row_begin; m < row_end; ++m) {
    const int8_t* xr = x + m * cols;
    int64_t sum = 0;
    for (int64_t j = 0; j < cols; ++j) sum += xr[j];
    const int64_t mean = floor_div(sum, cols);
    int64_t sq = 0;
    for (int64_t j = 0; j < cols; ++j) sq += (xr[j] - mean) * (xr[j] - mean);
    const int64_t var = floor_div(sq, cols);
    int64_t sd = orc_isqrt10(var);
    if (sd == 0) sd = 1;
    const int64_t fs = floor_div(pow2(intdiv_m), sd);
    if (stat_dump) {
      stat_dump[m * 4 + 0] = mean;
      stat_dump[m * 4 + 1] = var;
      stat_dump[m * 4 + 2] = sd;
      stat_dump[m * 4 + 3] = fs;
    }
    for (int64_t j = 0; j < cols; ++j) {
      const int64_t n = floor_div((xr[j] - mean) * fs, pow2(intdiv_m - norm_frac_bits));
      const int64_t y = n * gamma[j] + beta[j];
      out[m * cols + j] = (int8_t)orc_requant(y, b, c);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- linear attention
 * LA1 ReLU acts on the int8 codes: the symmetric quantiser's scale is positive,
 *     so max(S q, 0) = S max(q, 0).
 * LA2 The two sums over the tokens (steps i and ii of the page's five) are
 *     integers on the scales S_K S_V and S_K; each is requantised to int8 by
 *     its own dyadic pair before the products with ReLU(Q) (the page names a
 *     scale of its own for the summed keys, so the sum is a quantised tensor;
 *     KV is taken the same way).
 * LA3 The divisor X = ReLU(Q_i) . ksq (step iv) is an integer >= 0; its log2
 *     is the leading-one index plus the next lower bit (Eq. 11, the rule the
 *     page cites), the same ilog2r as the LIS codes.  The constant
 *     log2(S_Q S_ks) of Eq. 11 is folded into the output pair (out_b, out_c).
 * LA4 The division (step v) is the shift by that code, after the output
 *     multiplier: out = clip((out_b num) >> (out_c + L), -127, 127), floor
 *     semantics; the clip (-a, b) of Eq. 11 is not reached by codes of int32
 *     divisors (L in [0, 32]).
 * LA5 A divisor of 0 (ReLU(Q_i) = 0, or ksq = 0 where Q_i is positive) makes
 *     every numerator 0 as well; the code is taken as 0 and the output is 0.
 * LA6 No 1/sqrt(d) or other scaling: the ReLU similarity has none.          */
int orc_linattn(const orc_linattn_params* p, const int8_t* q, const int8_t* k, const int8_t* v,
                int8_t* out, int64_t head_begin, int64_t head_end, int64_t* dump) {
  if (!p || p->batch < 0 || p->heads < 1 || p->seq_len < 1 || p->head_dim < 1 ||
      p->head_dim > 1024)
    return -1;
  const int32_t bs[3] = {p->kv_b, p->ks_b, p->out_b}, cs[3] = {p->kv_c, p->ks_c, p->out_c};
  for (int i = 0; i < 3; ++i)
    if (bs[i] < 1 || cs[i] < 0 || cs[i] > 62) return -1;
  const int64_t NH = p->batch * p->heads, N = p->seq_len, d = p->head_dim;
  if (head_begin < 0 || head_end > NH || head_begin > head_end) return -1;
  int64_t* kv = (int64_t*)malloc((size_t)(d * d + d) * sizeof(int64_t));
  int64_t* num = (int64_t*)malloc((size_t)d * sizeof(int64_t));
  if (!kv || !num) {
    free(kv);
    free(num);
    return -1;
  }
  int64_t* ks = kv + d * d;
  for (int64_t hh = head_begin; hh < head_end; ++hh) {
    const int8_t* Q = q + hh * N * d;
    const int8_t* K = k + hh * N * d;
    const int8_t* V = v + hh * N * d;
    /* steps i and ii, then LA2 */
    for (int64_t a = 0; a < d; ++a) {
      int64_t sk = 0;
      for (int64_t j = 0; j < N; ++j) sk += K[j * d + a] > 0 ? K[j * d + a] : 0;
      ks[a] = orc_requant(sk, p->ks_b, p->ks_c);
      for (int64_t b = 0; b < d; ++b) {
        int64_t acc = 0;
        for (int64_t j = 0; j < N; ++j) {
          const int64_t kr = K[j * d + a] > 0 ? K[j * d + a] : 0;
          acc += kr * V[j * d + b];
        }
        kv[a * d + b] = orc_requant(acc, p->kv_b, p->kv_c);
      }
    }
    if (dump)
      for (int64_t t = 0; t < d * d + d; ++t) dump[(hh - head_begin) * (d * d + d) + t] = kv[t];
    /* steps iii, iv, v */
    for (int64_t i = 0; i < N; ++i) {
      int64_t den = 0;
      for (int64_t a = 0; a < d; ++a) {
        const int64_t qr = Q[i * d + a] > 0 ? Q[i * d + a] : 0;
        den += qr * ks[a];
      }
      for (int64_t b = 0; b < d; ++b) {
        int64_t acc = 0;
        for (int64_t a = 0; a < d; ++a) {
          const int64_t qr = Q[i * d + a] > 0 ? Q[i * d + a] : 0;
          acc += qr * kv[a * d + b];
        }
        num[b] = acc;
      }
      const int64_t L = den > 0 ? orc_ilog2r(den) : 0; /* LA3, LA5 */
      for (int64_t b = 0; b < d; ++b) {
        const int64_t sh = p->out_c + L;
        const int64_t prod = (int64_t)p->out_b * num[b];
        const int64_t y = sh >= 63 ? (prod < 0 ? -1 : 0) : floor_div(prod, pow2(sh));
        out[hh * N * d + i * d + b] = (int8_t)clip64(y, -127, 127);
      }
    }
  }
  free(kv);
  free(num);
  return 0;
}
