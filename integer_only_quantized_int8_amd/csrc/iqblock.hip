// iqblock.hip -- ShiftGELU and I-LayerNorm: the row-wise integer operators
// around the attention of a vision-transformer block.
//
// Method passages: I-ViT (mer.run summary) sec. 3.4 "Integer-only GELU:
// ShiftGELU", sec. 3.5 "Integer-only LayerNorm: I-LayerNorm"; sec. 3.3 for the
// shift exponential and IntDiv; sec. 3.2 for the dyadic requantisation.
//
// Both kernels stream int8 rows from HBM once and write int8 rows once; the
// work per byte is a few VALU operations, so they are HBM-bound kernels laid
// out for coalescing: a group of G lanes (16 or 64) owns one row, each lane
// 16-byte chunks at column 16 * (lane + G * k), k < NCH, read and written with
// 128-bit buffer operations; the row reductions run over the G lanes.
//
// ShiftGELU: x is int8, so for a given row maximum the output is a function of
// x alone.  The row maximum enters only through Imax = Ip(max(0, row max)),
// 128 possible values; the operator's exact result for every (clamped row
// maximum, x) pair is a 128 x 256 table (32 KiB), built once on the device by
// iqgelu_build_table with the sec. 3.3/3.4 integer steps.  The streaming kernel
// then needs only the row maximum (packed 16-bit maxima of the biased bytes)
// and one LDS byte lookup per element, with the table resident in LDS.
//
// I-LayerNorm: the row sums sum x and sum x^2 come from v_dot4 (four bytes a
// step), the centred sum of squares from the exact integer identity
// sum (x - mean)^2 = sum x^2 - 2 mean sum x + cols mean^2; mean, var and
// floor(2^M / sd) are per-row scalars, the ten Newton steps per row use a
// float reciprocal with an exact integer correction; the per-element part is
// 24-bit multiplies, a saturating add and the dyadic multiply-high.
#include "iqattn_dev.h"
#include "iqattn.h"
#include "iqblock.h"

#include <stdlib.h>
#include <string.h>

namespace iqattn {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kTabSlices = 128;               // clamped row maximum 0..127
constexpr int kTabBytes = kTabSlices * 256;   // x biased by 128: 0..255
constexpr int kGeluThreads = 512;
constexpr int kLnThreads = 256;
constexpr int kMaxCols = 16384;

struct GeluDev {
  const int8_t* x;
  int8_t* out;
  const uint8_t* tab;
  int32_t rows, cols;
};

struct LnDev {
  const int8_t* x;
  const int8_t* gamma;
  const int32_t* beta;
  int8_t* out;
  int32_t rows, cols;
  int32_t m, f;        // IntDiv exponent M, fraction bits F
  int32_t b, c;        // dyadic pair
  int32_t bm;          // b << (32 - c) (RQ_MULHI)
  int32_t ylo, yhi;    // -floor(127 * 2^c / b), ceil(127 * 2^c / b) (RQ_WIN)
  uint32_t sqmask[6];  // bit k: ten Newton steps on k^2 - 1 end on k (not k - 1)
};

// ---------------------------------------------------------------- ShiftGELU
__device__ __forceinline__ int32_t ip1702(int32_t v) {  // 1.1011b * v, floored shifts
  return v + (v >> 1) + (v >> 3) + (v >> 4);
}

// Shift exponential of d <= 0 at scale 1/i0 with n extra fraction bits.
__device__ __forceinline__ int64_t shift_exp(int32_t d, int32_t i0, int32_t n) {
  const int32_t t = d + (d >> 1) - (d >> 4);  // log2 e ~ 1.0111b
  const int32_t np = -t;                       // >= 0
  const int32_t q = np / i0, r = np - q * i0;
  const int64_t mant = (int64_t)i0 + ((-r) >> 1);
  return q >= 63 ? 0 : ((mant << n) >> q);
}

// tab[m * 256 + u] = ShiftGELU output for x = u - 128 in a row whose maximum,
// clamped at 0, is m.  Entries with x > m never occur and hold 0.
__global__ void iqgelu_build_table(uint8_t* tab, int32_t i0, int32_t n, int32_t mbits,
                                   int32_t k_out, int32_t b, int32_t c) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= kTabBytes) return;
  const int32_t m = idx >> 8, x = (idx & 255) - 128;
  int32_t res = 0;
  if (x <= m) {
    const int32_t imax = ip1702(m);  // >= 0
    const int64_t e1 = shift_exp(ip1702(x) - imax, i0, n);
    const int64_t e2 = shift_exp(-imax, i0, n);
    int64_t sig = 0;
    if (e1 > 0) {
      const int64_t f = ((int64_t)1 << mbits) / (e1 + e2);
      sig = min((f * e1) >> (mbits - k_out + 1), ((int64_t)1 << (k_out - 1)) - 1);
    }
    const int64_t y = ((int64_t)b * ((int64_t)x * sig)) >> c;
    res = (int32_t)(y < -127 ? -127 : (y > 127 ? 127 : y));
  }
  tab[idx] = (uint8_t)(int8_t)res;
}

// Reductions over the G lanes of a row group, every lane receiving the result.
// G = 16 (one DPP row): the pair and quad swaps (quad_perm [1,0,3,2] and
// [2,3,0,1]), then row_half_mirror and row_mirror, which pair each lane with
// one in the other quad and the other half-row -- VALU operations only.
// G = 64: lane-index shuffles.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (G == 16) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
  } else {
#pragma unroll
    for (int s = 1; s < G; s <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, s, 64));
  }
  return v;
}

template <int G>
__device__ __forceinline__ int32_t group_sum_i32(int32_t v) {
  if constexpr (G == 16) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
  } else {
#pragma unroll
    for (int s = 1; s < G; s <<= 1) v += __shfl_xor(v, s, 64);
  }
  return v;
}

template <int G, int NCH>
__global__ __launch_bounds__(kGeluThreads) void iqgelu_fwd(GeluDev p) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[kTabBytes];
  for (int i = threadIdx.x; i < kTabBytes / 16; i += kGeluThreads)
    reinterpret_cast<v4i*>(tab)[i] = reinterpret_cast<const v4i*>(p.tab)[i];
  __syncthreads();

  constexpr int RPW = 64 / G;                       // rows per wave
  constexpr int RPB = RPW * (kGeluThreads / 64);    // rows per block step
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane % G, sub = lane / G;
  const uint32_t total = (uint32_t)p.rows * (uint32_t)p.cols;
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(p.x, total);
  const __amdgpu_buffer_rsrc_t orr = buf_rsrc(p.out, total);
  const uint32_t tab_base = lds_addr(tab);

  for (int r0 = blockIdx.x * RPB; r0 < p.rows; r0 += gridDim.x * RPB) {
    const int row = r0 + wave * RPW + sub;
    const bool rv = row < p.rows;
    const int rowc = rv ? row : p.rows - 1;
    v4i d[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int col = 16 * (gl + G * k);
      const bool cv = col < p.cols;
      d[k] = buf_load<v4i>(xr, rowc * p.cols + (cv ? col : 0));
#pragma unroll
      for (int j = 0; j < 4; ++j) d[k][j] = cv ? (d[k][j] ^ 0x80808080) : 0;  // u = x + 128
    }
    // row maximum of u over packed 16-bit lanes (even and odd bytes)
    u16x2 mx = {0, 0};
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)d[k][j];
        const uint32_t ev = __builtin_amdgcn_perm(0u, w, 0x0c020c00u);  // bytes 0, 2
        const uint32_t od = __builtin_amdgcn_perm(0u, w, 0x0c030c01u);  // bytes 1, 3
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, ev));
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, od));
      }
    uint32_t um = group_max_u32<G>(max((uint32_t)mx[0], (uint32_t)mx[1]));
    const uint32_t m = um > 128u ? um - 128u : 0u;     // max(row max of x, 0)
    const uint32_t base = tab_base + (m << 8);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int col = 16 * (gl + G * k);
      v4i o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (uint32_t)d[k][j];
        uint32_t t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t a = base + ((w >> (8 * i)) & 0xffu);
          t[i] = *(const __attribute__((address_space(3))) uint8_t*)(uintptr_t)a;
        }
        o[j] = (int32_t)(t[0] | (t[1] << 8) | (t[2] << 16) | (t[3] << 24));
      }
      if (rv && col < p.cols) __builtin_amdgcn_raw_buffer_store_b128(o, orr, row * p.cols + col, 0, 0);
    }
  }
}

// ---------------------------------------------------------------- I-LayerNorm
// floor(a / b) for 0 <= a < 2^15, b >= 1: float reciprocal, then one exact
// integer correction step each way (the float estimate is off by at most 1).
__device__ __forceinline__ int32_t udiv_small(int32_t a, int32_t b) {
  int32_t q = (int32_t)((float)a * __builtin_amdgcn_rcpf((float)b));
  int32_t r = a - q * b;
  if (r < 0) { --q; r += b; }
  if (r >= b) ++q;
  return q;
}

// The ten Newton steps I <- (I + floor(v / I)) >> 1 from I = 2^floor(bits(v)/2)
// for 0 <= v < 2^15.
__device__ __forceinline__ int32_t isqrt_newton10(int32_t v) {
  if (v <= 0) return 0;
  const int bits = 32 - __builtin_clz((uint32_t)v);
  int32_t r = 1 << (bits >> 1);
#pragma unroll
  for (int it = 0; it < 10; ++it) r = (r + udiv_small(v, r)) >> 1;
  return r;
}

// For v < 2^15 the ten steps end on floor(sqrt v), except at v = k^2 - 1, where
// the integer iteration alternates between k - 1 and k and the tenth step may
// hold either; flags[k] records which (k < 192), so that the streaming kernel
// can take the exact square root and one mask bit instead of ten divisions.
__global__ void iqln_newton_flags(uint8_t* flags) {
  const int k = threadIdx.x;
  if (k >= 192) return;
  const int32_t v = k * k - 1;
  flags[k] = (v >= 1 && v < (1 << 15) && isqrt_newton10(v) == k) ? 1 : 0;
}

// The ten-step result for 1 <= v < 2^15: floor(sqrt v) by the float square
// root with an exact integer correction, raised to k where v = k^2 - 1 and
// the mask bit k is set.
__device__ __forceinline__ int32_t isqrt_newton10_fast(int32_t v, const uint32_t* mask) {
  int32_t s = (int32_t)__builtin_sqrtf((float)v);
  if (s * s > v) --s;
  if ((s + 1) * (s + 1) <= v) ++s;
  const int32_t k = s + 1;
  if (k * k - 1 == v) {
    const uint64_t lo = ((uint64_t)mask[1] << 32) | mask[0];
    const uint64_t mid = ((uint64_t)mask[3] << 32) | mask[2];
    const uint64_t hi = ((uint64_t)mask[5] << 32) | mask[4];
    const uint64_t m = k < 64 ? lo : (k < 128 ? mid : hi);
    if ((m >> (k & 63)) & 1) s = k;
  }
  return s;
}

// floor(a / b) for b >= 1 and |a / b| < 2^22 with rb ~ 1/b from v_rcp_f32:
// the float estimate is within 1 of the quotient (relative error below
// 2^-22), and up to two exact integer correction steps each way make it exact.
__device__ __forceinline__ int32_t floordiv_est(int32_t a, int32_t b, float rb) {
  int32_t q = (int32_t)floorf((float)a * rb);
  int32_t r = a - q * b;
  if (r < 0) { --q; r += b; if (r < 0) { --q; r += b; } }
  if (r >= b) { ++q; r -= b; if (r >= b) ++q; }
  return q;
}

// sat32(a * b + c) for a, b in the signed 24-bit range: v_mad_i32_i24 with the
// clamp bit, which saturates the integer result.
__device__ __forceinline__ int32_t mad24_sat(int32_t a, int32_t b, int32_t c) {
  int32_t r;
  asm("v_mad_i32_i24 %0, %1, %2, %3 clamp" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// median of (x, lo, hi) = clamp of x to [lo, hi] for lo <= hi (one v_med3_i32;
// the compiler emits a min and a max when it cannot see lo <= hi).
__device__ __forceinline__ int32_t med3_i32(int32_t x, int32_t lo, int32_t hi) {
  int32_t r;
  asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(lo), "s"(hi));
  return r;
}

// Requantisation of y = nrm * gamma + beta, exact in all three forms:
//   RQ_WIDE: 64-bit (b * y) >> c;
//   RQ_MULHI: int32 y saturated, mulhi(y, b << (32 - c)) (when b << (32 - c) <
//     2^31 and a saturated y clips either way);
//   RQ_WIN: y saturated, then clamped to [ylo, yhi] = [-floor(127 * 2^c / b),
//     ceil(127 * 2^c / b)], then a 24-bit multiply by b and a shift.  With
//     b <= 2^c the clamped bounds give exactly -127 and 127 and every y beyond
//     them clips to those values, so no further clip is needed; b, yhi < 2^23
//     and 127 * 2^c + b < 2^31 keep the product exact.
constexpr int RQ_WIDE = 0, RQ_MULHI = 1, RQ_WIN = 2;

// RQ_WIN's last step for one 16-column chunk: the 16 products t[j][i]
// (column 4 j + i) shifted right by c land as bytes i of the words w[j]
// through the SDWA destination select, byte-major over the four words: a
// write that keeps the other bytes reads the old word without an interlock,
// so two such writes to one word need other instructions between them.  The
// closing s_nop covers the same for the first later reader.
__device__ __forceinline__ void ln_shift_pack16(const int32_t (&t)[4][4], int32_t c, v4i& w) {
  int32_t w0, w1, w2, w3;
  asm("v_ashrrev_i32_sdwa %0, %20, %4 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %1, %20, %8 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %2, %20, %12 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %3, %20, %16 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %0, %20, %5 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %1, %20, %9 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %2, %20, %13 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %3, %20, %17 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %0, %20, %6 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %1, %20, %10 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %2, %20, %14 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %3, %20, %18 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %0, %20, %7 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %1, %20, %11 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %2, %20, %15 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_ashrrev_i32_sdwa %3, %20, %19 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "s_nop 4"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
      : "v"(t[0][0]), "v"(t[0][1]), "v"(t[0][2]), "v"(t[0][3]), "v"(t[1][0]), "v"(t[1][1]),
        "v"(t[1][2]), "v"(t[1][3]), "v"(t[2][0]), "v"(t[2][1]), "v"(t[2][2]), "v"(t[2][3]),
        "v"(t[3][0]), "v"(t[3][1]), "v"(t[3][2]), "v"(t[3][3]), "s"(c));
  w = v4i{w0, w1, w2, w3};
}

// gamma and beta sit in LDS, one copy per block, laid out chunk-major: entry
// ((k * 4 + j) * G + lane) holds the 4 columns 16 * (lane + G * k) + 4 j ..,
// so that the 16-byte reads of consecutive lanes hit consecutive banks
// (column-major order would put every fourth lane on the same banks).  This
// measured faster than keeping them in registers, which costs waves.
template <int G, int NCH, int RQ>
__global__ __launch_bounds__(kLnThreads) void iqln_fwd(LnDev p) {
  constexpr int RPW = 64 / G;
  constexpr int RPB = RPW * (kLnThreads / 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane % G, sub = lane / G;
  const uint32_t total = (uint32_t)p.rows * (uint32_t)p.cols;
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(p.x, total);
  const __amdgpu_buffer_rsrc_t orr = buf_rsrc(p.out, total);
  const __amdgpu_buffer_rsrc_t gr = buf_rsrc(p.gamma, (uint32_t)p.cols);
  const __amdgpu_buffer_rsrc_t br = buf_rsrc(p.beta, (uint32_t)p.cols * 4u);

  // this lane's chunks of the group of rows starting at r0 (zeros past the row
  // end; a row past the last reads the last row and is not stored)
  auto load_rows = [&](int r0, v4i* d) {
    const int row = r0 + wave * RPW + sub;
    const int rowc = row < p.rows ? row : p.rows - 1;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int col = 16 * (gl + G * k);
      d[k] = buf_load<v4i>(xr, rowc * p.cols + (col < p.cols ? col : 0));
    }
  };
  const int step = gridDim.x * RPB;
  int r0 = blockIdx.x * RPB;
  v4i d[NCH];
  load_rows(r0, d);  // in flight while gamma and beta are staged

  // LDS copy: beta entries, then gamma widened to int32, NENT of each
  extern __shared__ __attribute__((aligned(16))) int32_t ln_aff[];
  constexpr int NENT = 4 * G * NCH;  // 16-byte entries per table
  for (int i = threadIdx.x; i < NENT; i += kLnThreads) {
    const int gi = i % G, kj = i / G;
    const int col = 16 * (gi + G * (kj >> 2)) + 4 * (kj & 3);  // past cols: zeros
    reinterpret_cast<v4i*>(ln_aff)[i] = buf_load<v4i>(br, 4 * col);
    const int32_t g4 = __builtin_amdgcn_raw_buffer_load_b32(gr, col, 0, 0);
    v4i g;
#pragma unroll
    for (int t = 0; t < 4; ++t) g[t] = (int8_t)(g4 >> (8 * t));
    reinterpret_cast<v4i*>(ln_aff)[NENT + i] = g;
  }
  __syncthreads();
  const float rcols = __builtin_amdgcn_rcpf((float)p.cols);
  const int32_t sh = p.m - p.f;
  const int32_t ylo = p.ylo;

  for (; r0 < p.rows; r0 += step) {
    const int row = r0 + wave * RPW + sub;
    const bool rv = row < p.rows;
    int32_t s1 = 0, s2 = 0;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int col = 16 * (gl + G * k);
      const bool cv = col < p.cols;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d[k][j] = cv ? d[k][j] : 0;
        s1 = __builtin_amdgcn_sdot4(d[k][j], 0x01010101, s1, false);
        s2 = __builtin_amdgcn_sdot4(d[k][j], d[k][j], s2, false);
      }
    }
    s1 = group_sum_i32<G>(s1);   // |s1| <= 128 * 16384 = 2^21
    s2 = group_sum_i32<G>(s2);   // s2 <= 2^14 * 2^14 = 2^28
    const int32_t mean = floordiv_est(s1, p.cols, rcols);          // in [-128, 127]
    const int32_t cen = s2 - 2 * mean * s1 + p.cols * mean * mean; // sum (x - mean)^2 <= 2^30
    const int32_t var = floordiv_est(cen, p.cols, rcols);          // < 2^15
    const int32_t sd = var > 0 ? isqrt_newton10_fast(var, p.sqmask) : 1;
    const int32_t fs = floordiv_est(1 << p.m, sd, __builtin_amdgcn_rcpf((float)sd));  // <= 2^22
    const int32_t mfs = mean * fs;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int col = 16 * (gl + G * k);
      v4i o;
      v4i gk[4], bk[4];  // gamma (int32) and beta of the chunk's 16 columns
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bk[j] = reinterpret_cast<const v4i*>(ln_aff)[(k * 4 + j) * G + gl];
        gk[j] = reinterpret_cast<const v4i*>(ln_aff)[NENT + (k * 4 + j) * G + gl];
      }
      int32_t tw[4][4];  // RQ_WIN: the products before the final shift
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int32_t w = d[k][j];
        uint32_t res = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int32_t xv = (int8_t)(w >> (8 * i));  // signed byte i
          const int32_t gv = gk[j][i];
          // (x - mean) * fs with |x - mean| <= 255 and fs <= 2^22: fits 31 bits
          const int32_t nrm = (__mul24(xv, fs) - mfs) >> sh;  // |nrm| <= 2^16
          const int32_t bv = bk[j][i];
          int32_t y;
          if constexpr (RQ == RQ_WIN) {
            const int32_t ys = mad24_sat(nrm, gv, bv);
            const int32_t yc = med3_i32(ys, ylo, p.yhi);
            // (yc b) >> c lies in [-127, 127] by the choice of bounds; the shift
            // and the byte packing happen in ln_shift_pack16
            tw[j][i] = __mul24(yc, p.b);
            continue;
          } else if constexpr (RQ == RQ_MULHI) {
            const int32_t ys = mad24_sat(nrm, gv, bv);
            y = clamp127(__mulhi(ys, p.bm));
          } else {
            const int64_t yl = (int64_t)__mul24(nrm, gv) + bv;
            const int64_t t = ((int64_t)p.b * yl) >> p.c;
            y = (int32_t)(t < -127 ? -127 : (t > 127 ? 127 : t));
          }
          res |= ((uint32_t)y & 0xffu) << (8 * i);
        }
        o[j] = (int32_t)res;
      }
      if constexpr (RQ == RQ_WIN) ln_shift_pack16(tw, p.c, o);
      if (rv && col < p.cols) __builtin_amdgcn_raw_buffer_store_b128(o, orr, row * p.cols + col, 0, 0);
      // one chunk's gamma/beta reads at a time: keeps the register count low
      __builtin_amdgcn_sched_barrier(0);
    }
    if (r0 + step < p.rows) load_rows(r0 + step, d);
  }
}

// ---------------------------------------------------------------- dispatch
// G = 16 lanes per row for rows up to 2048 bytes (NCH = 1..8 chunks a lane),
// else G = 64 with NCH rounded up to 3, 4, 6, 8, 12 or 16 (rows up to 16384).
struct Shape {
  int g, nch;
};

Shape pick_shape(int cols) {
  if (cols <= 2048) return {16, (cols + 255) / 256};
  const int n = (cols + 1023) / 1024;
  static const int steps[] = {3, 4, 6, 8, 12, 16};
  for (int s : steps)
    if (n <= s) return {64, s};
  return {64, 16};
}

typedef void (*GeluKernel)(GeluDev);
typedef void (*LnKernel)(LnDev);

template <int G, int NCH>
void* gelu_ptr() { return (void*)&iqgelu_fwd<G, NCH>; }

template <int G, int NCH>
void* ln_ptr(int rq) {
  return rq == RQ_WIN ? (void*)&iqln_fwd<G, NCH, RQ_WIN>
       : rq == RQ_MULHI ? (void*)&iqln_fwd<G, NCH, RQ_MULHI> : (void*)&iqln_fwd<G, NCH, RQ_WIDE>;
}

template <bool LN>
void* pick_kernel(Shape s, int rq) {
#define IQB_CASE(GG, NN) \
  if (s.g == GG && s.nch == NN) return LN ? ln_ptr<GG, NN>(rq) : gelu_ptr<GG, NN>();
  IQB_CASE(16, 1) IQB_CASE(16, 2) IQB_CASE(16, 3) IQB_CASE(16, 4)
  IQB_CASE(16, 5) IQB_CASE(16, 6) IQB_CASE(16, 7) IQB_CASE(16, 8)
  IQB_CASE(64, 3) IQB_CASE(64, 4) IQB_CASE(64, 6) IQB_CASE(64, 8) IQB_CASE(64, 12) IQB_CASE(64, 16)
#undef IQB_CASE
  return nullptr;
}

int check_device(int* dev) {
  hipDeviceProp_t prop;
  if (hipGetDevice(dev) != hipSuccess || hipGetDeviceProperties(&prop, *dev) != hipSuccess)
    return IQATTN_E_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return IQATTN_E_DEVICE;
  return IQATTN_OK;
}

int check_rows_cols(int32_t rows, int32_t cols) {
  if (rows < 0 || cols < 16 || cols > kMaxCols || cols % 16) return IQATTN_E_SHAPE;
  if ((int64_t)rows * cols > INT32_MAX) return IQATTN_E_SHAPE;
  return IQATTN_OK;
}

// One block per group of rows; the hardware hands the blocks to the CUs as
// earlier ones finish (measured faster here than persistent blocks looping
// over the groups, for both kernels).  The kernels still loop when the grid
// is capped.
unsigned grid_for(int32_t rows, int rows_per_block) {
  const int64_t need = ((int64_t)rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = (int64_t)1 << 30;
  return (unsigned)(need < 1 ? 1 : (need > cap ? cap : need));
}

}  // namespace
}  // namespace iqattn

using namespace iqattn;

struct iqgelu_ctx {
  GeluDev dp;
  uint8_t* tab;
  void* kernel;
  unsigned grid;
  int device;
};

struct iqlayernorm_ctx {
  LnDev dp;
  void* kernel;
  unsigned grid;
  unsigned lds_bytes;
  int device;
};

extern "C" int iqgelu_create(const iqgelu_params* p, iqgelu_ctx** out) {
  if (!out) return IQATTN_E_NULL;
  *out = NULL;
  if (!p) return IQATTN_E_NULL;
  int rc = check_rows_cols(p->rows, p->cols);
  if (rc) return rc;
  if (p->i0 < 1 || p->i0 > 32768 || p->exp_frac_bits < 0 || p->exp_frac_bits > 30 ||
      p->k_out < 2 || p->k_out > 8 || p->intdiv_m < p->k_out - 1 || p->intdiv_m > 40 ||
      p->b < 1 || p->c < 0 || p->c > 62)
    return IQATTN_E_INVAL;
  int dev = 0;
  if ((rc = check_device(&dev))) return rc;
  const Shape s = pick_shape(p->cols);
  void* k = pick_kernel<false>(s, 0);
  if (!k) return IQATTN_E_SHAPE;
  iqgelu_ctx* c = (iqgelu_ctx*)calloc(1, sizeof(iqgelu_ctx));
  if (!c) return IQATTN_E_ALLOC;
  c->device = dev;
  c->kernel = k;
  const int rpb = (64 / s.g) * (kGeluThreads / 64);
  c->grid = grid_for(p->rows, rpb);
  if (hipMalloc((void**)&c->tab, kTabBytes) != hipSuccess) {
    free(c);
    return IQATTN_E_ALLOC;
  }
  hipLaunchKernelGGL(iqgelu_build_table, dim3(kTabBytes / 256), dim3(256), 0, 0, c->tab, p->i0,
                     p->exp_frac_bits, p->intdiv_m, p->k_out, p->b, p->c);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipFree(c->tab);
    free(c);
    return set_hip_error(e, "iqgelu table");
  }
  c->dp.tab = c->tab;
  c->dp.rows = p->rows;
  c->dp.cols = p->cols;
  *out = c;
  return IQATTN_OK;
}

extern "C" int iqgelu_forward(iqgelu_ctx* c, const int8_t* x, int8_t* out, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  if (c->dp.rows == 0) return IQATTN_OK;
  if (!x || !out) return IQATTN_E_NULL;
  if (((uintptr_t)x | (uintptr_t)out) & 15u) return IQATTN_E_ALIGN;
  GeluDev dp = c->dp;
  dp.x = x;
  dp.out = out;
  hipLaunchKernelGGL((GeluKernel)c->kernel, dim3(c->grid), dim3(kGeluThreads), 0,
                     (hipStream_t)hip_stream, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqgelu launch");
  return IQATTN_OK;
}

extern "C" int iqgelu_destroy(iqgelu_ctx* c) {
  if (!c) return IQATTN_OK;
  if (c->tab) (void)hipFree(c->tab);
  free(c);
  return IQATTN_OK;
}

extern "C" int iqlayernorm_create(const iqlayernorm_params* p, iqlayernorm_ctx** out) {
  if (!out) return IQATTN_E_NULL;
  *out = NULL;
  if (!p) return IQATTN_E_NULL;
  int rc = check_rows_cols(p->rows, p->cols);
  if (rc) return rc;
  if (p->norm_frac_bits < 0 || p->norm_frac_bits > 8 || p->intdiv_m < p->norm_frac_bits ||
      p->intdiv_m > 22 || p->b < 1 || p->c < 0 || p->c > 62)
    return IQATTN_E_INVAL;
  int dev = 0;
  if ((rc = check_device(&dev))) return rc;
  // The requantisation form: RQ_WIN when b <= 2^c, b, yhi < 2^23 and
  // 127 * 2^c + b < 2^31; else RQ_MULHI when b << (32 - c) < 2^31 and
  // (2^31 - 1) b / 2^c >= 128 (a saturated y clips either way); else the
  // 64-bit form.
  int rq = RQ_WIDE;
  int32_t bm = 0, ylo = 0, yhi = 0;
  if (p->c <= 31 && (int64_t)p->b <= ((int64_t)1 << p->c)) {
    const int64_t a = (int64_t)127 << p->c;
    const int64_t hi = (a + p->b - 1) / p->b, lo = -(a / p->b);
    if (p->b < (1 << 23) && hi < (1 << 23) && a + p->b < ((int64_t)1 << 31)) {
      rq = RQ_WIN;
      ylo = (int32_t)lo;
      yhi = (int32_t)hi;
    }
  }
  if (rq == RQ_WIDE && p->c >= 1 && p->c <= 32) {
    const int64_t v = (int64_t)p->b << (32 - p->c);
    const bool sat_ok = (((int64_t)INT32_MAX * p->b) >> p->c) >= 128;
    if (v < ((int64_t)1 << 31) && sat_ok) {
      rq = RQ_MULHI;
      bm = (int32_t)v;
    }
  }
  const Shape s = pick_shape(p->cols);
  void* k = pick_kernel<true>(s, rq);
  if (!k) return IQATTN_E_SHAPE;
  iqlayernorm_ctx* c = (iqlayernorm_ctx*)calloc(1, sizeof(iqlayernorm_ctx));
  if (!c) return IQATTN_E_ALLOC;
  c->device = dev;
  c->kernel = k;
  const int rpb = (64 / s.g) * (kLnThreads / 64);
  c->lds_bytes = (unsigned)(128 * s.g * s.nch);
  if (c->lds_bytes > 65536u) {
    // more than 64 KiB of dynamic LDS needs the kernel to opt in
    if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)c->lds_bytes) !=
        hipSuccess) {
      free(c);
      return IQATTN_E_DEVICE;
    }
  }
  c->grid = grid_for(p->rows, rpb);
  LnDev& d = c->dp;
  d.rows = p->rows;
  d.cols = p->cols;
  d.m = p->intdiv_m;
  d.f = p->norm_frac_bits;
  d.b = p->b;
  d.c = p->c;
  d.bm = bm;
  d.ylo = ylo;
  d.yhi = yhi;
  {
    uint8_t* flags = NULL;
    uint8_t host[192];
    hipError_t e = hipMalloc((void**)&flags, sizeof(host));
    if (e != hipSuccess) {
      free(c);
      return IQATTN_E_ALLOC;
    }
    hipLaunchKernelGGL(iqln_newton_flags, dim3(1), dim3(192), 0, 0, flags);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(host, flags, sizeof(host), hipMemcpyDeviceToHost);
    (void)hipFree(flags);
    if (e != hipSuccess) {
      free(c);
      return set_hip_error(e, "iqlayernorm newton flags");
    }
    for (int k = 0; k < 192; ++k)
      if (host[k]) d.sqmask[k >> 5] |= 1u << (k & 31);
  }
  *out = c;
  return IQATTN_OK;
}

extern "C" int iqlayernorm_forward(iqlayernorm_ctx* c, const int8_t* x, const int8_t* gamma,
                                   const int32_t* beta, int8_t* out, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  if (c->dp.rows == 0) return IQATTN_OK;
  if (!x || !gamma || !beta || !out) return IQATTN_E_NULL;
  if (((uintptr_t)x | (uintptr_t)gamma | (uintptr_t)beta | (uintptr_t)out) & 15u)
    return IQATTN_E_ALIGN;
  LnDev dp = c->dp;
  dp.x = x;
  dp.gamma = gamma;
  dp.beta = beta;
  dp.out = out;
  hipLaunchKernelGGL((LnKernel)c->kernel, dim3(c->grid), dim3(kLnThreads), c->lds_bytes,
                     (hipStream_t)hip_stream, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqlayernorm launch");
  return IQATTN_OK;
}

extern "C" int iqlayernorm_destroy(iqlayernorm_ctx* c) {
  free(c);
  return IQATTN_OK;
}
