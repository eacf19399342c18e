// iqattn_dev.h -- device-side definitions shared by the kernels of libiqattn.
//
// Integer conventions of the method (I-ViT, mer.run summary, sec. 3.2-3.3;
// FQ-ViT abstract; Trio-ViT sec. IV Eq. 11 and Eq. 12):
//   requantisation  floor((b * x) / 2^c), saturated to [-127, 127];
//   exponential     e(delta) for delta = L - max(L) in [-254, 0], read from a
//                   256-entry table built on the device at create time;
//   IntDiv          P = (floor(2^M / sum e) * e) >> (M - (k_out - 1));
//   LIS             Ph = (floor(2^M / sum e) * e) >> (M - F), code from the
//                   leading one of Ph plus the next bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqattn {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kExpRep = 32;  // copies of the exponential table in LDS (generic kernel)

// back ends of the specialised kernels
constexpr int kFastShiftmax = 0;
constexpr int kFastLisValu = 1;
constexpr int kFastLisMfma = 2;

struct DevParams {
  const int8_t* q;
  const int8_t* k;
  const int8_t* v;
  int8_t* out;
  const uint32_t* exp_tab;   // [256] e(-idx), or e(-idx) << e_shift for the fast kernels
  const int32_t* bias;       // [heads][Np][Np] expanded, query-major, or null
  int32_t heads, n, units;
  int32_t n_full;            // blocks [0, n_full) take whole heads, later blocks quarter heads
  int32_t qk_b, qk_c, pv_b, pv_c;
  int32_t exp_last;          // first table index whose entry is 0 (or 255)
  int32_t intdiv_m, p_shift, p_max;
  int32_t lis_f;
  // constants of the fast kernels (see the host's eligibility checks)
  int32_t qk_bm, mask_s;         // L_raw = mulhi(S, qk_bm); padded keys carry mask_s
  int32_t e_shift, f_shift;      // table holds e << e_shift; F = f_adj << f_shift
  int32_t e0, e0_pow2;           // e(0) and whether it divides 2^M
  int32_t pv_fast, pv_bm;        // output requantisation as mulhi(o, pv_bm)
};

typedef void (*KernelFn)(DevParams);

// ---------------------------------------------------------------- arithmetic
// floor((b * x) / 2^c) saturated to [-127, 127]; 64-bit product.
__device__ __forceinline__ int32_t requant_i8(int32_t x, int32_t b, int32_t c) {
  int64_t y = ((int64_t)b * (int64_t)x) >> c;  // arithmetic shift = floor
  y = y < -127 ? -127 : (y > 127 ? 127 : y);
  return (int32_t)y;
}


// floor(a * b / 2^32) for unsigned 32-bit a, b: v_mul_hi_u32 (full rate).
__device__ __forceinline__ uint32_t mulhi_u32(uint32_t a, uint32_t b) {
  return (uint32_t)(((uint64_t)a * (uint64_t)b) >> 32);
}

__device__ __forceinline__ int32_t clamp127(int32_t x) { return min(max(x, -127), 127); }

// floor(x * bm / 2^32) = floor((b x) / 2^c) for bm = b << (32 - c) < 2^31:
// the requantised logit before saturation, one v_mul_hi_i32 (full rate).
__device__ __forceinline__ int32_t mulhi_i32(int32_t x, int32_t bm) {
  return (int32_t)(((int64_t)x * (int64_t)bm) >> 32);
}

// Byte address of the exponential-table entry for accumulator x of a row
// whose entry-0 address is rb: clamp(rb + estr_neg * L_raw(x), lo, hi); the
// clamp is the [-127, 127] saturation of the logit.  Three VALU instructions
// (v_mul_hi_i32, v_mad_i32_i24, v_med3_i32).
__device__ __forceinline__ int32_t exp_offset(int32_t x, int32_t bm, int32_t estr_neg,
                                              int32_t rb, int32_t lo, int32_t hi) {
  int32_t a;
  asm("v_mul_hi_i32 %0, %1, %2\n\t"
      "v_mad_i32_i24 %0, %0, %3, %4\n\t"
      "v_med3_i32 %0, %0, %5, %6"
      : "=&v"(a)
      : "v"(x), "s"(bm), "s"(estr_neg), "v"(rb), "v"(lo), "v"(hi));
  return a;
}

// Four Shiftmax probabilities P = (e f) >> (M - k_out + 1) = mulhi(e 2^a, f 2^b)
// packed little-endian into one int8 word of the P.V MFMA operand.  The asm
// block makes the two 16-bit halves; the final merge is a compiler-visible
// v_perm so that the MFMA hazard checks see the instruction that feeds it.
__device__ __forceinline__ uint32_t p4_pack(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3,
                                            uint32_t F) {
  uint32_t lo, hi, t;
  asm("v_mul_hi_u32 %0, %3, %7\n\t"
      "v_mul_hi_u32 %2, %4, %7\n\t"
      "v_lshl_or_b32 %0, %2, 8, %0\n\t"
      "v_mul_hi_u32 %1, %5, %7\n\t"
      "v_mul_hi_u32 %2, %6, %7\n\t"
      "v_lshl_or_b32 %1, %2, 8, %1"
      : "=&v"(lo), "=&v"(hi), "=&v"(t)
      : "v"(e0), "v"(e1), "v"(e2), "v"(e3), "v"(F));
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Inline asm never reads an MFMA result first: the compiler's hazard checks do
// not look inside asm blocks, so the first reader of every accumulator is
// ordinary code (which gets the required wait states).

typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// 32-bit LDS address of a pointer into dynamic shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

__device__ __forceinline__ uint32_t lds_read_u32(uint32_t addr) {
  return *(lds_u32*)(uintptr_t)addr;
}


// Reductions over the four lanes l, l^16, l^32, l^48 (the 16-lane rows of a
// wave64): v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap pairs
// the two halves; each lane ends with the reduction of all four.
__device__ __forceinline__ int32_t wave_max4(int32_t x) {
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  x = max((int32_t)a[0], (int32_t)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  return max((int32_t)b[0], (int32_t)b[1]);
}

__device__ __forceinline__ uint32_t wave_sum4(uint32_t x) {
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] + a[1];
  auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] + b[1];
}

// low bytes of four values packed little-endian into one word
__device__ __forceinline__ uint32_t pack4_lowbytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                    uint32_t b3) {
  uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// position of key kappa inside its 64-key block of the staged V^T rows:
// key 16*tt + 4*g + r sits at byte 16*g + 4*tt + r, so that the P.V MFMA's
// A-operand k-slot (lane group g, byte p) holds the key that the B operand
// (P, straight from the Q.K^T accumulator layout) has in that slot.
__device__ __forceinline__ int vperm_pos(int kappa) {
  int base = kappa & ~63, w = kappa & 63;
  return base + ((w & 15) >> 2) * 16 + (w >> 4) * 4 + (w & 3);
}

// leading-one log2 with rounding: index of the leading one plus the next bit
// (Trio-ViT sec. IV, Eq. 11).  x >= 1.
__device__ __forceinline__ int32_t ilog2r_dev(uint32_t x) {
  int32_t k = 31 - __clz((int)x);
  int32_t nb = (k >= 1) ? (int32_t)((x >> (k - 1)) & 1u) : 0;
  return k + nb;
}

// ---------------------------------------------------------------- MFMA
template <int D>
struct Mfma;

template <>
struct Mfma<64> {
  typedef v4i Op;  // 16 int8 per lane
  static __device__ __forceinline__ v4i run(Op a, Op b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<32> {
  typedef int64_t Op;  // 8 int8 per lane
  static __device__ __forceinline__ v4i run(Op a, Op b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
  }
};

// 16x16x64 int8 MFMA, used for P.V (64 keys per instruction)
__device__ __forceinline__ v4i mfma64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// host-side selectors, one per translation unit
KernelFn generic_kernel(int d, int ktm, int variant, bool bias);
KernelFn fast_kernel(int d, int kt, bool bias, int var);  // null if not instantiated

}  // namespace iqattn
