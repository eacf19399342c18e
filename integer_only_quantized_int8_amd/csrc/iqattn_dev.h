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
  int32_t out_tok;           // output [B][N][H][d] (1) or [B][H][N][d] (0)
  int32_t n_full;            // work items [0, n_full) are whole heads, later items quarter heads
  int32_t n_items;           // whole heads plus quarter-head items (fast kernels)
  int32_t qk_b, qk_c, pv_b, pv_c;
  int32_t exp_last;          // first table index whose entry is 0 (or 255)
  int32_t intdiv_m, p_shift, p_max;
  int32_t lis_f;
  // constants of the fast kernels (see the host's eligibility checks)
  int32_t qk_bm, mask_s;         // L_raw = mulhi(S, qk_bm); padded keys carry mask_s
  int32_t e_shift, f_shift;      // table holds e << e_shift; F = f_adj << f_shift
  int32_t e0, e0_pow2;           // e(0) and whether it divides 2^M
  int32_t pv_fast, pv_bm;        // output requantisation as mulhi(o, pv_bm)
  int32_t p_u24;                 // Shiftmax: e << e_shift and F below 2^24 (p16_pack24)
  int32_t bias_lds;              // windowed bias of 64-key rows staged in LDS (fast kernels)
  uint32_t* status;              // context status word: kStatus* bits of waits that gave up
  int32_t spin_limit;            // polls of a bounded wait before it gives up
};

// Bits of the status word.  A wave whose bounded wait gives up sets its bit
// (one device atomic from lane 0, a vector memory operation) and exits; the
// output rows it would have written stay unwritten.
constexpr uint32_t kStatusLoader = 1u;    // loader wave: a buffer was never released
constexpr uint32_t kStatusKQ = 2u;        // compute wave: K and Q never arrived
constexpr uint32_t kStatusV = 4u;         // compute wave: V never arrived

__device__ __forceinline__ void report_giveup(const DevParams& p, uint32_t bit) {
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(p.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef void (*KernelFn)(DevParams);

// Byte offset of head u's row 0 in the output and the byte distance between
// its rows: [B][H][N][d] (u N d, d) or [B][N][H][d] ((b N H + h) d, H d) for
// u = b H + h.
__device__ __forceinline__ int64_t out_head_base(const DevParams& p, int u, int D) {
  return p.out_tok ? ((int64_t)(u / p.heads) * p.n * p.heads + (u % p.heads)) * D
                   : (int64_t)u * p.n * D;
}
__device__ __forceinline__ int32_t out_row_stride(const DevParams& p, int D) {
  return p.out_tok ? p.heads * D : D;
}

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

// Sixteen Shiftmax probabilities (four operand words) with e << a and f << b
// below 2^24: v_mul_hi_u32_u24 returns bits 32..47 of the 48-bit product, and
// its SDWA form writes the low byte of that result (P < 2^7) straight into byte
// k of a word, so a word costs four instructions.  A byte write that keeps the
// other bytes reads the old word without an interlock against the previous
// write, so the sixteen writes go byte-major: writes to one word are four
// instructions apart.  The closing s_nop gives the MFMA that reads the words
// the wait states a VALU write needs, which the compiler cannot insert for an
// asm block.
__device__ __forceinline__ void p16_pack24(const v4i& e0, const v4i& e1, const v4i& e2,
                                           const v4i& e3, uint32_t F, v4i& w) {
  uint32_t w0, w1, w2, w3;
  asm(
      "v_mul_hi_u32_u24_sdwa %0, %4, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %1, %8, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %2, %12, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %3, %16, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %0, %5, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %1, %9, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %2, %13, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %3, %17, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %0, %6, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %1, %10, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %2, %14, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %3, %18, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %0, %7, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %1, %11, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %2, %15, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_u32_u24_sdwa %3, %19, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "s_nop 4"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
      : "v"(e0[0]), "v"(e0[1]), "v"(e0[2]), "v"(e0[3]), "v"(e1[0]), "v"(e1[1]), "v"(e1[2]),
        "v"(e1[3]), "v"(e2[0]), "v"(e2[1]), "v"(e2[2]), "v"(e2[3]), "v"(e3[0]), "v"(e3[1]),
        "v"(e3[2]), "v"(e3[3]), "v"(F));
  w = v4i{(int32_t)w0, (int32_t)w1, (int32_t)w2, (int32_t)w3};
}

// Inline asm never reads an MFMA result first: the compiler's hazard checks do
// not look inside asm blocks, so the first reader of every accumulator is
// ordinary code (which gets the required wait states).

typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef int32_t v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const int8_t lds_i8;
typedef __attribute__((address_space(3))) uint32_t lds_u32w;

// buffer_load_dwordx4 ... lds: each lane's 16 bytes at rsrc.base + voffset go to
// LDS at (lds + 16 * lane); offsets at or past rsrc.num_records read as zero.
__device__ void raw_buffer_load_lds(v4i rsrc, lds_u32w* lds, int size, int voffset, int soffset,
                                    int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// buffer resource (typed) of a byte range [base, base + bytes): raw access;
// accesses through it take a 32-bit per-lane offset and the base in SGPRs
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// operand-sized loads through a buffer resource
template <typename Op>
__device__ __forceinline__ Op buf_load(__amdgpu_buffer_rsrc_t r, int off);
template <>
__device__ __forceinline__ v4i buf_load<v4i>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
template <>
__device__ __forceinline__ int64_t buf_load<int64_t>(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(int64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// buffer resource of a byte range [base, base + bytes): stride 0, raw access
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  v4i r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)(uint32_t)(a >> 32);
  r[2] = (int32_t)bytes;
  r[3] = 0x00020000;
  return r;
}

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

// ---------------------------------------------------------------- fast-kernel LDS plan
// K and V of one head occupy one region each, a whole number of 1 KB direct
// global->LDS blocks (rows beyond N arrive as zeros).  Two buffers (V0 K0 V1 K1)
// let the next head's loads run under the current head's compute; the
// exponential table and the LIS shift scratch follow.
constexpr int fast_region_bytes(int d, int kt) { return ((kt * 16 * d + 1023) / 1024) * 1024; }
constexpr int kFastTableBytes = 1024;  // LDS copy of the 256-entry table
// Rows of up to 256 keys run workgroups of 15 compute waves and one loader
// wave over four (V, K, Q) buffers (three for the LIS VALU back end, whose
// shift scratch needs the room); at 197 keys one such workgroup fills a CU,
// so all waves of a CU share one tile queue (two workgroups on a CU drift
// apart: the older one's waves win the issue arbitration and the younger one
// finishes alone).
// Rows of 209 to 256 keys (14 to 16 tiles) run 11 compute waves over three
// buffers: at 16 waves their accumulators would not fit the registers, and at
// d = 64 four buffers would not fit the LDS.
// Longer rows hold about 250 VGPRs per lane, two waves per SIMD.  When two
// (V, K) buffers, the table and the LIS shift scratch fit the LDS, one
// workgroup of 7 compute waves and the loader fills a CU (its waves sit on all
// four SIMDs); otherwise two workgroups of 3 compute waves and one buffer
// each share it.
constexpr bool fast_big(int kt, bool bias) { return kt <= 16; }
constexpr bool fast_mid(int kt, bool bias) { return kt >= 14 && kt <= 16; }
constexpr bool fast_long2(int d, int kt, int var) {
  return kt > 16 && 4 * fast_region_bytes(d, kt) + kFastTableBytes + (var == kFastLisValu ? 7 * 1024 : 0) + 64 <=
                        160 * 1024;
}
constexpr int fast_nbuf(int d, int kt, bool bias, int var) {
  return fast_big(kt, bias) ? (var == kFastLisValu || fast_mid(kt, bias) ? 3 : 4) : (fast_long2(d, kt, var) ? 2 : 1);
}
constexpr int fast_nreg(int kt, bool bias) { return fast_big(kt, bias) ? 3 : 2; }
constexpr int fast_cw(int d, int kt, bool bias, int var) {
  return fast_big(kt, bias) ? (fast_mid(kt, bias) ? 11 : 15) : (fast_long2(d, kt, var) ? 7 : 3);
}
// minimum waves per SIMD the register allocation must allow
// (rows of up to 64 keys: 8 waves per SIMD, so that two 16-wave workgroups
// share a CU; the bound keeps the scalar registers within what eight waves
// per SIMD can hold)
constexpr int fast_waves_per_eu(int kt, bool bias) {
  return kt <= 4 ? 8 : (fast_big(kt, bias) ? (fast_mid(kt, bias) ? 3 : 4) : 2);
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

// ---------------------------------------------------------------- LDS layouts of K and V
// XOR swizzles of the 16-byte chunk index of an LDS row.  K (b128 / b64
// operand reads of 16 rows): d = 64 by (row >> 1) & 3, d = 32 by (row >> 3) & 1.
// V (transpose reads of keys 16 tt + 4 g + r): d = 64 by bits 2 and 4 of the
// key, d = 32 by bit 4; both spread a half-wave over distinct banks.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 64 ? (row >> 1) & 3 : (row >> 3) & 1;
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 64 ? (((row >> 2) & 1) | ((row >> 3) & 2)) : (row >> 4) & 1;
}

// V^T operands by transpose reads: two ds_read_b64_tr_b8 per 16-feature tile
// at the lane offsets vtr[0], vtr[1], the feature tile entering as an XOR of
// the 16-byte chunk index.  vt_addr forms a tile's eight lane addresses once;
// read_vt adds the 64-key step's byte offset, a constant the reads carry in
// their offset field.
template <int FT>
__device__ __forceinline__ void vt_addr(uint32_t vb, const int (&vtr)[2], uint32_t (&va)[FT][2]) {
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    va[ft][0] = vb + (uint32_t)(vtr[0] ^ (ft << 4));
    va[ft][1] = vb + (uint32_t)(vtr[1] ^ (ft << 4));
  }
}
template <int FT>
__device__ __forceinline__ void read_vt(const uint32_t (&va)[FT][2], uint32_t off, v4i (&vop)[FT]) {
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(uintptr_t)(va[ft][0] + off));
    const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(uintptr_t)(va[ft][1] + off));
    vop[ft] = v4i{r0[0], r0[1], r1[0], r1[1]};
  }
}

// LIS bit-plane operand bytes of four shifts (w in the low four bits of each
// word): plane 0 gets -2^w for w < 8, plane 1 gets -2^(w-8) for w >= 8 (as
// int8 bytes 0xFF << l).
__device__ __forceinline__ void lis_planes(const v4i& w, int32_t& lo, int32_t& hi) {
  uint32_t y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {  // 16-bit (plane 1 byte, plane 0 byte)
    const uint32_t l = (uint32_t)w[r] & 15u;
    y[r] = (0xFFu << l) & (0xFFu << (l & 8));
  }
  const uint32_t t01 = __builtin_amdgcn_perm(y[1], y[0], 0x05010400u);
  const uint32_t t23 = __builtin_amdgcn_perm(y[3], y[2], 0x05010400u);
  lo = (int32_t)__builtin_amdgcn_perm(t23, t01, 0x05040100u);
  hi = (int32_t)__builtin_amdgcn_perm(t23, t01, 0x07060302u);
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

// records the HIP error text for iqattn_strerror and returns IQATTN_E_LAUNCH
int set_hip_error(hipError_t e, const char* what);

// host-side selectors, one per translation unit
KernelFn generic_kernel(int d, int ktm, int variant, bool bias);
KernelFn fast_kernel(int d, int kt, bool bias, int var);  // null if not instantiated
// rows of 641..1024 keys (three passes over LDS-resident K); var is a kFast* back end
KernelFn long_kernel(int d, int var, bool bias);
size_t long_lds_bytes(int d, int n, int var);
int long_threads();

}  // namespace iqattn
