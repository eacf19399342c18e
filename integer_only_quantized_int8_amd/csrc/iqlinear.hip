// iqlinear.hip -- integer-only int8 linear layer: Y = requant(X W^T) with a
// dyadic (b, c) per output tensor, fused into the GEMM epilogue.
//
// Method passage: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" (integer product, then (b * acc) >> c to int8); sec. 3.1
// (the MSA projections).
//
// Kernel (iqlinear_tile below): Y^T = W . X^T with v_mfma_i32_16x16x64_i8,
// W rows fed in an order that leaves each lane with 16 adjacent output
// columns of one row; their requantised bytes leave as one 16-byte store,
// straight into the head-split layout when asked.
#include "iqattn_dev.h"
#include "iqattn.h"
#include "iqlinear.h"

#include <stdlib.h>
#include <string.h>

#include <type_traits>
#include <vector>

namespace iqattn {
namespace {

constexpr int kStep = 64;   // k bytes per step

struct LinParams {
  const int8_t* x;
  const int8_t* w;
  int8_t* out[3];
  int32_t rows, in_f, out_f;
  int32_t layout;
  int32_t seq_len, heads, head_dim, width;  // width = heads * head_dim (QKV)
  int32_t b[3], c[3], bm[3];  // bm = b << (32 - c) when it is below 2^31, else 0
  // Window path (w24 = 1 when every pair in use qualifies): for b <= 2^c the
  // saturated result equals floor(b y / 2^c) of y = acc clamped to
  // [ylo, yhi] = [ceil(-127 2^c / b), floor((128 2^c - 1) / b)] (floor(b y /
  // 2^c) moves by at most 1 per unit of y, so it is -127 at ylo and 127 at
  // yhi); when the window and bm24 = b 2^(32 - c) fit in 24 signed bits that
  // is one v_mul_hi_i32_i24 of the clamped y and bm24.
  int32_t ylo[3], yhi[3], bm24[3];
  int32_t w24;
  // floor(m / seq_len) = (m + mulhi(seq_magic, m)) >> seq_shift for 0 <= m < 2^31
  // (Granlund and Montgomery's division by an invariant integer)
  uint32_t seq_magic;
  int32_t seq_shift;
  const int2* order;   // tile table: (row tile, column tile) of tile index t
  int32_t ntiles;
};

template <typename T>
__device__ __forceinline__ T pick3(int which, T a0, T a1, T a2) {
  return which == 0 ? a0 : (which == 1 ? a1 : a2);
}

// floor(x * m / 2^32) for x, m in the signed 24-bit range: v_mul_hi_i32_i24
__device__ __forceinline__ int32_t mulhi_i24(int32_t x, int32_t m) {
  const int64_t xs = (int32_t)((uint32_t)x << 8) >> 8, ms = (int32_t)((uint32_t)m << 8) >> 8;
  return (int32_t)((xs * ms) >> 32);
}

__device__ __forceinline__ int32_t div_seq(const LinParams& p, int32_t m) {
  return (int32_t)(((uint32_t)m + mulhi_u32(p.seq_magic, (uint32_t)m)) >> p.seq_shift);
}

// The four requantised bytes of accumulator block v (4 adjacent columns of
// one row, all under the pair `which`), packed little-endian.
template <bool W24>
__device__ __forceinline__ uint32_t requant4(const LinParams& p, int which, v4i v) {
  if (W24) {
    const int32_t lo = pick3(which, p.ylo[0], p.ylo[1], p.ylo[2]);
    const int32_t hi = pick3(which, p.yhi[0], p.yhi[1], p.yhi[2]);
    const int32_t m = pick3(which, p.bm24[0], p.bm24[1], p.bm24[2]);
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      r[k] = (uint32_t)mulhi_i24(__builtin_elementwise_max(__builtin_elementwise_min(v[k], hi), lo), m);
    return pack4_lowbytes(r[0], r[1], r[2], r[3]);
  }
  const int32_t bm = pick3(which, p.bm[0], p.bm[1], p.bm[2]);
  if (bm)
    return pack4_lowbytes((uint32_t)clamp127(mulhi_i32(v[0], bm)), (uint32_t)clamp127(mulhi_i32(v[1], bm)),
                          (uint32_t)clamp127(mulhi_i32(v[2], bm)), (uint32_t)clamp127(mulhi_i32(v[3], bm)));
  const int32_t bb = pick3(which, p.b[0], p.b[1], p.b[2]), cc = pick3(which, p.c[0], p.c[1], p.c[2]);
  return pack4_lowbytes((uint32_t)requant_i8(v[0], bb, cc), (uint32_t)requant_i8(v[1], bb, cc),
                        (uint32_t)requant_i8(v[2], bb, cc), (uint32_t)requant_i8(v[3], bb, cc));
}

// Destination of output row m (its part of the offset): plain m out; head
// split (bidx H N + t) d = m d + bidx (H - 1) N d for m = bidx N + t.
__device__ __forceinline__ int64_t row_offset(const LinParams& p, bool qkv, int m) {
  if (!qkv) return (int64_t)m * p.out_f;
  const int bidx = div_seq(p, m);
  return (int64_t)m * p.head_dim + (int64_t)bidx * (p.heads - 1) * p.seq_len * p.head_dim;
}

// Column part of the destination of output column n (a multiple of 4) and the
// tensor it belongs to: plain n; head split (h N d + i) for column n = which
// width + h d + i.  n / head_dim runs once per lane and tile.
__device__ __forceinline__ int col_part(const LinParams& p, bool qkv, int n, int& which) {
  if (!qkv) {
    which = 0;
    return n;
  }
  which = (n >= p.width) + (n >= 2 * p.width);
  const int col = n - which * p.width, h = col / p.head_dim;
  return h * p.seq_len * p.head_dim + (col - h * p.head_dim);
}

// Epilogue of one wave's TN x TM accumulator tiles, one 4-byte word at a
// time: acc[a][b][r] is output column n + 4 a + r of row m + 16 b;
// requantised, packed to 4 bytes and stored.  Rows past the end are skipped.
template <int TM, int TN, bool W24>
__device__ __forceinline__ void store_tile(const LinParams& p, const v4i (&acc)[TN][TM], int m_base,
                                           int n_base) {
  const bool qkv = p.layout == IQLINEAR_QKV_HEADS;
  int64_t rofs[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b) rofs[b] = row_offset(p, qkv, m_base + 16 * b);
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n_base + 4 * a;
    if (n >= p.out_f) continue;  // out is a multiple of 16: the lane's whole 16 columns
    int which;
    const int cofs = col_part(p, qkv, n, which);
    int8_t* const out = pick3(which, p.out[0], p.out[1], p.out[2]);
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      if (m_base + 16 * b >= p.rows) continue;
      *(uint32_t*)(out + rofs[b] + cofs) = requant4<W24>(p, which, acc[a][b]);
    }
  }
}

// Window path, four words at once: byte r of word a is
// floor(yc[a][r] m[a] / 2^32) (v_mul_hi_i32_i24 with an SDWA byte
// destination, the clamped accumulator and m both within 24 signed bits),
// written byte-major over the four words: a write that keeps the other bytes
// reads the old word without an interlock, so two such writes to one word
// need other instructions between them; the closing s_nop covers the first
// later reader.  (Each word takes its own multiplier, so words under
// different pairs can share a call.)
__device__ __forceinline__ void w24_pack4x4(const int32_t (&yc)[4][4], const int32_t (&m)[4], uint32_t (&w)[4]) {
  uint32_t w0, w1, w2, w3;
  asm("v_mul_hi_i32_i24_sdwa %0, %4, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %8, %21 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %12, %22 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %16, %23 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %0, %5, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %9, %21 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %13, %22 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %17, %23 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %0, %6, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %10, %21 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %14, %22 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %18, %23 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %0, %7, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %11, %21 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %15, %22 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %19, %23 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "s_nop 4"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
      : "v"(yc[0][0]), "v"(yc[0][1]), "v"(yc[0][2]), "v"(yc[0][3]), "v"(yc[1][0]), "v"(yc[1][1]),
        "v"(yc[1][2]), "v"(yc[1][3]), "v"(yc[2][0]), "v"(yc[2][1]), "v"(yc[2][2]), "v"(yc[2][3]),
        "v"(yc[3][0]), "v"(yc[3][1]), "v"(yc[3][2]), "v"(yc[3][3]), "v"(m[0]), "v"(m[1]), "v"(m[2]),
        "v"(m[3]));
  w[0] = w0;
  w[1] = w1;
  w[2] = w2;
  w[3] = w3;
}

// s_waitcnt immediate for vmcnt(n), other counters untouched (n < 64)
constexpr int pipe_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// ---------------------------------------------------------------- tiled GEMM
// Persistent workgroups of 2 WN waves, each SIMD running two waves: two
// 4-wave workgroups per CU (while one is in its epilogue or at a barrier, the
// other keeps the matrix core busy), or one 8-wave workgroup per CU (fewer
// operand bytes loaded per product).  A workgroup computes BM x BN output
// tiles, each wave a (BM/2) x (BN/WN) block: (BM/32) x (BN/(16 WN)) MFMA tiles
// of 16 x 16 with their accumulators in VGPRs.  Workgroup w takes the tiles
// order[w], order[w + G], ... of a table the host builds (see
// build_tile_order).  The k loop runs over 64-byte k-blocks through a ring of
// three LDS stages.  Every wave fills its share of a stage with direct
// global->LDS loads two steps ahead, waits for its own loads of the current
// stage, and one workgroup barrier per step makes every share visible (and
// frees the stage read in the step before for refilling).  The direct loads
// are written in asm: the compiler then does not treat them as LDS writes,
// which would make it wait for all of them before every operand read; the
// waits on them are the explicit ones below.  Rows are 64 bytes.
//
// A wave's W rows enter its MFMAs permuted: fragment a, A-row i is the
// wave's output column 16 (i / 4) + 4 a + i % 4.  Lane l of an MFMA result
// holds A-rows 4 (l / 16) .. + 3 of one B-column (an X row), so over the four
// fragments a lane holds the 16 adjacent output columns 16 (l / 16) .. + 15
// of one row: its 16 bytes go straight to memory.  The 16-byte chunk c of an
// X row r sits at position c ^ ((r >> 1) & 3), of a W row at position
// c ^ (((r >> 1) ^ (2 (r >> 4))) & 3): either way the b128 operand reads
// (eight lanes per LDS cycle) fall on distinct banks.
constexpr int kTileNS = 3;

template <int BM, int BN, int WN>
struct TileCfg {
  static constexpr int NW = 2 * WN;                         // waves: 2 along M, WN along N
  static constexpr int TMF = BM / 32, TNF = BN / (16 * WN);  // X and W fragments of a wave per k-block
  static constexpr int XB = BM * kStep, WB = BN * kStep, SB = XB + WB;
  static constexpr int XI = XB / (1024 * NW), WI = WB / (1024 * NW);  // 1 KB loads per wave and stage
  static constexpr int L = XI + WI;
};

// buffer_load_dwordx4 ... lds: lane l's 16 bytes at rsrc.base + voff go to LDS
// at m0 + 16 l (offsets at or past rsrc.num_records read as zeros).  The
// resource and the LDS address are wave-uniform by construction; the
// read-first-lane makes that visible to the compiler, which must place them
// in scalar registers.
// Entry t of the tile table through the scalar cache (a vector load here
// would make the compiler wait for every direct load in flight, since it
// counts only its own).  The wait is inside the asm, so the result registers
// are complete when the compiler first reads them.
__device__ __forceinline__ int2 tile_entry(const int2* order, int t) {
  const uint64_t base = (uint64_t)(uintptr_t)order;
  const uint32_t b0 = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t b1 = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  const uint32_t off = __builtin_amdgcn_readfirstlane((uint32_t)t * 8u);
  const uint64_t addr = ((uint64_t)b1 << 32) | b0;
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(addr), "s"(off));
  return int2{(int)(uint32_t)v, (int)(uint32_t)(v >> 32)};
}

__device__ __forceinline__ void dma16(v4i rsrc, uint32_t voff, uint32_t lds) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(l) : "memory");
}

template <int BM, int BN, int WN>
__global__ __launch_bounds__(128 * WN, 2) void iqlinear_tile(LinParams p) {
  typedef TileCfg<BM, BN, WN> C;
  constexpr int TMF = C::TMF, TNF = C::TNF, XI = C::XI, WI = C::WI, SB = C::SB, NW = C::NW;
  static_assert(XI * 1024 * NW == C::XB && WI * 1024 * NW == C::WB, "stage split");
  static_assert(C::L < 16, "vmcnt range");
  static_assert(TNF == 4, "one 16-byte output chunk per lane and block");
  static_assert(NW % 2 == 0, "W block parity is the wave's");
  __shared__ __attribute__((aligned(1024))) int8_t sSt[kTileNS * SB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int G = (int)gridDim.x;
  const int ntiles = p.ntiles;
  const int nkb = p.in_f / kStep;
  const uint32_t in_f = (uint32_t)p.in_f;
  const int t0 = blockIdx.x;
  if (t0 >= ntiles) return;  // uniform over the workgroup, before any barrier

  // ---- loads: this wave's 1 KB blocks (wave, wave + 4, ...) of a stage;
  //      block i holds rows 16 i .. 16 i + 15; lane l fills row 16 i + l / 4 at
  //      position l % 4, i.e. source chunk (l % 4) ^ ((l >> 3) & 3) of the
  //      k-block (the swizzle applied on the source side, since the load writes
  //      LDS in lane order); W rows also flip chunk bit 1 in odd blocks, i.e.
  //      in the odd waves' blocks.  The buffer resource starts at the tile's first
  //      row and k-block and ends with the operand's last row, so rows past the
  //      end read as zeros (the range check of a raw buffer covers the
  //      per-lane offset only).
  constexpr int NV = XI > WI ? XI : WI;
  uint32_t voff[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j)
    voff[j] = (uint32_t)(16 * (wave + NW * j) + (lane >> 2)) * in_f +
              16u * (uint32_t)((lane & 3) ^ ((lane >> 3) & 3));
  const uint32_t wflip = 32u * (uint32_t)(wave & 1);
  const uint32_t st0 = lds_addr(sSt);
  int lt = t0, lkb = 0, lst = 0;  // next (tile, k-block) to load, and its stage
  int2 ltile = tile_entry(p.order, lt);  // (row tile, column tile)
  auto issue = [&]() __attribute__((always_inline)) {
    if (lt >= ntiles) return;
    const uint32_t kofs = (uint32_t)lkb * kStep;
    const uint32_t x0 = (uint32_t)(ltile.x * BM) * in_f, w0 = (uint32_t)(ltile.y * BN) * in_f;
    const v4i xr = make_rsrc(p.x + x0 + kofs, (uint32_t)p.rows * in_f - x0 - kofs);
    const v4i wr = make_rsrc(p.w + w0 + kofs, (uint32_t)p.out_f * in_f - w0 - kofs);
    const uint32_t sb = st0 + (uint32_t)(lst * SB);
#pragma unroll
    for (int j = 0; j < XI; ++j) dma16(xr, voff[j], sb + 1024u * (uint32_t)(wave + NW * j));
#pragma unroll
    for (int j = 0; j < WI; ++j) dma16(wr, voff[j] ^ wflip, sb + (uint32_t)C::XB + 1024u * (uint32_t)(wave + NW * j));
    lst = lst == kTileNS - 1 ? 0 : lst + 1;
    if (++lkb == nkb) {
      lkb = 0;
      lt += G;
      if (lt < ntiles) ltile = tile_entry(p.order, lt);
    }
  };

  // prologue: stages 0 and 1.  The wait of a step counts the loads of the
  // next stage as the only younger operations; output stores issued in
  // between only make it wait longer (loads complete in order among
  // themselves), and a step with no next stage waits for everything.
  issue();
  issue();
  int cst = 0;  // stage of the current step
  const bool qkv = p.layout == IQLINEAR_QKV_HEADS;
  const bool wide_ep = !qkv || p.head_dim % 16 == 0;
  // this lane's W fragment rows (see the permutation above) and their chunk
  // positions, as byte offsets in a stage's W part
  int wofs[TNF];
#pragma unroll
  for (int a = 0; a < TNF; ++a) {
    const int r = 16 * TNF * wn + 16 * (li >> 2) + 4 * a + (li & 3);
    wofs[a] = r * kStep + 16 * (g ^ (((r >> 1) ^ (2 * (r >> 4))) & 3));
  }

  for (int t = t0; t < ntiles; t += G) {
    const int2 tile = tile_entry(p.order, t);
    const bool last = t + G >= ntiles;
    v4i acc[TNF][TMF];
    // one k-step: wait for this wave's loads of the stage, barrier, read the
    // operands and multiply (the first step of a tile starts the accumulators
    // from zero); the refill of the stage read in the previous step goes out
    // after the first half of the MFMAs, so that the wave does not stall on
    // issuing loads while its matrix core has no work queued
    auto kstep = [&](int kb, auto firstc) __attribute__((always_inline)) {
      constexpr bool first = decltype(firstc)::value;
      if (kb + 1 < nkb || !last)
        __builtin_amdgcn_s_waitcnt(pipe_vmcnt(C::L));
      else
        __builtin_amdgcn_s_waitcnt(pipe_vmcnt(0));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      const int8_t* const sx = sSt + cst * SB;
      const int8_t* const sw = sx + C::XB;
      // X fragment rows 16 f + li, chunk g at position g ^ ((li >> 1) & 3)
      const int cpos = 16 * (g ^ ((li >> 1) & 3));
      v4i fx[TMF], fw[TNF];
#pragma unroll
      for (int a = 0; a < TNF; ++a) fw[a] = *(const v4i*)(sw + wofs[a]);
#pragma unroll
      for (int b = 0; b < TMF; ++b) fx[b] = *(const v4i*)(sx + (16 * (TMF * wm + b) + li) * kStep + cpos);
#pragma unroll
      for (int b = 0; b < TMF / 2; ++b)
#pragma unroll
        for (int a = 0; a < TNF; ++a)
          acc[a][b] = mfma64(fw[a], fx[b], first ? v4i{0, 0, 0, 0} : acc[a][b]);
      __builtin_amdgcn_sched_barrier(0);
      issue();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = TMF / 2; b < TMF; ++b)
#pragma unroll
        for (int a = 0; a < TNF; ++a)
          acc[a][b] = mfma64(fw[a], fx[b], first ? v4i{0, 0, 0, 0} : acc[a][b]);
      cst = cst == kTileNS - 1 ? 0 : cst + 1;
    };
    kstep(0, std::true_type());
    for (int kb = 1; kb < nkb; ++kb) kstep(kb, std::false_type());

    const int m_w = tile.x * BM + 16 * TMF * wm, n_w = tile.y * BN + 16 * TNF * wn;
    if (!wide_ep) {
      // head_dim % 16 != 0: each lane stores its 4-byte words directly
      if (p.w24)
        store_tile<TMF, TNF, true>(p, acc, m_w + li, n_w + 16 * g);
      else
        store_tile<TMF, TNF, false>(p, acc, m_w + li, n_w + 16 * g);
      continue;
    }
    // epilogue: in block b the lane holds output columns n .. n + 15 of row
    // m0 + 16 b, all under one pair; requantised, they leave as one 16-byte
    // store.  The pair's window constants are selected once per tile and kept
    // in VGPRs (the clamps and multiplies read them as vector operands).
    const int n = n_w + 16 * g;
    int which;
    const int cofs = col_part(p, qkv, n, which);
    int32_t lo = pick3(which, p.ylo[0], p.ylo[1], p.ylo[2]);
    int32_t hi = pick3(which, p.yhi[0], p.yhi[1], p.yhi[2]);
    int32_t mm = pick3(which, p.bm24[0], p.bm24[1], p.bm24[2]);
    int8_t* outp = pick3(which, p.out[0], p.out[1], p.out[2]) + cofs;
    asm("" : "+v"(lo), "+v"(hi), "+v"(mm), "+v"(outp));
    typedef __attribute__((address_space(1))) int8_t gint8;
    gint8* const out = (gint8*)outp;
    const int32_t mm4[4] = {mm, mm, mm, mm};
    const bool col_ok = n < p.out_f;
    // The lane's row in block b is m0 + 16 b: its offset ro is advanced by 16
    // rows per block (in the head-split layout, a row step that crosses into
    // the next image also skips the other heads' rows; with at least 16
    // tokens per image one block crosses at most once).
    const int m0 = m_w + li;
    int64_t ro = row_offset(p, qkv, m0);
    int tk = qkv ? m0 - div_seq(p, m0) * p.seq_len : 0;  // token of row m0 + 16 b
    const bool inc = !qkv || p.seq_len >= 16;
    const int64_t step16 = 16 * (int64_t)(qkv ? p.head_dim : p.out_f);
    const int64_t wrap = qkv ? (int64_t)(p.heads - 1) * p.seq_len * p.head_dim : 0;
    // The window path's clamps are asm (the compiler would emit min and max:
    // it cannot tell that the bounds are ordered), and the compiler inserts no
    // wait states before an asm read of an MFMA result: the last MFMA's result
    // is complete at most 19 wait states after it issues; the nops give 24.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < TMF; ++b) {
      uint32_t w[TNF];
      if (p.w24) {
        int32_t yc[TNF][4];
#pragma unroll
        for (int a = 0; a < TNF; ++a)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            asm("v_med3_i32 %0, %1, %2, %3" : "=v"(yc[a][r]) : "v"(acc[a][b][r]), "v"(lo), "v"(hi));
        w24_pack4x4(yc, mm4, w);
      } else {
#pragma unroll
        for (int a = 0; a < TNF; ++a) w[a] = requant4<false>(p, which, acc[a][b]);
      }
      const int m = m0 + 16 * b;
      if (col_ok && m < p.rows)
        *(__attribute__((address_space(1))) v4i*)(out + (inc ? ro : row_offset(p, qkv, m))) =
            v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      tk += 16;
      const bool crosses = qkv && tk >= p.seq_len;
      tk = crosses ? tk - p.seq_len : tk;
      ro += step16 + (crosses ? wrap : 0);
    }
  }
}

}  // namespace
}  // namespace iqattn

using namespace iqattn;

struct iqlinear_ctx {
  LinParams lp;
  int device;
  unsigned grid;  // persistent grid
  int tile;       // 0: 256 x 128 tiles, 1: 128 x 128, 2: 256 x 256 (8 waves)
  int2* order;    // device copy of the tile table
};

namespace {

// The tile table: workgroup w runs on XCD w % 8 (workgroups are dealt to the
// eight XCDs in turn) and takes the table entries w, w + G, w + 2 G, ...  With
// G a multiple of 8, entry t is computed on XCD t % 8, so the entries
// t = x + 8 u are XCD x's tiles, in the order u in which its workgroups take
// them.  Each XCD gets the row tiles r with r % 8 == x, all column tiles of a
// row tile in a row (so a row tile's X rows reach that XCD's L2 once and are
// reused from there), up to its share of the table; tiles beyond an XCD's
// share go, in order, to the XCDs with fewer tiles of their own.  The shares
// differ by at most one, so every workgroup takes the same number of tiles up
// to one.
std::vector<int2> build_tile_order(int ntm, int ntn, unsigned grid) {
  const int64_t n = (int64_t)ntm * ntn;
  std::vector<int2> order((size_t)n);
  if (grid % 8 != 0) {  // small grids (one tile per workgroup): any order
    for (int64_t t = 0; t < n; ++t) order[(size_t)t] = int2{(int)(t / ntn), (int)(t % ntn)};
    return order;
  }
  std::vector<std::vector<int2>> xt(8);
  std::vector<int2> spill;
  for (int x = 0; x < 8; ++x) {
    const int64_t share = n / 8 + (x < n % 8 ? 1 : 0);
    for (int r = x; r < ntm; r += 8)
      for (int c = 0; c < ntn; ++c) {
        if ((int64_t)xt[x].size() < share)
          xt[x].push_back(int2{r, c});
        else
          spill.push_back(int2{r, c});
      }
  }
  size_t k = 0;
  for (int x = 0; x < 8; ++x) {
    const int64_t share = n / 8 + (x < n % 8 ? 1 : 0);
    while ((int64_t)xt[x].size() < share) xt[x].push_back(spill[k++]);
    for (size_t u = 0; u < xt[x].size(); ++u) order[(size_t)x + 8 * u] = xt[x][u];
  }
  return order;
}

}  // namespace

extern "C" int iqlinear_create(const iqlinear_params* p, iqlinear_ctx** out) {
  if (!out) return IQATTN_E_NULL;
  *out = NULL;
  if (!p) return IQATTN_E_NULL;
  if (p->rows < 0) return IQATTN_E_SHAPE;
  if (p->in_features < kStep || p->in_features % kStep) return IQATTN_E_SHAPE;
  if (p->out_features < 16 || p->out_features % 16) return IQATTN_E_SHAPE;
  if ((int64_t)p->rows * p->in_features > INT32_MAX ||
      (int64_t)p->out_features * p->in_features > INT32_MAX)
    return IQATTN_E_SHAPE;
  int npairs = 1;
  if (p->layout == IQLINEAR_QKV_HEADS) {
    npairs = 3;
    if (p->batch < 1 || p->seq_len < 1 || p->heads < 1 || p->head_dim < 4 || p->head_dim % 4)
      return IQATTN_E_SHAPE;
    if ((int64_t)p->batch * p->seq_len != p->rows) return IQATTN_E_SHAPE;
    if ((int64_t)3 * p->heads * p->head_dim != p->out_features) return IQATTN_E_SHAPE;
    if ((p->heads * p->head_dim) % 16) return IQATTN_E_SHAPE;
  } else if (p->layout != IQLINEAR_PLAIN) {
    return IQATTN_E_INVAL;
  }
  for (int i = 0; i < npairs; ++i) {
    if (p->b[i] < 1) return IQATTN_E_INVAL;
    if (p->c[i] < 0 || p->c[i] > 62) return IQATTN_E_INVAL;
  }
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return IQATTN_E_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return IQATTN_E_DEVICE;
  iqlinear_ctx* c = (iqlinear_ctx*)calloc(1, sizeof(iqlinear_ctx));
  if (!c) return IQATTN_E_ALLOC;
  c->device = dev;
  LinParams& lp = c->lp;
  lp.rows = p->rows;
  lp.in_f = p->in_features;
  lp.out_f = p->out_features;
  lp.layout = p->layout;
  lp.seq_len = p->seq_len;
  lp.heads = p->heads;
  lp.head_dim = p->head_dim;
  lp.width = p->heads * p->head_dim;
  lp.w24 = 1;
  for (int i = 0; i < 3; ++i) {
    const int k = i < npairs ? i : 0;
    const int64_t b = p->b[k];
    const int c = p->c[k];
    lp.b[i] = (int32_t)b;
    lp.c[i] = c;
    const bool fast = c >= 1 && c <= 32 && (b << (32 - c)) < ((int64_t)1 << 31);
    lp.bm[i] = fast ? (int32_t)(b << (32 - c)) : 0;
    // window path: bm24 = b 2^(32 - c) < 2^23 (so b <= 2^c) and the window
    // [ceil(-127 2^c / b), floor((128 2^c - 1) / b)] inside [-2^23, 2^23 - 1]
    bool w = c <= 32 && (b << (32 - c)) < ((int64_t)1 << 23);
    if (w) {
      const int64_t lo = -((127 * ((int64_t)1 << c)) / b);
      const int64_t hi = (128 * ((int64_t)1 << c) - 1) / b;
      w = lo >= -((int64_t)1 << 23) && hi <= ((int64_t)1 << 23) - 1;
      lp.ylo[i] = w ? (int32_t)lo : 0;
      lp.yhi[i] = w ? (int32_t)hi : 0;
      lp.bm24[i] = w ? (int32_t)(b << (32 - c)) : 0;
    }
    if (!w) lp.w24 = 0;
  }
  // floor(m / seq_len) for the head split: l = ceil(log2 seq_len), magic =
  // floor(2^32 (2^l - seq_len) / seq_len) + 1 (below 2^32 since 2^l - seq_len
  // < seq_len); exact for 0 <= m < 2^31
  lp.seq_magic = 0;
  lp.seq_shift = 0;
  if (p->layout == IQLINEAR_QKV_HEADS) {
    const uint64_t d = (uint64_t)p->seq_len;
    int l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    lp.seq_magic = (uint32_t)(((((uint64_t)1 << l) - d) << 32) / d + 1);
    lp.seq_shift = l;
  }
  // persistent grid; the tile shape with the least work on the busiest CU:
  // the most tiles a CU takes (the table balances them to within one) times
  // the tile's size in 128 x 128 units times a measured cost per unit (the
  // 8-wave 256 x 256 tile moves the fewest operand bytes per product, the
  // 128 x 128 tile's 64 x 64 wave tiles the most)
  {
    const int64_t cus = prop.multiProcessorCount;
    const int64_t rows = p->rows, n128 = (p->out_features + 127) / 128, n256 = (p->out_features + 255) / 256;
    const int64_t t[3] = {(rows + 255) / 256 * n128, (rows + 127) / 128 * n128, (rows + 255) / 256 * n256};
    const int64_t units[3] = {2, 1, 4}, per_unit[3] = {100, 135, 80};
    int best = 0;
    int64_t best_cost = 0;
    for (int k = 0; k < 3; ++k) {
      const int64_t cost = (t[k] + cus - 1) / cus * units[k] * per_unit[k];
      if (k == 0 || cost < best_cost) {
        best = k;
        best_cost = cost;
      }
    }
    c->tile = best;
    const int64_t tiles = t[best];
    const int64_t slots = best == 2 ? cus : 2 * cus;  // one 8-wave or two 4-wave workgroups per CU
    if (tiles > INT32_MAX / 2) {
      free(c);
      return IQATTN_E_SHAPE;
    }
    c->grid = (unsigned)(tiles < slots ? (tiles > 0 ? tiles : 1) : slots);
    lp.ntiles = (int32_t)tiles;
  }
  if (lp.ntiles > 0) {
    const int bm = c->tile == 1 ? 128 : 256, bn = c->tile == 2 ? 256 : 128;
    const std::vector<int2> order =
        build_tile_order((p->rows + bm - 1) / bm, (p->out_features + bn - 1) / bn, c->grid);
    if (hipMalloc((void**)&c->order, order.size() * sizeof(int2)) != hipSuccess) {
      free(c);
      return IQATTN_E_ALLOC;
    }
    if (hipMemcpy(c->order, order.data(), order.size() * sizeof(int2), hipMemcpyHostToDevice) !=
        hipSuccess) {
      (void)hipFree(c->order);
      free(c);
      return IQATTN_E_DEVICE;
    }
  }
  lp.order = c->order;
  *out = c;
  return IQATTN_OK;
}

extern "C" int iqlinear_forward(iqlinear_ctx* c, const int8_t* x, const int8_t* w, int8_t* out0,
                                int8_t* out1, int8_t* out2, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  if (c->lp.rows == 0) return IQATTN_OK;
  const bool qkv = c->lp.layout == IQLINEAR_QKV_HEADS;
  if (!x || !w || !out0 || (qkv && (!out1 || !out2))) return IQATTN_E_NULL;
  uintptr_t al = (uintptr_t)x | (uintptr_t)w | (uintptr_t)out0;
  if (qkv) al |= (uintptr_t)out1 | (uintptr_t)out2;
  if (al & 15u) return IQATTN_E_ALIGN;
  LinParams lp = c->lp;
  lp.x = x;
  lp.w = w;
  lp.out[0] = out0;
  lp.out[1] = qkv ? out1 : out0;
  lp.out[2] = qkv ? out2 : out0;
  if (c->tile == 1)
    hipLaunchKernelGGL((iqlinear_tile<128, 128, 2>), dim3(c->grid), dim3(256), 0, (hipStream_t)hip_stream, lp);
  else if (c->tile == 2)
    hipLaunchKernelGGL((iqlinear_tile<256, 256, 4>), dim3(c->grid), dim3(512), 0, (hipStream_t)hip_stream, lp);
  else
    hipLaunchKernelGGL((iqlinear_tile<256, 128, 2>), dim3(c->grid), dim3(256), 0, (hipStream_t)hip_stream, lp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqlinear launch");
  return IQATTN_OK;
}

extern "C" int iqlinear_destroy(iqlinear_ctx* c) {
  if (!c) return IQATTN_OK;
  if (c->order) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipSetDevice(c->device);
    (void)hipFree(c->order);
    (void)hipSetDevice(dev);
  }
  free(c);
  return IQATTN_OK;
}
