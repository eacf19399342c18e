// iqlinear.hip -- integer-only int8 linear layer: Y = requant(X W^T) with a
// dyadic (b, c) per output tensor, fused into the GEMM epilogue.
//
// Method passage: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" (integer product, then (b * acc) >> c to int8); sec. 3.1
// (the MSA projections).
//
// Kernel (iqlinear_pipe below): persistent workgroups, one per CU, of 4 MFMA
// waves and 4 loader waves.  Each workgroup computes 128 x 128 output tiles as
// Y^T = W . X^T with v_mfma_i32_16x16x64_i8, so a lane ends
// with 4 adjacent output columns of one row (one 4-byte store after the fused
// requantisation, straight into the head-split layout when asked).  Each
// compute wave owns a quarter of the tile (64 x 64: 16 MFMA tiles, 64
// accumulators).  The k loop runs through a ring of LDS stages of 128 k-bytes a
// row (whole cache lines per load request), filled by the loader waves with
// direct global->LDS loads; the 16-byte chunks of a 128-byte LDS row are
// XOR-swizzled by (row >> 1) & 7, which makes the b128 operand reads of 16
// rows bank-conflict free.
#include "iqattn_dev.h"
#include "iqattn.h"
#include "iqlinear.h"

#include <stdlib.h>
#include <string.h>

#include <type_traits>

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
  uint32_t* status;    // context status word: bit 0 loader, bit 1 compute wave gave up
  int32_t spin_limit;  // polls of a bounded wait before it gives up
};

__device__ __forceinline__ void lin_giveup(const LinParams& p, uint32_t bit) {
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(p.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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

// Epilogue of one wave's TN x TM accumulator tiles: acc[a][b][r] is output
// column n + 16 a + r of row m + 16 b; requantised, packed to 4 bytes and
// stored.  Rows past the end are skipped.
template <int TM, int TN, bool W24>
__device__ __forceinline__ void store_tile(const LinParams& p, const v4i (&acc)[TN][TM], int m_base,
                                           int n_base) {
  const bool qkv = p.layout == IQLINEAR_QKV_HEADS;
  int64_t rofs[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b) rofs[b] = row_offset(p, qkv, m_base + 16 * b);
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n_base + 16 * a;
    if (n >= p.out_f) continue;  // out is a multiple of 16: the whole 16-column tile
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

// The same epilogue through a wave-private LDS block: the requantised bytes of
// the wave's (16 TM) x (16 TN) block go to LDS rows of kEpPitch bytes (the
// pitch keeps the 4-byte writes of 16 rows bank-conflict free), then each lane
// stores whole 16-byte row chunks (4 x fewer store instructions, contiguous
// 16-byte writes).  Needs 16-column groups that stay inside one output row
// segment: always for the plain layout, head_dim % 16 == 0 for the head split.
// The pair of a 16-column group is wave-uniform (n_w is), so it is picked from
// scalar registers; the output tensor of a lane's chunk is picked by selects.
constexpr int kEpPitch = 16 * 4 + 16;  // (16 TN = 64) bytes + 16 of padding

// Window path, four 4-column blocks at once: byte r of word b is
// floor(yc[b][r] m / 2^32) (v_mul_hi_i32_i24 with an SDWA byte destination,
// the clamped accumulator and m both within 24 signed bits), written
// byte-major over the four words: a write that keeps the other bytes reads
// the old word without an interlock, so two such writes to one word need
// other instructions between them; the closing s_nop covers the first later
// reader.  The clamps before it are plain code, the first readers of the MFMA
// results.
__device__ __forceinline__ void w24_pack16(const int32_t (&yc)[4][4], int32_t m, uint32_t (&w)[4]) {
  uint32_t w0, w1, w2, w3;
  asm("v_mul_hi_i32_i24_sdwa %0, %4, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %8, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %12, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %16, %20 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %0, %5, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %9, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %13, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %17, %20 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %0, %6, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %10, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %14, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %18, %20 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %0, %7, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %1, %11, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %2, %15, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "v_mul_hi_i32_i24_sdwa %3, %19, %20 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD\n\t"
      "s_nop 4"
      : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
      : "v"(yc[0][0]), "v"(yc[0][1]), "v"(yc[0][2]), "v"(yc[0][3]), "v"(yc[1][0]), "v"(yc[1][1]),
        "v"(yc[1][2]), "v"(yc[1][3]), "v"(yc[2][0]), "v"(yc[2][1]), "v"(yc[2][2]), "v"(yc[2][3]),
        "v"(yc[3][0]), "v"(yc[3][1]), "v"(yc[3][2]), "v"(yc[3][3]), "v"(m));
  w[0] = w0;
  w[1] = w1;
  w[2] = w2;
  w[3] = w3;
}

template <int TM, int TN, bool W24>
__device__ __forceinline__ void store_tile_lds(const LinParams& p, const v4i (&acc)[TN][TM],
                                               int8_t* scr, int m_w, int n_w, int li, int g,
                                               int lane) {
  static_assert(16 * TN + 16 == kEpPitch, "pitch");
  static_assert(64 % TN == 0, "a lane's chunks share one column group");
  const bool qkv = p.layout == IQLINEAR_QKV_HEADS;
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n_w + 16 * a;
    const int which = qkv ? (n >= p.width) + (n >= 2 * p.width) : 0;
    if constexpr (W24 && TM == 4) {
      const int32_t lo = pick3(which, p.ylo[0], p.ylo[1], p.ylo[2]);
      const int32_t hi = pick3(which, p.yhi[0], p.yhi[1], p.yhi[2]);
      const int32_t m = pick3(which, p.bm24[0], p.bm24[1], p.bm24[2]);
      int32_t yc[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          yc[b][r] = __builtin_elementwise_max(__builtin_elementwise_min(acc[a][b][r], hi), lo);
      uint32_t w[4];
      w24_pack16(yc, m, w);
#pragma unroll
      for (int b = 0; b < 4; ++b) *(uint32_t*)(scr + (16 * b + li) * kEpPitch + 16 * a + 4 * g) = w[b];
    } else {
#pragma unroll
      for (int b = 0; b < TM; ++b)
        *(uint32_t*)(scr + (16 * b + li) * kEpPitch + 16 * a + 4 * g) = requant4<W24>(p, which, acc[a][b]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block is in LDS (one wave: in order)
  // lane chunk k: row lane / TN + (64 / TN) k of the block, column group lane % TN
  const int cg = lane % TN, n = n_w + 16 * cg;
  int which;
  const int cofs = col_part(p, qkv, n, which);
  int8_t* const out = pick3(which, p.out[0], p.out[1], p.out[2]) + cofs;
  const bool col_ok = n < p.out_f;
#pragma unroll
  for (int k = 0; k < (16 * TM * TN) / 64; ++k) {
    const int row = lane / TN + (64 / TN) * k, m = m_w + row;
    const v4i v = *(const v4i*)(scr + row * kEpPitch + 16 * cg);
    if (m < p.rows && col_ok) *(v4i*)(out + row_offset(p, qkv, m)) = v;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the block is reused
}

// ---------------------------------------------------------------- pipelined GEMM
// Persistent workgroups (one per CU) of 4 compute waves and kPipeNL loader
// waves.  The loaders stream 128-byte k-slices of a tile's X rows and W rows
// (two 64-byte MFMA k-blocks) into a ring of kPipeNS LDS stages with direct
// global->LDS loads, each loader wave a quarter of every stage (the swizzle is
// applied on the source side: lane l of a 1 KB block fills LDS bytes
// [1024 i + 16 l, +16) = (row, chunk position cp) from source chunk
// cp ^ ((row >> 1) & 7)), kPipeLag stages in flight per wave, running ahead
// across tile boundaries.  Monotonic LDS counters per stage slot: ready[b]
// (loader waves that finished a fill), done[b] (compute waves that finished
// reading it).  Compute waves read a k-block's fragments while the MFMAs of the
// previous one run.  Tiles are dealt XCD-aware: the workgroups of one XCD
// (every 8th) take all column tiles of one block of X rows in turn, so those
// rows reach that XCD's L2 once.
constexpr int kPipeKB = 128;  // k bytes of a row per stage: whole cache lines per request
constexpr int kPipeNS = 4;
constexpr int kPipeLag = 2;
constexpr int kPipeNL = 4;
constexpr int kPipeThreads = 64 * (4 + kPipeNL);

constexpr int pipe_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

template <int BM, int BN>
struct PipeCfg {
  static constexpr int TM = BM / 32, TN = BN / 32;  // 16 x 16 tiles per wave (2 x 2 waves)
  static constexpr int KB = kPipeKB, NCH = KB / 16, KPS = KB / kStep;  // chunks, k-blocks per stage
  static constexpr int XB = BM * KB, WB = BN * KB, SB = XB + WB;
  static constexpr int XI = XB / 1024 / kPipeNL, WI = WB / 1024 / kPipeNL;  // loads per loader wave
  static constexpr int LDS = kPipeNS * SB + 64 + 4 * (16 * TM) * kEpPitch;  // + epilogue blocks
};

__device__ __forceinline__ void pipe_decode(int t, int ntn, int& tm, int& tn) {
  const int x = t & 7, r = t >> 3, q = r / ntn;
  tm = q * 8 + x;
  tn = r - q * ntn;
}

template <int BM, int BN>
__global__ __launch_bounds__(kPipeThreads) void iqlinear_pipe(LinParams p) {
  typedef PipeCfg<BM, BN> C;
  constexpr int TM = C::TM, TN = C::TN, NS = kPipeNS, NL = kPipeNL;
  static_assert((C::XI + C::WI) * kPipeLag < 64, "vmcnt range");
  static_assert(C::XI * NL * 1024 == C::XB && C::WI * NL * 1024 == C::WB, "stage split");
  static_assert(kPipeLag < NS, "ring depth");
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  int* const ready = (int*)(smem + NS * C::SB);
  int* const done = ready + NS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x;
  const int ntm = (p.rows + BM - 1) / BM, ntn = (p.out_f + BN - 1) / BN;
  const int total_t = 8 * ntn * ((ntm + 7) / 8);
  constexpr int KB = C::KB, NCH = C::NCH, KPS = C::KPS;
  const int nkb = p.in_f / kStep;              // 64-byte k-blocks per tile
  const int nks = (nkb + KPS - 1) / KPS;       // stages per tile
  if (tid < NS) {
    ready[tid] = 0;
    done[tid] = 0;
  }
  __syncthreads();
  const uint32_t sm0 = lds_addr(smem);

  if (wave >= 4) {
    // ---- loader wave wl: 1 KB blocks wl, wl + NL, ... of each stage's X and W parts
    const int wl = wave - 4;
    const v4i xr = make_rsrc(p.x, (uint32_t)(p.rows * p.in_f));
    const v4i wr = make_rsrc(p.w, (uint32_t)(p.out_f * p.in_f));
    auto mark = [&](int step) {
      if (lane == 0)
        __hip_atomic_fetch_add(&ready[step % NS], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int s = 0;
    for (int t = blockIdx.x; t < total_t; t += G) {
      int tm, tn;
      pipe_decode(t, ntn, tm, tn);
      if (tm >= ntm) continue;
      const int m0 = tm * BM, n0 = tn * BN;
      for (int ks = 0; ks < nks; ++ks, ++s) {
        const int b = s % NS;
        if (s >= NS) {  // the slot's previous step has been read by every compute wave
          const int need = 4 * (s / NS);
          int spins = 0;
          while (__hip_atomic_load(&done[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
            if (++spins > p.spin_limit) {
              lin_giveup(p, 1u);
              __builtin_amdgcn_s_waitcnt(0);  // no direct loads left in flight
              return;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        const uint32_t sb = sm0 + b * C::SB;
#pragma unroll
        for (int j = 0; j < C::XI; ++j) {
          const int i = wl + NL * j;
          const int o = 1024 * i + 16 * lane, row = o / KB, cp = (o >> 4) & (NCH - 1);
          raw_buffer_load_lds(xr, (lds_u32w*)(uintptr_t)(sb + 1024 * i), 16,
                              (m0 + row) * p.in_f + KB * ks + 16 * (cp ^ ((row >> 1) & (NCH - 1))), 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < C::WI; ++j) {
          const int i = wl + NL * j;
          const int o = 1024 * i + 16 * lane, row = o / KB, cp = (o >> 4) & (NCH - 1);
          raw_buffer_load_lds(wr, (lds_u32w*)(uintptr_t)(sb + C::XB + 1024 * i), 16,
                              (n0 + row) * p.in_f + KB * ks + 16 * (cp ^ ((row >> 1) & (NCH - 1))), 0, 0, 0);
        }
        // this wave's share of the stage issued kPipeLag steps ago has landed
        if (s >= kPipeLag) {
          __builtin_amdgcn_s_waitcnt(pipe_vmcnt(kPipeLag * (C::XI + C::WI)));
          mark(s - kPipeLag);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(pipe_vmcnt(0));
    for (int q = s - kPipeLag; q < s; ++q)
      if (q >= 0) mark(q);
    return;
  }

  // ---- compute waves: wave (wm, wn) owns rows 16 (TM wm + b) + li and columns
  //      16 (TN wn + a) + 4 g + r of the tile
  const int wm = wave & 1, wn = wave >> 1;
  int8_t* const ep_scr = smem + NS * C::SB + 64 + wave * (16 * TM) * kEpPitch;
  const bool wide_ep = p.layout != IQLINEAR_QKV_HEADS || p.head_dim % 16 == 0;
  auto wait_ready = [&](int step) -> bool {
    const int need = NL * (step / NS + 1);
    int spins = 0;
    while (__hip_atomic_load(&ready[step % NS], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
      if (++spins > p.spin_limit) {
        lin_giveup(p, 2u);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };
  // operand fragments of k-block j of a stage: row r, chunk (4 j + g) ^ swizzle(r)
  auto lds_off = [&](int r, int j) { return r * KB + 16 * ((4 * j + g) ^ ((r >> 1) & (NCH - 1))); };
  typedef std::integral_constant<int, 0> J0;
  typedef std::integral_constant<int, 1> J1;
  auto read_frags = [&](int step, auto jc, v4i (&fx)[TM], v4i (&fw)[TN]) {
    constexpr int j = decltype(jc)::value;
    const int8_t* sb = smem + (step % NS) * C::SB;
#pragma unroll
    for (int b = 0; b < TM; ++b) fx[b] = *(const v4i*)(sb + lds_off(16 * (TM * wm + b) + li, j));
#pragma unroll
    for (int a = 0; a < TN; ++a) fw[a] = *(const v4i*)(sb + C::XB + lds_off(16 * (TN * wn + a) + li, j));
  };
  auto signal_done = [&](int step) {
    if (lane == 0) __hip_atomic_fetch_add(&done[step % NS], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  int s = 0;
  for (int t = blockIdx.x; t < total_t; t += G) {
    int tm, tn;
    pipe_decode(t, ntn, tm, tn);
    if (tm >= ntm) continue;
    const int m0 = tm * BM, n0 = tn * BN;
    v4i acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    // per stage: block 1's fragments are read while block 0's MFMAs run, the
    // stage is released once they are in registers, and the next stage's
    // block 0 is read while block 1's MFMAs run.  The MFMAs of the loop body
    // are unconditional (a conditional accumulator update makes the compiler
    // copy every accumulator register each iteration); an odd k-block count
    // ends with a one-block stage after the loop.
    v4i fx0[TM], fw0[TN], fx1[TM], fw1[TN];
    if (!wait_ready(s)) return;
    read_frags(s, J0(), fx0, fw0);
    const int nfull = nkb >> 1;  // stages holding two k-blocks
    for (int st = 0; st < nfull; ++st) {
      read_frags(s + st, J1(), fx1, fw1);
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma64(fw0[a], fx0[b], acc[a][b]);
      // the MFMAs are issued before the wait (the scheduler would otherwise
      // hoist the wait above them and expose the fragment reads' latency)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every fragment of the stage is in registers
      signal_done(s + st);
      if (st + 1 < nks) {
        if (!wait_ready(s + st + 1)) return;
        read_frags(s + st + 1, J0(), fx0, fw0);
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma64(fw1[a], fx1[b], acc[a][b]);
    }
    if (nkb & 1) {  // the last stage's single k-block is in fx0, fw0
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma64(fw0[a], fx0[b], acc[a][b]);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      signal_done(s + nfull);
    }
    s += nks;
    if (wide_ep) {
      if (p.w24)
        store_tile_lds<TM, TN, true>(p, acc, ep_scr, m0 + 16 * TM * wm, n0 + 16 * TN * wn, li, g, lane);
      else
        store_tile_lds<TM, TN, false>(p, acc, ep_scr, m0 + 16 * TM * wm, n0 + 16 * TN * wn, li, g, lane);
    } else {
      if (p.w24)
        store_tile<TM, TN, true>(p, acc, m0 + 16 * TM * wm + li, n0 + 16 * TN * wn + 4 * g);
      else
        store_tile<TM, TN, false>(p, acc, m0 + 16 * TM * wm + li, n0 + 16 * TN * wn + 4 * g);
    }
  }
}

}  // namespace
}  // namespace iqattn

using namespace iqattn;

struct iqlinear_ctx {
  LinParams lp;
  int device;
  unsigned grid;  // persistent grid of the pipelined kernel
  uint32_t* status;
};

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
  // persistent kernels: one workgroup per CU, 128 x 128 tiles
  {
    const int cus = prop.multiProcessorCount;
    const int64_t tiles = ((int64_t)p->rows + 127) / 128 * ((p->out_features + 127) / 128);
    c->grid = (unsigned)(tiles < cus ? (tiles > 0 ? tiles : 1) : cus);
    if (hipFuncSetAttribute((const void*)&iqlinear_pipe<128, 128>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            PipeCfg<128, 128>::LDS) != hipSuccess) {
      free(c);
      return IQATTN_E_DEVICE;
    }
  }
  if (hipMalloc((void**)&c->status, sizeof(uint32_t)) != hipSuccess) {
    free(c);
    return IQATTN_E_ALLOC;
  }
  if (hipMemset(c->status, 0, sizeof(uint32_t)) != hipSuccess) {
    (void)hipFree(c->status);
    free(c);
    return IQATTN_E_DEVICE;
  }
  lp.status = c->status;
  lp.spin_limit = 1 << 22;  // polls of about 64 clocks: only a broken invariant gives up
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
  constexpr int lds = PipeCfg<128, 128>::LDS;
  hipLaunchKernelGGL((iqlinear_pipe<128, 128>), dim3(c->grid), dim3(kPipeThreads), lds,
                     (hipStream_t)hip_stream, lp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqlinear launch");
  return IQATTN_OK;
}

extern "C" int iqlinear_check(iqlinear_ctx* c, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  hipError_t e = hipStreamSynchronize((hipStream_t)hip_stream);
  if (e != hipSuccess) return set_hip_error(e, "iqlinear_check synchronize");
  uint32_t word = 0;
  if ((e = hipMemcpy(&word, c->status, sizeof(word), hipMemcpyDeviceToHost)) != hipSuccess)
    return set_hip_error(e, "iqlinear_check read");
  if (word == 0) return IQATTN_OK;
  const uint32_t zero = 0;
  if ((e = hipMemcpy(c->status, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess)
    return set_hip_error(e, "iqlinear_check clear");
  return IQATTN_E_INCOMPLETE;
}

extern "C" int iqlinear_set_spin_limit(iqlinear_ctx* c, int32_t polls) {
  if (!c) return IQATTN_E_NULL;
  if (polls < 1) return IQATTN_E_INVAL;
  c->lp.spin_limit = polls;
  return IQATTN_OK;
}

extern "C" int iqlinear_destroy(iqlinear_ctx* c) {
  if (!c) return IQATTN_OK;
  if (c->status) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipSetDevice(c->device);
    (void)hipFree(c->status);
    (void)hipSetDevice(dev);
  }
  free(c);
  return IQATTN_OK;
}
