// iqattn_fast.hip -- fused integer-only attention specialised on the number of
// 16-key tiles (KT, so N in (16(KT-1), 16 KT]) for the parameter ranges in
// which every step fits 32-bit VALU arithmetic (the host checks them).
//
// Work distribution: a persistent grid (as many workgroups as fit on the chip)
// walks a list of work items -- whole heads, then the heads of a last partial
// round split into quarter heads.  K and V of a head reach LDS through direct
// global->LDS loads (buffer_load ... lds, no registers); with two buffers the
// next item's loads run while the current item is computed.
//
// Front end, per 16-query tile of a wave (shared by every variant):
//   S^T = K . Q^T   one int8 MFMA per 16-key tile, accumulators in VGPRs;
//   pass 1          row max (plain max: the first reads of MFMA results);
//   pass 2          v_mul_hi_i32 (requantisation), v_mad_i32_i24 + v_med3_i32
//                   (saturation folded into the exponential-table address),
//                   one ds_read_b32, one add;  f = floor(2^M / sum) from a
//                   reciprocal estimate and an exact one-step fix-up.
// Back ends:
//   Shiftmax        P = (e f) >> (M - k_out + 1) as one v_mul_hi_u32 per logit,
//                   packed to int8, O^T = V^T . P^T by MFMA;
//   LIS, VALU       shift w = F - code per logit, then sum_j V_j << w_ij with one
//                   v_lshl_add_u32 per (query, key, feature) -- the BitShift P.V;
//   LIS, MFMA       the same sum, exact, as two int8 MFMA products: the weight
//                   2^w = 2^(8h) 2^l (h = w >> 3, l = w & 7) enters as the int8
//                   -2^l in bit plane h (-128 fits where +128 does not), so
//                   o = -(O_0 + 256 O_1).
// Padded keys (j >= N) get the accumulator init mask_s below every real
// accumulator, so they never win the row max; their table entry is removed
// from the row sum once per lane, and their K and V rows are zero in LDS.
//
// LDS: V and K as row-major regions of whole 1 KB load blocks, 16-byte chunks
// XOR-swizzled per row so that the MFMA operand reads are bank-conflict free;
// the V^T operand of P.V comes from ds_read_b64_tr_b8 (8 keys x 16 features
// per 16-lane group), so V needs no transpose on the way in.  One exponential
// table per workgroup.
//
// Method passages: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" and sec. 3.3 "Integer-only Softmax: Shiftmax"; FQ-ViT
// abstract (Log-Int-Softmax, 4-bit log2 codes, BitShift); Trio-ViT sec. IV
// Eq. 11 (leading-one log2 with the next bit).
#include "iqattn_dev.h"
#include "iqattn.h"

namespace iqattn {
namespace {


// LIS shift w = F - code of the probability Ph = (f e) >> (M - F).  Ph <= 2^F
// (e is at most the row sum s and f = floor(2^M / s)), so w = ilog2r(max(Ph, 1))
// with no clamp: Ph = 0 and Ph = 1 both give code F.  ilog2r(x) is the
// leading-one index plus the next bit; for x < 2^24 the float conversion is
// exact, its mantissa's top bit is that next bit, and adding 2^22 to the bit
// pattern carries it into the exponent.  Adding 2^23 more returns the biased
// exponent plus one, w + 128: w in the low four and the low five bits.
// (The empty asm keeps the conversion a 32-bit one: without it the compiler
// sees that ph is the high half of a 64-bit product and converts that as a
// 64-bit integer, five instructions instead of one.)
__device__ __forceinline__ uint32_t lis_exp(uint32_t ph) {
  asm("" : "+v"(ph));
  return (__float_as_uint((float)max(ph, 1u)) + 0xC00000u) >> 23;
}

// o + (v << w) as one v_lshl_add_u32 (the empty asm keeps every step a single
// instruction: without it the compiler pairs two shifts into a v_add3_u32, three
// instructions per two steps)
__device__ __forceinline__ int32_t shl_add(int32_t v, int32_t w, int32_t o) {
  int32_t r = (int32_t)(((uint32_t)v << (w & 31)) + (uint32_t)o);
  asm("" : "+v"(r));
  return r;
}


// The two bit-plane operand words of sixteen LIS shifts at once (four 16-key
// tiles of four keys).  Each input holds w (mod 16) in byte 0 and w + 8 (mod
// 16) in byte 1.  v_lshlrev_b16 shifts by the low four bits of its amount, so
// the low byte of 0xFF << (w mod 16) is the plane-0 byte (0 for w >= 8) and
// that of 0xFF << ((w + 8) mod 16) the plane-1 byte (0 for w < 8); the SDWA
// form takes the amount from byte 0 or byte 1 of the input and writes that low
// byte straight into byte r of the operand word.  The writes go byte-major
// (eight instructions between writes to one word) and end with the wait
// states an MFMA reading the words needs, as in p16_pack24.
__device__ __forceinline__ void lis_planes16(const v4i& x0, const v4i& x1, const v4i& x2,
                                             const v4i& x3, uint32_t ff, v4i& lo, v4i& hi) {
  uint32_t l0, l1, l2, l3, h0, h1, h2, h3;
  asm(
      "v_lshlrev_b16_sdwa %0, %8, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %1, %12, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %2, %16, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %3, %20, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %4, %8, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %5, %12, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %6, %16, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %7, %20, %24 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %0, %9, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %1, %13, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %2, %17, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %3, %21, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %4, %9, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %5, %13, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %6, %17, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %7, %21, %24 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %0, %10, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %1, %14, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %2, %18, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %3, %22, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %4, %10, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %5, %14, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %6, %18, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %7, %22, %24 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %0, %11, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %1, %15, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %2, %19, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %3, %23, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %4, %11, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %5, %15, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %6, %19, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "v_lshlrev_b16_sdwa %7, %23, %24 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1 src1_sel:WORD_0\n\t"
      "s_nop 4"
      : "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3), "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3)
      : "v"(x0[0]), "v"(x0[1]), "v"(x0[2]), "v"(x0[3]), "v"(x1[0]), "v"(x1[1]), "v"(x1[2]),
        "v"(x1[3]), "v"(x2[0]), "v"(x2[1]), "v"(x2[2]), "v"(x2[3]), "v"(x3[0]), "v"(x3[1]),
        "v"(x3[2]), "v"(x3[3]), "v"(ff));
  lo = v4i{(int32_t)l0, (int32_t)l1, (int32_t)l2, (int32_t)l3};
  hi = v4i{(int32_t)h0, (int32_t)h1, (int32_t)h2, (int32_t)h3};
}

// One work item: head u (-1 past the end) and its query tiles qt0, qt0 + qstep,
// ... (T of them).  Whole heads take every tile; a head of the last partial
// round is split into four quarter items (tiles q, q + 4, ...).  The quarters
// of a head sit 8 items apart, so with a grid that is a multiple of 8 they run
// on one XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2
// for the K/V reads.
struct Item {
  int u, qt0, qstep, T;
};

template <int KT>
__device__ __forceinline__ Item decode_item(const DevParams& p, int k) {
  Item it;
  it.u = -1;
  it.qt0 = 0;
  it.qstep = 1;
  it.T = 0;
  if (k >= p.n_items) return it;
  if (k < p.n_full) {
    it.u = k;
    it.T = KT;
  } else {
    const int r = k - p.n_full, kk = r >> 3, q = kk & 3;
    const int u = p.n_full + (kk >> 2) * 8 + (r & 7);
    if (u < p.units) it.u = u;
    it.qt0 = q;
    it.qstep = 4;
    it.T = q < KT ? (KT - q + 3) / 4 : 0;
  }
  return it;
}

// Key held by accumulator row 4 g + r of the last 16-key tile when its rows
// are transposed: 4 r + g.
__device__ __forceinline__ int kt_perm(int pos) { return ((pos & 3) << 2) | (pos >> 2); }

// Direct loads of head u's K (and Q), then V (R / 1024 blocks each) into the
// LDS regions at vbuf + R (and vbuf + 2R) and vbuf, issued by one wave.  Lane l of block i fills LDS bytes
// [1024 i + 16 l, +16) = (row, chunk position cp) from source chunk
// cp ^ swizzle(row).  Rows >= N lie past the buffer range and arrive as zeros.
template <int D, int R, bool WITH_Q, int KT, bool PERM>
__device__ __forceinline__ void stage_head(const DevParams& p, int u, uint32_t vbuf, int lane) {
  constexpr int NB = R / 1024;
  constexpr int LT = (KT - 1) * 16;  // first key of the last 16-key tile
  const int64_t hb = (int64_t)u * p.n * D;
  const uint32_t bytes = (uint32_t)(p.n * D);
  const v4i rk = make_rsrc(p.k + hb, bytes);
  const v4i rv = make_rsrc(p.v + hb, bytes);
  const v4i rq = make_rsrc(p.q + hb, bytes);
  // K and V rows of the last tile are transposed 4 x 4 (kt_perm): its real
  // keys fill the accumulator rows r = 0 first, so that every lane's rows
  // r >= ceil(real keys / 4) hold padding only
  auto kv_row = [&](int row) { return (PERM && row >= LT && row < LT + 16) ? LT + kt_perm(row - LT) : row; };
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int o = blk * 1024 + 16 * lane;
    const int row = o / D, cp = (o % D) >> 4;
    const int sw = 16 * (cp ^ kswz<D>(row));
    raw_buffer_load_lds(rk, (lds_u32w*)(uintptr_t)(vbuf + R + blk * 1024), 16, kv_row(row) * D + sw,
                        0, 0, 0);
    if (WITH_Q)
      raw_buffer_load_lds(rq, (lds_u32w*)(uintptr_t)(vbuf + 2 * R + blk * 1024), 16, row * D + sw, 0,
                          0, 0);
  }
  // V last: the Q.K^T part of a tile may start once the loads above are in
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int o = blk * 1024 + 16 * lane;
    const int row = o / D, cp = (o % D) >> 4;
    raw_buffer_load_lds(rv, (lds_u32w*)(uintptr_t)(vbuf + blk * 1024), 16,
                        kv_row(row) * D + 16 * (cp ^ vswz<D>(row)), 0, 0, 0);
  }
}

// s_waitcnt immediate for vmcnt(n), other counters untouched (n < 64)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }


// Output stores of rows of up to 64 keys (many small heads, two workgroups
// per CU) go through LDS as whole-row chunks with cache policy sc1 (written
// through while the kernel runs instead of left dirty in L2 for the
// end-of-kernel write-back); longer rows store each lane's words directly
// (measured faster there).
constexpr int kOutStorePolicy = 16;
constexpr bool fast_staged_out(int kt) { return kt <= 4; }

// Output requantisation and store of a lane's 4 x FT int32 sums (features
// 16 ft + 4 g + r of one query, at byte offset dst + 16 ft of the head).
template <int FT>
__device__ __forceinline__ void store_out(const DevParams& p, const v4i (&O)[FT],
                                          __amdgpu_buffer_rsrc_t ores, int dst) {
  if (p.pv_fast) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      __builtin_amdgcn_raw_buffer_store_b32(
          pack4_lowbytes((uint32_t)clamp127(mulhi_i32(O[ft][0], p.pv_bm)),
                         (uint32_t)clamp127(mulhi_i32(O[ft][1], p.pv_bm)),
                         (uint32_t)clamp127(mulhi_i32(O[ft][2], p.pv_bm)),
                         (uint32_t)clamp127(mulhi_i32(O[ft][3], p.pv_bm))),
          ores, dst + ft * 16, 0, 0);
  } else {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      __builtin_amdgcn_raw_buffer_store_b32(
          pack4_lowbytes((uint32_t)requant_i8(O[ft][0], p.pv_b, p.pv_c),
                         (uint32_t)requant_i8(O[ft][1], p.pv_b, p.pv_c),
                         (uint32_t)requant_i8(O[ft][2], p.pv_b, p.pv_c),
                         (uint32_t)requant_i8(O[ft][3], p.pv_b, p.pv_c)),
          ores, dst + ft * 16, 0, 0);
  }
}



// Output requantisation and store of a tile through LDS: each lane's four
// words (features 16 ft + 4 g .. + 3 of query row li) go to the wave's own
// 16 Q rows in LDS (dead once its Q operand is loaded), and the tile leaves as
// 16-byte chunks of whole rows (one store instruction covers 16 rows).  Rows
// past N lie outside the output range and are dropped by the buffer store.
template <int D, int FT>
__device__ __forceinline__ void store_out_staged(const DevParams& p, const v4i (&O)[FT],
                                                 __amdgpu_buffer_rsrc_t ores, int8_t* stage,
                                                 int li, int g, int lane, int row0, int ostride) {
  uint32_t wd[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    if (p.pv_fast)
      wd[ft] = pack4_lowbytes((uint32_t)clamp127(mulhi_i32(O[ft][0], p.pv_bm)),
                              (uint32_t)clamp127(mulhi_i32(O[ft][1], p.pv_bm)),
                              (uint32_t)clamp127(mulhi_i32(O[ft][2], p.pv_bm)),
                              (uint32_t)clamp127(mulhi_i32(O[ft][3], p.pv_bm)));
    else
      wd[ft] = pack4_lowbytes((uint32_t)requant_i8(O[ft][0], p.pv_b, p.pv_c),
                              (uint32_t)requant_i8(O[ft][1], p.pv_b, p.pv_c),
                              (uint32_t)requant_i8(O[ft][2], p.pv_b, p.pv_c),
                              (uint32_t)requant_i8(O[ft][3], p.pv_b, p.pv_c));
  }
  volatile uint32_t* sw = (volatile uint32_t*)(stage + li * D + 4 * g);
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) sw[4 * ft] = wd[ft];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int r = lane >> 2, c = lane & 3;
  if (D == 64) {
    const v4i val = *(volatile v4i*)(stage + r * 64 + 16 * c);
    __builtin_amdgcn_raw_buffer_store_b128(val, ores, (row0 + r) * ostride + 16 * c, 0,
                                           kOutStorePolicy);
  } else {
    const v2i val = *(volatile v2i*)(stage + r * 32 + 8 * c);
    __builtin_amdgcn_raw_buffer_store_b64(val, ores, (row0 + r) * ostride + 8 * c, 0,
                                          kOutStorePolicy);
  }
  // (the next tile's writes to these rows come after these reads)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int KT, bool BIAS, int VAR>
__global__ __launch_bounds__(64 * (fast_cw(D, KT, BIAS, VAR) + 1), fast_waves_per_eu(KT, BIAS)) void iqattn_fast(
    DevParams p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  constexpr int CW = fast_cw(D, KT, BIAS, VAR);         // compute waves; wave CW loads
  constexpr int NBUF = fast_nbuf(D, KT, BIAS, VAR);
  constexpr int R = fast_region_bytes(D, KT);  // bytes of one V, K or Q region
  constexpr int BS = fast_nreg(KT, BIAS) * R;  // bytes of one buffer
  constexpr bool QLDS = fast_nreg(KT, BIAS) == 3;
  constexpr int KPL = D / 4;                   // k-bytes per lane in the Q.K^T MFMA
  constexpr int KS = (KT + 3) / 4;             // 64-key steps of the P.V MFMA
  constexpr int FT = D / 16;
  typedef typename Mfma<D>::Op Op;

  const int N = p.n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x;

  const uint32_t smem0 = lds_addr(smem);
  const char* sE = (const char*)(smem + NBUF * BS);
  int32_t* sW = (int32_t*)(smem + NBUF * BS + kFastTableBytes);
  // work-queue words: next tile of the workgroup's sequence, then per buffer
  // the item it holds and the number of that item's tiles finished
  int* ctl = (int*)(smem + NBUF * BS + kFastTableBytes + (VAR == kFastLisValu ? CW * 1024 : 0));
  // windowed bias of 64-key rows staged in LDS (p.bias_lds): [heads][64][64] int32,
  // the 16-byte chunk c of row r at slot c ^ (r & 15), so that the b128 reads of
  // sixteen query rows (one chunk each) fall on distinct banks
  const int32_t* sBias = (const int32_t*)(smem + NBUF * BS + kFastTableBytes +
                                          (VAR == kFastLisValu ? CW * 1024 : 0) + 64);
  constexpr bool BIAS64 = BIAS && KT == 4;
  // last key tile transposed (no bias: the expanded bias keeps the natural
  // key order of its rows)
  constexpr bool PERM = !BIAS;
  int* const ctl_next = ctl;
  int* const ctl_ready = ctl + 1;
  int* const ctl_done = ctl + 1 + NBUF;
  int* const ctl_vready = ctl + 1 + 2 * NBUF;  // item whose V is in the buffer

  const Item item0 = decode_item<KT>(p, blockIdx.x);
  if (item0.u < 0) return;  // uniform, before the barrier
  if (wave == CW) {
    // the loader issues its first loads before the barrier (they go to the
    // table, bias and buffer-0 regions, not to the work-queue words that
    // thread 0 initialises): the exponential table (entries e << e_shift,
    // 1 KB), every head's windowed bias for rows of 64 keys (read from L2: it is
    // the same for every workgroup), then item 0's K, Q and V
    raw_buffer_load_lds(make_rsrc(p.exp_tab, kFastTableBytes), (lds_u32w*)(uintptr_t)lds_addr(sE),
                        16, 16 * lane, 0, 0, 0);
    if (BIAS64 && p.bias_lds) {
      const v4i rb = make_rsrc(p.bias, (uint32_t)(p.heads * 64 * 64 * 4));
      const uint32_t b0 = lds_addr(sBias);
      for (int blk = 0; blk < p.heads * 16; ++blk) {
        const int row = 4 * blk + (lane >> 4), slot = lane & 15;
        raw_buffer_load_lds(rb, (lds_u32w*)(uintptr_t)(b0 + blk * 1024), 16,
                            row * 256 + 16 * (slot ^ (row & 15)), 0, 0, 0);
      }
    }
    stage_head<D, R, QLDS, KT, PERM>(p, item0.u, smem0, lane);
  }
  if (tid == 0) {
    ctl_next[0] = 0;
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      ctl_ready[b] = -1;
      ctl_done[b] = 0;
      ctl_vready[b] = -1;
    }
  }
  // the only workgroup barrier; it orders the work-queue words that thread 0
  // wrote (a fence in the loader wave would make it wait for its loads into
  // LDS first)
  if (wave != CW) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  if (wave == CW) {
    // ---- loader wave: item j of the workgroup's sequence into buffer
    //      j % NBUF once every tile of item j - NBUF is finished (item 0 and
    //      the table were issued before the barrier; the flags of item 0 cover
    //      them)
    for (int j = 0;; ++j) {
      const Item it = decode_item<KT>(p, (int)blockIdx.x + j * G);
      if (it.u < 0) break;
      const int b = j % NBUF;
      if (j >= NBUF) {
        const int tprev = decode_item<KT>(p, (int)blockIdx.x + (j - NBUF) * G).T;
        // (bounded: p.spin_limit polls of about 64 clocks each; only a broken
        // invariant, or a test's tiny limit, makes a wave give up)
        int spins = 0;
        while (__hip_atomic_load(&ctl_done[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) !=
               tprev) {
          if (++spins > p.spin_limit) {
            report_giveup(p, kStatusLoader);
            return;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      // (the counters start at 0; resetting only reused buffers keeps the
      // first items' loads from waiting behind a vmcnt(0) the compiler puts
      // before any LDS access that follows a direct load)
      if (j >= NBUF && lane == 0)
        __hip_atomic_store(&ctl_done[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (j > 0) stage_head<D, R, QLDS, KT, PERM>(p, it.u, smem0 + b * BS, lane);
      // (in effect both flags below are set once K, Q and V are all in: the
      // compiler puts a vmcnt(0) before every LDS access that follows a direct
      // load into LDS, the release stores included.  Loaders that set the K/Q
      // flag first, or kept two items in flight, through flag accesses in asm,
      // measured slower on every short-row shape.)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(R / 1024));  // K and Q are in LDS
      if (lane == 0) __hip_atomic_store(&ctl_ready[b], j, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      __builtin_amdgcn_s_waitcnt(0);  // and V
      if (lane == 0) __hip_atomic_store(&ctl_vready[b], j, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return;
  }

  // ---- compute waves
  // padded keys of the last tile held by this lane: accumulator init and count
  // (with the transposed last tile, row 4 g + r holds key 4 r + g of it, and
  // rows r >= rl of every lane hold padding only: pass 2 skips them)
  const int nl = N - (KT - 1) * 16;       // real keys of the last tile, 1..16
  const int rl = PERM ? (nl + 3) >> 2 : 4;
  v4i cmask;
  int npad = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool pad = PERM ? 4 * r + g >= nl : (KT - 1) * 16 + 4 * g + r >= N;
    cmask[r] = pad ? p.mask_s : 0;
    npad += (pad && r < rl) ? 1 : 0;
  }
  const int32_t tab0 = (int32_t)lds_addr(sE);  // absolute LDS address of entry 0
  // per-lane operand offsets inside a K region (the swizzle depends on li only)
  const int koff = (D == 64 ? li * 64 + 16 * g : li * 32 + 8 * g) ^ (kswz<D>(li) << 4);
  // transpose-read offsets inside a 64-key block of a V region: lane (g, 2b + h)
  // reads 8 features (16 ft + 8 h ...) of key 16 (2 hr + (b >> 2)) + 4 g + (b & 3)
  // for read hr; the chunk index (ft) enters by XOR
  int vtr[2];
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
    const int kap = 16 * (2 * hr + (li >> 3)) + 4 * g + ((li >> 1) & 3);
    vtr[hr] = kap * D + 8 * (li & 1) + 16 * vswz<D>(kap);
  }
  const int32_t qk_bm = p.qk_bm;
  const int32_t lpad = mulhi_i32(p.mask_s, qk_bm);

  int jw = 0, base = 0, have = -1, havev = -1;
  Item it = decode_item<KT>(p, blockIdx.x);
  // tile numbers are taken one tile ahead, so the atomic's latency is hidden
  int sq = 0;
  if (lane == 0) sq = __hip_atomic_fetch_add(ctl_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (;;) {
    // this tile of the workgroup's sequence: item jw, tile s - base of it
    const int s = __builtin_amdgcn_readfirstlane(sq);
    if (lane == 0) sq = __hip_atomic_fetch_add(ctl_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (it.u >= 0 && s >= base + it.T) {
      base += it.T;
      ++jw;
      it = decode_item<KT>(p, (int)blockIdx.x + jw * G);
    }
    if (it.u < 0) break;
    // the workgroup's last item runs at the highest priority (its tiles end the kernel)
    const bool last_item = decode_item<KT>(p, (int)blockIdx.x + (jw + 1) * G).u < 0;
    const int b = jw % NBUF;
    if (have < jw) {
      int spins = 0;
      while (__hip_atomic_load(&ctl_ready[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != jw) {
        if (++spins > p.spin_limit) {
          report_giveup(p, kStatusKQ);
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      have = jw;
    }
    const int qt = it.qt0 + (s - base) * it.qstep;

    const uint32_t vbase = smem0 + b * BS;  // V region; K (and Q) regions follow
    const int8_t* sV = smem + b * BS;
    const int8_t* sK = sV + R;
    const int8_t* sQ = sV + 2 * R;
    const int u = it.u;
    const int64_t hbase = (int64_t)u * N * D;
    const int h = u % p.heads;
    // Query rows past N are clamped to N - 1 for every load, bias read and
    // store: such a lane computes query N - 1 exactly and stores the same bytes.
    const __amdgpu_buffer_rsrc_t qres = buf_rsrc(p.q + hbase, (uint32_t)(N * D));
    const __amdgpu_buffer_rsrc_t bres =
        buf_rsrc(p.bias, BIAS ? (uint32_t)((int64_t)p.heads * (KT * 16) * (KT * 16) * 4) : 0u);
    // output rows of this head: `ostride` bytes apart (head-major or token-major)
    const int ostride = out_row_stride(p, D);
    const __amdgpu_buffer_rsrc_t ores =
        buf_rsrc(p.out + out_head_base(p, u, D), (uint32_t)((N - 1) * ostride + D));

    {
      const int qrow = min(qt * 16 + li, N - 1);
      Op qop;
      if (QLDS)
        qop = *(const Op*)(sQ + ((D == 64 ? qrow * 64 + 16 * g : qrow * 32 + 8 * g) ^
                                 (kswz<D>(qrow) << 4)));
      else
        qop = buf_load<Op>(qres, qrow * D + KPL * g);

      // ---- S^T = K . Q^T (+ bias / padding mask in the accumulator).  K
      //      operands are read one tile ahead; the scheduling barriers keep the
      //      compiler from hoisting every LDS read of a phase (registers)
      constexpr int KPF = 3;  // K operand reads in flight ahead of the MFMA
      v4i S[KT];
      Op kb[KPF];
#pragma unroll
      for (int i = 0; i < KPF; ++i)
        if (i < KT) kb[i] = *(const Op*)(sK + i * 16 * D + koff);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const Op kop = kb[kt % KPF];
        if (kt + KPF < KT) kb[kt % KPF] = *(const Op*)(sK + (kt + KPF) * 16 * D + koff);
        v4i c0 = {0, 0, 0, 0};
        if (BIAS) {
          // (an LDS-typed read and a buffer load: a generic pointer chosen at run
          // time would become a flat load, which waits for the stores too)
          if (BIAS64 && p.bias_lds)
            c0 = *(lds_v4i*)(uintptr_t)(lds_addr(sBias) +
                                        4u * ((h * 64 + qrow) * 64 + 4 * ((kt * 4 + g) ^ (qrow & 15))));
          else
            c0 = __builtin_amdgcn_raw_buffer_load_b128(
                bres, (int)(((h * (KT * 16) + qrow) * (KT * 16) + kt * 16 + 4 * g) * 4), 0, 0);
        } else if (kt == KT - 1) {
          c0 = cmask;
        }
        S[kt] = Mfma<D>::run(kop, qop, c0);
        __builtin_amdgcn_sched_barrier(0);
      }

      if (last_item)
        __builtin_amdgcn_s_setprio(3);
      else
        __builtin_amdgcn_s_setprio(2);
      // ---- pass 1: row max of the accumulators (plain code: these are the first
      //      reads of the MFMA results)
      // (four independent chains)
      // (the empty asm keeps each chain step one v_max3: without it the compiler
      // re-associates the chain into v_max pairs, 3 instructions per 4 values)
      int32_t mx[4] = {S[0][0], S[0][1], S[0][2], S[0][3]};
#pragma unroll
      for (int kt = 1; kt + 1 < KT; kt += 2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mx[r] = max(mx[r], max(S[kt][r], S[kt + 1][r]));  // v_max3
          asm volatile("" : "+v"(mx[r]));
        }
      if ((KT & 1) == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx[r] = max(mx[r], S[KT - 1][r]);
      int32_t amax = max(max(mx[0], mx[1]), max(mx[2], mx[3]));
      amax = wave_max4(amax);
      const int32_t m = clamp127(mulhi_i32(amax, qk_bm));
      // table address of index (m - L) is rb - 4 L; saturating L to [-127, 127]
      // clamps it to [lo, hi] (entries past exp_last are 0)
      const int32_t rb = tab0 + m * 4;
      const int32_t lo = rb - 127 * 4;
      const int32_t hi = tab0 + min(m + 127, p.exp_last) * 4;

      // ---- pass 2: e << e_shift from the table, row sum (two chains)
      uint32_t sacc[2] = {0, 0};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (PERM && kt == KT - 1 && r > 0 && r >= rl) {
            S[kt][r] = 0;  // padding only: e = 0
            continue;
          }
          const int32_t a = exp_offset(S[kt][r], qk_bm, -4, rb, lo, hi);
          const uint32_t e = lds_read_u32((uint32_t)a);
          S[kt][r] = (int32_t)e;
          sacc[r >> 1] += e;
        }
      }
      uint32_t s = sacc[0] + sacc[1];
      if (npad) s -= (uint32_t)npad * lds_read_u32((uint32_t)min(max(rb - lpad * 4, lo), hi));
      s = wave_sum4(s);
      const uint32_t st = s >> p.e_shift;

      // ---- IntDiv: f = floor(2^M / st).  |estimate - 2^M/st| <= 1/2 (2^M/st
      //      <= 2^22, one-ulp reciprocal), so the truncated estimate is off by at
      //      most one; f st < 2^31 keeps 32 bits exact
      const uint32_t two_m = 1u << p.intdiv_m;
      uint32_t f = (uint32_t)(__builtin_amdgcn_rcpf((float)st) * (float)two_m);
      int32_t rem = (int32_t)(two_m - f * st);
      if (rem < 0) { f -= 1; rem += (int32_t)st; }
      if (rem >= (int32_t)st) { f += 1; }
      // Shiftmax: one key holding the whole row would give P = 2^(k_out-1); f - 1
      // yields the clamped 2^(k_out-1) - 1 for it (every other key has e = 0)
      if (VAR == kFastShiftmax && p.e0_pow2 && st == (uint32_t)p.e0) f -= 1;
      const uint32_t F = f << p.f_shift;
      // V of the item (loaded after K and Q) is needed from here on
      if (havev < jw) {
        int spins = 0;
        while (__hip_atomic_load(&ctl_vready[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != jw) {
          if (++spins > p.spin_limit) {
            report_giveup(p, kStatusV);
            return;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        havev = jw;
      }
      __builtin_amdgcn_sched_barrier(0);

      if (VAR == kFastShiftmax) {
        // ---- P = (f e) >> (M - k_out + 1) as one mulhi, O^T = V^T . P^T; the
        //      V^T operands of the next 64-key step are read during this one
        v4i O[FT];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) O[ft] = v4i{0, 0, 0, 0};
        v4i vcur[FT], vnxt[FT];
        uint32_t va[FT][2];
        vt_addr<FT>(vbase, vtr, va);
        read_vt<FT>(va, 0, vcur);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) read_vt<FT>(va, (ks + 1) * 64 * D, vnxt);
          v4i pop;
          if (ks * 4 + 3 < KT && p.p_u24) {
            p16_pack24(S[ks * 4], S[ks * 4 + 1], S[ks * 4 + 2], S[ks * 4 + 3], F, pop);
          } else {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              const int kt = ks * 4 + tt;
              uint32_t word = 0;
              if (kt < KT)
                word = p4_pack((uint32_t)S[kt][0], (uint32_t)S[kt][1], (uint32_t)S[kt][2],
                               (uint32_t)S[kt][3], F);
              pop[tt] = (int32_t)word;
            }
          }
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) O[ft] = mfma64(vcur[ft], pop, O[ft]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) vcur[ft] = vnxt[ft];
        }
        // lane holds features 16 ft + 4 g + r of query qrow
        if (QLDS && fast_staged_out(KT))
          store_out_staged<D, FT>(p, O, ores, const_cast<int8_t*>(sQ) + qt * 16 * D, li, g, lane,
                                  qt * 16, ostride);
        else
          store_out<FT>(p, O, ores, qrow * ostride + 4 * g);
      } else {
        // ---- LIS: Ph = (f e) >> (M - F) as one mulhi, shift w = F - code as
        //      w + 128 (VALU engine: the amount of a 32-bit shift, formed one
        //      16-key tile at a time in the P.V loop) or as the two plane-shift
        //      bytes w + 128 and w + 136 (MFMA engine)
        if (VAR == kFastLisMfma) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              S[kt][r] = (int32_t)(lis_exp(mulhi_u32((uint32_t)S[kt][r], F)) * 257u + 2048u);
          // ---- o = -(O_0 + 256 O_1), O_h = V^T . (plane h of -2^w)^T
          v4i O0[FT], O1[FT];
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) O0[ft] = O1[ft] = v4i{0, 0, 0, 0};
          // (at 609-640 keys the V^T operands of a step are read at its start:
          // one step of read-ahead would not fit the registers)
          constexpr bool VPF = KT < 39;
          v4i vcur[FT], vnxt[FT];
          uint32_t va[FT][2];
          vt_addr<FT>(vbase, vtr, va);
          if (VPF) read_vt<FT>(va, 0, vcur);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (!VPF) read_vt<FT>(va, ks * 64 * D, vcur);
            if (VPF && ks + 1 < KS) read_vt<FT>(va, (ks + 1) * 64 * D, vnxt);
            v4i plo, phi;
            if (ks * 4 + 3 < KT) {
              lis_planes16(S[ks * 4], S[ks * 4 + 1], S[ks * 4 + 2], S[ks * 4 + 3], 0xFFu, plo, phi);
            } else {
#pragma unroll
              for (int tt = 0; tt < 4; ++tt) {
                const int kt = ks * 4 + tt;
                int32_t lo_w = 0, hi_w = 0;
                if (kt < KT) lis_planes(S[kt], lo_w, hi_w);
                plo[tt] = lo_w;
                phi[tt] = hi_w;
              }
            }
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
              O0[ft] = mfma64(vcur[ft], plo, O0[ft]);
              O1[ft] = mfma64(vcur[ft], phi, O1[ft]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (VPF)
#pragma unroll
              for (int ft = 0; ft < FT; ++ft) vcur[ft] = vnxt[ft];
          }
#pragma unroll
          for (int ft = 0; ft < FT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r) O0[ft][r] = -(O0[ft][r] + (O1[ft][r] << 8));
          if (QLDS && fast_staged_out(KT))
            store_out_staged<D, FT>(p, O0, ores, const_cast<int8_t*>(sQ) + qt * 16 * D, li, g,
                                    lane, qt * 16, ostride);
          else
            store_out<FT>(p, O0, ores, qrow * ostride + 4 * g);
        } else {
          // ---- VALU P.V: lane owns 4 queries x NF = D / 16 features (lanes
          //      16 qg + fg: queries 4 qg.., features NF fg..); the wave's shifts
          //      go through LDS one 16-key tile at a time (16 keys x 16
          //      queries).  Per key a lane reads its 4 shifts (one b128, the
          //      same for the 16 lanes of its query group) and its NF V bytes
          //      for 4 NF shift-adds: half the LDS bytes per shift-add of one
          //      query per lane at D = 64
          constexpr int NF = D / 16;
          const int fg = lane & 15, qg = lane >> 4;
          const int q0 = 4 * qg, f0 = NF * fg;
          int32_t* sWw = sW + wave * 256;
          // this lane's column block of the shift rows, held in a VGPR (the empty
          // asm): a wave-uniform address would be formed in SGPRs and copied to a
          // VGPR for every read instead of riding in the reads' offset field
          uint32_t wcol = lds_addr(sWw + q0);
          asm volatile("" : "+v"(wcol));
          int32_t o[4][NF];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int f = 0; f < NF; ++f) o[i][f] = 0;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              sWw[(4 * g + r) * 16 + li] = (int32_t)lis_exp(mulhi_u32((uint32_t)S[kt][r], F));
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 4
            for (int jj = 0; jj < 16; ++jj) {
              const int row = kt * 16 + jj;  // rows >= N are zero
              // f0.. f0 + NF - 1 lie in one 16-byte chunk, which the swizzle moves
              // whole; one sign-extending byte read per feature (volatile: merged
              // into one dword read, each byte would cost an extract instruction)
              const volatile lds_i8* vrow =
                  (const volatile lds_i8*)(uintptr_t)lds_addr(sV + row * D + (f0 ^ (vswz<D>(row) << 4)));
              int32_t v[NF];
#pragma unroll
              for (int f = 0; f < NF; ++f) v[f] = (int32_t)vrow[f];
              const v4i w4 = *(lds_v4i*)(uintptr_t)(wcol + (uint32_t)(jj * 16) * 4u);
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int f = 0; f < NF; ++f) o[i][f] = shl_add(v[f], w4[i], o[i][f]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __builtin_amdgcn_sched_barrier(0);
          }
          // requantise, pack the NF bytes of a query, one store per query
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t y[NF];
#pragma unroll
            for (int f = 0; f < NF; ++f)
              y[f] = (uint32_t)(p.pv_fast ? clamp127(mulhi_i32(o[i][f], p.pv_bm))
                                          : requant_i8(o[i][f], p.pv_b, p.pv_c));
            const int dst = min(qt * 16 + q0 + i, N - 1) * ostride + f0;
            if (NF == 4)
              __builtin_amdgcn_raw_buffer_store_b32(pack4_lowbytes(y[0], y[1], y[2], y[3]), ores,
                                                    dst, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16(
                  (uint16_t)__builtin_amdgcn_perm(y[NF - 1], y[0], 0x0c0c0400u), ores, dst, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // this tile's LDS reads have returned: count it against the buffer
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (lane == 0) __hip_atomic_fetch_add(&ctl_done[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

}  // namespace

#define IQ_FAST_CASE(D, KT, B, V) \
  if (d == D && kt == KT && bias == B && var == V) return iqattn_fast<D, KT, B, V>;

// every row of up to 256 keys (KT <= 16) for both head sizes and all three back
// ends;
// Shiftmax with the windowed bias for every window up to 25 x 25 (N = w^2
// keys: every tile count up to 16, then those of w = 17..25); every longer row
// up to 640 keys
#define IQ_FAST_ALL_VAR(D, KT)                 \
  IQ_FAST_CASE(D, KT, false, kFastShiftmax) \
  IQ_FAST_CASE(D, KT, false, kFastLisValu)  \
  IQ_FAST_CASE(D, KT, false, kFastLisMfma)
#define IQ_FAST_SHORT13(D)                                                                \
  IQ_FAST_ALL_VAR(D, 1) IQ_FAST_ALL_VAR(D, 2) IQ_FAST_ALL_VAR(D, 3) IQ_FAST_ALL_VAR(D, 4)     \
  IQ_FAST_ALL_VAR(D, 5) IQ_FAST_ALL_VAR(D, 6) IQ_FAST_ALL_VAR(D, 7) IQ_FAST_ALL_VAR(D, 8)     \
  IQ_FAST_ALL_VAR(D, 9) IQ_FAST_ALL_VAR(D, 10) IQ_FAST_ALL_VAR(D, 11) IQ_FAST_ALL_VAR(D, 12)  \
  IQ_FAST_ALL_VAR(D, 13)

#define IQ_FAST_LONG(D)                                                                    \
  IQ_FAST_ALL_VAR(D, 17) IQ_FAST_ALL_VAR(D, 18) IQ_FAST_ALL_VAR(D, 19) IQ_FAST_ALL_VAR(D, 20)  \
  IQ_FAST_ALL_VAR(D, 21) IQ_FAST_ALL_VAR(D, 22) IQ_FAST_ALL_VAR(D, 23) IQ_FAST_ALL_VAR(D, 24)  \
  IQ_FAST_ALL_VAR(D, 25) IQ_FAST_ALL_VAR(D, 26) IQ_FAST_ALL_VAR(D, 27) IQ_FAST_ALL_VAR(D, 28)  \
  IQ_FAST_ALL_VAR(D, 29) IQ_FAST_ALL_VAR(D, 30) IQ_FAST_ALL_VAR(D, 31) IQ_FAST_ALL_VAR(D, 32)  \
  IQ_FAST_ALL_VAR(D, 33) IQ_FAST_ALL_VAR(D, 34) IQ_FAST_ALL_VAR(D, 35) IQ_FAST_ALL_VAR(D, 36)  \
  IQ_FAST_ALL_VAR(D, 37) IQ_FAST_ALL_VAR(D, 38) IQ_FAST_ALL_VAR(D, 39) IQ_FAST_ALL_VAR(D, 40)

#define IQ_FAST_B(D, KT) IQ_FAST_CASE(D, KT, true, kFastShiftmax)
// Log-Int-Softmax with the windowed bias (both engines): 7 x 7, 8 x 8 and 12 x 12 windows
#define IQ_FAST_LB(D, KT) \
  IQ_FAST_CASE(D, KT, true, kFastLisValu) IQ_FAST_CASE(D, KT, true, kFastLisMfma)
#define IQ_FAST_BIAS(D)                                                                     \
  IQ_FAST_B(D, 1) IQ_FAST_B(D, 2) IQ_FAST_B(D, 3) IQ_FAST_B(D, 4) IQ_FAST_B(D, 5)               \
  IQ_FAST_B(D, 6) IQ_FAST_B(D, 7) IQ_FAST_B(D, 8) IQ_FAST_B(D, 9) IQ_FAST_B(D, 10)              \
  IQ_FAST_B(D, 11) IQ_FAST_B(D, 12) IQ_FAST_B(D, 13) IQ_FAST_B(D, 14) IQ_FAST_B(D, 15)          \
  IQ_FAST_B(D, 16) IQ_FAST_B(D, 19) IQ_FAST_B(D, 21) IQ_FAST_B(D, 23) IQ_FAST_B(D, 25)         \
  IQ_FAST_B(D, 28) IQ_FAST_B(D, 31) IQ_FAST_B(D, 34) IQ_FAST_B(D, 36) IQ_FAST_B(D, 40)

KernelFn fast_kernel(int d, int kt, bool bias, int var) {
  IQ_FAST_SHORT13(64)
  IQ_FAST_ALL_VAR(64, 14)
  IQ_FAST_ALL_VAR(64, 15)
  IQ_FAST_ALL_VAR(64, 16)
  IQ_FAST_SHORT13(32)
  IQ_FAST_ALL_VAR(32, 14)
  IQ_FAST_ALL_VAR(32, 15)
  IQ_FAST_ALL_VAR(32, 16)
  IQ_FAST_BIAS(64)
  IQ_FAST_BIAS(32)
  IQ_FAST_LB(64, 4) IQ_FAST_LB(64, 9) IQ_FAST_LB(32, 4) IQ_FAST_LB(32, 9)
  IQ_FAST_LONG(64)
  IQ_FAST_LONG(32)
  return nullptr;
}

}  // namespace iqattn
