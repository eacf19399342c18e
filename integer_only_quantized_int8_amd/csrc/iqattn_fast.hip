// iqattn_fast.hip -- fused Shiftmax attention specialised on the number of
// 16-key tiles (KT, so N in (16(KT-1), 16 KT]) for the parameter ranges in
// which every step fits 24/32-bit VALU arithmetic (the host checks them).
//
// Per logit, after the MFMA:  pass 1  one v_max3 per two logits;
//   pass 2  v_mul_hi_i32 (requantisation), v_mad_i32_i24 + v_med3_i32
//           (saturation folded into the exponential-table address), one
//           ds_read_b32, one add;
//   pass 3  v_mul_hi_u32_u24 (IntDiv product and shift in one), byte packing
//           into the P.V MFMA operand.
// Padded keys (j >= N) get the accumulator init mask_s below every real
// accumulator, so they never win the row max; their table entry is removed
// from the row sum once per lane, and their V rows are zero in LDS.
//
// LDS layout (no padding): K as 64-byte rows (d = 64) whose four 16-byte
// chunks are XOR-swizzled by (row >> 1) & 3, which makes the b128 operand
// reads of 16 rows x 4 chunks bank-conflict free on gfx950 (d = 32 keeps
// 48-byte padded rows); V^T as [64-key step][feature][64 bytes] with the same
// swizzle; the exponential table with kRep copies (entry stride 4 kRep bytes).
//
// Method passages: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" and sec. 3.3 "Integer-only Softmax: Shiftmax".
#include "iqattn_dev.h"
#include "iqattn.h"

namespace iqattn {
namespace {

// byte offset of 16-byte chunk `c` of 64-byte row `r` after the XOR swizzle
__device__ __forceinline__ int swz64(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

template <int D, int KT, bool BIAS>
__global__ __launch_bounds__(kThreads) void iqattn_shiftmax_fast(DevParams p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  constexpr bool KSWZ = (D == 64);      // swizzled 64-byte K rows
  constexpr int KSTR = KSWZ ? 64 : D + 16;
  constexpr int KPL = D / 4;            // k-bytes per lane in the Q.K^T MFMA
  constexpr int KS = (KT + 3) / 4;      // 64-key steps of the P.V MFMA
  constexpr int NP = KT * 16;
  constexpr int FT = D / 16;
  constexpr int K_BYTES = NP * KSTR;
  constexpr int V_BYTES = KS * D * 64;
  constexpr int kRep = kFastExpRep;
  typedef typename Mfma<D>::Op Op;

  const int N = p.n;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;

  int8_t* sK = smem;
  int8_t* sV = smem + K_BYTES;
  const char* sE = (const char*)(smem + K_BYTES + V_BYTES);

  const int64_t hbase = (int64_t)u * N * D;
  const int8_t* gK = p.k + hbase;
  const int8_t* gV = p.v + hbase;

  // ---- stage K (rows >= N are zero)
  for (int i = tid; i < NP * (D / 16); i += kThreads) {
    const int row = i / (D / 16), c16 = i % (D / 16);
    v4i val = {0, 0, 0, 0};
    if (row < N) val = *(const v4i*)(gK + row * D + c16 * 16);
    *(v4i*)(sK + (KSWZ ? swz64(row, c16) : row * KSTR + c16 * 16)) = val;
  }
  // ---- stage V^T with the key permutation: a unit is 4 keys x 16 features
  //      (four 16-byte loads), transposed in registers 4 x 4 bytes at a time;
  //      keys 4q..4q+3 land on 4 contiguous bytes of each feature row
  for (int i = tid; i < KS * 16 * FT; i += kThreads) {
    const int kq = i % (KS * 16), fb = i / (KS * 16);
    const int key0 = kq * 4;
    const int8_t* src = gV + key0 * D + fb * 16;
    v4i r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = v4i{0, 0, 0, 0};
      if (key0 + j < N) r[j] = *(const v4i*)(src + j * D);
    }
    const int pos = vperm_pos(key0) & 63, c = pos >> 4;
    int8_t* base = sV + (key0 >> 6) * (D * 64) + fb * 16 * 64 + (pos & 15);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = r[0][q], w1 = r[1][q], w2 = r[2][q], w3 = r[3][q];
      const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
      const uint32_t b = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
      const uint32_t cc = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
      const uint32_t d = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
      const uint32_t out[4] = {__builtin_amdgcn_perm(b, a, 0x05040100u),
                               __builtin_amdgcn_perm(b, a, 0x07060302u),
                               __builtin_amdgcn_perm(d, cc, 0x05040100u),
                               __builtin_amdgcn_perm(d, cc, 0x07060302u)};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = 4 * q + jj;  // feature within the block; row swizzle (t >> 1) & 3
        *(uint32_t*)(base + t * 64 + 16 * (c ^ ((t >> 1) & 3))) = out[jj];
      }
    }
  }
  // ---- stage the exponential table (entries e << e_shift), kRep copies
  {
    uint32_t* dstE = (uint32_t*)sE;
    const int nexp = (p.exp_last + 1) * kRep;
    for (int i = tid; i < nexp; i += kThreads) dstE[i] = p.exp_tab[i / kRep];
  }
  __syncthreads();

  // padded keys of the last tile held by this lane: accumulator init and count
  v4i cmask;
  int npad = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool pad = (KT - 1) * 16 + 4 * g + r >= N;
    cmask[r] = pad ? p.mask_s : 0;
    npad += pad ? 1 : 0;
  }
  // absolute LDS address of this lane's copy of table entry 0
  const int32_t tab0 = (int32_t)lds_addr(sE) + (lane & (kRep - 1)) * 4;
  constexpr int ESTR = 4 * kRep;  // bytes between consecutive table entries
  // per-lane operand offsets (swizzled rows: the swizzle depends on li only)
  const int koff = KSWZ ? swz64(li, g) : li * KSTR + KPL * g;
  const int voff = swz64(li, g);
  const int h = u % p.heads;
  const int32_t qk_bm = p.qk_bm;
  const int32_t lpad = mulhi_i32(p.mask_s, qk_bm);

  // tiles rotate over the waves from one head to the next so that the wave
  // with one extra tile is not always the same SIMD's
  for (int qt = (wave + kWaves - (u & (kWaves - 1))) & (kWaves - 1); qt < KT; qt += kWaves) {
    const int qrow = qt * 16 + li;
    Op qop = Op{};
    if (qrow < N) qop = *(const Op*)(p.q + hbase + (int64_t)qrow * D + KPL * g);

    // ---- S^T = K . Q^T (+ bias / padding mask in the accumulator)
    // K operands are read one tile ahead; the scheduling barriers keep the
    // compiler from hoisting every LDS read of a phase (which costs registers)
    v4i S[KT];
    Op knext = *(const Op*)(sK + koff);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const Op kop = knext;
      if (kt + 1 < KT) knext = *(const Op*)(sK + (kt + 1) * 16 * KSTR + koff);
      v4i c0 = {0, 0, 0, 0};
      if (BIAS) {
        c0 = *(const v4i*)(p.bias + ((int64_t)h * NP + qrow) * NP + kt * 16 + 4 * g);
      } else if (kt == KT - 1) {
        c0 = cmask;
      }
      S[kt] = Mfma<D>::run(kop, qop, c0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- pass 1: row max of the accumulators (plain code: these are the first
    //      reads of the MFMA results)
    int32_t amax = max(S[0][0], S[0][1]);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      if (kt > 0) amax = max(amax, max(S[kt][0], S[kt][1]));
      amax = max(amax, max(S[kt][2], S[kt][3]));
    }
    amax = wave_max4(amax);
    const int32_t m = clamp127(mulhi_i32(amax, qk_bm));
    // table byte offset of index (m - L) is rb - ESTR L; saturating L to
    // [-127, 127] clamps that offset to [lo, hi] (entries past exp_last are 0)
    const int32_t rb = tab0 + m * ESTR;
    const int32_t lo = rb - 127 * ESTR;
    const int32_t hi = tab0 + min(m + 127, p.exp_last) * ESTR;

    // ---- pass 2: e << e_shift from the table, row sum
    uint32_t s = 0;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t a = exp_offset(S[kt][r], qk_bm, -ESTR, rb, lo, hi);
        const uint32_t e = lds_read_u32((uint32_t)a);
        S[kt][r] = (int32_t)e;
        s += e;
      }
    }
    if (npad) {
      const int32_t a = min(max(rb - lpad * ESTR, lo), hi);
      s -= (uint32_t)npad * lds_read_u32((uint32_t)a);
    }
    s = wave_sum4(s);
    const uint32_t st = s >> p.e_shift;

    // ---- IntDiv: f = floor(2^M / st), reciprocal estimate then exact fix-up
    const uint32_t two_m = 1u << p.intdiv_m;
    // |estimate - 2^M/st| <= 1/2 (2^M/st <= 2^22, one-ulp reciprocal), so the
    // truncated estimate is off by at most one; f st < 2^31 keeps 32 bits exact
    uint32_t f = (uint32_t)(__builtin_amdgcn_rcpf((float)st) * (float)two_m);
    int32_t rem = (int32_t)(two_m - __umul24(f, st));
    if (rem < 0) { f -= 1; rem += (int32_t)st; }
    if (rem >= (int32_t)st) { f += 1; }
    // one key holding the whole row would give P = 2^(k_out-1): f - 1 yields
    // the clamped value 2^(k_out-1) - 1 for it (all other keys have e = 0)
    if (p.e0_pow2 && st == (uint32_t)p.e0) f -= 1;
    const uint32_t F = f << p.f_shift;

    __builtin_amdgcn_sched_barrier(0);
    // ---- pass 3: P = (f e) >> (M - k_out + 1) as one mulhi, O^T = V^T . P^T
    v4i O[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) O[ft] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v4i pop;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int kt = ks * 4 + tt;
        uint32_t word = 0;
        if (kt < KT)
          word = p4_pack((uint32_t)S[kt][0], (uint32_t)S[kt][1], (uint32_t)S[kt][2],
                         (uint32_t)S[kt][3], F);
        pop[tt] = (int32_t)word;
      }
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const v4i vop = *(const v4i*)(sV + ks * (D * 64) + ft * 16 * 64 + voff);
        O[ft] = mfma64(vop, pop, O[ft]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- epilogue: lane holds features 16 ft + 4 g + r of query qrow
    if (qrow < N) {
      int8_t* dst = p.out + hbase + (int64_t)qrow * D + 4 * g;
      if (p.pv_fast) {  // pv_b << (32 - pv_c) < 2^31: one v_mul_hi_i32
        const int32_t pv_bm = p.pv_bm;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
          *(uint32_t*)(dst + ft * 16) = pack4_lowbytes(
              (uint32_t)clamp127(mulhi_i32(O[ft][0], pv_bm)),
              (uint32_t)clamp127(mulhi_i32(O[ft][1], pv_bm)),
              (uint32_t)clamp127(mulhi_i32(O[ft][2], pv_bm)),
              (uint32_t)clamp127(mulhi_i32(O[ft][3], pv_bm)));
      } else {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
          *(uint32_t*)(dst + ft * 16) = pack4_lowbytes(
              (uint32_t)requant_i8(O[ft][0], p.pv_b, p.pv_c),
              (uint32_t)requant_i8(O[ft][1], p.pv_b, p.pv_c),
              (uint32_t)requant_i8(O[ft][2], p.pv_b, p.pv_c),
              (uint32_t)requant_i8(O[ft][3], p.pv_b, p.pv_c));
      }
    }
  }
}

}  // namespace

#define IQ_FAST_CASE(D, KT, B) \
  if (d == D && kt == KT && bias == B) return iqattn_shiftmax_fast<D, KT, B>;

KernelFn fast_shiftmax_kernel(int d, int kt, bool bias) {
  IQ_FAST_CASE(64, 13, false)
  IQ_FAST_CASE(64, 37, false)
  IQ_FAST_CASE(64, 1, false)
  IQ_FAST_CASE(64, 2, false)
  IQ_FAST_CASE(64, 4, false)
  IQ_FAST_CASE(64, 12, false)
  IQ_FAST_CASE(64, 4, true)
  IQ_FAST_CASE(32, 4, true)
  IQ_FAST_CASE(32, 4, false)
  IQ_FAST_CASE(32, 13, false)
  return nullptr;
}

}  // namespace iqattn
