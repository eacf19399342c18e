// iqattn_fast.hip -- fused Shiftmax attention specialised on the number of
// 16-key tiles (KT, so N in (16(KT-1), 16 KT]) for the parameter ranges in
// which every step fits 24/32-bit VALU arithmetic (the host checks them).
//
// Per logit, after the MFMA:  pass 1  one v_max3 per two logits;
//   pass 2  v_lshlrev + v_mul_hi_i32_i24 (requantisation), v_mad_i32_i24 +
//           v_med3_i32 (saturation folded into the exponential-table address),
//           one ds_read_b32 (table replicated once per LDS bank), v_add3;
//   pass 3  v_mul_hi_u32_u24 (IntDiv product and shift in one), byte packing
//           into the P.V MFMA operand.
// Padded keys (j >= N) get the accumulator init mask_s below every real
// accumulator, so they never win the row max; their table entry is removed
// from the row sum once per lane, and their V rows are zero in LDS.
//
// Method passages: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" and sec. 3.3 "Integer-only Softmax: Shiftmax".
#include "iqattn_dev.h"
#include "iqattn.h"

namespace iqattn {
namespace {

template <int D, int KT, bool BIAS>
__global__ __launch_bounds__(kThreads) void iqattn_shiftmax_fast(DevParams p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  constexpr int KSTR = D + 16;          // padded K row (bank spread of the b128 reads)
  constexpr int KPL = D / 4;            // k-bytes per lane in the Q.K^T MFMA
  constexpr int KS = (KT + 3) / 4;      // 64-key steps of the P.V MFMA
  constexpr int NP = KT * 16;
  constexpr int VTSTR = KS * 64 + 16;   // padded V^T row
  constexpr int FT = D / 16;
  constexpr int K_BYTES = NP * KSTR;
  constexpr int V_BYTES = D * VTSTR;
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

  // ---- stage K row-major (rows >= N are zero)
  for (int i = tid; i < NP * (D / 16); i += kThreads) {
    const int row = i / (D / 16), c16 = i % (D / 16);
    v4i val = {0, 0, 0, 0};
    if (row < N) val = *(const v4i*)(gK + row * D + c16 * 16);
    *(v4i*)(sK + row * KSTR + c16 * 16) = val;
  }
  // ---- stage V^T with the key permutation: 4 keys x 4 features per thread,
  //      transposed in registers (keys 4q..4q+3 land on 4 contiguous bytes)
  for (int i = tid; i < KS * 16 * (D / 4); i += kThreads) {
    const int kq = i / (D / 4), c4 = i % (D / 4);
    const int key0 = kq * 4;
    uint32_t r0 = 0, r1 = 0, r2 = 0, r3 = 0;
    const int8_t* src = gV + key0 * D + c4 * 4;
    if (key0 + 0 < N) r0 = *(const uint32_t*)(src);
    if (key0 + 1 < N) r1 = *(const uint32_t*)(src + D);
    if (key0 + 2 < N) r2 = *(const uint32_t*)(src + 2 * D);
    if (key0 + 3 < N) r3 = *(const uint32_t*)(src + 3 * D);
    const uint32_t a = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
    const uint32_t b = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    const uint32_t c = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
    const uint32_t d = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
    int8_t* dst = sV + (c4 * 4) * VTSTR + vperm_pos(key0);
    *(uint32_t*)(dst) = __builtin_amdgcn_perm(b, a, 0x05040100u);
    *(uint32_t*)(dst + VTSTR) = __builtin_amdgcn_perm(b, a, 0x07060302u);
    *(uint32_t*)(dst + 2 * VTSTR) = __builtin_amdgcn_perm(d, c, 0x05040100u);
    *(uint32_t*)(dst + 3 * VTSTR) = __builtin_amdgcn_perm(d, c, 0x07060302u);
  }
  // ---- stage the exponential table (entries e << e_shift), one copy per bank
  {
    uint32_t* dstE = (uint32_t*)sE;
    const int nexp = (p.exp_last + 1) * kExpRep;
    for (int i = tid; i < nexp; i += kThreads) dstE[i] = p.exp_tab[i / kExpRep];
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
  const int32_t tab0 = (int32_t)lds_addr(sE) + (lane & (kExpRep - 1)) * 4;
  const int h = u % p.heads;
  const int32_t alpha = p.alpha, qk_bm = p.qk_bm;
  const int32_t lpad = requant_raw24(p.mask_s, alpha, qk_bm);

  // tiles rotate over the waves from one head to the next so that the wave
  // with one extra tile is not always the same SIMD's
  for (int qt = (wave + kWaves - (u & (kWaves - 1))) & (kWaves - 1); qt < KT; qt += kWaves) {
    const int qrow = qt * 16 + li;
    Op qop = Op{};
    if (qrow < N) qop = *(const Op*)(p.q + hbase + (int64_t)qrow * D + KPL * g);

    // ---- S^T = K . Q^T (+ bias / padding mask in the accumulator)
    v4i S[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const Op kop = *(const Op*)(sK + (kt * 16 + li) * KSTR + KPL * g);
      v4i c0 = {0, 0, 0, 0};
      if (BIAS) {
        c0 = *(const v4i*)(p.bias + ((int64_t)h * NP + qrow) * NP + kt * 16 + 4 * g);
      } else if (kt == KT - 1) {
        c0 = cmask;
      }
      S[kt] = Mfma<D>::run(kop, qop, c0);
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
    const int32_t m = clamp127(requant_raw24(amax, alpha, qk_bm));
    // table byte offset of index (m - L) is rb - 128 L; saturating L to
    // [-127, 127] clamps that offset to [lo, hi] (entries past exp_last are 0)
    const int32_t rb = tab0 + m * 128;
    const int32_t lo = rb - 127 * 128;
    const int32_t hi = tab0 + min(m + 127, p.exp_last) * 128;

    // ---- pass 2: e << e_shift from the table, row sum
    uint32_t s = 0;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t a = exp_offset(S[kt][r], alpha, qk_bm, -128, rb, lo, hi);
        const uint32_t e = lds_read_u32((uint32_t)a);
        S[kt][r] = (int32_t)e;
        s += e;
      }
    }
    if (npad) {
      const int32_t a = min(max(rb - lpad * 128, lo), hi);
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
        const v4i vop = *(const v4i*)(sV + (ft * 16 + li) * VTSTR + ks * 64 + 16 * g);
        O[ft] = mfma64(vop, pop, O[ft]);
      }
    }

    // ---- epilogue: lane holds features 16 ft + 4 g + r of query qrow
    if (qrow < N) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        int32_t y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (p.pv_fast)
            y[r] = clamp127(__mul24(O[ft][r], p.pv_b) >> p.pv_c);
          else
            y[r] = requant_i8(O[ft][r], p.pv_b, p.pv_c);
        }
        *(uint32_t*)(p.out + hbase + (int64_t)qrow * D + ft * 16 + 4 * g) =
            pack4_lowbytes((uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]);
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
