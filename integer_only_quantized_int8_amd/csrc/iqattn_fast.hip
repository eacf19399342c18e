// iqattn_fast.hip -- fused integer-only attention specialised on the number of
// 16-key tiles (KT, so N in (16(KT-1), 16 KT]) for the parameter ranges in
// which every step fits 32-bit VALU arithmetic (the host checks them).
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
// from the row sum once per lane, and their V rows are zero in LDS.
//
// LDS layout (no padding): K as 64-byte rows (d = 64) whose four 16-byte
// chunks are XOR-swizzled by (row >> 1) & 3, which makes the b128 operand
// reads of 16 rows x 4 chunks bank-conflict free on gfx950 (d = 32 keeps
// 48-byte padded rows); V^T as [64-key step][feature][64 bytes] with the same
// swizzle (V row-major for the VALU LIS back end); one exponential table.
//
// Method passages: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" and sec. 3.3 "Integer-only Softmax: Shiftmax"; FQ-ViT
// abstract (Log-Int-Softmax, 4-bit log2 codes, BitShift); Trio-ViT sec. IV
// Eq. 11 (leading-one log2 with the next bit).
#include "iqattn_dev.h"
#include "iqattn.h"

namespace iqattn {
namespace {

// byte offset of 16-byte chunk `c` of 64-byte row `r` after the XOR swizzle
__device__ __forceinline__ int swz64(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

// LIS shift w = F - code for the probability Ph (Ph < 2^24):
// code = F - ilog2r(Ph) clipped to [0, F], Ph = 0 -> code F.  ilog2r(x) is the
// leading-one index plus the next bit; for x < 2^24 the float conversion is
// exact, its mantissa's top bit is that next bit, and adding 2^22 to the bit
// pattern carries it into the exponent.
__device__ __forceinline__ int32_t lis_shift(uint32_t ph, int32_t F) {
  const uint32_t bits = __float_as_uint((float)ph) + 0x400000u;
  return min(max((int32_t)(bits >> 23) - 127, 0), F);
}

// LIS bit-plane operand bytes of four shifts: plane 0 gets -2^w for w < 8,
// plane 1 gets -2^(w-8) for w >= 8 (as int8 bytes 0xFF << l).
__device__ __forceinline__ void lis_planes(const v4i& w, int32_t& lo, int32_t& hi) {
  uint32_t y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)  // 16-bit (plane 1 byte, plane 0 byte)
    y[r] = (0xFFu << w[r]) & (0xFFu << (w[r] & 8));
  const uint32_t t01 = __builtin_amdgcn_perm(y[1], y[0], 0x05010400u);
  const uint32_t t23 = __builtin_amdgcn_perm(y[3], y[2], 0x05010400u);
  lo = (int32_t)__builtin_amdgcn_perm(t23, t01, 0x05040100u);
  hi = (int32_t)__builtin_amdgcn_perm(t23, t01, 0x07060302u);
}

template <int D, int KT, bool BIAS, int VAR>
__global__ __launch_bounds__(kThreads) void iqattn_fast(DevParams p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  constexpr bool KSWZ = (D == 64);      // swizzled 64-byte K rows
  constexpr int KSTR = KSWZ ? 64 : D + 16;
  constexpr int KPL = D / 4;            // k-bytes per lane in the Q.K^T MFMA
  constexpr int KS = (KT + 3) / 4;      // 64-key steps of the P.V MFMA
  constexpr int NP = KT * 16;
  constexpr int FT = D / 16;
  constexpr int K_BYTES = NP * KSTR;
  constexpr bool VROW = (VAR == kFastLisValu);  // V row-major instead of V^T
  constexpr int V_BYTES = VROW ? NP * D : KS * D * 64;
  typedef typename Mfma<D>::Op Op;

  const int N = p.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;

  // Work unit.  Blocks below n_full take one whole head; the heads left over
  // for a last, partial round of blocks are split into quarter heads (query
  // tiles q, q+4, ... for quarter q), so that round is a quarter as long.  The
  // four quarters of a head sit 8 blocks apart: blocks are dealt to the 8
  // XCDs round-robin, so they share an L2 for the K/V reads.
  int u, qt0, qstep;
  if ((int)blockIdx.x < p.n_full) {
    u = blockIdx.x;
    qt0 = (wave + kWaves - (u & (kWaves - 1))) & (kWaves - 1);  // rotate the extra tile
    qstep = kWaves;
  } else {
    const int r = blockIdx.x - p.n_full;
    const int k = r >> 3, q = k & 3;
    u = p.n_full + (k >> 2) * 8 + (r & 7);
    if (u >= p.units) return;  // uniform over the block, before any barrier
    qt0 = q + 4 * wave;
    qstep = 4 * kWaves;
  }

  int8_t* sK = smem;
  int8_t* sV = smem + K_BYTES;
  const char* sE = (const char*)(smem + K_BYTES + V_BYTES);
  int32_t* sW = (int32_t*)(smem + K_BYTES + V_BYTES + (((p.exp_last + 1) * 4 + 15) & ~15));

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
  if (VROW) {
    // ---- stage V row-major (rows >= N are zero)
    for (int i = tid; i < NP * (D / 16); i += kThreads) {
      const int row = i / (D / 16), c16 = i % (D / 16);
      v4i val = {0, 0, 0, 0};
      if (row < N) val = *(const v4i*)(gV + row * D + c16 * 16);
      *(v4i*)(sV + row * D + c16 * 16) = val;
    }
  } else {
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
  }
  // ---- stage the exponential table (entries e << e_shift)
  {
    uint32_t* dstE = (uint32_t*)sE;
    for (int i = tid; i <= p.exp_last; i += kThreads) dstE[i] = p.exp_tab[i];
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
  const int32_t tab0 = (int32_t)lds_addr(sE);  // absolute LDS address of entry 0
  // per-lane operand offsets (swizzled rows: the swizzle depends on li only)
  const int koff = KSWZ ? swz64(li, g) : li * KSTR + KPL * g;
  const int voff = swz64(li, g);
  const int h = u % p.heads;
  const int32_t qk_bm = p.qk_bm;
  const int32_t lpad = mulhi_i32(p.mask_s, qk_bm);

  for (int qt = qt0; qt < KT; qt += qstep) {
    const int qrow = qt * 16 + li;
    Op qop = Op{};
    if (qrow < N) qop = *(const Op*)(p.q + hbase + (int64_t)qrow * D + KPL * g);

    // ---- S^T = K . Q^T (+ bias / padding mask in the accumulator).  K
    //      operands are read one tile ahead; the scheduling barriers keep the
    //      compiler from hoisting every LDS read of a phase (registers)
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
    // table address of index (m - L) is rb - 4 L; saturating L to [-127, 127]
    // clamps it to [lo, hi] (entries past exp_last are 0)
    const int32_t rb = tab0 + m * 4;
    const int32_t lo = rb - 127 * 4;
    const int32_t hi = tab0 + min(m + 127, p.exp_last) * 4;

    // ---- pass 2: e << e_shift from the table, row sum
    uint32_t s = 0;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t a = exp_offset(S[kt][r], qk_bm, -4, rb, lo, hi);
        const uint32_t e = lds_read_u32((uint32_t)a);
        S[kt][r] = (int32_t)e;
        s += e;
      }
    }
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
    __builtin_amdgcn_sched_barrier(0);

    if (VAR == kFastShiftmax) {
      // ---- P = (f e) >> (M - k_out + 1) as one mulhi, O^T = V^T . P^T
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
      // lane holds features 16 ft + 4 g + r of query qrow
      if (qrow < N) {
        int8_t* dst = p.out + hbase + (int64_t)qrow * D + 4 * g;
        if (p.pv_fast) {
#pragma unroll
          for (int ft = 0; ft < FT; ++ft)
            *(uint32_t*)(dst + ft * 16) = pack4_lowbytes(
                (uint32_t)clamp127(mulhi_i32(O[ft][0], p.pv_bm)),
                (uint32_t)clamp127(mulhi_i32(O[ft][1], p.pv_bm)),
                (uint32_t)clamp127(mulhi_i32(O[ft][2], p.pv_bm)),
                (uint32_t)clamp127(mulhi_i32(O[ft][3], p.pv_bm)));
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
    } else {
      // ---- LIS: Ph = (f e) >> (M - F) as one mulhi, shift w = F - code
      const int32_t Fl = p.lis_f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[kt][r] = lis_shift(mulhi_u32((uint32_t)S[kt][r], F), Fl);

      if (VAR == kFastLisMfma) {
        // ---- o = -(O_0 + 256 O_1), O_h = V^T . (plane h of -2^w)^T
        v4i O0[FT], O1[FT];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) O0[ft] = O1[ft] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          v4i plo, phi;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int kt = ks * 4 + tt;
            int32_t lo_w = 0, hi_w = 0;
            if (kt < KT) lis_planes(S[kt], lo_w, hi_w);
            plo[tt] = lo_w;
            phi[tt] = hi_w;
          }
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            const v4i vop = *(const v4i*)(sV + ks * (D * 64) + ft * 16 * 64 + voff);
            O0[ft] = mfma64(vop, plo, O0[ft]);
            O1[ft] = mfma64(vop, phi, O1[ft]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (qrow < N) {
          int8_t* dst = p.out + hbase + (int64_t)qrow * D + 4 * g;
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            int32_t y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int32_t o = -(O0[ft][r] + (O1[ft][r] << 8));
              y[r] = p.pv_fast ? clamp127(mulhi_i32(o, p.pv_bm)) : requant_i8(o, p.pv_b, p.pv_c);
            }
            *(uint32_t*)(dst + ft * 16) =
                pack4_lowbytes((uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]);
          }
        }
      } else {
        // ---- VALU P.V: lane owns feature t of QPL queries; the wave's shifts
        //      go through LDS one 16-key tile at a time (16 keys x 16 queries)
        constexpr int QPL = 16 * D / 64;
        const int t = lane % D;
        const int qsub = (lane / D) * QPL;
        int32_t* sWw = sW + wave * 256;
        int32_t o[QPL];
#pragma unroll
        for (int i = 0; i < QPL; ++i) o[i] = 0;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sWw[(4 * g + r) * 16 + li] = S[kt][r];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 4
          for (int jj = 0; jj < 16; ++jj) {
            const int32_t vj = (int32_t)sV[(kt * 16 + jj) * D + t];  // 0 for padded keys
            const v4i* wrow = (const v4i*)(sWw + jj * 16 + qsub);
#pragma unroll
            for (int i4 = 0; i4 < QPL / 4; ++i4) {
              const v4i w4 = wrow[i4];
#pragma unroll
              for (int r = 0; r < 4; ++r) o[4 * i4 + r] += (int32_t)((uint32_t)vj << w4[r]);
            }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < QPL; ++i) {
          const int qi = qt * 16 + qsub + i;
          if (qi < N) {
            const int32_t y = p.pv_fast ? clamp127(mulhi_i32(o[i], p.pv_bm))
                                        : requant_i8(o[i], p.pv_b, p.pv_c);
            p.out[hbase + (int64_t)qi * D + t] = (int8_t)y;
          }
        }
      }
    }
  }
}

}  // namespace

#define IQ_FAST_CASE(D, KT, B, V) \
  if (d == D && kt == KT && bias == B && var == V) return iqattn_fast<D, KT, B, V>;

KernelFn fast_kernel(int d, int kt, bool bias, int var) {
  // Shiftmax: the workload shapes and the tile counts the tests use
  IQ_FAST_CASE(64, 13, false, kFastShiftmax)
  IQ_FAST_CASE(64, 37, false, kFastShiftmax)
  IQ_FAST_CASE(64, 1, false, kFastShiftmax)
  IQ_FAST_CASE(64, 2, false, kFastShiftmax)
  IQ_FAST_CASE(64, 4, false, kFastShiftmax)
  IQ_FAST_CASE(64, 12, false, kFastShiftmax)
  IQ_FAST_CASE(64, 4, true, kFastShiftmax)
  IQ_FAST_CASE(32, 4, true, kFastShiftmax)
  IQ_FAST_CASE(32, 4, false, kFastShiftmax)
  IQ_FAST_CASE(32, 13, false, kFastShiftmax)
  // Log-Int-Softmax, both P.V engines
  IQ_FAST_CASE(64, 37, false, kFastLisValu)
  IQ_FAST_CASE(64, 37, false, kFastLisMfma)
  IQ_FAST_CASE(64, 1, false, kFastLisValu)
  IQ_FAST_CASE(64, 1, false, kFastLisMfma)
  IQ_FAST_CASE(64, 5, false, kFastLisValu)
  IQ_FAST_CASE(64, 5, false, kFastLisMfma)
  IQ_FAST_CASE(64, 13, false, kFastLisValu)
  IQ_FAST_CASE(64, 13, false, kFastLisMfma)
  IQ_FAST_CASE(32, 4, false, kFastLisValu)
  IQ_FAST_CASE(32, 4, false, kFastLisMfma)
  return nullptr;
}

}  // namespace iqattn
