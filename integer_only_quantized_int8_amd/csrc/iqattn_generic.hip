// iqattn_generic.hip -- the generic fused kernel: any supported shape and
// parameter set, 64-bit requantisation, runtime tile counts.
//
// One work-group (4 wave64s) per attention head (b, h).  The head's K and V
// are staged once into LDS; each wave takes 16-query tiles in turn and keeps
// the tile's whole logit block in registers:
//   S^T = K . Q^T  by int8 MFMA (bias preloaded into the accumulator);
//   pass 1  row max of the accumulators (requantisation is monotone);
//   pass 2  L = requant(S); e = table[max - L]; row sum;  f = floor(2^M / sum);
//   pass 3  Shiftmax: P = min((f e) >> (M - k_out + 1), pmax), O^T = V^T . P^T
//           by MFMA;  LIS: shift w = F - code, P.V as sum_j V_j << w_ij (VALU);
//   Out = clip((pv_b o) >> pv_c).
// MFMA 16x16 accumulator layout: lane l holds rows 4*(l/16)+r of column l%16,
// so with A = K (rows = keys), B = Q^T (columns = queries) lane l owns query
// l%16 and keys 16*kt + 4*(l/16) + r.
#include "iqattn_dev.h"
#include "iqattn.h"

namespace iqattn {
namespace {

// ---------------------------------------------------------------- kernel
// LDS layout (bytes):
//   sK   [Np][D + 16]         keys row-major (rows padded against bank conflicts)
//   sV   Shiftmax: V^T [D][KS*64 + 16] keys permuted (vperm_pos)
//        LIS:      V   [Np][D]          row-major
//   sExp [exp_last + 1][kExpRep] uint32
//   sW   LIS only: [kWaves][16 keys][16 queries] int32 shift amounts
template <int D, int KTM, int VAR, bool BIAS>
__global__ __launch_bounds__(kThreads) void iqattn_generic(DevParams p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  constexpr int KSTR = D + 16;
  constexpr int KPL = D / 4;                 // k-bytes per lane in the QK MFMA
  const int N = p.n;
  const int KT = (N + 15) >> 4;              // key (and query) tiles
  const int KS = (KT + 3) >> 2;              // 64-key steps of the P.V MFMA
  const int Np = KT * 16;
  const int VTSTR = KS * 64 + 16;
  const int u = blockIdx.x;
  const int h = u % p.heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;

  int8_t* sK = smem;
  int8_t* sV = sK + Np * KSTR;
  const int vbytes = (VAR == IQATTN_SHIFTMAX) ? D * VTSTR : Np * D;
  uint32_t* sExp = (uint32_t*)(sV + ((vbytes + 15) & ~15));
  int32_t* sW = (int32_t*)(sExp + (p.exp_last + 1) * kExpRep);

  const int64_t hbase = (int64_t)u * N * D;
  int8_t* const gO = p.out + out_head_base(p, u, D);  // output rows ostride bytes apart
  const int64_t ostride = out_row_stride(p, D);
  const int8_t* gK = p.k + hbase;
  const int8_t* gV = p.v + hbase;

  // ---- stage K (zero rows beyond N)
  for (int i = tid; i < Np * (D / 16); i += kThreads) {
    int row = i / (D / 16), c16 = i % (D / 16);
    v4i val = {0, 0, 0, 0};
    if (row < N) val = *(const v4i*)(gK + row * D + c16 * 16);
    *(v4i*)(sK + row * KSTR + c16 * 16) = val;
  }
  // ---- stage V
  if (VAR == IQATTN_SHIFTMAX) {
    for (int i = tid; i < D * (VTSTR / 4); i += kThreads) ((int32_t*)sV)[i] = 0;
    __syncthreads();
    for (int i = tid; i < N * (D / 4); i += kThreads) {
      int row = i / (D / 4), c4 = i % (D / 4);
      int32_t word = *(const int32_t*)(gV + row * D + c4 * 4);
      int pos = vperm_pos(row);
#pragma unroll
      for (int b = 0; b < 4; ++b) sV[(c4 * 4 + b) * VTSTR + pos] = (int8_t)(word >> (8 * b));
    }
  } else {
    for (int i = tid; i < Np * (D / 16); i += kThreads) {
      int row = i / (D / 16), c16 = i % (D / 16);
      v4i val = {0, 0, 0, 0};
      if (row < N) val = *(const v4i*)(gV + row * D + c16 * 16);
      *(v4i*)(sV + row * D + c16 * 16) = val;
    }
  }
  // ---- stage the exponential table, one copy per bank
  for (int i = tid; i < (p.exp_last + 1) * kExpRep; i += kThreads) sExp[i] = p.exp_tab[i / kExpRep];
  __syncthreads();

  typedef typename Mfma<D>::Op Op;
  const int erep = lane & (kExpRep - 1);

  for (int qt = wave; qt < KT; qt += kWaves) {
    // ---- Q operand: query qt*16 + li, k-bytes [KPL*g, KPL*g + KPL)
    const int qrow = qt * 16 + li;
    Op qop;
    if (qrow < N) {
      qop = *(const Op*)(p.q + hbase + (int64_t)qrow * D + KPL * g);
    } else {
      qop = Op{};
    }
    // ---- S^T = K . Q^T
    v4i S[KTM];
#pragma unroll
    for (int kt = 0; kt < KTM; ++kt) {
      if (kt < KT) {
        Op kop = *(const Op*)(sK + (kt * 16 + li) * KSTR + KPL * g);
        v4i c0 = {0, 0, 0, 0};
        if (BIAS) c0 = *(const v4i*)(p.bias + ((int64_t)h * Np + qrow) * Np + kt * 16 + 4 * g);
        S[kt] = Mfma<D>::run(kop, qop, c0);
      }
    }
    // ---- pass 1: row max of the accumulators (keys < N only)
    int32_t amax = INT32_MIN;
#pragma unroll
    for (int kt = 0; kt < KTM; ++kt) {
      if (kt < KT - 1) {
        amax = max(amax, max(max(S[kt][0], S[kt][1]), max(S[kt][2], S[kt][3])));
      } else if (kt == KT - 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt * 16 + 4 * g + r < N) amax = max(amax, S[kt][r]);
      }
    }
    amax = wave_max4(amax);
    const int32_t m = requant_i8(amax, p.qk_b, p.qk_c);
    // ---- pass 2: exponentials from the table, row sum
    uint32_t s = 0;
#pragma unroll
    for (int kt = 0; kt < KTM; ++kt) {
      if (kt < KT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int32_t L = requant_i8(S[kt][r], p.qk_b, p.qk_c);
          int32_t idx = min(max(m - L, 0), p.exp_last);
          uint32_t e = sExp[idx * kExpRep + erep];
          if (kt == KT - 1 && kt * 16 + 4 * g + r >= N) e = 0;
          S[kt][r] = (int32_t)e;
          s += e;
        }
      }
    }
    s = wave_sum4(s);
    const uint32_t f = (1u << p.intdiv_m) / s;

    if (VAR == IQATTN_SHIFTMAX) {
      // ---- pass 3: P and O^T = V^T . P^T
      constexpr int FT = D / 16;
      v4i O[FT];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) O[ft] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < (KTM + 3) / 4; ++ks) {
        if (ks < KS) {
          v4i pop;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int kt = ks * 4 + tt;
            uint32_t word = 0;
            if (kt < KTM && kt < KT) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                uint32_t pr = (f * (uint32_t)S[kt][r]) >> p.p_shift;
                pr = min(pr, (uint32_t)p.p_max);
                word |= pr << (8 * r);
              }
            }
            pop[tt] = (int32_t)word;
          }
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            v4i vop = *(const v4i*)(sV + (ft * 16 + li) * VTSTR + ks * 64 + 16 * g);
            O[ft] = mfma64(vop, pop, O[ft]);
          }
        }
      }
      // ---- epilogue: lane holds features 16*ft + 4*g + r of query qrow
      if (qrow < N) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          uint32_t word = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int32_t y = requant_i8(O[ft][r], p.pv_b, p.pv_c);
            word |= ((uint32_t)y & 0xffu) << (8 * r);
          }
          *(uint32_t*)(gO + qrow * ostride + ft * 16 + 4 * g) = word;
        }
      }
    } else {
      // ---- pass 3 (LIS): shift amounts w = F - code, then VALU P.V
      const uint32_t lis_shift = (uint32_t)(p.intdiv_m - p.lis_f);
      constexpr int QPL = 16 * D / 64;        // queries per lane in the VALU P.V
      const int t = lane % D;
      const int qsub = (lane / D) * QPL;      // first query of this lane
      int32_t* sWw = sW + wave * 256;
      int32_t o[QPL];
#pragma unroll
      for (int i = 0; i < QPL; ++i) o[i] = 0;
#pragma unroll
      for (int kt = 0; kt < KTM; ++kt) {
        if (kt < KT) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint32_t ph = (f * (uint32_t)S[kt][r]) >> lis_shift;
            int32_t w = (ph == 0) ? 0 : min(ilog2r_dev(ph), p.lis_f);
            sWw[(4 * g + r) * 16 + li] = w;
          }
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          const int nk = min(16, N - kt * 16);
          for (int jj = 0; jj < nk; ++jj) {
            const int32_t vj = (int32_t)sV[(kt * 16 + jj) * D + t];
            const int32_t* wrow = sWw + jj * 16 + qsub;
#pragma unroll
            for (int i = 0; i < QPL; ++i) o[i] += (int32_t)((uint32_t)vj << wrow[i]);
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      }
#pragma unroll
      for (int i = 0; i < QPL; ++i) {
        const int qi = qt * 16 + qsub + i;
        if (qi < N) gO[qi * ostride + t] = (int8_t)requant_i8(o[i], p.pv_b, p.pv_c);
      }
    }
  }
}

}  // namespace

template <int D, int KTM, int VAR, bool BIAS>
static KernelFn ptr() { return iqattn_generic<D, KTM, VAR, BIAS>; }

template <int D, int KTM>
static KernelFn pick3(int variant, bool bias) {
  if (variant == IQATTN_SHIFTMAX) return bias ? ptr<D, KTM, 0, true>() : ptr<D, KTM, 0, false>();
  return bias ? ptr<D, KTM, 1, true>() : ptr<D, KTM, 1, false>();
}

template <int D>
static KernelFn pick2(int kt, int variant, bool bias) {
  if (kt <= 4) return pick3<D, 4>(variant, bias);
  if (kt <= 13) return pick3<D, 13>(variant, bias);
  return pick3<D, 40>(variant, bias);
}

KernelFn generic_kernel(int d, int kt, int variant, bool bias) {
  return d == 64 ? pick2<64>(kt, variant, bias) : pick2<32>(kt, variant, bias);
}

}  // namespace iqattn
