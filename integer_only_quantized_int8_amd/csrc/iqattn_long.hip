// iqattn_long.hip -- fused integer-only attention for rows longer than the
// register-resident kernels hold (641 to 1024 keys), every parameter set of
// the header, all three back ends.
//
// One workgroup of 16 waves per head (b, h).  K and V of the head reach LDS
// through direct global->LDS loads (rows beyond N arrive as zeros), in the
// swizzled row-major layouts of the specialised kernels; then each wave takes
// 16-query tiles in turn.  A tile's row of up to 64 16-key tiles does not fit
// the registers, so the tile walks the keys three times in blocks of 64
// (four Q.K^T MFMAs per block, recomputed from the LDS-resident K each time):
//   pass A  row max of the accumulators over the real keys (the requantisation
//           is monotone, so it is applied to the maximum alone);
//   pass B  L = clip((b1 acc) >> c1), e = exponential table[m - L], row sum;
//           f = floor(2^M / sum);
//   pass C  e again, then Shiftmax P = min((f e) >> (M - k_out + 1), pmax) and
//           O^T = V^T . P^T by MFMA; or the LIS shift w = F - code with the
//           BitShift sum on VALU or by two bit-plane MFMAs;
//   Out = clip((b2 o) >> c2).
// The arithmetic is the 64-bit form of the generic kernel, so no parameter
// range needs a host check.
//
// Method passages: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" and sec. 3.3 "Integer-only Softmax: Shiftmax"; FQ-ViT
// abstract (Log-Int-Softmax, 4-bit log2 codes, BitShift); Trio-ViT sec. IV
// Eq. 11 (leading-one log2 with the next bit).
#include "iqattn_dev.h"
#include "iqattn.h"

namespace iqattn {
namespace {

constexpr int kLongWaves = 16;  // waves per workgroup (one workgroup per CU: K and V fill LDS)
constexpr int kLongBlk = 4;     // 16-key tiles per key block of a pass (one 64-key P.V step)

// e for the accumulators of one 16-key tile: requantise, index the table by
// m - L (clamped to the table), zero for padded keys (j >= N).
__device__ __forceinline__ void tile_exp(const DevParams& p, const uint32_t* sE, int32_t m,
                                         int kt, int KT, int g, v4i& S) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int32_t L = requant_i8(S[r], p.qk_b, p.qk_c);
    const int32_t idx = min(max(m - L, 0), p.exp_last);
    uint32_t e = sE[idx];
    if (kt == KT - 1 && kt * 16 + 4 * g + r >= p.n) e = 0;
    S[r] = (int32_t)e;
  }
}

template <int D, int VAR, bool BIAS>
__global__ __launch_bounds__(64 * kLongWaves) void iqattn_long(DevParams p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  constexpr int KPL = D / 4;   // k-bytes per lane in the Q.K^T MFMA
  constexpr int FT = D / 16;   // 16-feature tiles of the output
  typedef typename Mfma<D>::Op Op;

  const int N = p.n;
  const int KT = (N + 15) >> 4;           // 16-key (and 16-query) tiles
  const int KS = (KT + 3) >> 2;           // 64-key steps of the P.V MFMA
  const int R = ((KT * 16 * D + 1023) / 1024) * 1024;  // K region bytes (whole 1 KB blocks)
  const int RV = max(R, KS * 64 * D);     // V region: the last step's operand reads reach KS*64 rows
  const int u = blockIdx.x;
  const int h = u % p.heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;

  int8_t* sV = smem;
  int8_t* sK = smem + RV;
  uint32_t* sE = (uint32_t*)(smem + RV + R);
  int32_t* sW = (int32_t*)(smem + RV + R + 1024);  // LIS VALU: [waves][16 keys][16 queries]

  const int64_t hbase = (int64_t)u * N * D;
  const uint32_t hbytes = (uint32_t)(N * D);
  // ---- stage K and V (direct loads, 1 KB per wave instruction; rows >= N
  //      lie past the range and arrive as zeros) and the exponential table
  {
    const v4i rk = make_rsrc(p.k + hbase, hbytes);
    const v4i rv = make_rsrc(p.v + hbase, hbytes);
    const uint32_t kb0 = lds_addr(sK), vb0 = lds_addr(sV);
    for (int blk = wave; blk < R / 1024; blk += kLongWaves) {
      const int o = blk * 1024 + 16 * lane;
      const int row = o / D, cp = (o % D) >> 4;
      raw_buffer_load_lds(rk, (lds_u32w*)(uintptr_t)(kb0 + blk * 1024), 16,
                          row * D + 16 * (cp ^ kswz<D>(row)), 0, 0, 0);
      raw_buffer_load_lds(rv, (lds_u32w*)(uintptr_t)(vb0 + blk * 1024), 16,
                          row * D + 16 * (cp ^ vswz<D>(row)), 0, 0, 0);
    }
    // V rows from R / D up to the last step's reach: zeros
    for (int i = R + 16 * tid; i < RV; i += 16 * 64 * kLongWaves) *(v4i*)(sV + i) = v4i{0, 0, 0, 0};
    for (int i = tid; i <= p.exp_last; i += 64 * kLongWaves) sE[i] = p.exp_tab[i];
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  // per-lane operand offsets: K rows (swizzle depends on li only), V^T
  // transpose reads (as in the specialised kernels)
  const int koff = (D == 64 ? li * 64 + 16 * g : li * 32 + 8 * g) ^ (kswz<D>(li) << 4);
  int vtr[2];
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
    const int kap = 16 * (2 * hr + (li >> 3)) + 4 * g + ((li >> 1) & 3);
    vtr[hr] = kap * D + 8 * (li & 1) + 16 * vswz<D>(kap);
  }
  uint32_t va[FT][2];
  vt_addr<FT>(lds_addr(sV), vtr, va);
  const __amdgpu_buffer_rsrc_t qres = buf_rsrc(p.q + hbase, hbytes);
  int8_t* const gO = p.out + out_head_base(p, u, D);
  const int32_t ostride = out_row_stride(p, D);
  const int Np = KT * 16;

  for (int qt = wave; qt < KT; qt += kLongWaves) {
    const int qrow = min(qt * 16 + li, N - 1);
    const Op qop = buf_load<Op>(qres, qrow * D + KPL * g);
    const int32_t* brow = BIAS ? p.bias + ((int64_t)h * Np + qrow) * Np + 4 * g : nullptr;

    // the Q.K^T accumulators of key block kb (tiles kb .. kb + 3 that exist)
    auto qk_block = [&](int kb, v4i (&S)[kLongBlk]) {
#pragma unroll
      for (int t = 0; t < kLongBlk; ++t) {
        const int kt = kb + t;
        if (kt < KT) {
          const Op kop = *(const Op*)(sK + kt * 16 * D + koff);
          v4i c0 = {0, 0, 0, 0};
          if (BIAS) c0 = *(const v4i*)(brow + kt * 16);
          S[t] = Mfma<D>::run(kop, qop, c0);
        }
      }
    };

    // ---- pass A: row max over the real keys
    int32_t amax = INT32_MIN;
    for (int kb = 0; kb < KT; kb += kLongBlk) {
      v4i S[kLongBlk];
      qk_block(kb, S);
#pragma unroll
      for (int t = 0; t < kLongBlk; ++t) {
        const int kt = kb + t;
        if (kt < KT) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt < KT - 1 || kt * 16 + 4 * g + r < N) amax = max(amax, S[t][r]);
        }
      }
    }
    amax = wave_max4(amax);
    const int32_t m = requant_i8(amax, p.qk_b, p.qk_c);

    // ---- pass B: exponentials and row sum
    uint32_t s = 0;
    for (int kb = 0; kb < KT; kb += kLongBlk) {
      v4i S[kLongBlk];
      qk_block(kb, S);
#pragma unroll
      for (int t = 0; t < kLongBlk; ++t) {
        const int kt = kb + t;
        if (kt < KT) {
          tile_exp(p, sE, m, kt, KT, g, S[t]);
          s += (uint32_t)S[t][0] + (uint32_t)S[t][1] + (uint32_t)S[t][2] + (uint32_t)S[t][3];
        }
      }
    }
    s = wave_sum4(s);
    const uint32_t f = (uint32_t)(((uint64_t)1 << p.intdiv_m) / s);

    // ---- pass C: probabilities (or LIS shifts) and P.V
    if (VAR == kFastShiftmax || VAR == kFastLisMfma) {
      v4i O0[FT], O1[FT];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) O0[ft] = O1[ft] = v4i{0, 0, 0, 0};
      const uint32_t lis_sh = (uint32_t)(p.intdiv_m - p.lis_f);
      for (int kb = 0; kb < KT; kb += kLongBlk) {
        v4i S[kLongBlk];
        qk_block(kb, S);
#pragma unroll
        for (int ksl = 0; ksl < kLongBlk / 4; ++ksl) {
          v4i plo = {0, 0, 0, 0}, phi = {0, 0, 0, 0};
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int t = 4 * ksl + tt, kt = kb + t;
            if (kt < KT) {
              tile_exp(p, sE, m, kt, KT, g, S[t]);
              if (VAR == kFastShiftmax) {
                uint32_t word = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const uint32_t pr = min((f * (uint32_t)S[t][r]) >> p.p_shift, (uint32_t)p.p_max);
                  word |= pr << (8 * r);
                }
                plo[tt] = (int32_t)word;
              } else {
                v4i w;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const uint32_t ph = (f * (uint32_t)S[t][r]) >> lis_sh;
                  w[r] = (ph == 0) ? 0 : min(ilog2r_dev(ph), p.lis_f);
                }
                int32_t lo_w, hi_w;
                lis_planes(w, lo_w, hi_w);
                plo[tt] = lo_w;
                phi[tt] = hi_w;
              }
            }
          }
          const int ks = kb / 4 + ksl;
          if (ks < KS) {
            v4i vop[FT];
            read_vt<FT>(va, (uint32_t)(ks * 64 * D), vop);
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
              O0[ft] = mfma64(vop[ft], plo, O0[ft]);
              if (VAR == kFastLisMfma) O1[ft] = mfma64(vop[ft], phi, O1[ft]);
            }
          }
        }
      }
      // lane holds features 16 ft + 4 g + r of query qt * 16 + li
      if (qt * 16 + li < N) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          uint32_t word = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int32_t o = (VAR == kFastLisMfma) ? -(O0[ft][r] + (O1[ft][r] << 8)) : O0[ft][r];
            word |= ((uint32_t)requant_i8(o, p.pv_b, p.pv_c) & 0xffu) << (8 * r);
          }
          *(uint32_t*)(gO + (int64_t)qrow * ostride + ft * 16 + 4 * g) = word;
        }
      }
    } else {
      // ---- LIS, VALU: lane owns feature t of QPL queries; per 16-key tile the
      //      wave's shifts go through its LDS block [16 keys][16 queries]
      constexpr int QPL = 16 * D / 64;
      const int t = lane % D;
      const int qsub = (lane / D) * QPL;
      const uint32_t lis_sh = (uint32_t)(p.intdiv_m - p.lis_f);
      int32_t* sWw = sW + wave * 256;
      int32_t o[QPL];
#pragma unroll
      for (int i = 0; i < QPL; ++i) o[i] = 0;
      for (int kb = 0; kb < KT; kb += kLongBlk) {
        v4i S[kLongBlk];
        qk_block(kb, S);
#pragma unroll
        for (int tt = 0; tt < kLongBlk; ++tt) {
          const int kt = kb + tt;
          if (kt < KT) {
            tile_exp(p, sE, m, kt, KT, g, S[tt]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t ph = (f * (uint32_t)S[tt][r]) >> lis_sh;
              sWw[(4 * g + r) * 16 + li] = (ph == 0) ? 0 : min(ilog2r_dev(ph), p.lis_f);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int nk = min(16, N - kt * 16);
            for (int jj = 0; jj < nk; ++jj) {
              const int row = kt * 16 + jj;
              const int32_t vj = (int32_t)sV[row * D + (t ^ (vswz<D>(row) << 4))];
              const int32_t* wrow = sWw + jj * 16 + qsub;
#pragma unroll
              for (int i = 0; i < QPL; ++i) o[i] += (int32_t)((uint32_t)vj << wrow[i]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          }
        }
      }
#pragma unroll
      for (int i = 0; i < QPL; ++i) {
        const int qi = qt * 16 + qsub + i;
        if (qi < N) gO[(int64_t)qi * ostride + t] = (int8_t)requant_i8(o[i], p.pv_b, p.pv_c);
      }
    }
  }
}

}  // namespace

// LDS bytes of the long-row kernel: V region, K region, table, LIS VALU scratch
size_t long_lds_bytes(int d, int n, int var) {
  const int kt = (n + 15) / 16, ks = (kt + 3) / 4;
  const size_t r = ((size_t)kt * 16 * d + 1023) / 1024 * 1024;
  const size_t rv = r > (size_t)ks * 64 * d ? r : (size_t)ks * 64 * d;
  return rv + r + 1024 + (var == kFastLisValu ? (size_t)kLongWaves * 1024 : 0);
}

int long_threads() { return 64 * kLongWaves; }

template <int D>
static KernelFn long_pick(int var, bool bias) {
  if (var == kFastShiftmax) return bias ? iqattn_long<D, kFastShiftmax, true> : iqattn_long<D, kFastShiftmax, false>;
  if (var == kFastLisValu) return bias ? iqattn_long<D, kFastLisValu, true> : iqattn_long<D, kFastLisValu, false>;
  return bias ? iqattn_long<D, kFastLisMfma, true> : iqattn_long<D, kFastLisMfma, false>;
}

KernelFn long_kernel(int d, int var, bool bias) {
  return d == 64 ? long_pick<64>(var, bias) : long_pick<32>(var, bias);
}

}  // namespace iqattn
