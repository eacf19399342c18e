// iqattn.hip -- fused integer-only int8 multi-head self-attention for gfx950.
//
// One work-group (4 wave64s) per attention head (b, h).  The head's K and V
// are staged once into LDS; each wave takes 16-query tiles in turn and, for
// its tile, keeps the whole logit row block in registers:
//
//   S^T = K . Q^T   v_mfma_i32_16x16x64_i8 (d = 64) / 16x16x32_i8 (d = 32),
//                   one MFMA per 16-key tile, bias preloaded into the
//                   accumulator for windowed attention;
//   pass 1          row max on the int32 accumulators (requantisation is
//                   monotone, so max(L) = requant(max acc)); 4-lane exchange;
//   pass 2          L = requant(acc); e = exp_table[max - L] (LDS, one copy per
//                   bank); row sum; 4-lane exchange;  f = floor(2^M / sum);
//   pass 3 Shiftmax P = min((f e) >> (M - k_out + 1), pmax), packed to int8
//                   in the MFMA B layout, O^T = V^T . P^T by MFMA;
//   pass 3 LIS      code -> shift w = F - code, P.V as sum_j V_j << w_ij on the
//                   VALU (one v_lshl_add per (i, j, t));
//   epilogue        Out = clip((pv_b o) >> pv_c), int8 stores.
//
// MFMA 16x16 accumulator layout (CDNA3/4): lane l holds rows 4*(l/16)+r
// (r = 0..3) of column l%16.  With A = K (rows = keys) and B = Q^T (columns =
// queries), lane l owns query l%16 and keys 16*kt + 4*(l/16) + r, so every
// row reduction is lane-local plus an exchange among lanes l, l^16, l^32, l^48.
// For P.V the same lane already holds P in the B-operand layout (query l%16,
// k-group l/16); V^T is staged with its keys permuted so that the A operand's
// k-slot (group g, byte p) holds the key the B operand has in that slot.
//
// Method passages: I-ViT (mer.run summary) sec. 3.2 (dyadic requantisation)
// and sec. 3.3 (Shiftmax); FQ-ViT abstract (Log-Int-Softmax, 4-bit log2,
// BitShift); Trio-ViT sec. IV Eq. 11 (leading-one log2) and Eq. 12 (b, c).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "iqattn.h"

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef int32_t v2i __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kExpRep = 32;  // copies of the exponential table, one per LDS bank

struct DevParams {
  const int8_t* q;
  const int8_t* k;
  const int8_t* v;
  int8_t* out;
  const uint32_t* exp_tab;  // [256]: e(-idx)
  const int32_t* bias;      // [heads][Np][Np] expanded, zero-padded (query-major)
  int32_t heads, n, units;
  int32_t qk_b, qk_c, pv_b, pv_c;
  int32_t exp_last;         // entries 0..exp_last are staged; all later ones are 0
  int32_t intdiv_m, p_shift, p_max;
  int32_t lis_f;
};

// ---------------------------------------------------------------- helpers
// floor((b * x) / 2^c) saturated to [-127, 127]; 64-bit product.
__device__ __forceinline__ int32_t requant_i8(int32_t x, int32_t b, int32_t c) {
  int64_t y = ((int64_t)b * (int64_t)x) >> c;  // arithmetic shift = floor
  y = y < -127 ? -127 : (y > 127 ? 127 : y);
  return (int32_t)y;
}

__device__ __forceinline__ int32_t wave_max4(int32_t x) {
  x = max(x, __shfl_xor(x, 16));
  x = max(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ uint32_t wave_sum4(uint32_t x) {
  x += (uint32_t)__shfl_xor((int)x, 16);
  x += (uint32_t)__shfl_xor((int)x, 32);
  return x;
}

// position of key kappa inside its 64-key block of the staged V^T rows:
// key 16*tt + 4*g + r sits at byte 16*g + 4*tt + r.
__device__ __forceinline__ int vperm_pos(int kappa) {
  int base = kappa & ~63, w = kappa & 63;
  return base + ((w & 15) >> 2) * 16 + (w >> 4) * 4 + (w & 3);
}

// leading-one log2 with rounding: index of the leading one plus the next bit.
__device__ __forceinline__ int32_t ilog2r_dev(uint32_t x) {
  int32_t k = 31 - __clz((int)x);
  int32_t nb = (k >= 1) ? (int32_t)((x >> (k - 1)) & 1u) : 0;
  return k + nb;
}

template <int D>
struct Mfma;

template <>
struct Mfma<64> {
  typedef v4i Op;
  static __device__ __forceinline__ v4i run(Op a, Op b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<32> {
  typedef int64_t Op;
  static __device__ __forceinline__ v4i run(Op a, Op b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- kernel
// LDS layout (bytes):
//   sK   [Np][D + 16]         keys row-major (rows padded against bank conflicts)
//   sV   Shiftmax: V^T [D][KS*64 + 16] keys permuted (vperm_pos)
//        LIS:      V   [Np][D]          row-major
//   sExp [exp_last + 1][kExpRep] uint32
//   sW   LIS only: [kWaves][16 keys][16 queries] int32 shift amounts
template <int D, int KTM, int VAR, bool BIAS>
__global__ __launch_bounds__(kThreads) void iqattn_fused(DevParams p) {
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
            O[ft] = __builtin_amdgcn_mfma_i32_16x16x64_i8(vop, pop, O[ft], 0, 0, 0);
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
          *(uint32_t*)(p.out + hbase + (int64_t)qrow * D + ft * 16 + 4 * g) = word;
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
        if (qi < N) p.out[hbase + (int64_t)qi * D + t] = (int8_t)requant_i8(o[i], p.pv_b, p.pv_c);
      }
    }
  }
}

// ---------------------------------------------------------------- set-up kernels
// e(-idx) for idx = 0..255: the Shiftmax exponential of delta = -idx
// (I-ViT sec. 3.3), with exp_frac_bits extra fraction bits.
__global__ void iqattn_build_exp(uint32_t* tab, int32_t i0, int32_t nfrac) {
  const int idx = threadIdx.x;
  if (idx > 255) return;
  const int32_t d = -idx;
  const int32_t ip = d + (d >> 1) - (d >> 4);
  const int32_t np = -ip;                   // >= 0
  const int32_t q = np / i0, r = np - q * i0;
  const int64_t mant = (int64_t)i0 + ((-r) >> 1);
  tab[idx] = (q >= 62) ? 0u : (uint32_t)((mant << nfrac) >> q);
}

// bias[h][i][j] = T[h][(ri - rj + w - 1)(2w - 1) + (ci - cj + w - 1)] for
// query i < N and key j < N, zero elsewhere; [heads][Np][Np].
__global__ void iqattn_expand_bias(int32_t* out, const int32_t* table, int32_t heads,
                                   int32_t n, int32_t np, int32_t w) {
  const int64_t total = (int64_t)heads * np * np;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(x % np), i = (int)((x / np) % np), h = (int)(x / ((int64_t)np * np));
    int32_t val = 0;
    if (i < n && j < n) {
      const int dr = i / w - j / w, dc = i % w - j % w;
      val = table[(int64_t)h * (2 * w - 1) * (2 * w - 1) + (dr + w - 1) * (2 * w - 1) + dc + w - 1];
    }
    out[x] = val;
  }
}

// ---------------------------------------------------------------- host side
typedef void (*KernelFn)(DevParams);

template <int D, int KTM, int VAR, bool BIAS>
KernelFn kernel_ptr() { return iqattn_fused<D, KTM, VAR, BIAS>; }

template <int D, int KTM>
KernelFn pick3(int variant, bool bias) {
  if (variant == IQATTN_SHIFTMAX) return bias ? kernel_ptr<D, KTM, 0, true>() : kernel_ptr<D, KTM, 0, false>();
  return bias ? kernel_ptr<D, KTM, 1, true>() : kernel_ptr<D, KTM, 1, false>();
}

template <int D>
KernelFn pick2(int kt, int variant, bool bias) {
  if (kt <= 4) return pick3<D, 4>(variant, bias);
  if (kt <= 13) return pick3<D, 13>(variant, bias);
  return pick3<D, 40>(variant, bias);
}

thread_local char g_errbuf[256];

int set_hip_error(hipError_t e, const char* what) {
  snprintf(g_errbuf, sizeof(g_errbuf), "%s: %s", what, hipGetErrorString(e));
  return IQATTN_E_LAUNCH;
}

}  // namespace

struct iqattn_ctx {
  iqattn_params p;
  int device;
  uint32_t* exp_tab;
  int32_t* bias;
  KernelFn fn;
  size_t lds_bytes;
  DevParams dp;
};

static int validate(const iqattn_params* p) {
  if (!p) return IQATTN_E_NULL;
  if (p->batch < 0 || p->heads < 1) return IQATTN_E_SHAPE;
  if (p->seq_len < 1 || p->seq_len > IQATTN_MAX_SEQ) return IQATTN_E_SHAPE;
  if (p->head_dim != 32 && p->head_dim != 64) return IQATTN_E_SHAPE;
  if ((int64_t)p->batch * p->heads > INT32_MAX) return IQATTN_E_SHAPE;
  if (p->qk_b < 1 || p->pv_b < 1) return IQATTN_E_INVAL;
  if (p->qk_c < 0 || p->qk_c > 62 || p->pv_c < 0 || p->pv_c > 62) return IQATTN_E_INVAL;
  if (p->i0 < 1 || p->exp_frac_bits < 0 || p->exp_frac_bits > 22) return IQATTN_E_INVAL;
  if ((int64_t)p->i0 << p->exp_frac_bits > (1 << 22)) return IQATTN_E_INVAL;
  if (p->k_out < 2 || p->k_out > 8) return IQATTN_E_INVAL;
  if (p->intdiv_m < p->k_out - 1 || p->intdiv_m > 31) return IQATTN_E_INVAL;
  if (p->variant != IQATTN_SHIFTMAX && p->variant != IQATTN_LIS) return IQATTN_E_INVAL;
  if (p->variant == IQATTN_LIS) {
    if (p->lis_bits < 1 || p->lis_bits > 4) return IQATTN_E_INVAL;
    if (p->intdiv_m < (1 << p->lis_bits) - 1) return IQATTN_E_INVAL;
  }
  if (p->rel_bias == NULL) {
    if (p->window != 0) return IQATTN_E_INVAL;
  } else {
    if (p->window < 1 || (int64_t)p->window * p->window != p->seq_len) return IQATTN_E_SHAPE;
    const int64_t span = (int64_t)(2 * p->window - 1) * (2 * p->window - 1) * p->heads;
    for (int64_t i = 0; i < span; ++i)
      if (p->rel_bias[i] > (1 << 30) || p->rel_bias[i] < -(1 << 30)) return IQATTN_E_INVAL;
  }
  return IQATTN_OK;
}

extern "C" int iqattn_create(const iqattn_params* p, iqattn_ctx** out) {
  if (!out) return IQATTN_E_NULL;
  *out = NULL;
  int rc = validate(p);
  if (rc) return rc;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return IQATTN_E_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return IQATTN_E_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return IQATTN_E_DEVICE;

  iqattn_ctx* c = (iqattn_ctx*)calloc(1, sizeof(iqattn_ctx));
  if (!c) return IQATTN_E_ALLOC;
  c->p = *p;
  c->p.rel_bias = NULL;
  c->device = dev;

  const int N = p->seq_len, D = p->head_dim;
  const int KT = (N + 15) / 16, KS = (KT + 3) / 4, Np = KT * 16;
  hipError_t e;
  if ((e = hipMalloc((void**)&c->exp_tab, 256 * sizeof(uint32_t))) != hipSuccess) {
    free(c);
    return IQATTN_E_ALLOC;
  }
  hipLaunchKernelGGL(iqattn_build_exp, dim3(1), dim3(256), 0, 0, c->exp_tab, p->i0,
                     p->exp_frac_bits);
  if ((e = hipGetLastError()) != hipSuccess) { rc = set_hip_error(e, "build_exp"); goto fail; }
  if (p->rel_bias) {
    const size_t tbytes = (size_t)p->heads * (2 * p->window - 1) * (2 * p->window - 1) * 4;
    const size_t ebytes = (size_t)p->heads * Np * Np * 4;
    int32_t* tab = NULL;
    if (hipMalloc((void**)&c->bias, ebytes) != hipSuccess) { rc = IQATTN_E_ALLOC; goto fail; }
    if (hipMalloc((void**)&tab, tbytes) != hipSuccess) { rc = IQATTN_E_ALLOC; goto fail; }
    if ((e = hipMemcpy(tab, p->rel_bias, tbytes, hipMemcpyHostToDevice)) != hipSuccess) {
      (void)hipFree(tab);
      rc = set_hip_error(e, "bias copy");
      goto fail;
    }
    hipLaunchKernelGGL(iqattn_expand_bias, dim3(256), dim3(256), 0, 0, c->bias, tab, p->heads,
                       N, Np, p->window);
    e = hipDeviceSynchronize();
    (void)hipFree(tab);
    if (e != hipSuccess) { rc = set_hip_error(e, "expand_bias"); goto fail; }
  }
  {
    uint32_t host_tab[256];
    if ((e = hipMemcpy(host_tab, c->exp_tab, sizeof(host_tab), hipMemcpyDeviceToHost)) != hipSuccess) {
      rc = set_hip_error(e, "exp table");
      goto fail;
    }
    int last = 255;
    for (int i = 0; i < 256; ++i)
      if (host_tab[i] == 0) { last = i; break; }
    c->dp.exp_last = last;
  }
  {
    const size_t kbytes = (size_t)Np * (D + 16);
    const size_t vbytes = (p->variant == IQATTN_SHIFTMAX) ? (size_t)D * (KS * 64 + 16) : (size_t)Np * D;
    c->lds_bytes = kbytes + ((vbytes + 15) & ~(size_t)15) + (size_t)(c->dp.exp_last + 1) * kExpRep * 4 +
                   (p->variant == IQATTN_LIS ? (size_t)kWaves * 256 * 4 : 0);
    int maxlds = 0, optin = 0;
    (void)hipDeviceGetAttribute(&maxlds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    (void)hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev);
    if (optin > maxlds) maxlds = optin;
    if ((int64_t)c->lds_bytes > maxlds) { rc = IQATTN_E_SHAPE; goto fail; }
    c->fn = (D == 64) ? pick2<64>(KT, p->variant, p->rel_bias != NULL)
                      : pick2<32>(KT, p->variant, p->rel_bias != NULL);
    if ((e = hipFuncSetAttribute((const void*)c->fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)c->lds_bytes)) != hipSuccess) {
      rc = set_hip_error(e, "lds attribute");
      goto fail;
    }
  }
  c->dp.exp_tab = c->exp_tab;
  c->dp.bias = c->bias;
  c->dp.heads = p->heads;
  c->dp.n = N;
  c->dp.units = p->batch * p->heads;
  c->dp.qk_b = p->qk_b;
  c->dp.qk_c = p->qk_c;
  c->dp.pv_b = p->pv_b;
  c->dp.pv_c = p->pv_c;
  c->dp.intdiv_m = p->intdiv_m;
  c->dp.p_shift = p->intdiv_m - (p->k_out - 1);
  c->dp.p_max = (1 << (p->k_out - 1)) - 1;
  c->dp.lis_f = (1 << p->lis_bits) - 1;
  if ((e = hipDeviceSynchronize()) != hipSuccess) { rc = set_hip_error(e, "create"); goto fail; }
  *out = c;
  return IQATTN_OK;
fail:
  if (c->exp_tab) (void)hipFree(c->exp_tab);
  if (c->bias) (void)hipFree(c->bias);
  free(c);
  return rc;
}

extern "C" int iqattn_forward(iqattn_ctx* c, const int8_t* q, const int8_t* k, const int8_t* v,
                              int8_t* out, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  if (c->dp.units == 0) return IQATTN_OK;
  if (!q || !k || !v || !out) return IQATTN_E_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return IQATTN_E_ALIGN;
  DevParams dp = c->dp;
  dp.q = q;
  dp.k = k;
  dp.v = v;
  dp.out = out;
  hipLaunchKernelGGL(c->fn, dim3(dp.units), dim3(kThreads), c->lds_bytes, (hipStream_t)hip_stream, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqattn_fused launch");
  return IQATTN_OK;
}

extern "C" int iqattn_destroy(iqattn_ctx* c) {
  if (!c) return IQATTN_OK;
  int dev = 0;
  (void)hipGetDevice(&dev);
  (void)hipSetDevice(c->device);
  if (c->exp_tab) (void)hipFree(c->exp_tab);
  if (c->bias) (void)hipFree(c->bias);
  (void)hipSetDevice(dev);
  free(c);
  return IQATTN_OK;
}

extern "C" const char* iqattn_strerror(int code) {
  switch (code) {
    case IQATTN_OK: return "success";
    case IQATTN_E_INVAL: return "invalid parameter value";
    case IQATTN_E_SHAPE: return "unsupported shape (B, H, N, d or window)";
    case IQATTN_E_ALLOC: return "device allocation failed";
    case IQATTN_E_LAUNCH: return g_errbuf[0] ? g_errbuf : "HIP launch failed";
    case IQATTN_E_NULL: return "required pointer is NULL";
    case IQATTN_E_ALIGN: return "tensor pointer not 16-byte aligned";
    case IQATTN_E_DEVICE: return "no usable gfx950 device";
    default: return "unknown error code";
  }
}
