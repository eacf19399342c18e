// iqattn_api.hip -- the C ABI of libiqattn (include/iqattn.h): parameter
// checks, device constants built by set-up kernels, kernel selection, launch.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "iqattn.h"
#include "iqattn_dev.h"

using namespace iqattn;

namespace iqattn {
// last HIP error text of this thread, for iqattn_strerror(IQATTN_E_LAUNCH)
thread_local char g_errbuf[256];

int set_hip_error(hipError_t e, const char* what) {
  snprintf(g_errbuf, sizeof(g_errbuf), "%s: %s", what, hipGetErrorString(e));
  return IQATTN_E_LAUNCH;
}
}  // namespace iqattn

namespace {

// e(-idx) << shift for idx = 0..255: the Shiftmax exponential of
// delta = -idx (I-ViT sec. 3.3) with exp_frac_bits extra fraction bits:
//   I_p = d + (d >> 1) - (d >> 4);  -I_p = q i0 + r;  e = ((i0 + ((-r) >> 1)) << n) >> q
__global__ void iqattn_build_exp(uint32_t* tab, int32_t i0, int32_t nfrac, int32_t shift,
                                 uint32_t* status_clear) {
  const int idx = threadIdx.x;
  if (idx == 0 && status_clear) *status_clear = 0u;
  if (idx > 255) return;
  const int32_t d = -idx;
  const int32_t ip = d + (d >> 1) - (d >> 4);
  const int32_t np = -ip;  // >= 0
  const int32_t q = np / i0, r = np - q * i0;
  const int64_t mant = (int64_t)i0 + ((-r) >> 1);
  const uint64_t e = (q >= 62) ? 0u : (uint64_t)((mant << nfrac) >> q);
  tab[idx] = (uint32_t)(e << shift);
}

// bias[h][i][j] = T[h][(ri - rj + w - 1)(2w - 1) + (ci - cj + w - 1)] for
// query i < N and key j < N, `pad` elsewhere; layout [heads][Np][Np].
__global__ void iqattn_expand_bias(int32_t* out, const int32_t* table, int32_t heads, int32_t n,
                                   int32_t np, int32_t w, int32_t pad) {
  const int64_t total = (int64_t)heads * np * np;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(x % np), i = (int)((x / np) % np), h = (int)(x / ((int64_t)np * np));
    int32_t val = pad;
    if (i < n && j < n) {
      const int dr = i / w - j / w, dc = i % w - j % w;
      val = table[(int64_t)h * (2 * w - 1) * (2 * w - 1) + (dr + w - 1) * (2 * w - 1) + dc + w - 1];
    }
    out[x] = val;
  }
}

// Index of the first zero entry of the table iqattn_build_exp writes (255 if
// none): the same integer steps on the host, so that no read-back is needed.
int host_exp_last(int32_t i0, int32_t nfrac, int32_t shift) {
  for (int idx = 0; idx < 256; ++idx) {
    const int32_t d = -idx;
    const int32_t ip = d + (d >> 1) - (d >> 4);
    const int32_t np = -ip;
    const int32_t q = np / i0, r = np - q * i0;
    const int64_t mant = (int64_t)i0 + ((-r) >> 1);
    const uint64_t e = (q >= 62) ? 0u : (uint64_t)((mant << nfrac) >> q);
    if ((uint32_t)(e << shift) == 0) return idx;
  }
  return 255;
}

// The relative-position table passed by value (the no-allocation entry point
// has no device buffer to copy it into).
constexpr int kArgBiasMax = 960;  // int32 entries: heads * (2w - 1)^2
struct BiasArg {
  int32_t v[kArgBiasMax];
};

__global__ void iqattn_expand_bias_arg(int32_t* out, BiasArg table, int32_t heads, int32_t n,
                                       int32_t np, int32_t w, int32_t pad) {
  const int64_t total = (int64_t)heads * np * np;
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(x % np), i = (int)((x / np) % np), h = (int)(x / ((int64_t)np * np));
    int32_t val = pad;
    if (i < n && j < n) {
      const int dr = i / w - j / w, dc = i % w - j % w;
      val = table.v[h * (2 * w - 1) * (2 * w - 1) + (dr + w - 1) * (2 * w - 1) + dc + w - 1];
    }
    out[x] = val;
  }
}

int validate(const iqattn_params* p) {
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
    if (p->lis_engine != IQATTN_LIS_VALU && p->lis_engine != IQATTN_LIS_MFMA) return IQATTN_E_INVAL;
  }
  if (p->out_layout != IQATTN_OUT_HEADS && p->out_layout != IQATTN_OUT_TOKENS) return IQATTN_E_INVAL;
  // token-major output: one head's rows span (N - 1) H d + d bytes, addressed
  // with 32-bit offsets in the kernels
  if (p->out_layout == IQATTN_OUT_TOKENS &&
      (int64_t)p->heads * p->seq_len * p->head_dim > INT32_MAX)
    return IQATTN_E_SHAPE;
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

// Back end of the specialised kernel for these parameters.
int fast_variant(const iqattn_params* p) {
  if (p->variant == IQATTN_SHIFTMAX) return kFastShiftmax;
  return p->lis_engine == IQATTN_LIS_MFMA ? kFastLisMfma : kFastLisValu;
}

// Constants of the specialised kernel, or false if some step of it would
// leave its 32-bit range for these parameters (the generic kernel runs then).
bool fast_constants(const iqattn_params* p, int kt, int64_t bias_max, DevParams* dp) {
  const int var = fast_variant(p);
  if (!fast_kernel(p->head_dim, kt, p->rel_bias != NULL, var)) return false;
  // requantisation: floor(b x / 2^c) = mulhi32(x, b << (32 - c)) for
  // b << (32 - c) < 2^31; padded keys carry mask_s = -(smax + 1), below every
  // real accumulator; every raw logit then fits the 24-bit v_mad_i32_i24.
  // Inputs are any int8 values: |q_t k_t| <= 128 * 128 (both -128), so
  // |acc| <= d * 128 * 128 + bias_max.
  if (p->qk_c > 32 || p->qk_c < 1) return false;
  if (((int64_t)p->qk_b << (32 - p->qk_c)) >= ((int64_t)1 << 31)) return false;
  const int64_t smax = (int64_t)p->head_dim * 128 * 128 + bias_max;
  if ((((smax + 1) * p->qk_b) >> p->qk_c) >= (1 << 22)) return false;
  // IntDiv product: floor(e f / 2^sh) = mulhi32(e 2^ea, f 2^fb), ea + fb = 32 - sh,
  // sh = M - (k_out - 1) (Shiftmax) or M - F (LIS); the table holds e 2^ea
  const int64_t e0 = (int64_t)p->i0 << p->exp_frac_bits;
  const int64_t two_m = (int64_t)1 << p->intdiv_m;
  const int F = (1 << p->lis_bits) - 1;
  const int sh = (var == kFastShiftmax) ? p->intdiv_m - (p->k_out - 1) : p->intdiv_m - F;
  if (sh < 0 || sh > 32 || p->intdiv_m > 30) return false;
  const int64_t np = (int64_t)kt * 16;
  if (np * e0 >= (1 << 24)) return false;           // exact float row sum
  // the expanded bias is read through a buffer resource with 32-bit offsets
  if (p->rel_bias && (int64_t)p->heads * np * np * 4 > INT32_MAX) return false;
  if (two_m / e0 > (1 << 22)) return false;         // reciprocal estimate within 1/2
  const bool pow2 = (e0 & (e0 - 1)) == 0 && e0 <= two_m;
  if (var == kFastShiftmax && e0 > ((int64_t)1 << sh)) return false;  // f - 1 clamp case
  const int tot = 32 - sh;
  const int64_t fmax = two_m / e0;
  int ea = 0, fb = 0;
  bool u24 = false;
  if (var == kFastShiftmax) {
    // 24-bit operands (p4_pack24): the largest e shift that keeps e0 << ea and
    // the row sum in range, if f << fb then fits 24 bits as well
    for (int a = tot; a >= 0; --a) {
      const int b = tot - a;
      if ((e0 << a) < (1 << 24) && np * (e0 << a) < ((int64_t)1 << 32) && (fmax << b) < (1 << 24)) {
        ea = a;
        fb = b;
        u24 = true;
        break;
      }
    }
  }
  if (!u24) {
    while (ea < tot && np * (e0 << (ea + 1)) < ((int64_t)1 << 32)) ++ea;  // row sum fits
    fb = tot - ea;
    if ((fmax << fb) >= ((int64_t)1 << 32)) return false;
  }
  dp->qk_bm = (int32_t)((int64_t)p->qk_b << (32 - p->qk_c));
  dp->mask_s = (int32_t)(-(smax + 1));
  dp->e_shift = ea;
  dp->f_shift = fb;
  dp->p_u24 = u24 ? 1 : 0;
  dp->e0 = (int32_t)e0;
  dp->e0_pow2 = pow2 ? 1 : 0;
  dp->pv_fast = (p->pv_c >= 1 && p->pv_c <= 32 &&
                 ((int64_t)p->pv_b << (32 - p->pv_c)) < ((int64_t)1 << 31)) ? 1 : 0;
  dp->pv_bm = dp->pv_fast ? (int32_t)((int64_t)p->pv_b << (32 - p->pv_c)) : 0;
  return true;
}

// Polls of a bounded work-queue wait (each followed by s_sleep 1, about 64
// clocks) before a wave gives up; only a broken invariant could reach it.
constexpr int32_t kDefaultSpinLimit = 1 << 22;

// Everything a launch needs except the device pointers: kernel, launch shape,
// constants.  No device memory is touched.
struct Plan {
  DevParams dp;
  KernelFn fn;
  size_t lds_bytes;
  int fast;
  int grid;
  int block;  // threads per workgroup
  int np;     // 16 * number of key tiles (rows of the expanded bias)
};

int make_plan(const iqattn_params* p, int dev, const hipDeviceProp_t& prop, Plan* pl) {
  memset(pl, 0, sizeof(*pl));
  const int N = p->seq_len, D = p->head_dim;
  const int KT = (N + 15) / 16, KS = (KT + 3) / 4, Np = KT * 16;
  pl->np = Np;
  int64_t bias_max = 0;
  if (p->rel_bias) {
    const int64_t span = (int64_t)(2 * p->window - 1) * (2 * p->window - 1) * p->heads;
    for (int64_t i = 0; i < span; ++i) {
      const int64_t a = p->rel_bias[i] < 0 ? -(int64_t)p->rel_bias[i] : p->rel_bias[i];
      if (a > bias_max) bias_max = a;
    }
  }
  DevParams& dp = pl->dp;
  pl->fast = fast_constants(p, KT, bias_max, &dp) ? 1 : 0;
  dp.exp_last = host_exp_last(p->i0, p->exp_frac_bits, pl->fast ? dp.e_shift : 0);
  const size_t kbytes = (size_t)Np * (D + 16);
  if (pl->fast) {
    // buffers (V, K regions of R bytes each), table, LIS shift scratch; the
    // last V region's operand reads reach KS * 64 rows past its start
    const int var = fast_variant(p);
    const bool bias = p->rel_bias != NULL;
    const size_t R = (size_t)fast_region_bytes(D, KT);
    const size_t nbuf = (size_t)fast_nbuf(D, KT, bias, var);
    const size_t cw = (size_t)fast_cw(D, KT, bias, var);
    const size_t bs = (size_t)fast_nreg(KT, bias) * R;  // bytes per buffer
    const size_t used = nbuf * bs + kFastTableBytes + (var == kFastLisValu ? cw * 1024 : 0) + 64;
    const size_t reach = (nbuf - 1) * bs + (size_t)KS * 64 * D;
    pl->fn = fast_kernel(D, KT, bias, var);
    pl->lds_bytes = used > reach ? used : reach;
    pl->block = (int)(64 * (cw + 1));
    // rows of 64 keys: the expanded bias of every head in LDS after the
    // work-queue words, when it fits (the per-tile reads then leave global
    // memory, where they also waited for the previous tile's stores)
    const size_t bias_bytes = (size_t)p->heads * 64 * 64 * 4;
    if (bias && KT == 4 && used + bias_bytes <= 160 * 1024) {
      dp.bias_lds = 1;
      pl->lds_bytes = used + bias_bytes;
    }
  } else if (KT > 40) {
    // rows of 641..1024 keys: three passes over LDS-resident K, every back end
    const int var = fast_variant(p);
    pl->fn = long_kernel(D, var, p->rel_bias != NULL);
    pl->block = long_threads();
    pl->lds_bytes = long_lds_bytes(D, N, var);
  } else {
    const size_t vbytes =
        (p->variant == IQATTN_SHIFTMAX) ? (size_t)D * (KS * 64 + 16) : (size_t)Np * D;
    pl->fn = generic_kernel(D, KT, p->variant, p->rel_bias != NULL);
    pl->block = kThreads;
    pl->lds_bytes = kbytes + ((vbytes + 15) & ~(size_t)15) + (size_t)(dp.exp_last + 1) * kExpRep * 4 +
                    (p->variant == IQATTN_LIS ? (size_t)kWaves * 256 * 4 : 0);
  }
  int maxlds = 0, optin = 0;
  (void)hipDeviceGetAttribute(&maxlds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  (void)hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev);
  if (optin > maxlds) maxlds = optin;
  if ((int64_t)pl->lds_bytes > maxlds) return IQATTN_E_SHAPE;
  dp.spin_limit = kDefaultSpinLimit;
  dp.heads = p->heads;
  dp.n = N;
  dp.out_tok = p->out_layout == IQATTN_OUT_TOKENS;
  dp.units = p->batch * p->heads;
  dp.n_full = dp.units;
  dp.n_items = dp.units;
  pl->grid = dp.units;
  if (pl->fast && dp.units > 0) {
    // persistent grid: one workgroup per slot the chip holds at once, walking
    // the work items; the heads of a last, partial round are split into
    // quarter heads (groups of 8 heads x 4 quarters)
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)pl->fn, pl->block,
                                                     pl->lds_bytes) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    const int64_t slots = (int64_t)per_cu * prop.multiProcessorCount;
    const int64_t rem = dp.units % slots;
    if (rem > 0 && rem * 2 <= slots) {
      dp.n_full = (int32_t)(dp.units - rem);
      dp.n_items = (int32_t)(dp.n_full + ((rem + 7) / 8) * 32);
    }
    pl->grid = (int)(dp.n_items < slots ? dp.n_items : slots);
  }
  dp.qk_b = p->qk_b;
  dp.qk_c = p->qk_c;
  dp.pv_b = p->pv_b;
  dp.pv_c = p->pv_c;
  dp.intdiv_m = p->intdiv_m;
  dp.p_shift = p->intdiv_m - (p->k_out - 1);
  dp.p_max = (1 << (p->k_out - 1)) - 1;
  dp.lis_f = (1 << p->lis_bits) - 1;
  return IQATTN_OK;
}

int set_lds_attribute(const Plan& pl) {
  const hipError_t e = hipFuncSetAttribute((const void*)pl.fn,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)pl.lds_bytes);
  return e == hipSuccess ? IQATTN_OK : set_hip_error(e, "lds attribute");
}

int check_device(int* dev, hipDeviceProp_t* prop) {
  if (hipGetDevice(dev) != hipSuccess) return IQATTN_E_DEVICE;
  if (hipGetDeviceProperties(prop, *dev) != hipSuccess) return IQATTN_E_DEVICE;
  if (strncmp(prop->gcnArchName, "gfx950", 6) != 0) return IQATTN_E_DEVICE;
  return IQATTN_OK;
}

}  // namespace

struct iqattn_ctx {
  iqattn_params p;
  int device;
  uint32_t* exp_tab;
  int32_t* bias;
  uint32_t* status;  // bits of bounded waits that gave up (iqattn_check)
  Plan pl;
};

extern "C" int iqattn_create(const iqattn_params* p, iqattn_ctx** out) {
  if (!out) return IQATTN_E_NULL;
  *out = NULL;
  int rc = validate(p);
  if (rc) return rc;

  int dev = 0;
  hipDeviceProp_t prop;
  if ((rc = check_device(&dev, &prop))) return rc;

  iqattn_ctx* c = (iqattn_ctx*)calloc(1, sizeof(iqattn_ctx));
  if (!c) return IQATTN_E_ALLOC;
  c->p = *p;
  c->p.rel_bias = NULL;
  c->device = dev;
  Plan& pl = c->pl;
  hipError_t e;
  if ((rc = make_plan(p, dev, prop, &pl))) goto fail;
  if ((rc = set_lds_attribute(pl))) goto fail;
  if (hipMalloc((void**)&c->exp_tab, 256 * sizeof(uint32_t)) != hipSuccess) {
    rc = IQATTN_E_ALLOC;
    goto fail;
  }
  if (hipMalloc((void**)&c->status, sizeof(uint32_t)) != hipSuccess) { rc = IQATTN_E_ALLOC; goto fail; }
  if ((e = hipMemset(c->status, 0, sizeof(uint32_t))) != hipSuccess) {
    rc = set_hip_error(e, "status word");
    goto fail;
  }
  hipLaunchKernelGGL(iqattn_build_exp, dim3(1), dim3(256), 0, 0, c->exp_tab, p->i0,
                     p->exp_frac_bits, pl.fast ? pl.dp.e_shift : 0, (uint32_t*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) { rc = set_hip_error(e, "build_exp"); goto fail; }
  if (p->rel_bias) {
    const size_t tbytes = (size_t)p->heads * (2 * p->window - 1) * (2 * p->window - 1) * 4;
    const size_t ebytes = (size_t)p->heads * pl.np * pl.np * 4;
    int32_t* tab = NULL;
    if (hipMalloc((void**)&c->bias, ebytes) != hipSuccess) { rc = IQATTN_E_ALLOC; goto fail; }
    if (hipMalloc((void**)&tab, tbytes) != hipSuccess) { rc = IQATTN_E_ALLOC; goto fail; }
    if ((e = hipMemcpy(tab, p->rel_bias, tbytes, hipMemcpyHostToDevice)) != hipSuccess) {
      (void)hipFree(tab);
      rc = set_hip_error(e, "bias copy");
      goto fail;
    }
    hipLaunchKernelGGL(iqattn_expand_bias, dim3(256), dim3(256), 0, 0, c->bias, tab, p->heads,
                       p->seq_len, pl.np, p->window, pl.fast ? pl.dp.mask_s : 0);
    e = hipDeviceSynchronize();
    (void)hipFree(tab);
    if (e != hipSuccess) { rc = set_hip_error(e, "expand_bias"); goto fail; }
  }
  {
    // the table on the device must end where the host expects it to
    uint32_t host_tab[256];
    if ((e = hipMemcpy(host_tab, c->exp_tab, sizeof(host_tab), hipMemcpyDeviceToHost)) !=
        hipSuccess) {
      rc = set_hip_error(e, "exp table");
      goto fail;
    }
    int last = 255;
    for (int i = 0; i < 256; ++i)
      if (host_tab[i] == 0) { last = i; break; }
    if (last != pl.dp.exp_last) {
      snprintf(g_errbuf, sizeof(g_errbuf), "exponential table ends at %d, host expects %d", last,
               pl.dp.exp_last);
      rc = IQATTN_E_LAUNCH;
      goto fail;
    }
  }
  pl.dp.exp_tab = c->exp_tab;
  pl.dp.bias = c->bias;
  pl.dp.status = c->status;
  if ((e = hipDeviceSynchronize()) != hipSuccess) { rc = set_hip_error(e, "create"); goto fail; }
  *out = c;
  return IQATTN_OK;
fail:
  if (c->exp_tab) (void)hipFree(c->exp_tab);
  if (c->bias) (void)hipFree(c->bias);
  if (c->status) (void)hipFree(c->status);
  free(c);
  return rc;
}

extern "C" int iqattn_forward(iqattn_ctx* c, const int8_t* q, const int8_t* k, const int8_t* v,
                              int8_t* out, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  if (c->pl.dp.units == 0) return IQATTN_OK;
  if (!q || !k || !v || !out) return IQATTN_E_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return IQATTN_E_ALIGN;
  DevParams dp = c->pl.dp;
  dp.q = q;
  dp.k = k;
  dp.v = v;
  dp.out = out;
  hipLaunchKernelGGL(c->pl.fn, dim3(c->pl.grid), dim3(c->pl.block), c->pl.lds_bytes,
                     (hipStream_t)hip_stream, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqattn launch");
  return IQATTN_OK;
}

// ---------------------------------------------------------------- no-allocation entry point
// Static device memory of iqattn_forward_noalloc (one copy per GPU, held until
// the process ends): the exponential table, the status word and the expanded
// windowed bias.  Host code never uses the symbol itself as an address (on the
// host it is only a stand-in): each device's address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kScratchTab = 0;          // 256 u32
constexpr size_t kScratchStatus = 1024;    // u32 status word
constexpr size_t kScratchBias = 4096;      // expanded bias, heads * Np * Np int32
constexpr size_t kScratchBiasBytes = (size_t)256 << 10;
static __device__ __align__(256) uint8_t scratch[kScratchBias + kScratchBiasBytes];

namespace {
constexpr int kMaxDevices = 64;
struct DeviceState {
  bool ready;
  int rc;
  uint8_t* scratch;  // device address of `scratch` on this device
  hipDeviceProp_t prop;
};
DeviceState g_dev[kMaxDevices];
std::mutex g_dev_mutex;

// Set-up of the current device, once: its properties and the device address of
// its copy of `scratch`.
int device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return IQATTN_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceState& st = g_dev[dev];
  if (!st.ready) {
    int d2 = 0;
    st.rc = check_device(&d2, &st.prop);
    if (st.rc == IQATTN_OK) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        st.rc = set_hip_error(e == hipSuccess ? hipErrorInvalidSymbol : e, "scratch address");
      st.scratch = (uint8_t*)ptr;
    }
    st.ready = true;
  }
  *out = &st;
  return st.rc;
}
}  // namespace

extern "C" int iqattn_forward_noalloc(const iqattn_params* p, const int8_t* q, const int8_t* k,
                                      const int8_t* v, int8_t* out, void* hip_stream) {
  int rc = validate(p);
  if (rc) return rc;
  if (p->batch == 0) return IQATTN_OK;
  if (!q || !k || !v || !out) return IQATTN_E_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return IQATTN_E_ALIGN;
  // sizes the static memory holds: the relative table travels as a kernel
  // argument, its expansion lives in `scratch`
  if (p->rel_bias) {
    const int64_t span = (int64_t)(2 * p->window - 1) * (2 * p->window - 1) * p->heads;
    const int64_t np = ((int64_t)p->seq_len + 15) / 16 * 16;
    if (span > kArgBiasMax || (int64_t)p->heads * np * np * 4 > (int64_t)kScratchBiasBytes)
      return IQATTN_E_TOOBIG;
  }
  DeviceState* st = nullptr;
  if ((rc = device_state(&st))) return rc;
  int dev = 0;
  (void)hipGetDevice(&dev);
  Plan pl;
  if ((rc = make_plan(p, dev, st->prop, &pl))) return rc;
  if ((rc = set_lds_attribute(pl))) return rc;
  uint32_t* tab = (uint32_t*)(st->scratch + kScratchTab);
  uint32_t* status = (uint32_t*)(st->scratch + kScratchStatus);
  int32_t* bias = (int32_t*)(st->scratch + kScratchBias);
  hipStream_t stream = (hipStream_t)hip_stream;
  // the table and a cleared status word (a kernel, not a memset: callers may
  // capture this call in a graph), then the expanded bias, then the attention
  hipLaunchKernelGGL(iqattn_build_exp, dim3(1), dim3(256), 0, stream, tab, p->i0,
                     p->exp_frac_bits, pl.fast ? pl.dp.e_shift : 0, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "build_exp");
  if (p->rel_bias) {
    BiasArg ba;
    const int span = (2 * p->window - 1) * (2 * p->window - 1) * p->heads;
    memcpy(ba.v, p->rel_bias, (size_t)span * sizeof(int32_t));
    hipLaunchKernelGGL(iqattn_expand_bias_arg, dim3(64), dim3(256), 0, stream, bias, ba, p->heads,
                       p->seq_len, pl.np, p->window, pl.fast ? pl.dp.mask_s : 0);
    if ((e = hipGetLastError()) != hipSuccess) return set_hip_error(e, "expand_bias");
  }
  DevParams dp = pl.dp;
  dp.exp_tab = tab;
  dp.bias = p->rel_bias ? bias : nullptr;
  dp.status = status;
  dp.q = q;
  dp.k = k;
  dp.v = v;
  dp.out = out;
  hipLaunchKernelGGL(pl.fn, dim3(pl.grid), dim3(pl.block), pl.lds_bytes, stream, dp);
  if ((e = hipGetLastError()) != hipSuccess) return set_hip_error(e, "iqattn launch");
  return IQATTN_OK;
}

extern "C" int iqattn_check(iqattn_ctx* c, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  hipError_t e = hipStreamSynchronize((hipStream_t)hip_stream);
  if (e != hipSuccess) return set_hip_error(e, "iqattn_check synchronize");
  uint32_t word = 0;
  if ((e = hipMemcpy(&word, c->status, sizeof(word), hipMemcpyDeviceToHost)) != hipSuccess)
    return set_hip_error(e, "iqattn_check read");
  if (word == 0) return IQATTN_OK;
  const uint32_t zero = 0;
  if ((e = hipMemcpy(c->status, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess)
    return set_hip_error(e, "iqattn_check clear");
  return IQATTN_E_INCOMPLETE;
}

extern "C" int iqattn_set_spin_limit(iqattn_ctx* c, int32_t polls) {
  if (!c) return IQATTN_E_NULL;
  if (polls < 1) return IQATTN_E_INVAL;
  c->pl.dp.spin_limit = polls;
  return IQATTN_OK;
}

extern "C" int iqattn_destroy(iqattn_ctx* c) {
  if (!c) return IQATTN_OK;
  int dev = 0;
  (void)hipGetDevice(&dev);
  (void)hipSetDevice(c->device);
  if (c->exp_tab) (void)hipFree(c->exp_tab);
  if (c->bias) (void)hipFree(c->bias);
  if (c->status) (void)hipFree(c->status);
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
    case IQATTN_E_INCOMPLETE: return "a bounded wait in the kernel gave up: output incomplete";
    case IQATTN_E_TOOBIG:
      return "the windowed bias exceeds the static memory of iqattn_forward_noalloc";
    default: return "unknown error code";
  }
}
