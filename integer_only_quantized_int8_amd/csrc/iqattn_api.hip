// iqattn_api.hip -- the C ABI of libiqattn (include/iqattn.h): parameter
// checks, device constants built by set-up kernels, kernel selection, launch.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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
__global__ void iqattn_build_exp(uint32_t* tab, int32_t i0, int32_t nfrac, int32_t shift) {
  const int idx = threadIdx.x;
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
  // real accumulator; every raw logit then fits the 24-bit v_mad_i32_i24
  if (p->qk_c > 32 || p->qk_c < 1) return false;
  if (((int64_t)p->qk_b << (32 - p->qk_c)) >= ((int64_t)1 << 31)) return false;
  const int64_t smax = (int64_t)p->head_dim * 127 * 127 + bias_max;
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

}  // namespace

struct iqattn_ctx {
  iqattn_params p;
  int device;
  uint32_t* exp_tab;
  int32_t* bias;
  KernelFn fn;
  size_t lds_bytes;
  DevParams dp;
  int fast;
  int grid;
  int block;  // threads per workgroup
};

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
  int64_t bias_max = 0;
  if (p->rel_bias) {
    const int64_t span = (int64_t)(2 * p->window - 1) * (2 * p->window - 1) * p->heads;
    for (int64_t i = 0; i < span; ++i) {
      const int64_t a = p->rel_bias[i] < 0 ? -(int64_t)p->rel_bias[i] : p->rel_bias[i];
      if (a > bias_max) bias_max = a;
    }
  }
  c->fast = fast_constants(p, KT, bias_max, &c->dp) ? 1 : 0;

  hipError_t e;
  if (hipMalloc((void**)&c->exp_tab, 256 * sizeof(uint32_t)) != hipSuccess) {
    free(c);
    return IQATTN_E_ALLOC;
  }
  hipLaunchKernelGGL(iqattn_build_exp, dim3(1), dim3(256), 0, 0, c->exp_tab, p->i0,
                     p->exp_frac_bits, c->fast ? c->dp.e_shift : 0);
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
    hipLaunchKernelGGL(iqattn_expand_bias, dim3(256), dim3(256), 0, 0, c->bias, tab, p->heads, N,
                       Np, p->window, c->fast ? c->dp.mask_s : 0);
    e = hipDeviceSynchronize();
    (void)hipFree(tab);
    if (e != hipSuccess) { rc = set_hip_error(e, "expand_bias"); goto fail; }
  }
  {
    uint32_t host_tab[256];
    if ((e = hipMemcpy(host_tab, c->exp_tab, sizeof(host_tab), hipMemcpyDeviceToHost)) !=
        hipSuccess) {
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
    size_t vbytes;
    if (c->fast) {
      // buffers (V, K regions of R bytes each), table, LIS shift scratch; the
      // last V region's operand reads reach KS * 64 rows past its start
      const int var = fast_variant(p);
      const bool bias = p->rel_bias != NULL;
      const size_t R = (size_t)fast_region_bytes(D, KT);
      const size_t nbuf = (size_t)fast_nbuf(KT, bias, var);
      const size_t cw = (size_t)fast_cw(KT, bias);
      const size_t bs = (size_t)fast_nreg(KT, bias) * R;  // bytes per buffer
      const size_t used = nbuf * bs + kFastTableBytes + (var == kFastLisValu ? cw * 1024 : 0) + 64;
      const size_t reach = (nbuf - 1) * bs + (size_t)KS * 64 * D;
      c->fn = fast_kernel(D, KT, bias, var);
      c->lds_bytes = used > reach ? used : reach;
      c->block = (int)(64 * (cw + 1));
    } else {
      vbytes = (p->variant == IQATTN_SHIFTMAX) ? (size_t)D * (KS * 64 + 16) : (size_t)Np * D;
      c->fn = generic_kernel(D, KT, p->variant, p->rel_bias != NULL);
      c->block = kThreads;
      c->lds_bytes = kbytes + ((vbytes + 15) & ~(size_t)15) +
                     (size_t)(c->dp.exp_last + 1) * kExpRep * 4 +
                     (p->variant == IQATTN_LIS ? (size_t)kWaves * 256 * 4 : 0);
    }
    int maxlds = 0, optin = 0;
    (void)hipDeviceGetAttribute(&maxlds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    (void)hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev);
    if (optin > maxlds) maxlds = optin;
    if ((int64_t)c->lds_bytes > maxlds) { rc = IQATTN_E_SHAPE; goto fail; }
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
  c->dp.out_tok = p->out_layout == IQATTN_OUT_TOKENS;
  c->dp.units = p->batch * p->heads;
  c->dp.n_full = c->dp.units;
  c->dp.n_items = c->dp.units;
  c->grid = c->dp.units;
  if (c->fast && c->dp.units > 0) {
    // persistent grid: one workgroup per slot the chip holds at once, walking
    // the work items; the heads of a last, partial round are split into
    // quarter heads (groups of 8 heads x 4 quarters)
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)c->fn, c->block,
                                                     c->lds_bytes) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    const int64_t slots = (int64_t)per_cu * prop.multiProcessorCount;
    const int64_t rem = c->dp.units % slots;
    if (rem > 0 && rem * 2 <= slots) {
      c->dp.n_full = (int32_t)(c->dp.units - rem);
      c->dp.n_items = (int32_t)(c->dp.n_full + ((rem + 7) / 8) * 32);
    }
    c->grid = (int)(c->dp.n_items < slots ? c->dp.n_items : slots);
  }
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
  hipLaunchKernelGGL(c->fn, dim3(c->grid), dim3(c->block), c->lds_bytes,
                     (hipStream_t)hip_stream, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqattn launch");
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
