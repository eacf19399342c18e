// iqlinear.hip -- integer-only int8 linear layer: Y = requant(X W^T) with a
// dyadic (b, c) per output tensor, fused into the GEMM epilogue.
//
// Method passage: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" (integer product, then (b * acc) >> c to int8); sec. 3.1
// (the MSA projections).
//
// Kernel: a workgroup of 2 x 2 waves computes a 128 (rows) x 128 (output
// columns) tile as Y^T = W . X^T with v_mfma_i32_16x16x64_i8, so a lane ends
// with 4 adjacent output columns of one row (one 4-byte store).  Each wave owns
// 64 x 64: 4 x 4 MFMA tiles, 64 accumulator registers (larger wave tiles need
// so many registers that one wave per SIMD remains, which measured slower).
// The k loop steps by 64 bytes: the next step's X and W tiles (2 x 8 KB) are
// loaded into registers while the current step runs from LDS, then written to
// the other LDS buffer (double buffering, one barrier per step).  LDS rows are 64 bytes
// with the 16-byte chunks XOR-swizzled by (row >> 1) & 3, which makes the
// b128 operand reads of 16 rows x 4 chunks bank-conflict free.
#include "iqattn_dev.h"
#include "iqattn.h"
#include "iqlinear.h"

#include <stdlib.h>
#include <string.h>

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
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 1) & 3)); }

// Workgroup of WM x WN waves; each wave owns TM x TN MFMA tiles (16 x 16) of
// rows x output columns, so the workgroup tile is (16 WM TM) x (16 WN TN).
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(64 * WM * WN) void iqlinear_gemm(LinParams p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BM = 16 * WM * TM, BN = 16 * WN * TN;   // workgroup tile
  constexpr int XCH = BM * 4 / NT, WCH = BN * 4 / NT;   // 16-byte chunks per thread per step
  static_assert(BM * 4 % NT == 0 && BN * 4 % NT == 0, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) int8_t sX[2][BM * kStep];
  __shared__ __attribute__((aligned(16))) int8_t sW[2][BN * kStep];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int wm = wave % WM, wn = wave / WM;
  const int m0 = blockIdx.x * BM, n0 = blockIdx.y * BN;

  // global tile loads (rows past the end read as zeros: buffer range)
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(p.x, (uint32_t)(p.rows * p.in_f));
  const __amdgpu_buffer_rsrc_t wr = buf_rsrc(p.w, (uint32_t)(p.out_f * p.in_f));
  int xoff[XCH], xls[XCH], woff[WCH], wls[WCH];
  bool xin[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int idx = tid + NT * i, row = idx >> 2, ch = idx & 3;
    xin[i] = m0 + row < p.rows;
    xoff[i] = (xin[i] ? m0 + row : 0) * p.in_f + 16 * ch;
    xls[i] = swz(row, ch);
  }
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int idx = tid + NT * i, row = idx >> 2, ch = idx & 3;
    woff[i] = (n0 + row) * p.in_f + 16 * ch;
    wls[i] = swz(row, ch);
  }
  v4i xv[XCH], wv[WCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[i] + k0, 0, 0);
#pragma unroll
    for (int i = 0; i < WCH; ++i) wv[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[i] + k0, 0, 0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) *(v4i*)(sX[buf] + xls[i]) = xin[i] ? xv[i] : v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < WCH; ++i) *(v4i*)(sW[buf] + wls[i]) = wv[i];
  };

  v4i acc[TN][TM];  // [n tile][m tile]
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = v4i{0, 0, 0, 0};

  const int nks = p.in_f / kStep;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nks) gload((ks + 1) * kStep);
    v4i bf[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) bf[t] = *(const v4i*)(sX[buf] + swz(16 * (TM * wm + t) + li, g));
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const v4i af = *(const v4i*)(sW[buf] + swz(16 * (TN * wn + a) + li, g));  // output columns
#pragma unroll
      for (int b = 0; b < TM; ++b) acc[a][b] = mfma64(af, bf[b], acc[a][b]);
    }
    if (ks + 1 < nks) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds output columns n0 + 16 (TN wn + a) + 4 g + r of row
  // m0 + 16 (TM wm + b) + li
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int m = m0 + 16 * (TM * wm + b) + li;
    if (m >= p.rows) continue;
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int n = n0 + 16 * (TN * wn + a) + 4 * g;
      if (n >= p.out_f) continue;  // out is a multiple of 16: the whole 16-column tile
      int which = 0, col = n;
      if (p.layout == IQLINEAR_QKV_HEADS) {
        which = n / p.width;
        col = n - which * p.width;
      }
      int32_t y[4];
      if (p.bm[which]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = clamp127(mulhi_i32(acc[a][b][r], p.bm[which]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = requant_i8(acc[a][b][r], p.b[which], p.c[which]);
      }
      const uint32_t word = pack4_lowbytes((uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]);
      int64_t dst;
      if (p.layout == IQLINEAR_QKV_HEADS) {
        const int bidx = m / p.seq_len, t = m - bidx * p.seq_len;
        const int h = col / p.head_dim, i = col - h * p.head_dim;
        dst = (((int64_t)bidx * p.heads + h) * p.seq_len + t) * p.head_dim + i;
      } else {
        dst = (int64_t)m * p.out_f + n;
      }
      *(uint32_t*)(p.out[which] + dst) = word;
    }
  }
}

#ifndef IQLINEAR_CFG
#define IQLINEAR_CFG 2, 2, 4, 4
#endif
constexpr int kCfg[4] = {IQLINEAR_CFG};
#define IQLINEAR_KERNEL iqlinear_gemm<kCfg[0], kCfg[1], kCfg[2], kCfg[3]>
constexpr int kBM = 16 * kCfg[0] * kCfg[2], kBN = 16 * kCfg[1] * kCfg[3];
constexpr int kNT = 64 * kCfg[0] * kCfg[1];

}  // namespace
}  // namespace iqattn

using namespace iqattn;

struct iqlinear_ctx {
  LinParams lp;
  int device;
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
  for (int i = 0; i < 3; ++i) {
    const int k = i < npairs ? i : 0;
    lp.b[i] = p->b[k];
    lp.c[i] = p->c[k];
    const bool fast = p->c[k] >= 1 && p->c[k] <= 32 &&
                      ((int64_t)p->b[k] << (32 - p->c[k])) < ((int64_t)1 << 31);
    lp.bm[i] = fast ? (int32_t)((int64_t)p->b[k] << (32 - p->c[k])) : 0;
  }
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
  const dim3 grid((unsigned)((lp.rows + kBM - 1) / kBM), (unsigned)((lp.out_f + kBN - 1) / kBN));
  hipLaunchKernelGGL(IQLINEAR_KERNEL, grid, dim3(kNT), 0, (hipStream_t)hip_stream, lp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqlinear launch");
  return IQATTN_OK;
}

extern "C" int iqlinear_destroy(iqlinear_ctx* c) {
  free(c);
  return IQATTN_OK;
}
