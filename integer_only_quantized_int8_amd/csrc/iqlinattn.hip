// iqlinattn.hip -- softmax-free integer linear attention (ReLU global
// attention with a log2-quantised divisor and shift division).
//
// Method passages: Trio-ViT (cloud.tencent.com article) sec. III Eq. 4 (the
// ReLU attention of EfficientViT), sec. V "Distinct Computational Pattern of
// Attention" (steps i-v), sec. IV Eq. 11 (leading-one log2 of the divisor);
// I-ViT (mer.run summary) sec. 3.2 (dyadic requantisation).
//
// One workgroup of 8 waves per head; the head's Q, K, V and Out are each read
// or written once (4 N d bytes per head), so the kernel is HBM-bound and both
// contractions run on int8 MFMA (v_mfma_i32_16x16x32_i8):
//   phase 1 (steps i, ii): each wave streams 32-token chunks of K and V
//     through its own LDS slot (four chunks in flight in registers, the
//     first issued at kernel entry); ds_read_b64_tr_b8 turns the row-major chunk
//     into the token-major MFMA operands, so that one MFMA per 16 x 16 tile of
//     KV = ReLU(K)^T V sums 32 tokens; ks = sum ReLU(K) comes from v_dot4 on
//     the same operand bytes.  ReLU acts on the operand bytes (a byte mask).
//     The waves add their partial sums into LDS, where they are
//     requantised to int8 (KVq stored transposed, [b][a]).
//   phase 2 (steps iii-v): for 16 tokens at a time (four tiles of Q in flight
//     per wave, the first issued at kernel entry), num^T = KVq^T . ReLU(Q)^T
//     by MFMA leaves each lane 4 consecutive output features of one token;
//     den = ReLU(Q) . ksq by v_dot4 over the lane's operand bytes and a
//     reduction over the lane groups; the output is
//     clip((out_b num) >> (out_c + ilog2r(den))).
// Buffer resources per head make tokens past N read as zeros and drop their
// stores.
#include "iqattn_dev.h"
#include "iqattn.h"
#include "iqlinattn.h"

#include <stdlib.h>
#include <string.h>

namespace iqattn {
namespace {

#ifndef IQLA_WAVES
#define IQLA_WAVES 8
#endif
constexpr int kLaWaves = IQLA_WAVES;
constexpr int kLaThreads = 64 * kLaWaves;
constexpr int kChunk = 32;       // tokens per MFMA step of the token sums
constexpr int kKVDepth = 4;      // K/V chunks in flight per wave (phase 1)
constexpr int kQDepth = 4;       // 16-token Q tiles in flight per wave (phase 2)

struct LaParams {
  const int8_t* q;
  const int8_t* k;
  const int8_t* v;
  int8_t* out;
  int32_t n;  // tokens per head
  int32_t kv_b, kv_c, ks_b, ks_c, out_b, out_c;
};

// max(byte, 0) on the 4 signed bytes of w
__device__ __forceinline__ int32_t relu4(int32_t w) {
  const uint32_t s = ((uint32_t)w >> 7) & 0x01010101u;  // sign bit of each byte at its bit 0
  return (int32_t)((uint32_t)w & ~(s * 0xFFu));
}

__device__ __forceinline__ int64_t relu8(int64_t x) {
  const uint32_t lo = (uint32_t)relu4((int32_t)x), hi = (uint32_t)relu4((int32_t)(x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int32_t requant64(int64_t x, int32_t b, int32_t sh) {
  const int64_t t = (int64_t)b * x;
  const int64_t y = sh >= 63 ? (t < 0 ? -1 : 0) : (t >> sh);
  return (int32_t)(y < -127 ? -127 : (y > 127 ? 127 : y));
}

__device__ __forceinline__ v4i mfma32(int64_t a, int64_t b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
}

// One wave's share of a 32-token chunk of K and V (row-major, D bytes a
// token): D / 2 bytes of each per lane.
template <int D>
struct Stage {
  static constexpr int NP = D == 16 ? 1 : D / 32;  // 16-byte pieces (D >= 32)
  int64_t k8 = 0, v8 = 0;                          // D = 16
  v4i kp[NP] = {}, vp[NP] = {};                    // D >= 32

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                       int chunk, int lane) {
    const int base = chunk * kChunk * D;
    if constexpr (D == 16) {
      k8 = buf_load<int64_t>(kr, base + 8 * lane);
      v8 = buf_load<int64_t>(vr, base + 8 * lane);
    } else {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        kp[i] = buf_load<v4i>(kr, base + 1024 * i + 16 * lane);
        vp[i] = buf_load<v4i>(vr, base + 1024 * i + 16 * lane);
      }
    }
  }

  // K rows at stg, V rows at stg + 32 D
  __device__ __forceinline__ void store(int8_t* stg, int lane) const {
    if constexpr (D == 16) {
      *reinterpret_cast<int64_t*>(stg + 8 * lane) = k8;
      *reinterpret_cast<int64_t*>(stg + kChunk * D + 8 * lane) = v8;
    } else {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        *reinterpret_cast<v4i*>(stg + 1024 * i + 16 * lane) = kp[i];
        *reinterpret_cast<v4i*>(stg + kChunk * D + 1024 * i + 16 * lane) = vp[i];
      }
    }
  }
};

__device__ __forceinline__ int64_t read_tr8(const int8_t* p) {
  const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(uintptr_t)lds_addr(p));
  return (int64_t)(((uint64_t)(uint32_t)r[1] << 32) | (uint32_t)r[0]);
}

template <int D>
__global__ __launch_bounds__(kLaThreads) void iqlinattn_fwd(LaParams p) {
  constexpr int FT = D / 16;        // 16-feature tiles
  constexpr int KS = (D + 31) / 32; // 32-feature k steps of the output product
  constexpr int PR = 32 * KS;       // row length of KVq^T and ksq in LDS (zero padded)
  constexpr int STG = 2 * kChunk * D;
  __shared__ __attribute__((aligned(16))) int8_t stg[kLaWaves][STG];
  __shared__ int32_t kv_acc[D * D];
  __shared__ int32_t ks_acc[D];
  __shared__ __attribute__((aligned(16))) int8_t kvq_t[D * PR];
  __shared__ __attribute__((aligned(16))) int8_t ksq[PR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, m = lane & 15;
  const uint32_t hbytes = (uint32_t)p.n * D;
  const int64_t hoff = (int64_t)blockIdx.x * hbytes;
  const __amdgpu_buffer_rsrc_t qr = buf_rsrc(p.q + hoff, hbytes);
  const __amdgpu_buffer_rsrc_t kr = buf_rsrc(p.k + hoff, hbytes);
  const __amdgpu_buffer_rsrc_t vr = buf_rsrc(p.v + hoff, hbytes);
  const __amdgpu_buffer_rsrc_t orr = buf_rsrc(p.out + hoff, hbytes);
  const int nchunks = (p.n + kChunk - 1) / kChunk;
  const int ntiles = (p.n + 15) / 16;

  // ReLU(Q)^T operand bytes of tile t for this lane: token 16 t + m, features
  // 32 s + 8 g .. (zero past D and, through the buffer bounds, past N)
  auto load_q = [&](int t, int64_t (&qb)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qb[s] = 0;
      if (32 * s + 8 * g < D) qb[s] = buf_load<int64_t>(qr, (16 * t + m) * D + 32 * s + 8 * g);
    }
  };
  // the first Q tiles and K/V chunks of this wave load from the start, so that
  // their latency overlaps the zeroing, the token sums and the reduction
  int64_t qring[kQDepth][KS];
#pragma unroll
  for (int u = 0; u < kQDepth; ++u) {
    const int t = wave + kLaWaves * u;
#pragma unroll
    for (int s = 0; s < KS; ++s) qring[u][s] = 0;
    if (t < ntiles) load_q(t, qring[u]);
  }
  Stage<D> ring[kKVDepth];
#pragma unroll
  for (int u = 0; u < kKVDepth; ++u) {
    const int c = wave + kLaWaves * u;
    if (c < nchunks) ring[u].load(kr, vr, c, lane);
  }

  for (int i = tid; i < D * D; i += kLaThreads) kv_acc[i] = 0;
  if (tid < D) ks_acc[tid] = 0;
  __syncthreads();

  // ---------------------------------------------------------------- phase 1
  int8_t* my = stg[wave];
  // transposed-read address of this lane: token row 8 g + (m >> 1), bytes
  // 8 (m & 1) .. of the 16-feature tile
  const int tro = (8 * g + (m >> 1)) * D + 8 * (m & 1);
  v4i acc[FT][FT];
  int32_t ksa[FT];
#pragma unroll
  for (int a = 0; a < FT; ++a) {
    ksa[a] = 0;
#pragma unroll
    for (int b = 0; b < FT; ++b) acc[a][b] = v4i{0, 0, 0, 0};
  }
  for (int c0 = wave; c0 < nchunks; c0 += kLaWaves * kKVDepth) {
#pragma unroll
    for (int u = 0; u < kKVDepth; ++u) {
      const int c = c0 + kLaWaves * u;
      if (c >= nchunks) break;
      ring[u].store(my, lane);
      const int cn = c + kLaWaves * kKVDepth;
      if (cn < nchunks) ring[u].load(kr, vr, cn, lane);
      int64_t ka[FT], vb[FT];
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        ka[f] = relu8(read_tr8(my + tro + 16 * f));
        vb[f] = read_tr8(my + kChunk * D + tro + 16 * f);
        ksa[f] = __builtin_amdgcn_sdot4((int32_t)ka[f], 0x01010101, ksa[f], false);
        ksa[f] = __builtin_amdgcn_sdot4((int32_t)(ka[f] >> 32), 0x01010101, ksa[f], false);
      }
#pragma unroll
      for (int a = 0; a < FT; ++a)
#pragma unroll
        for (int b = 0; b < FT; ++b) acc[a][b] = mfma32(ka[a], vb[b], acc[a][b]);
    }
  }
  // lane (g, m): acc[a][b][r] = KV[16 a + 4 g + r][16 b + m]; ksa[a] sums the
  // tokens 8 g .. of feature 16 a + m
#pragma unroll
  for (int a = 0; a < FT; ++a) {
    int32_t s = ksa[a];
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (g == 0) atomicAdd(&ks_acc[16 * a + m], s);
#pragma unroll
    for (int b = 0; b < FT; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) atomicAdd(&kv_acc[(16 * a + 4 * g + r) * D + 16 * b + m], acc[a][b][r]);
  }
  __syncthreads();
  // requantised sums: KVq^T [b][a] and ksq [a], zero for a >= D
  for (int i = tid; i < D * PR; i += kLaThreads) {
    const int b = i / PR, a = i % PR;
    kvq_t[i] = (int8_t)(a < D ? requant64(kv_acc[a * D + b], p.kv_b, p.kv_c) : 0);
  }
  if (tid < PR) ksq[tid] = (int8_t)(tid < D ? requant64(ks_acc[tid], p.ks_b, p.ks_c) : 0);
  __syncthreads();

  // ---------------------------------------------------------------- phase 2
  int64_t aop[FT][KS], kq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    kq[s] = *reinterpret_cast<const int64_t*>(ksq + 32 * s + 8 * g);
#pragma unroll
    for (int f = 0; f < FT; ++f)
      aop[f][s] = *reinterpret_cast<const int64_t*>(kvq_t + (16 * f + m) * PR + 32 * s + 8 * g);
  }
  for (int t0 = wave; t0 < ntiles; t0 += kLaWaves * kQDepth) {
#pragma unroll
    for (int u = 0; u < kQDepth; ++u) {
      const int t = t0 + kLaWaves * u;
      if (t >= ntiles) break;
      const int row = 16 * t + m;  // this lane's token (past N: zeros, no store)
      int64_t qb[KS];
      int32_t den = 0;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qb[s] = relu8(qring[u][s]);
        den = __builtin_amdgcn_sdot4((int32_t)qb[s], (int32_t)kq[s], den, false);
        den = __builtin_amdgcn_sdot4((int32_t)(qb[s] >> 32), (int32_t)(kq[s] >> 32), den, false);
      }
      const int tn = t + kLaWaves * kQDepth;
      if (tn < ntiles) load_q(tn, qring[u]);
      den += __shfl_xor(den, 16, 64);
      den += __shfl_xor(den, 32, 64);
      const int32_t L = den > 0 ? ilog2r_dev((uint32_t)den) : 0;
      const int32_t sh = p.out_c + L;
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        v4i num = v4i{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) num = mfma32(aop[f][s], qb[s], num);
        // num[r] = numerator of feature 16 f + 4 g + r of token `row`
        const uint32_t word = pack4_lowbytes(
            (uint32_t)requant64(num[0], p.out_b, sh), (uint32_t)requant64(num[1], p.out_b, sh),
            (uint32_t)requant64(num[2], p.out_b, sh), (uint32_t)requant64(num[3], p.out_b, sh));
        __builtin_amdgcn_raw_buffer_store_b32(word, orr, row * D + 16 * f + 4 * g, 0, 0);
      }
    }
  }
}

}  // namespace
}  // namespace iqattn

using namespace iqattn;

struct iqlinattn_ctx {
  LaParams lp;
  int64_t heads;  // batch * heads
  int32_t d;
  int device;
};

extern "C" int iqlinattn_create(const iqlinattn_params* p, iqlinattn_ctx** out) {
  if (!out) return IQATTN_E_NULL;
  *out = NULL;
  if (!p) return IQATTN_E_NULL;
  if (p->batch < 0 || p->heads < 1 || p->seq_len < 1 || p->seq_len > 65536) return IQATTN_E_SHAPE;
  if (p->head_dim != 16 && p->head_dim != 32 && p->head_dim != 64) return IQATTN_E_SHAPE;
  if ((int64_t)p->batch * p->heads * p->seq_len * p->head_dim > INT32_MAX) return IQATTN_E_SHAPE;
  const int32_t bs[3] = {p->kv_b, p->ks_b, p->out_b}, cs[3] = {p->kv_c, p->ks_c, p->out_c};
  for (int i = 0; i < 3; ++i)
    if (bs[i] < 1 || cs[i] < 0 || cs[i] > 62) return IQATTN_E_INVAL;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return IQATTN_E_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return IQATTN_E_DEVICE;
  iqlinattn_ctx* c = (iqlinattn_ctx*)calloc(1, sizeof(iqlinattn_ctx));
  if (!c) return IQATTN_E_ALLOC;
  c->device = dev;
  c->heads = (int64_t)p->batch * p->heads;
  c->d = p->head_dim;
  LaParams& lp = c->lp;
  lp.n = p->seq_len;
  lp.kv_b = p->kv_b;
  lp.kv_c = p->kv_c;
  lp.ks_b = p->ks_b;
  lp.ks_c = p->ks_c;
  lp.out_b = p->out_b;
  lp.out_c = p->out_c;
  *out = c;
  return IQATTN_OK;
}

extern "C" int iqlinattn_forward(iqlinattn_ctx* c, const int8_t* q, const int8_t* k,
                                 const int8_t* v, int8_t* out, void* hip_stream) {
  if (!c) return IQATTN_E_NULL;
  if (c->heads == 0) return IQATTN_OK;
  if (!q || !k || !v || !out) return IQATTN_E_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15u) return IQATTN_E_ALIGN;
  LaParams lp = c->lp;
  lp.q = q;
  lp.k = k;
  lp.v = v;
  lp.out = out;
  const dim3 grid((unsigned)c->heads), block(kLaThreads);
  hipStream_t s = (hipStream_t)hip_stream;
  if (c->d == 16)
    hipLaunchKernelGGL(iqlinattn_fwd<16>, grid, block, 0, s, lp);
  else if (c->d == 32)
    hipLaunchKernelGGL(iqlinattn_fwd<32>, grid, block, 0, s, lp);
  else
    hipLaunchKernelGGL(iqlinattn_fwd<64>, grid, block, 0, s, lp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqlinattn launch");
  return IQATTN_OK;
}

extern "C" int iqlinattn_destroy(iqlinattn_ctx* c) {
  free(c);
  return IQATTN_OK;
}
