// iqlinear.hip -- integer-only int8 linear layer: Y = requant(X W^T) with a
// dyadic (b, c) per output tensor, fused into the GEMM epilogue.
//
// Method passage: I-ViT (mer.run summary) sec. 3.2 "Dyadic Arithmetic for
// Linear Operations" (integer product, then (b * acc) >> c to int8); sec. 3.1
// (the MSA projections).
//
// Kernel (iqlinear_pipe below): persistent workgroups, one per CU, of 4 MFMA
// waves and 4 loader waves.  Each workgroup computes 128 x 128 output tiles as
// Y^T = W . X^T with v_mfma_i32_16x16x64_i8, so a lane ends
// with 4 adjacent output columns of one row (one 4-byte store after the fused
// requantisation, straight into the head-split layout when asked).  Each
// compute wave owns a quarter of the tile (64 x 64: 16 MFMA tiles, 64
// accumulators).  The k loop runs through a ring of LDS stages of 128 k-bytes a
// row (whole cache lines per load request), filled by the loader waves with
// direct global->LDS loads; the 16-byte chunks of a 128-byte LDS row are
// XOR-swizzled by (row >> 1) & 7, which makes the b128 operand reads of 16
// rows bank-conflict free.
#include "iqattn_dev.h"
#include "iqattn.h"
#include "iqlinear.h"

#include <stdlib.h>
#include <string.h>

#include <type_traits>

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


// Epilogue of one wave's TN x TM accumulator tiles: acc[a][b][r] is output
// column n + 16 a + r of row m + 16 b; requantised, packed to 4 bytes and
// stored.  The destination offset splits into a row part and a column part
// (plain: m out + n; head split: ((bidx H + h) N + t) d + i = (bidx H N + t) d
// + (h N d + i)), so the divisions run once per row and once per column.
// Rows past the end are skipped.
template <int TM, int TN>
__device__ __forceinline__ void store_tile(const LinParams& p, const v4i (&acc)[TN][TM], int m_base,
                                           int n_base) {
  const bool qkv = p.layout == IQLINEAR_QKV_HEADS;
  int64_t rofs[TM];
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int m = m_base + 16 * b;
    if (qkv) {
      const int bidx = m / p.seq_len, t = m - bidx * p.seq_len;
      rofs[b] = ((int64_t)bidx * p.heads * p.seq_len + t) * p.head_dim;
    } else {
      rofs[b] = (int64_t)m * p.out_f;
    }
  }
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n_base + 16 * a;
    if (n >= p.out_f) continue;  // out is a multiple of 16: the whole 16-column tile
    int which = 0, cofs = n;
    if (qkv) {
      which = n / p.width;
      const int col = n - which * p.width;
      const int h = col / p.head_dim;
      cofs = h * p.seq_len * p.head_dim + (col - h * p.head_dim);
    }
    const int32_t bm = p.bm[which], bb = p.b[which], cc = p.c[which];
    int8_t* const out = p.out[which];
    if (bm) {  // uniform: the pair of this 16-column tile
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        if (m_base + 16 * b >= p.rows) continue;
        *(uint32_t*)(out + rofs[b] + cofs) = pack4_lowbytes(
            (uint32_t)clamp127(mulhi_i32(acc[a][b][0], bm)), (uint32_t)clamp127(mulhi_i32(acc[a][b][1], bm)),
            (uint32_t)clamp127(mulhi_i32(acc[a][b][2], bm)), (uint32_t)clamp127(mulhi_i32(acc[a][b][3], bm)));
      }
    } else {
#pragma unroll
      for (int b = 0; b < TM; ++b) {
        if (m_base + 16 * b >= p.rows) continue;
        *(uint32_t*)(out + rofs[b] + cofs) = pack4_lowbytes(
            (uint32_t)requant_i8(acc[a][b][0], bb, cc), (uint32_t)requant_i8(acc[a][b][1], bb, cc),
            (uint32_t)requant_i8(acc[a][b][2], bb, cc), (uint32_t)requant_i8(acc[a][b][3], bb, cc));
      }
    }
  }
}

// The same epilogue through a wave-private LDS block: the requantised bytes of
// the wave's (16 TM) x (16 TN) block go to LDS rows of kEpPitch bytes (the
// pitch keeps the 4-byte writes of 16 rows bank-conflict free), then each lane
// stores whole 16-byte row chunks (4 x fewer store instructions, contiguous
// 16-byte writes).  Needs 16-column groups that stay inside one output row
// segment: always for the plain layout, head_dim % 16 == 0 for the head split.
constexpr int kEpPitch = 16 * 4 + 16;  // (16 TN = 64) bytes + 16 of padding

template <int TM, int TN>
__device__ __forceinline__ void store_tile_lds(const LinParams& p, const v4i (&acc)[TN][TM],
                                               int8_t* scr, int m_w, int n_w, int li, int g,
                                               int lane) {
  static_assert(16 * TN + 16 == kEpPitch, "pitch");
  const bool qkv = p.layout == IQLINEAR_QKV_HEADS;
#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n_w + 16 * a;
    const int which = qkv ? n / p.width : 0;
    const int32_t bm = p.bm[which], bb = p.b[which], cc = p.c[which];
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      uint32_t word;
      if (bm)
        word = pack4_lowbytes(
            (uint32_t)clamp127(mulhi_i32(acc[a][b][0], bm)), (uint32_t)clamp127(mulhi_i32(acc[a][b][1], bm)),
            (uint32_t)clamp127(mulhi_i32(acc[a][b][2], bm)), (uint32_t)clamp127(mulhi_i32(acc[a][b][3], bm)));
      else
        word = pack4_lowbytes(
            (uint32_t)requant_i8(acc[a][b][0], bb, cc), (uint32_t)requant_i8(acc[a][b][1], bb, cc),
            (uint32_t)requant_i8(acc[a][b][2], bb, cc), (uint32_t)requant_i8(acc[a][b][3], bb, cc));
      *(uint32_t*)(scr + (16 * b + li) * kEpPitch + 16 * a + 4 * g) = word;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the block is in LDS (one wave: in order)
  constexpr int CH = TM * TN;          // 16-byte chunks per lane: (16 TM rows x TN chunks) / 16 ... / 64 lanes x 16
#pragma unroll
  for (int k = 0; k < (16 * TM * TN) / 64; ++k) {
    const int c = lane + 64 * k, row = c / TN, cg = c % TN;
    const int m = m_w + row, n = n_w + 16 * cg;
    const v4i v = *(const v4i*)(scr + row * kEpPitch + 16 * cg);
    if (m >= p.rows || n >= p.out_f) continue;
    int64_t dst;
    int which = 0;
    if (qkv) {
      which = n / p.width;
      const int col = n - which * p.width, h = col / p.head_dim;
      const int bidx = m / p.seq_len, t = m - bidx * p.seq_len;
      dst = (((int64_t)bidx * p.heads + h) * p.seq_len + t) * p.head_dim + (col - h * p.head_dim);
    } else {
      dst = (int64_t)m * p.out_f + n;
    }
    *(v4i*)(p.out[which] + dst) = v;
  }
  (void)CH;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // the reads are done before the block is reused
}

// ---------------------------------------------------------------- pipelined GEMM
// Persistent workgroups (one per CU) of 4 compute waves and kPipeNL loader
// waves.  The loaders stream 128-byte k-slices of a tile's X rows and W rows
// (two 64-byte MFMA k-blocks) into a ring of kPipeNS LDS stages with direct
// global->LDS loads, each loader wave a quarter of every stage (the swizzle is
// applied on the source side: lane l of a 1 KB block fills LDS bytes
// [1024 i + 16 l, +16) = (row, chunk position cp) from source chunk
// cp ^ ((row >> 1) & 7)), kPipeLag stages in flight per wave, running ahead
// across tile boundaries.  Monotonic LDS counters per stage slot: ready[b]
// (loader waves that finished a fill), done[b] (compute waves that finished
// reading it).  Compute waves read a k-block's fragments while the MFMAs of the
// previous one run.  Tiles are dealt XCD-aware: the workgroups of one XCD
// (every 8th) take all column tiles of one block of X rows in turn, so those
// rows reach that XCD's L2 once.
constexpr int kPipeKB = 128;  // k bytes of a row per stage: whole cache lines per request
constexpr int kPipeNS = 4;
constexpr int kPipeLag = 2;
constexpr int kPipeNL = 4;
constexpr int kPipeSpin = 1 << 22;
constexpr int kPipeThreads = 64 * (4 + kPipeNL);

constexpr int pipe_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

template <int BM, int BN>
struct PipeCfg {
  static constexpr int TM = BM / 32, TN = BN / 32;  // 16 x 16 tiles per wave (2 x 2 waves)
  static constexpr int KB = kPipeKB, NCH = KB / 16, KPS = KB / kStep;  // chunks, k-blocks per stage
  static constexpr int XB = BM * KB, WB = BN * KB, SB = XB + WB;
  static constexpr int XI = XB / 1024 / kPipeNL, WI = WB / 1024 / kPipeNL;  // loads per loader wave
  static constexpr int LDS = kPipeNS * SB + 64 + 4 * (16 * TM) * kEpPitch;  // + epilogue blocks
};

__device__ __forceinline__ void pipe_decode(int t, int ntn, int& tm, int& tn) {
  const int x = t & 7, r = t >> 3, q = r / ntn;
  tm = q * 8 + x;
  tn = r - q * ntn;
}

template <int BM, int BN>
__global__ __launch_bounds__(kPipeThreads) void iqlinear_pipe(LinParams p) {
  typedef PipeCfg<BM, BN> C;
  constexpr int TM = C::TM, TN = C::TN, NS = kPipeNS, NL = kPipeNL;
  static_assert((C::XI + C::WI) * kPipeLag < 64, "vmcnt range");
  static_assert(C::XI * NL * 1024 == C::XB && C::WI * NL * 1024 == C::WB, "stage split");
  static_assert(kPipeLag < NS, "ring depth");
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  int* const ready = (int*)(smem + NS * C::SB);
  int* const done = ready + NS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int G = (int)gridDim.x;
  const int ntm = (p.rows + BM - 1) / BM, ntn = (p.out_f + BN - 1) / BN;
  const int total_t = 8 * ntn * ((ntm + 7) / 8);
  constexpr int KB = C::KB, NCH = C::NCH, KPS = C::KPS;
  const int nkb = p.in_f / kStep;              // 64-byte k-blocks per tile
  const int nks = (nkb + KPS - 1) / KPS;       // stages per tile
  if (tid < NS) {
    ready[tid] = 0;
    done[tid] = 0;
  }
  __syncthreads();
  const uint32_t sm0 = lds_addr(smem);

  if (wave >= 4) {
    // ---- loader wave wl: 1 KB blocks wl, wl + NL, ... of each stage's X and W parts
    const int wl = wave - 4;
    const v4i xr = make_rsrc(p.x, (uint32_t)(p.rows * p.in_f));
    const v4i wr = make_rsrc(p.w, (uint32_t)(p.out_f * p.in_f));
    auto mark = [&](int step) {
      if (lane == 0)
        __hip_atomic_fetch_add(&ready[step % NS], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int s = 0;
    for (int t = blockIdx.x; t < total_t; t += G) {
      int tm, tn;
      pipe_decode(t, ntn, tm, tn);
      if (tm >= ntm) continue;
      const int m0 = tm * BM, n0 = tn * BN;
      for (int ks = 0; ks < nks; ++ks, ++s) {
        const int b = s % NS;
        if (s >= NS) {  // the slot's previous step has been read by every compute wave
          const int need = 4 * (s / NS);
          int spins = 0;
          while (__hip_atomic_load(&done[b], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
            if (++spins > kPipeSpin) return;
            __builtin_amdgcn_s_sleep(1);
          }
        }
        const uint32_t sb = sm0 + b * C::SB;
#pragma unroll
        for (int j = 0; j < C::XI; ++j) {
          const int i = wl + NL * j;
          const int o = 1024 * i + 16 * lane, row = o / KB, cp = (o >> 4) & (NCH - 1);
          raw_buffer_load_lds(xr, (lds_u32w*)(uintptr_t)(sb + 1024 * i), 16,
                              (m0 + row) * p.in_f + KB * ks + 16 * (cp ^ ((row >> 1) & (NCH - 1))), 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < C::WI; ++j) {
          const int i = wl + NL * j;
          const int o = 1024 * i + 16 * lane, row = o / KB, cp = (o >> 4) & (NCH - 1);
          raw_buffer_load_lds(wr, (lds_u32w*)(uintptr_t)(sb + C::XB + 1024 * i), 16,
                              (n0 + row) * p.in_f + KB * ks + 16 * (cp ^ ((row >> 1) & (NCH - 1))), 0, 0, 0);
        }
        // this wave's share of the stage issued kPipeLag steps ago has landed
        if (s >= kPipeLag) {
          __builtin_amdgcn_s_waitcnt(pipe_vmcnt(kPipeLag * (C::XI + C::WI)));
          mark(s - kPipeLag);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(pipe_vmcnt(0));
    for (int q = s - kPipeLag; q < s; ++q)
      if (q >= 0) mark(q);
    return;
  }

  // ---- compute waves: wave (wm, wn) owns rows 16 (TM wm + b) + li and columns
  //      16 (TN wn + a) + 4 g + r of the tile
  const int wm = wave & 1, wn = wave >> 1;
  int8_t* const ep_scr = smem + NS * C::SB + 64 + wave * (16 * TM) * kEpPitch;
  const bool wide_ep = p.layout != IQLINEAR_QKV_HEADS || p.head_dim % 16 == 0;
  auto wait_ready = [&](int step) -> bool {
    const int need = NL * (step / NS + 1);
    int spins = 0;
    while (__hip_atomic_load(&ready[step % NS], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
      if (++spins > kPipeSpin) return false;
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };
  // operand fragments of k-block j of a stage: row r, chunk (4 j + g) ^ swizzle(r)
  auto lds_off = [&](int r, int j) { return r * KB + 16 * ((4 * j + g) ^ ((r >> 1) & (NCH - 1))); };
  typedef std::integral_constant<int, 0> J0;
  typedef std::integral_constant<int, 1> J1;
  auto read_frags = [&](int step, auto jc, v4i (&fx)[TM], v4i (&fw)[TN]) {
    constexpr int j = decltype(jc)::value;
    const int8_t* sb = smem + (step % NS) * C::SB;
#pragma unroll
    for (int b = 0; b < TM; ++b) fx[b] = *(const v4i*)(sb + lds_off(16 * (TM * wm + b) + li, j));
#pragma unroll
    for (int a = 0; a < TN; ++a) fw[a] = *(const v4i*)(sb + C::XB + lds_off(16 * (TN * wn + a) + li, j));
  };
  auto signal_done = [&](int step) {
    if (lane == 0) __hip_atomic_fetch_add(&done[step % NS], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  int s = 0;
  for (int t = blockIdx.x; t < total_t; t += G) {
    int tm, tn;
    pipe_decode(t, ntn, tm, tn);
    if (tm >= ntm) continue;
    const int m0 = tm * BM, n0 = tn * BN;
    v4i acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) acc[a][b] = v4i{0, 0, 0, 0};
    // per stage: block 1's fragments are read while block 0's MFMAs run, the
    // stage is released once they are in registers, and the next stage's
    // block 0 is read while block 1's MFMAs run
    v4i fx0[TM], fw0[TN], fx1[TM], fw1[TN];
    if (!wait_ready(s)) return;
    read_frags(s, J0(), fx0, fw0);
    for (int st = 0; st < nks; ++st) {
      const bool two = 2 * st + 1 < nkb;  // the stage's second k-block exists
      if (two) read_frags(s + st, J1(), fx1, fw1);
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = mfma64(fw0[a], fx0[b], acc[a][b]);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every fragment of the stage is in registers
      signal_done(s + st);
      if (st + 1 < nks) {
        if (!wait_ready(s + st + 1)) return;
        read_frags(s + st + 1, J0(), fx0, fw0);
      }
      if (two) {
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
          for (int b = 0; b < TM; ++b) acc[a][b] = mfma64(fw1[a], fx1[b], acc[a][b]);
      }
    }
    s += nks;
    if (wide_ep)
      store_tile_lds<TM, TN>(p, acc, ep_scr, m0 + 16 * TM * wm, n0 + 16 * TN * wn, li, g, lane);
    else
      store_tile<TM, TN>(p, acc, m0 + 16 * TM * wm + li, n0 + 16 * TN * wn + 4 * g);
  }
}

}  // namespace
}  // namespace iqattn

using namespace iqattn;

struct iqlinear_ctx {
  LinParams lp;
  int device;
  unsigned grid;  // persistent grid of the pipelined kernel
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
  // pipelined kernel: one persistent workgroup per CU, 128 x 128 tiles
  {
    const int cus = prop.multiProcessorCount;
    const int64_t tiles = ((int64_t)p->rows + 127) / 128 * ((p->out_features + 127) / 128);
    c->grid = (unsigned)(tiles < cus ? (tiles > 0 ? tiles : 1) : cus);
    if (hipFuncSetAttribute((const void*)&iqlinear_pipe<128, 128>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            PipeCfg<128, 128>::LDS) != hipSuccess) {
      free(c);
      return IQATTN_E_DEVICE;
    }
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
  constexpr int lds = PipeCfg<128, 128>::LDS;
  hipLaunchKernelGGL((iqlinear_pipe<128, 128>), dim3(c->grid), dim3(kPipeThreads), lds,
                     (hipStream_t)hip_stream, lp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_hip_error(e, "iqlinear launch");
  return IQATTN_OK;
}

extern "C" int iqlinear_destroy(iqlinear_ctx* c) {
  free(c);
  return IQATTN_OK;
}
