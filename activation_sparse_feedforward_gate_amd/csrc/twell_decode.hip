// Forward for few tokens (decode-shaped batches, T <= 256, bf16 inputs,
// inference), and the dense few-token forward it is measured against.
//
// With a few dozen tokens every phase of the layer is a pass over weights:
// WgT whole, then the rows of WuT and Wd of the neurons active in any token
// (one row block, so one union: [IN] "Слитые CUDA-ядра для инференса и гибрид
// для обучения" keeps only the active neurons in the up/down phases).  The
// prefill kernels would run a handful of workgroups here, so each GEMM is
// split along K over many workgroups (64x64 output tiles of four waves on the
// direct-to-LDS mainloop, whose coalesced loads stream the weights at close
// to the rate of a plain copy) that write fp32 partial sums; small kernels
// then reduce the partials:
//   1 gate partials   Pg[s] = x . WgT[:, Ks]^T
//   2 pack            g = sum_s Pg[s] + b, TwELL pack of ReLU(g) (fp32
//                     values) and the OR of each 64-row slab's masks; one
//                     workgroup per 16x64 tile, four rows per wave
//   3 union list      (the prefill list kernel, one row block)
//   4 up partials     Pu[s] = x . WuT[ulist][:, Ks]^T
//   5 a               a = h * sum_s Pu[s] at the stored pairs, else 0, split
//                     into bf16 hi + lo (exact to about 2^-17 relative)
//   6 down partials   Py[s] = (a_hi + a_lo)[:, Ps] . Wd[ulist[Ps]]
//   7 reduce          y = sum_s Py[s]
// The dense few-token forward uses the same blocks: gate and up partials in
// one GEMM with two B operands, act = bf16(ReLU(sum Pg + b) * sum Pu), then
// 6 and 7 over all F neurons.  All sums are in a fixed order, so results do
// not depend on timing.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

// 64x64 output tiles, four waves of 32x32 each
using SplitCfg = DmaCfg<64, 64, 2, 2>;                      // K-major B
using SplitCfg2 = DmaCfg<64, 64, 2, 2, 2>;                  // two K-major B sharing A
using SplitCfgBT = DmaCfg<64, 64, 2, 2, 1, false, true>;    // [K][N] B, gathered K

constexpr int KS_GATE = 4, KS_UP = 8, KS_DOWN = 16;
constexpr int KS_DENSE_GU = 2;   // the dense gate/up GEMM reads twice the bytes per split: fewer splits are faster

struct DecArgs {
  const uint16_t* x;
  const uint16_t* WgT;
  const uint16_t* bg;
  const uint16_t* WuT;
  const uint16_t* Wd;
  int T, d, F, NT;
  const int* ulist;     // the row block's union list (block 0)
  const int* ucount;
  uint64_t* slabs;      // 64-row slab unions [ceil(T/64)][NT], filled by the pack
  float* pg;            // [KS_GATE][T][F]
  float* pu;            // [KS_UP][T][F]  (dense path: [KS_DENSE_GU][T][F], and pg likewise)
  uint16_t* ahi;        // [T][F]         (dense path: act)
  uint16_t* alo;        // [T][F]
  float* py;            // [KS_DOWN][T][d]
  void* y;
  int out_bf16;
  // TwELL of h
  uint8_t* cnt;
  uint8_t* width;
  float* hval;
  uint8_t* hidx;
  uint64_t* hmask;
};

namespace {

// K range of split s of KS over K, in whole 64-wide tiles.
__device__ __forceinline__ void split_range(int K, int KS, int s, int& k0, int& kn) {
  const int tiles = (K + 63) / 64;
  const int per = (tiles + KS - 1) / KS;
  k0 = min(s * per, tiles) * 64;
  kn = min(K, min(s * per + per, tiles) * 64) - k0;
}

template <class Cfg>
__device__ __forceinline__ void store_partial(const DmaTile<Cfg>& g, int b, float* P, int ld, int rows, int m0,
                                              int n0) {
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + DmaTile<Cfg>::row_of(i, e);
        if (r < rows) P[(int64_t)r * ld + n0 + DmaTile<Cfg>::col_of(j)] = g.acc[b][i][j][e];
      }
}

template <class Cfg>
__device__ __forceinline__ void zero_tile(DmaTile<Cfg>& g) {
#pragma unroll
  for (int b = 0; b < Cfg::NB; ++b)
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) g.acc[b][i][j][e] = 0.f;
}

}  // namespace

// 1 / 4: partial x . W^T over one K split; W rows gathered through the union
// list for the up-projection (positions past the list's end are clamped to
// its last entry and never read back).
template <bool UP>
__device__ __forceinline__ void dec_splitk(const DecArgs& a, char* st0, char* st1) {
  constexpr int KS = UP ? KS_UP : KS_GATE;
  const int s = blockIdx.y, n0 = blockIdx.x * 64, m0 = blockIdx.z * 64;
  if (!UP && s == 0 && threadIdx.x == 0) a.slabs[(int64_t)blockIdx.z * a.NT + blockIdx.x] = 0;   // cleared for the pack
  const int ncols = UP ? *a.ucount : a.F;
  if (n0 >= ncols) return;
  int k0, kn;
  split_range(a.d, KS, s, k0, kn);
  float* P = (UP ? a.pu : a.pg) + (int64_t)s * a.T * a.F;
  DmaTile<SplitCfg> g;
  if (kn > 0) {
    const Operand A{a.x + k0, a.d, nullptr, a.T};
    const Operand B{(UP ? a.WuT : a.WgT) + k0, a.d, UP ? a.ulist : nullptr, ncols};
    g.run(A, &B, m0, n0, kn, st0, st1);
  } else {
    zero_tile(g);
  }
  store_partial(g, 0, P, a.F, a.T, m0, n0);
}

__global__ __launch_bounds__(SplitCfg::NTH) void dec_gate_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfg::STAGE];
  dec_splitk<false>(a, st0, st1);
}

__global__ __launch_bounds__(SplitCfg::NTH) void dec_up_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfg::STAGE];
  dec_splitk<true>(a, st0, st1);
}

// 2: g = sum of the gate partials + bias; TwELL pack of ReLU(g).  One
// workgroup per (row tile, column tile); wave w takes rows 4w..4w+3, lane =
// column.  Every lane issues its 16 partial loads at once.
__global__ __launch_bounds__(256) void dec_pack_kernel(DecArgs a) {
  __shared__ int wmax[4];
  __shared__ uint64_t wor[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x / a.NT, j = blockIdx.x % a.NT;
  const int col = j * 64 + lane;
  const float b = a.bg ? bf16_to_f32(a.bg[col]) : 0.f;
  float v[4];
  uint64_t M[4];
  int wd = 0;
  uint64_t any = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = i * 16 + 4 * w + q;
    float g = 0.f;
    if (t < a.T) {
#pragma unroll
      for (int s = 0; s < KS_GATE; ++s) g += a.pg[((int64_t)s * a.T + t) * a.F + col];
      g += b;
    }
    v[q] = g;
    M[q] = ballot(t < a.T && g > 0.f);
    wd = max(wd, popc64(M[q]));
    any |= M[q];
  }
  if (lane == 0) {
    wmax[w] = wd;
    wor[w] = any;
  }
  __syncthreads();
  wd = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int64_t tile = (int64_t)i * a.NT + j;
  if (threadIdx.x == 0) {
    a.width[tile] = (uint8_t)wd;
    const uint64_t u = wor[0] | wor[1] | wor[2] | wor[3];
    if (u) atomicOr((unsigned long long*)&a.slabs[(int64_t)(i >> 2) * a.NT + j], (unsigned long long)u);
  }
  const int64_t tbase = tile * (64 * 16);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * w + q, t = i * 16 + r;
    const int c = popc64(M[q]);
    if (lane == 0 && t < a.T) {
      a.cnt[(int64_t)t * a.NT + j] = (uint8_t)c;
      a.hmask[(int64_t)t * a.NT + j] = M[q];
    }
    const int nb = popc64(M[q] & below(lane));
    const bool act = (M[q] >> lane) & 1ull;
    const int slot = act ? nb : c + (lane - nb);
    if (slot < wd) {
      a.hval[tbase + slot * 16 + r] = act ? v[q] : 0.f;
      a.hidx[tbase + slot * 16 + r] = act ? (uint8_t)lane : (uint8_t)0;
    }
  }
}

// 5: a[t][p] = h[t][ulist[p]] * sum of the up partials, stored as a bf16
// hi + lo pair; positions in [n, roundup64(n)) are zeros.
__global__ __launch_bounds__(256) void dec_a_kernel(DecArgs a) {
  const int n = *a.ucount;
  const int npad = (n + 63) & ~63;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)a.T * npad) return;
  const int t = (int)(e / npad), p = (int)(e % npad);
  float v = 0.f;
  if (p < n) {
    const int nn = a.ulist[p];
    const int tj = nn >> 6, c = nn & 63;
    const uint64_t M = a.hmask[(int64_t)t * a.NT + tj];
    if ((M >> c) & 1ull) {
      const int slot = popc64(M & below(c));
      const float h = a.hval[((int64_t)(t >> 4) * a.NT + tj) * 1024 + slot * 16 + (t & 15)];
      float u = 0.f;
#pragma unroll
      for (int s = 0; s < KS_UP; ++s) u += a.pu[((int64_t)s * a.T + t) * a.F + p];
      v = h * u;
    }
  }
  uint32_t hi, lo;
  split_bf16(v, hi, lo);
  a.ahi[(int64_t)t * a.F + p] = (uint16_t)hi;
  a.alo[(int64_t)t * a.F + p] = (uint16_t)lo;
}

// 6: y partial over one split of K: A[:, Ks] . Wd rows of Ks; K is the union
// positions (GATHER: Wd rows through the list, A = a_hi + a_lo) or all F
// neurons (A = act, bf16).
template <bool GATHER>
__device__ __forceinline__ void dec_down(const DecArgs& a, char* st0, char* st1) {
  const int s = blockIdx.y, n0 = blockIdx.x * 64, m0 = blockIdx.z * 64;
  int k0, kn;
  split_range(GATHER ? *a.ucount : a.F, KS_DOWN, s, k0, kn);
  DmaTile<SplitCfgBT> g;
  if (kn > 0) {
    const Operand B = GATHER ? Operand{a.Wd, a.d, a.ulist + k0, a.F}
                             : Operand{a.Wd + (int64_t)k0 * a.d, a.d, nullptr, a.F};
    const Operand A0{a.ahi + k0, a.F, nullptr, a.T};
    g.run(A0, &B, m0, n0, kn, st0, st1);
    if constexpr (GATHER) {
      const Operand A1{a.alo + k0, a.F, nullptr, a.T};
      g.run(A1, &B, m0, n0, kn, st0, st1, false);
    }
  } else {
    zero_tile(g);
  }
  store_partial(g, 0, a.py + (int64_t)s * a.T * a.d, a.d, a.T, m0, n0);
}

__global__ __launch_bounds__(SplitCfgBT::NTH) void dec_down_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfgBT::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfgBT::STAGE];
  dec_down<true>(a, st0, st1);
}

__global__ __launch_bounds__(SplitCfgBT::NTH) void dense_few_down_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfgBT::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfgBT::STAGE];
  dec_down<false>(a, st0, st1);
}

// 7: y = sum of the down partials.
__global__ __launch_bounds__(256) void dec_reduce_kernel(DecArgs a) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)a.T * a.d) return;
  float v = 0.f;
#pragma unroll
  for (int s = 0; s < KS_DOWN; ++s) v += a.py[(int64_t)s * a.T * a.d + e];
  if (a.out_bf16) ((uint16_t*)a.y)[e] = (uint16_t)f32_to_bf16_bits(v);
  else ((float*)a.y)[e] = v;
}

// Dense path, 1: gate and up partials of one K split, one GEMM with the two
// weight matrices as B operands sharing the x tiles.
__global__ __launch_bounds__(SplitCfg2::NTH) void dense_few_gu_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfg2::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfg2::STAGE];
  const int s = blockIdx.y, n0 = blockIdx.x * 64, m0 = blockIdx.z * 64;
  int k0, kn;
  split_range(a.d, KS_DENSE_GU, s, k0, kn);
  DmaTile<SplitCfg2> g;
  if (kn > 0) {
    const Operand A{a.x + k0, a.d, nullptr, a.T};
    const Operand B[2] = {{a.WgT + k0, a.d, nullptr, a.F}, {a.WuT + k0, a.d, nullptr, a.F}};
    g.run(A, B, m0, n0, kn, st0, st1);
  } else {
    zero_tile(g);
  }
  store_partial(g, 0, a.pg + (int64_t)s * a.T * a.F, a.F, a.T, m0, n0);
  store_partial(g, 1, a.pu + (int64_t)s * a.T * a.F, a.F, a.T, m0, n0);
}

// Dense path, 2: act = bf16(ReLU(sum Pg + b) * sum Pu).
__global__ __launch_bounds__(256) void dense_few_act_kernel(DecArgs a) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)a.T * a.F) return;
  const int n = (int)(e % a.F);
  float gs = 0.f, u = 0.f;
#pragma unroll
  for (int s = 0; s < KS_DENSE_GU; ++s) {
    gs += a.pg[(int64_t)s * a.T * a.F + e];
    u += a.pu[(int64_t)s * a.T * a.F + e];
  }
  const float g = gs + (a.bg ? bf16_to_f32(a.bg[n]) : 0.f);
  a.ahi[e] = (uint16_t)f32_to_bf16_bits(g > 0.f ? g * u : 0.f);
}

namespace {

size_t r256(size_t v) { return (v + 255) & ~(size_t)255; }

DecArgs dec_args(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd, int T, int d,
                 int F, void* y, int out_dt) {
  DecArgs a{};
  a.x = (const uint16_t*)x; a.WgT = (const uint16_t*)WgT; a.bg = (const uint16_t*)bg;
  a.WuT = (const uint16_t*)WuT; a.Wd = (const uint16_t*)Wd;
  a.T = T; a.d = d; a.F = F; a.NT = F / 64;
  a.y = y; a.out_bf16 = out_dt == DT_BF16;
  return a;
}

void launch_down_reduce(const DecArgs& a, bool gather, hipStream_t s) {
  const dim3 grid(a.d / 64, KS_DOWN, (a.T + 63) / 64);
  if (gather) hipLaunchKernelGGL(dec_down_kernel, grid, dim3(SplitCfgBT::NTH), 0, s, a);
  else hipLaunchKernelGGL(dense_few_down_kernel, grid, dim3(SplitCfgBT::NTH), 0, s, a);
  hipLaunchKernelGGL(dec_reduce_kernel, dim3((unsigned)(((int64_t)a.T * a.d + 255) / 256)), dim3(256), 0, s, a);
}

}  // namespace

size_t decode_ws_bytes(int T, int d, int F) {
  return r256((size_t)KS_GATE * T * F * 4) + r256((size_t)KS_UP * T * F * 4) + 2 * r256((size_t)T * F * 2) +
         r256((size_t)KS_DOWN * T * d * 4);
}

hipError_t launch_decode_fwd(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd, int T,
                             int d, int F, const TwellView& h, void* ws, void* uni_ws, void* y, int out_dt,
                             hipStream_t s, hipEvent_t ev_gate, hipEvent_t ev_lists, hipEvent_t ev_up) {
  if (T == 0) return hipSuccess;
  char* w = (char*)ws;
  DecArgs a = dec_args(x, WgT, bg, WuT, Wd, T, d, F, y, out_dt);
  a.pg = (float*)w; w += r256((size_t)KS_GATE * T * F * 4);
  a.pu = (float*)w; w += r256((size_t)KS_UP * T * F * 4);
  a.ahi = (uint16_t*)w; w += r256((size_t)T * F * 2);
  a.alo = (uint16_t*)w; w += r256((size_t)T * F * 2);
  a.py = (float*)w;
  a.cnt = h.cnt; a.width = h.width; a.hval = (float*)h.val; a.hidx = h.idx; a.hmask = h.mask;
  int* ulist = nullptr;
  int* ucount = nullptr;
  uint64_t* slabs = nullptr;
  union_lists_only(T, F, h, uni_ws, &ulist, &ucount, &slabs);
  a.ulist = ulist; a.ucount = ucount; a.slabs = slabs;
  const int mt = (T + 63) / 64;
  hipLaunchKernelGGL(dec_gate_kernel, dim3(F / 64, KS_GATE, mt), dim3(SplitCfg::NTH), 0, s, a);
  const int NR = (T + 15) / 16;
  hipLaunchKernelGGL(dec_pack_kernel, dim3((unsigned)((int64_t)NR * a.NT)), dim3(256), 0, s, a);
  if (ev_gate) (void)hipEventRecord(ev_gate, s);
  hipError_t e = launch_union_lists(T, F, h, uni_ws, s, true);
  if (e != hipSuccess) return e;
  if (ev_lists) (void)hipEventRecord(ev_lists, s);
  hipLaunchKernelGGL(dec_up_kernel, dim3(F / 64, KS_UP, mt), dim3(SplitCfg::NTH), 0, s, a);
  hipLaunchKernelGGL(dec_a_kernel, dim3((unsigned)(((int64_t)T * F + 255) / 256)), dim3(256), 0, s, a);
  if (ev_up) (void)hipEventRecord(ev_up, s);
  launch_down_reduce(a, true, s);
  return hipGetLastError();
}

size_t dense_few_ws_bytes(int T, int d, int F) {
  return 2 * r256((size_t)KS_DENSE_GU * T * F * 4) + r256((size_t)T * F * 2) + r256((size_t)KS_DOWN * T * d * 4);
}

hipError_t launch_dense_few_fwd(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd,
                                int T, int d, int F, void* ws, int out_dt, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  char* w = (char*)ws;
  DecArgs a = dec_args(x, WgT, bg, WuT, Wd, T, d, F, y, out_dt);
  a.pg = (float*)w; w += r256((size_t)KS_DENSE_GU * T * F * 4);
  a.pu = (float*)w; w += r256((size_t)KS_DENSE_GU * T * F * 4);
  a.ahi = (uint16_t*)w; w += r256((size_t)T * F * 2);
  a.py = (float*)w;
  hipLaunchKernelGGL(dense_few_gu_kernel, dim3(F / 64, KS_DENSE_GU, (T + 63) / 64), dim3(SplitCfg2::NTH), 0, s, a);
  hipLaunchKernelGGL(dense_few_act_kernel, dim3((unsigned)(((int64_t)T * F + 255) / 256)), dim3(256), 0, s, a);
  launch_down_reduce(a, false, s);
  return hipGetLastError();
}

}  // namespace twell
