// Forward for few tokens (decode-shaped batches, T <= 256, bf16 inputs).
//
// With a few dozen tokens every phase of the layer is a pass over weights:
// Wg whole, then the rows of Wu and Wd of the neurons active in any token
// (one row block, so one union: [IN] "Слитые CUDA-ядра для инференса и гибрид
// для обучения" keeps only the active neurons in the up/down phases).  The
// prefill kernels would run a handful of workgroups here, so each GEMM is
// split along K over many one-wave workgroups (64x64 output tiles on the
// direct-to-LDS mainloop) that write fp32 partial sums; small kernels then
// reduce the partials:
//   1 gate partials   Pg[s] = x . WgT[:, Ks]^T
//   2 pack            g = sum_s Pg[s] + b, TwELL pack of ReLU(g) (fp32 values)
//   3 union list      (the prefill list kernel, one row block; the pack has
//                     already OR-ed each 64-row slab's masks)
//   4 up partials     Pu[s] = x . WuT[ulist][:, Ks]^T
//   5 a               a = h * sum_s Pu[s] at the stored pairs, else 0, split
//                     into bf16 hi + lo (exact to about 2^-17 relative)
//   6 down partials   Py[s] = (a_hi + a_lo)[:, Ps] . Wd[ulist[Ps]]
//   7 reduce          y = sum_s Py[s]
// All sums are in a fixed order, so the result does not depend on timing.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

// 64x64 output tiles, four waves of 32x32 each
using SplitCfg = DmaCfg<64, 64, 2, 2>;                      // K-major B
using SplitCfgBT = DmaCfg<64, 64, 2, 2, 1, false, true>;    // [K][N] B, gathered K

constexpr int KS_GATE = 4, KS_UP = 8, KS_DOWN = 16;

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
  float* pu;            // [KS_UP][T][F]
  uint16_t* ahi;        // [T][F]
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

__device__ __forceinline__ void store_partial(const DmaTile<SplitCfg>& g, float* P, int ld, int rows, int m0,
                                              int n0) {
#pragma unroll
  for (int j = 0; j < SplitCfg::TN; ++j)
#pragma unroll
    for (int i = 0; i < SplitCfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + DmaTile<SplitCfg>::row_of(i, e);
        if (r < rows) P[(int64_t)r * ld + n0 + DmaTile<SplitCfg>::col_of(j)] = g.acc[0][i][j][e];
      }
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
#pragma unroll
    for (int i = 0; i < SplitCfg::TM; ++i)
#pragma unroll
      for (int j = 0; j < SplitCfg::TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) g.acc[0][i][j][e] = 0.f;
  }
  store_partial(g, P, a.F, a.T, m0, n0);
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

// 2: g = sum of the gate partials + bias; TwELL pack of ReLU(g).  One wave
// per (row tile, column tile), lane = column, as the standalone pack.
__global__ __launch_bounds__(256) void dec_pack_kernel(DecArgs a) {
  const int lane = threadIdx.x & 63;
  const int NR = (a.T + 15) / 16;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= (int64_t)NR * a.NT) return;
  const int i = (int)(tile / a.NT), j = (int)(tile % a.NT);
  const int col = j * 64 + lane;
  const float b = a.bg ? bf16_to_f32(a.bg[col]) : 0.f;
  float v[16];
  uint64_t M[16];
  int w = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = i * 16 + r;
    float g = 0.f;
    if (t < a.T) {
#pragma unroll
      for (int s = 0; s < KS_GATE; ++s) g += a.pg[((int64_t)s * a.T + t) * a.F + col];
      g += b;
    }
    v[r] = g;
    M[r] = ballot(t < a.T && g > 0.f);
    w = max(w, popc64(M[r]));
  }
  if (lane == 0) {
    a.width[tile] = (uint8_t)w;
    uint64_t u = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) u |= M[r];
    if (u) atomicOr((unsigned long long*)&a.slabs[(int64_t)(i >> 2) * a.NT + j], (unsigned long long)u);
  }
  const int64_t tbase = tile * (64 * 16);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = i * 16 + r;
    const int c = popc64(M[r]);
    if (lane == 0 && t < a.T) {
      a.cnt[(int64_t)t * a.NT + j] = (uint8_t)c;
      a.hmask[(int64_t)t * a.NT + j] = M[r];
    }
    const int nb = popc64(M[r] & below(lane));
    const bool act = (M[r] >> lane) & 1ull;
    const int slot = act ? nb : c + (lane - nb);
    if (slot < w) {
      a.hval[tbase + slot * 16 + r] = act ? v[r] : 0.f;
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

// 6: y partial over one split of the union positions: (a_hi + a_lo) . Wd rows.
__global__ __launch_bounds__(SplitCfgBT::NTH) void dec_down_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfgBT::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfgBT::STAGE];
  const int s = blockIdx.y, n0 = blockIdx.x * 64, m0 = blockIdx.z * 64;
  int k0, kn;
  split_range(*a.ucount, KS_DOWN, s, k0, kn);
  DmaTile<SplitCfgBT> g;
  if (kn > 0) {
    const Operand B{a.Wd, a.d, a.ulist + k0, a.F};
    const Operand A0{a.ahi + k0, a.F, nullptr, a.T}, A1{a.alo + k0, a.F, nullptr, a.T};
    g.run(A0, &B, m0, n0, kn, st0, st1);
    g.run(A1, &B, m0, n0, kn, st0, st1, false);
  } else {
#pragma unroll
    for (int i = 0; i < SplitCfgBT::TM; ++i)
#pragma unroll
      for (int j = 0; j < SplitCfgBT::TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) g.acc[0][i][j][e] = 0.f;
  }
  float* P = a.py + (int64_t)s * a.T * a.d;
#pragma unroll
  for (int j = 0; j < SplitCfgBT::TN; ++j)
#pragma unroll
    for (int i = 0; i < SplitCfgBT::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + DmaTile<SplitCfgBT>::row_of(i, e);
        if (r < a.T) P[(int64_t)r * a.d + n0 + DmaTile<SplitCfgBT>::col_of(j)] = g.acc[0][i][j][e];
      }
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

size_t decode_ws_bytes(int T, int d, int F) {
  auto r = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return r((size_t)KS_GATE * T * F * 4) + r((size_t)KS_UP * T * F * 4) + 2 * r((size_t)T * F * 2) +
         r((size_t)KS_DOWN * T * d * 4);
}

hipError_t launch_decode_fwd(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd, int T,
                             int d, int F, const TwellView& h, void* ws, void* uni_ws, void* y, int out_dt,
                             hipStream_t s, hipEvent_t ev_gate, hipEvent_t ev_lists, hipEvent_t ev_up) {
  if (T == 0) return hipSuccess;
  auto r = [](size_t v) { return (v + 255) & ~(size_t)255; };
  char* w = (char*)ws;
  DecArgs a{};
  a.x = (const uint16_t*)x; a.WgT = (const uint16_t*)WgT; a.bg = (const uint16_t*)bg;
  a.WuT = (const uint16_t*)WuT; a.Wd = (const uint16_t*)Wd;
  a.T = T; a.d = d; a.F = F; a.NT = F / 64;
  a.pg = (float*)w; w += r((size_t)KS_GATE * T * F * 4);
  a.pu = (float*)w; w += r((size_t)KS_UP * T * F * 4);
  a.ahi = (uint16_t*)w; w += r((size_t)T * F * 2);
  a.alo = (uint16_t*)w; w += r((size_t)T * F * 2);
  a.py = (float*)w;
  a.y = y; a.out_bf16 = out_dt == DT_BF16;
  a.cnt = h.cnt; a.width = h.width; a.hval = (float*)h.val; a.hidx = h.idx; a.hmask = h.mask;
  int* ulist = nullptr;
  int* ucount = nullptr;
  uint64_t* slabs = nullptr;
  union_lists_only(T, F, h, uni_ws, &ulist, &ucount, &slabs);
  a.ulist = ulist; a.ucount = ucount; a.slabs = slabs;
  const int mt = (T + 63) / 64;
  hipLaunchKernelGGL(dec_gate_kernel, dim3(F / 64, KS_GATE, mt), dim3(SplitCfg::NTH), 0, s, a);
  const int NR = (T + 15) / 16;
  hipLaunchKernelGGL(dec_pack_kernel, dim3((unsigned)(((int64_t)NR * a.NT + 3) / 4)), dim3(256), 0, s, a);
  if (ev_gate) (void)hipEventRecord(ev_gate, s);
  hipError_t e = launch_union_lists(T, F, h, uni_ws, s, true);
  if (e != hipSuccess) return e;
  if (ev_lists) (void)hipEventRecord(ev_lists, s);
  hipLaunchKernelGGL(dec_up_kernel, dim3(F / 64, KS_UP, mt), dim3(SplitCfg::NTH), 0, s, a);
  hipLaunchKernelGGL(dec_a_kernel, dim3((unsigned)(((int64_t)T * F + 255) / 256)), dim3(256), 0, s, a);
  if (ev_up) (void)hipEventRecord(ev_up, s);
  hipLaunchKernelGGL(dec_down_kernel, dim3(d / 64, KS_DOWN, mt), dim3(SplitCfgBT::NTH), 0, s, a);
  hipLaunchKernelGGL(dec_reduce_kernel, dim3((unsigned)(((int64_t)T * d + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace twell
