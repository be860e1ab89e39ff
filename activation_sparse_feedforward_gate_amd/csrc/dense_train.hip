// Dense training step of the ReLU-gated FFN on the direct-to-LDS mainloop:
// the speedup denominator of the hybrid sparse/dense training path.  Forward
// and backward of
//
//   g = x.WgT^T + b,  h = ReLU(g),  u = x.WuT^T,  a = h*u,  y = a.Wd
//
// with bf16 intermediates (h, u, a, dG, dU stored as bf16 [T][F]; h and u
// interleaved, one 32-bit word per element) and fp32 accumulation, nine GEMMs:
//   1  g, u    (dual GEMM; epilogue stores (h, u) and a)
//   2  y  = a.Wd
//   3  dA = dY.Wd^T  (epilogue: dG = dA*u*[g>0], dU = dA*h, per-block dbg sums)
//   4  dX = dG.WgT + dU.WuT
//   5  dWgT = dG^T.x,  6  dWuT = dU^T.x,  7  dWd = a^T.dY
// The hybrid training step it is compared with is [IN] "Слитые CUDA-ядра для
// инференса и гибрид для обучения"; this file is the plain dense version of
// the same layer.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

namespace {

struct TrainArgs {
  const uint16_t* x;
  const uint16_t* WgT;
  const uint16_t* bg;
  const uint16_t* WuT;
  const uint16_t* Wd;
  const uint16_t* dY;
  int T, d, F;
  uint32_t* hu32;   // [T][F]: bf16 h in the low half, bf16 u in the high half
  uint16_t* a16;
  uint16_t* dg16;
  uint16_t* du16;
  float* dbg_part;  // [ceil(T/256)][F]
};

__device__ __forceinline__ void order(int id, int nbm, int nbn, int& bm, int& bn) {
  constexpr int GM = 8;
  const int per_group = GM * nbn;
  const int group = id / per_group;
  const int first = group * GM;
  const int gsize = min(nbm - first, GM);
  const int r = id - group * per_group;
  bm = first + r % gsize;
  bn = r / gsize;
}

__device__ __forceinline__ uint16_t bf(float v) { return (uint16_t)f32_to_bf16_bits(v); }

}  // namespace

// 1: g and u for a 256x128 tile; stores h, u and a = h*u as bf16.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void train_gateup_kernel(TrainArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  int bm, bn;
  order(xcd_remap(blockIdx.x, gridDim.x), (a.T + Cfg::BM - 1) / Cfg::BM, a.F / Cfg::BN, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B[2] = {{a.WgT, a.d, nullptr, a.F}, {a.WuT, a.d, nullptr, a.F}};
  g.run(A, B, m0, n0, a.d, st0, st1);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
    const float b = a.bg ? bf16_to_f32(a.bg[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + Tile::row_of(i, e);
        if (row < a.T) {
          const float gv = g.acc[0][i][j][e] + b;
          const float h = gv > 0.f ? gv : 0.f;
          const float u = g.acc[1][i][j][e];
          const int64_t o = (int64_t)row * a.F + col;
          a.hu32[o] = (uint32_t)bf(h) | ((uint32_t)bf(u) << 16);
          a.a16[o] = bf(h * u);
        }
      }
  }
}

// 3: dA = dY.Wd^T for a 256x256 tile of [T][F]; epilogue dG, dU (bf16) and
// the tile's column sums of dG (one partial per 256-row block).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void train_da_kernel(TrainArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  static_assert(Cfg::BM == 256, "one dbg partial per 256-row block");
  int bm, bn;
  order(xcd_remap(blockIdx.x, gridDim.x), (a.T + Cfg::BM - 1) / Cfg::BM, a.F / Cfg::BN, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.dY, a.d, nullptr, a.T};
  const Operand B{a.Wd, a.d, nullptr, a.F};
  g.run(A, &B, m0, n0, a.d, st0, st1);
  // Lanes l and l^1 hold neighbouring columns of the same rows: for each
  // group of 4 rows, the even lane loads rows 0 and 2 of the column pair and
  // the odd lane rows 1 and 3 (8-byte loads of two (h, u) words), one
  // exchange gives each lane its own column, and dG, dU go out as 4-byte
  // stores of column pairs (the even lane rows 0 and 2, the odd lane rows 1
  // and 3).  Column sums of dG: per lane over its rows, then across the two
  // row halves of the wave (lanes l and l^32) and across the waves of a
  // column (LDS).
  float* csum = (float*)st0;                       // [WM][BN]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool odd = lane & 1;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int cl = Tile::col_of(j);
    const int ce = n0 + (cl & ~1);                 // even column of the lane pair
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int r0 = m0 + Tile::row_of(i, 4 * qq);   // rows r0..r0+3
        uint32_t own[4];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int r = r0 + 2 * m + (odd ? 1 : 0);
          const uint2 L = r < a.T ? *(const uint2*)(a.hu32 + (int64_t)r * a.F + ce) : make_uint2(0u, 0u);
          const uint32_t recv = (uint32_t)__shfl_xor((int)(odd ? L.x : L.y), 1);
          own[2 * m] = odd ? recv : L.x;
          own[2 * m + 1] = odd ? L.y : recv;
        }
        float dg[4], du[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float h = bf16_lo(own[k]), u = bf16_hi(own[k]);
          const float dA = g.acc[0][i][j][4 * qq + k];
          dg[k] = h > 0.f ? dA * u : 0.f;
          du[k] = dA * h;
          if (r0 + k < a.T) s += dg[k];
        }
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          const int kr = odd ? k + 1 : k;                  // row this lane stores
          const float sg = __shfl_xor(odd ? dg[k] : dg[k + 1], 1);
          const float su = __shfl_xor(odd ? du[k] : du[k + 1], 1);
          if (r0 + kr < a.T) {
            const uint32_t pg = odd ? ((uint32_t)bf(sg) | ((uint32_t)bf(dg[k + 1]) << 16))
                                    : ((uint32_t)bf(dg[k]) | ((uint32_t)bf(sg) << 16));
            const uint32_t pu = odd ? ((uint32_t)bf(su) | ((uint32_t)bf(du[k + 1]) << 16))
                                    : ((uint32_t)bf(du[k]) | ((uint32_t)bf(su) << 16));
            const int64_t o = (int64_t)(r0 + kr) * a.F + ce;
            *(uint32_t*)(a.dg16 + o) = pg;
            *(uint32_t*)(a.du16 + o) = pu;
          }
        }
      }
    s += __shfl_xor(s, 32);
    if (lane < 32) csum[(wave / Cfg::WN) * Cfg::BN + cl] = s;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < Cfg::BN; c += Cfg::NTH) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < Cfg::WM; ++w) s += csum[w * Cfg::BN + c];
    a.dbg_part[(int64_t)bm * a.F + n0 + c] = s;
  }
}

// 4: dX = dG.WgT + dU.WuT (fp32 out).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void train_dx_kernel(TrainArgs a, float* dX) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  int bm, bn;
  order(xcd_remap(blockIdx.x, gridDim.x), (a.T + Cfg::BM - 1) / Cfg::BM, a.d / Cfg::BN, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A0{a.dg16, a.F, nullptr, a.T}, A1{a.du16, a.F, nullptr, a.T};
  const Operand B0{a.WgT, a.d, nullptr, a.F}, B1{a.WuT, a.d, nullptr, a.F};
  g.run(A0, &B0, m0, n0, a.F, st0, st1);
  g.run(A1, &B1, m0, n0, a.F, st0, st1, false);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + Tile::row_of(i, e);
        if (row < a.T) __builtin_nontemporal_store(g.acc[0][i][j][e], dX + (int64_t)row * a.d + col);   // streamed, as the TwELL step's
      }
  }
}

// 5-7: C[F][d] = P^T.Q with P [T][F] and Q [T][d] (K = T), fp32 out.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void train_wgrad_kernel(const uint16_t* P, const uint16_t* Q, int T, int d,
                                                               int F, float* C) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  int bm, bn;
  order(xcd_remap(blockIdx.x, gridDim.x), F / Cfg::BM, d / Cfg::BN, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{P, F, nullptr, T};
  const Operand B{Q, d, nullptr, T};
  g.run(A, &B, m0, n0, T, st0, st1);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) C[(int64_t)(m0 + Tile::row_of(i, e)) * d + col] = g.acc[0][i][j][e];
  }
}

__global__ __launch_bounds__(256) void train_dbg_kernel(const float* part, int nblk, int F, float* dbg) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= F) return;
  float s = 0.f;
  for (int b = 0; b < nblk; ++b) s += part[(int64_t)b * F + n];
  dbg[n] = s;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0 || !p) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

using TrainGateUp = DmaCfg<256, 128, 4, 2, 2>;
using TrainDA = DmaCfg<256, 256, 2, 4>;
using TrainDX = DmaCfg<256, 256, 2, 4, 1, false, true>;
using TrainWgrad = DmaCfg<256, 256, 2, 4, 1, false, true, true>;

size_t dense_train_ws_bytes(int T, int d, int F) {
  (void)d;
  const size_t tf = ((size_t)T * F * 2 + 255) & ~(size_t)255;
  return 5 * tf + (size_t)((T + 255) / 256) * F * 4;
}

hipError_t launch_dense_train(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd,
                              const void* dY, int T, int d, int F, void* ws, int out_dt, void* y, float* dX,
                              float* dWgT, float* dWuT, float* dWd, float* dbg, hipStream_t s) {
  const size_t tf = ((size_t)T * F * 2 + 255) & ~(size_t)255;
  char* w = (char*)ws;
  TrainArgs a{(const uint16_t*)x, (const uint16_t*)WgT, (const uint16_t*)bg, (const uint16_t*)WuT,
              (const uint16_t*)Wd, (const uint16_t*)dY, T, d, F,
              (uint32_t*)w, (uint16_t*)(w + 2 * tf), (uint16_t*)(w + 3 * tf),
              (uint16_t*)(w + 4 * tf), (float*)(w + 5 * tf)};
  const int nbm = (T + 255) / 256;
  hipLaunchKernelGGL(train_gateup_kernel<TrainGateUp>, dim3(nbm * (F / TrainGateUp::BN)), dim3(TrainGateUp::NTH), 0,
                     s, a);
  hipError_t e = launch_dense_down(a.a16, Wd, T, d, F, out_dt, y, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(train_da_kernel<TrainDA>, dim3(nbm * (F / TrainDA::BN)), dim3(TrainDA::NTH), 0, s, a);
  hipLaunchKernelGGL(train_dx_kernel<TrainDX>, dim3(nbm * (d / TrainDX::BN)), dim3(TrainDX::NTH), 0, s, a, dX);
  const dim3 gw((F / TrainWgrad::BM) * (d / TrainWgrad::BN));
  hipLaunchKernelGGL(train_wgrad_kernel<TrainWgrad>, gw, dim3(TrainWgrad::NTH), 0, s, a.dg16, a.x, T, d, F, dWgT);
  hipLaunchKernelGGL(train_wgrad_kernel<TrainWgrad>, gw, dim3(TrainWgrad::NTH), 0, s, a.du16, a.x, T, d, F, dWuT);
  hipLaunchKernelGGL(train_wgrad_kernel<TrainWgrad>, gw, dim3(TrainWgrad::NTH), 0, s, a.a16, a.dY, T, d, F, dWd);
  if (dbg) hipLaunchKernelGGL(train_dbg_kernel, dim3((F + 255) / 256), dim3(256), 0, s, a.dbg_part, nbm, F, dbg);
  return hipGetLastError();
}

}  // namespace twell
