// Dense ReLU-gated FFN on the same MFMA mainloop: the speedup denominator.
//
//   kernel 1 (dual GEMM): g = x.WgT^T, u = x.WuT^T on one A tile, epilogue
//                         act = bf16(ReLU(g + b) * u)       -> act [T][F]
//   kernel 2 (GEMM):      y = act . Wd  (Wd is [F][d]: its rows are K, so
//                         it is staged through LDS transposed)
// The act round trip through HBM in bf16 is what a standard bf16 FFN does.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

struct DenseArgs {
  const void* x;
  const void* WgT;
  const void* bg;
  const void* WuT;
  const void* Wd;
  int T, d, F;
  uint16_t* act;
  void* y;
  int out_bf16;
};

__device__ __forceinline__ void tile_order(int id, int nbm, int nbn, int& bm, int& bn) {
  constexpr int GM = 8;
  const int per_group = GM * nbn;
  const int group = id / per_group;
  const int first = group * GM;
  const int gsize = min(nbm - first, GM);
  const int r = id - group * per_group;
  bm = first + r % gsize;
  bn = r / gsize;
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void dense_gateup_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  const int nbm = (a.T + Cfg::BM - 1) / Cfg::BM, nbn = a.F / Cfg::BN;
  int bm, bn;
  tile_order(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B[2] = {{a.WgT, a.d, nullptr, a.F}, {a.WuT, a.d, nullptr, a.F}};
  g.run(A, B, m0, n0, a.d, st0, st1);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
    const float b = a.bg ? bf16_to_f32(((const uint16_t*)a.bg)[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + Tile::row_of(i, e);
        if (row < a.T) {
          const float gv = g.acc[0][i][j][e] + b;
          const float h = gv > 0.f ? gv : 0.f;
          a.act[(int64_t)row * a.F + col] = (uint16_t)f32_to_bf16_bits(h * g.acc[1][i][j][e]);
        }
      }
  }
}

// Non-gated layer: act = bf16(ReLU(x.W1T^T + b1)) (W1T passed as WgT).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void dense_relu_act_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  const int nbm = (a.T + Cfg::BM - 1) / Cfg::BM, nbn = a.F / Cfg::BN;
  int bm, bn;
  tile_order(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B{a.WgT, a.d, nullptr, a.F};
  g.run(A, &B, m0, n0, a.d, st0, st1);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
    const float b = a.bg ? bf16_to_f32(((const uint16_t*)a.bg)[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + Tile::row_of(i, e);
        if (row < a.T) {
          const float gv = g.acc[0][i][j][e] + b;
          a.act[(int64_t)row * a.F + col] = (uint16_t)f32_to_bf16_bits(gv > 0.f ? gv : 0.f);
        }
      }
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void dense_down_kernel(DenseArgs a) {
  const int nbm = (a.T + Cfg::BM - 1) / Cfg::BM, nbn = a.d / Cfg::BN;
  int bm, bn;
  tile_order(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  typedef typename TileFor<Cfg>::type Tile;
  Tile g;
  const Operand A{a.act, a.F, nullptr, a.T};
  const Operand B{a.Wd, a.d, nullptr, a.d};
  if constexpr (TileFor<Cfg>::dma) {
    __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
    __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
    g.run(A, &B, m0, n0, a.F, st0, st1);
  } else {
    __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
    g.run(A, &B, m0, n0, a.F, lds);
  }
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + Tile::row_of(i, e);
        if (row < a.T) {
          const float v = g.acc[0][i][j][e];
          // y streams past the caches, as the TwELL path's does
          if (a.out_bf16) __builtin_nontemporal_store((uint16_t)f32_to_bf16_bits(v), (uint16_t*)a.y + (int64_t)row * a.d + col);
          else __builtin_nontemporal_store(v, (float*)a.y + (int64_t)row * a.d + col);
        }
      }
  }
}

using DenseGateUp = DmaCfg<256, 128, 4, 2, 2>;
using DenseReluAct = DmaCfg<256, 128, 4, 2>;
using DenseDownBig = DmaCfg<256, 256, 2, 4, 1, false, true>;
using DenseDownSmall = GemmCfg<128, 64, 2, 1, OP_BF16_K, OP_BF16_T>;

template <class Cfg, class K>
static hipError_t launch_grid(K kernel, int M, int N, const DenseArgs& a, hipStream_t s) {
  const int grid = ((M + Cfg::BM - 1) / Cfg::BM) * (N / Cfg::BN);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(Cfg::NTH), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_down(const void* act, const void* Wd, int T, int d, int F, int out_dt, void* y,
                             hipStream_t s) {
  DenseArgs a{nullptr, nullptr, nullptr, nullptr, Wd, T, d, F, (uint16_t*)act, y, out_dt == DT_BF16};
  if (d % 256 == 0) return launch_grid<DenseDownBig>(dense_down_kernel<DenseDownBig>, T, d, a, s);
  return launch_grid<DenseDownSmall>(dense_down_kernel<DenseDownSmall>, T, d, a, s);
}

hipError_t launch_dense_relu_fwd(const void* x, const void* W1T, const void* b1, const void* W2, int T, int d, int F,
                                 void* act, int out_dt, void* y, hipStream_t s) {
  DenseArgs a{x, W1T, b1, nullptr, W2, T, d, F, (uint16_t*)act, y, out_dt == DT_BF16};
  hipError_t e = launch_grid<DenseReluAct>(dense_relu_act_kernel<DenseReluAct>, T, F, a, s);
  if (e != hipSuccess) return e;
  return launch_dense_down(act, W2, T, d, F, out_dt, y, s);
}

hipError_t launch_dense_fwd(const void* x, const void* WgT, const void* bg, const void* WuT,
                            const void* Wd, int T, int d, int F, void* act, int out_dt, void* y,
                            hipStream_t s) {
  DenseArgs a{x, WgT, bg, WuT, Wd, T, d, F, (uint16_t*)act, y, out_dt == DT_BF16};
  hipError_t e = launch_grid<DenseGateUp>(dense_gateup_kernel<DenseGateUp>, T, F, a, s);
  if (e != hipSuccess) return e;
  return launch_dense_down(act, Wd, T, d, F, out_dt, y, s);
}

}  // namespace twell
