// Hybrid sparse/dense training path: row classification, the dense branch
// (gathered-row MFMA GEMMs) and the neuron-major weight-gradient accumulation
// of the sparse branch.
//
// The intellectnews.ru TwELL article, section "Слитые CUDA-ядра для инференса
// и гибрид для обучения", describes the training format: rows of the
// activation matrix that are well sparse are kept in a compact sparse matrix,
// rows with many active values are routed to a dense branch.  Here a row is
// dense iff its non-zero count exceeds an integer threshold tau.
//
// Dense rows D (gathered, n_D of them, order of increasing token index):
//   forward :  g = x_D.WgT^T + b, u = x_D.WuT^T, A = ReLU(g)*u,  y_D = A.Wd
//   backward:  dA = dY_D.Wd^T, dG = (dA*u + l1)*1[g>0], dU = dA*ReLU(g)
//              (l1: gradient coefficient of an L1 penalty on h, else 0)
//              dX_D = dG.WgT + dU.WuT
//              dWgT = dG^T.x_D, dWuT = dU^T.x_D, dWd = A^T.dY_D, dbg = sum dG
// The fp32 intermediates (A, dG, dU) enter the bf16 matrix cores as a hi + lo
// pair of bf16 values; x, dY and the weights are exact in bf16.  For bf16
// inputs the act kernel's epilogue writes them split, as bf16 planes (per
// dense row: dG hi, dG lo, dU hi, dU lo, A hi, A lo, F values each; the
// forward keeps A hi, A lo), which the later GEMMs read directly.
//
// Sparse rows: the weight gradients are sums over the tokens that activate a
// neuron, i.e. over a column of the TwELL pattern.  A column-major index of
// the sparse rows' stored pairs (per neuron, tokens ascending) is built from
// the 64-bit tile masks with no atomics, and one workgroup per neuron sums
// coefficient * row over its list in that fixed order.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

// ------------------------------------------------------------------ classify

// One wave per row: nnz = sum of the row's per-tile counts; flag = nnz > tau.
__global__ __launch_bounds__(256) void row_classify_kernel(const uint8_t* cnt, int T, int NT, int tau,
                                                           const uint8_t* force, uint8_t* flag) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int s = 0;
  for (int j = lane; j < NT; j += 64) s += cnt[(int64_t)t * NT + j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) flag[t] = (s > tau || (force && force[t])) ? 1 : 0;
}

// Single workgroup: stable compaction of the flagged rows into list[0..n).
__global__ __launch_bounds__(1024) void row_compact_kernel(const uint8_t* flag, int T, int* list, int* n_out,
                                                           int* n_copy) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (T + 1023) / 1024;
  const int r0 = min(T, tid * per), r1 = min(T, r0 + per);
  int c = 0;
  for (int r = r0; r < r1; ++r) c += flag[r];
  part[tid] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int pos = part[tid] - c;
  for (int r = r0; r < r1; ++r)
    if (flag[r]) list[pos++] = r;
  if (tid == 1023) {
    *n_out = part[1023];
    if (n_copy) *n_copy = part[1023];
  }
}

hipError_t launch_classify(const TwellView& h, int tau, uint8_t* flag, int* list, int* n_out, int* n_copy,
                           hipStream_t s, const uint8_t* force) {
  if (h.T > 0)
    hipLaunchKernelGGL(row_classify_kernel, dim3((h.T + 3) / 4), dim3(256), 0, s, h.cnt, h.T, h.NT, tau, force,
                       flag);
  hipLaunchKernelGGL(row_compact_kernel, dim3(1), dim3(1024), 0, s, flag, h.T, list, n_out, n_copy);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dense branch

struct DenseRowsArgs {
  const void* x;
  const void* WgT;
  const void* bg;
  const void* WuT;
  const void* Wd;
  const void* dY;
  int T, d, F;
  const int* rows;    // dense row list
  const int* n_rows;  // device count n_D
  float* buf;         // forward: A [T][F]; backward: [dG | dU | A] [T][3F]
  void* y;            // forward output rows (out_bf16 selects bf16)
  int out_bf16;
  float* dX;
  float* dWgT;
  float* dWuT;
  float* dWd;
  float* dbg_part;    // [ceil(T/dbg_rows)][F]
  float* dbg;
  int dbg_rows;       // rows per dbg partial
  float l1;           // backward: added to dG where g > 0 (activation penalty)
  // rounds: the launch covers list entries [r0, r0 + cap) (rows already points
  // at entry r0; buf and dbg_part hold cap rows), accum: add the weight and
  // bias gradients to those of the earlier rounds
  int r0, cap, accum;
};

// dense rows of this round
__device__ __forceinline__ int round_rows(const DenseRowsArgs& a) {
  return min(max(*a.n_rows - a.r0, 0), a.cap);
}

template <bool BF16IN>
__device__ __forceinline__ float ld_bias(const void* b, int n) {
  if (b == nullptr) return 0.f;
  if constexpr (BF16IN) return bf16_to_f32(((const uint16_t*)b)[n]);
  else return ((const float*)b)[n];
}

// Gathered-row gate/up (and, backward, dY.Wd^T) GEMMs with the elementwise
// epilogue.  Tiles past n_D exit at once (n_D is only known on the device).
template <class Cfg2, class Cfg1, bool BF16IN, bool BWD>
__global__ __launch_bounds__(Cfg2::NTH) void dense_rows_act_kernel(DenseRowsArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg2::LDS_BYTES];
  const int nD = round_rows(a);
  const int nbn = a.F / Cfg2::BN;
  const int bm = blockIdx.x / nbn, bn = blockIdx.x % nbn;
  const int m0 = bm * Cfg2::BM, n0 = bn * Cfg2::BN;
  if (m0 >= nD) return;
  GemmTile<Cfg2> g;
  const Operand A{a.x, a.d, a.rows, nD};
  const Operand B[2] = {{a.WgT, a.d, nullptr, a.F}, {a.WuT, a.d, nullptr, a.F}};
  g.run(A, B, m0, n0, a.d, lds);
  GemmTile<Cfg1> gd;
  if constexpr (BWD) {
    const Operand A2{a.dY, a.d, a.rows, nD};
    const Operand B2{a.Wd, a.d, nullptr, a.F};
    gd.run(A2, &B2, m0, n0, a.d, lds);
  }
  const int64_t ldb = BWD ? 3 * (int64_t)a.F : a.F;
#pragma unroll
  for (int j = 0; j < Cfg2::TN; ++j) {
    const int col = n0 + GemmTile<Cfg2>::col_of(j);
    const float b = ld_bias<BF16IN>(a.bg, col);
#pragma unroll
    for (int i = 0; i < Cfg2::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + GemmTile<Cfg2>::row_of(i, e);
        if (r < nD) {
          const float gv = g.acc[0][i][j][e] + b;
          const float h = gv > 0.f ? gv : 0.f;
          const float u = g.acc[1][i][j][e];
          float* row = a.buf + (int64_t)r * ldb;
          if constexpr (BWD) {
            const float da = gd.acc[0][i][j][e];
            row[col] = gv > 0.f ? da * u + a.l1 : 0.f;
            row[a.F + col] = da * h;
            row[2 * a.F + col] = h * u;
          } else {
            row[col] = h * u;
          }
        }
      }
  }
}

// bf16 inputs: the same GEMMs and epilogue on the direct-to-LDS mainloop
// (single-stage tiles, two workgroups per CU; the gathered x and dY rows come
// through the A operand's row list).
template <class Cfg2, class Cfg1, bool BWD>
__global__ __launch_bounds__(Cfg2::NTH, WavesPerEU<Cfg2>::value) void dense_rows_act_dma_kernel(DenseRowsArgs a) {
  static_assert(Cfg2::SINGLE && Cfg1::SINGLE && Cfg2::STAGE >= Cfg1::STAGE, "one stage buffer for both GEMMs");
  __shared__ __attribute__((aligned(1024))) char st[Cfg2::STAGE];
  const int nD = round_rows(a);
  const int nbn = a.F / Cfg2::BN;
  const int bm = blockIdx.x / nbn, bn = blockIdx.x % nbn;
  const int m0 = bm * Cfg2::BM, n0 = bn * Cfg2::BN;
  if (m0 >= nD) return;
  typedef DmaTile<Cfg2> Tile;
  Tile g;
  const Operand A{a.x, a.d, a.rows, nD};
  const Operand B[2] = {{a.WgT, a.d, nullptr, a.F}, {a.WuT, a.d, nullptr, a.F}};
  g.run(A, B, m0, n0, a.d, st, st);
  DmaTile<Cfg1> gd;
  if constexpr (BWD) {
    const Operand A2{a.dY, a.d, a.rows, nD};
    const Operand B2{a.Wd, a.d, nullptr, a.F};
    gd.run(A2, &B2, m0, n0, a.d, st, st);
  }
  // bf16 planes: backward [dG hi | dG lo | dU hi | dU lo | A hi | A lo],
  // forward [A hi | A lo], F values each
  const int64_t ld16 = (BWD ? 6 : 2) * (int64_t)a.F;
  uint16_t* buf16 = (uint16_t*)a.buf;
  float dsum[Cfg2::TN];                             // backward: this lane's column sum of dG
#pragma unroll
  for (int j = 0; j < Cfg2::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
    const float b = ld_bias<true>(a.bg, col);
    dsum[j] = 0.f;
#pragma unroll
    for (int i = 0; i < Cfg2::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + Tile::row_of(i, e);
        if (r < nD) {
          const float gv = g.acc[0][i][j][e] + b;
          const float h = gv > 0.f ? gv : 0.f;
          const float u = g.acc[1][i][j][e];
          uint16_t* row = buf16 + (int64_t)r * ld16 + col;
          uint32_t hi, lo;
          if constexpr (BWD) {
            const float da = gd.acc[0][i][j][e];
            const float dg = gv > 0.f ? da * u + a.l1 : 0.f;
            dsum[j] += dg;
            split_bf16(dg, hi, lo);
            row[0] = (uint16_t)hi;
            row[a.F] = (uint16_t)lo;
            split_bf16(da * h, hi, lo);
            row[2 * a.F] = (uint16_t)hi;
            row[3 * a.F] = (uint16_t)lo;
            split_bf16(h * u, hi, lo);
            row[4 * a.F] = (uint16_t)hi;
            row[5 * a.F] = (uint16_t)lo;
          } else {
            split_bf16(h * u, hi, lo);
            row[0] = (uint16_t)hi;
            row[a.F] = (uint16_t)lo;
          }
        }
      }
  }
  if constexpr (BWD) {
    if (a.dbg) {
      // partial dbg of the tile's rows, in a fixed order: lanes l and l + 32
      // hold the same column (rows 4 apart), the WM waves of a column range
      // hold different rows (added through the free stage buffer)
      const int lane = threadIdx.x & 63, wm = (threadIdx.x >> 6) / Cfg2::WN;
      float* red = (float*)st;                      // [WM][BN]
#pragma unroll
      for (int j = 0; j < Cfg2::TN; ++j) {
        dsum[j] += __shfl_xor(dsum[j], 32);
        if (lane < 32) red[wm * Cfg2::BN + Tile::col_of(j)] = dsum[j];
      }
      __syncthreads();
      if (wm == 0 && lane < 32) {
#pragma unroll
        for (int j = 0; j < Cfg2::TN; ++j) {
          float sum = 0.f;
#pragma unroll
          for (int q = 0; q < Cfg2::WM; ++q) sum += red[q * Cfg2::BN + Tile::col_of(j)];
          a.dbg_part[(int64_t)(m0 / Cfg2::BM) * a.F + n0 + Tile::col_of(j)] = sum;
        }
      }
    }
  }
}

// bf16 inputs: out[rows[r]] from the bf16 planes (forward: y = A.Wd;
// backward: dX = dG.WgT + dU.WuT), each intermediate read as a hi/lo plane
// pair, so every weight tile serves both MFMAs as with the fp32 split.  The A
// operand starts at the tile's first row, so its 32-bit element offsets stay
// within one tile's rows.
template <class Cfg, bool BWD>
__global__ __launch_bounds__(Cfg::NTH) void dense_rows_out16_kernel(DenseRowsArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int nD = round_rows(a);
  const int nbn = a.d / Cfg::BN;
  const int bm = blockIdx.x / nbn, bn = blockIdx.x % nbn;
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  if (m0 >= nD) return;
  const int64_t ld16 = (BWD ? 6 : 2) * (int64_t)a.F;
  const uint16_t* tile = (const uint16_t*)a.buf + (int64_t)m0 * ld16;
  auto pair = [&](int p) { return Operand{tile + (int64_t)p * a.F, ld16, nullptr, nD - m0, a.F}; };
  GemmTile<Cfg> g;
  if constexpr (BWD) {
    const Operand Bg{a.WgT, a.d, nullptr, a.F}, Bu{a.WuT, a.d, nullptr, a.F};
    g.run(pair(0), &Bg, 0, n0, a.F, lds);
    g.run(pair(2), &Bu, 0, n0, a.F, lds, false);
  } else {
    const Operand Bd{a.Wd, a.d, nullptr, a.F};
    g.run(pair(0), &Bd, 0, n0, a.F, lds);
  }
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + GemmTile<Cfg>::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + GemmTile<Cfg>::row_of(i, e);
        if (r < nD) {
          const int64_t t = a.rows[r];
          const float v = g.acc[0][i][j][e];
          if constexpr (BWD) {
            __builtin_nontemporal_store(v, a.dX + t * a.d + col);   // streamed like the sparse rows' dX
          } else {
            if (a.out_bf16) ((uint16_t*)a.y)[t * a.d + col] = (uint16_t)f32_to_bf16_bits(v);
            else ((float*)a.y)[t * a.d + col] = v;
          }
        }
      }
  }
}

// bf16 inputs: dense-row weight gradients from the bf16 planes on the
// direct-to-LDS mainloop, written (not accumulated):
//   C rows [0, F): dWgT = dG^T.x_D, [F, 2F): dWuT = dU^T.x_D, [2F, 3F): dWd = A^T.dY_D
// A is a plane read as [K][M] (K = the dense rows), B the gathered x or dY
// rows; K runs in chunks of WG_KCH rows (hi and lo pass each) so the 32-bit
// byte offsets stay within one chunk; rows past n_D lie outside the A
// operand's range and read as zeros.
constexpr int WG_KCH = 1024;
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void dense_rows_wgrad16_kernel(DenseRowsArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  const int nD = round_rows(a);
  const int nbn = a.d / Cfg::BN;
  const int tl = xcd_remap(blockIdx.x, gridDim.x);
  const int bm = tl / nbn, bn = tl % nbn;
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  const int part = m0 / a.F;                        // 0: dWgT, 1: dWuT, 2: dWd (tiles never straddle)
  const int mp = m0 - part * a.F;
  const int64_t ld16 = 6 * (int64_t)a.F;
  const uint16_t* b16 = (const uint16_t*)a.buf;
  const void* V = part == 2 ? a.dY : a.x;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  if (nD == 0 && a.accum) return;                   // nothing to add in this round
  if (nD == 0) {
    const Operand A{b16, ld16, nullptr, 0};
    const Operand B{V, a.d, a.rows, a.T};
    g.run(A, &B, mp, n0, 0, st0, st1);              // no K tiles: zeros
  }
  for (int k0 = 0; k0 < nD; k0 += WG_KCH) {
    const int kn = min(WG_KCH, nD - k0);
#pragma unroll
    for (int lo = 0; lo < 2; ++lo) {
      const Operand A{b16 + (int64_t)k0 * ld16 + (int64_t)(2 * part + lo) * a.F, ld16, nullptr, kn};
      const Operand B{V, a.d, a.rows + k0, a.T};
      g.run(A, &B, mp, n0, kn, st0, st1, k0 == 0 && lo == 0);
    }
  }
  float* out = part == 0 ? a.dWgT : part == 1 ? a.dWuT : a.dWd;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float* o = out + (int64_t)(mp + Tile::row_of(i, e)) * a.d + col;
        *o = a.accum ? *o + g.acc[0][i][j][e] : g.acc[0][i][j][e];
      }
  }
}

// out[rows[r]] = sum_k buf[r][k].W[k]  (forward: y = A.Wd;  backward:
// dX = dG.WgT + dU.WuT, two passes into one accumulator).
template <class Cfg, bool BWD>
__global__ __launch_bounds__(Cfg::NTH) void dense_rows_out_kernel(DenseRowsArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int nD = round_rows(a);
  const int nbn = a.d / Cfg::BN;
  const int bm = blockIdx.x / nbn, bn = blockIdx.x % nbn;
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  if (m0 >= nD) return;
  GemmTile<Cfg> g;
  if constexpr (BWD) {
    const Operand A1{a.buf, 3 * (int64_t)a.F, nullptr, nD};
    const Operand B1{a.WgT, a.d, nullptr, a.F};
    g.run(A1, &B1, m0, n0, a.F, lds);
    const Operand A2{a.buf + a.F, 3 * (int64_t)a.F, nullptr, nD};
    const Operand B2{a.WuT, a.d, nullptr, a.F};
    g.run(A2, &B2, m0, n0, a.F, lds, false);
  } else {
    const Operand A1{a.buf, a.F, nullptr, nD};
    const Operand B1{a.Wd, a.d, nullptr, a.F};
    g.run(A1, &B1, m0, n0, a.F, lds);
  }
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + GemmTile<Cfg>::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + GemmTile<Cfg>::row_of(i, e);
        if (r < nD) {
          const int64_t t = a.rows[r];
          const float v = g.acc[0][i][j][e];
          if constexpr (BWD) {
            __builtin_nontemporal_store(v, a.dX + t * a.d + col);   // streamed like the sparse rows' dX
          } else {
            if (a.out_bf16) ((uint16_t*)a.y)[t * a.d + col] = (uint16_t)f32_to_bf16_bits(v);
            else ((float*)a.y)[t * a.d + col] = v;
          }
        }
      }
  }
}

// Dense-row weight gradients, written (not accumulated):
//   rows [0, F)   of C: dWgT = dG^T.x_D
//   rows [F, 2F)  of C: dWuT = dU^T.x_D
//   rows [2F, 3F) of C: dWd  = A^T.dY_D
// C = buf^T.V with K = n_D (device value; the transposed loaders zero-fill
// past it, so n_D == 0 writes zeros).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void dense_rows_wgrad_kernel(DenseRowsArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  const int nD = round_rows(a);
  const int nbn = a.d / Cfg::BN;
  const int bm = blockIdx.x / nbn, bn = blockIdx.x % nbn;
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;
  const int part = m0 / a.F;                      // 0: dWgT, 1: dWuT, 2: dWd (tiles never straddle)
  if (nD == 0 && a.accum) return;                 // nothing to add in this round
  GemmTile<Cfg> g;
  const Operand A{a.buf, 3 * (int64_t)a.F, nullptr, 3 * a.F};
  const Operand B{part == 2 ? a.dY : a.x, a.d, a.rows, a.T};
  g.run(A, &B, m0, n0, nD, lds);
  float* out = part == 0 ? a.dWgT : part == 1 ? a.dWuT : a.dWd;
  const int mrow0 = m0 - part * a.F;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + GemmTile<Cfg>::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = mrow0 + GemmTile<Cfg>::row_of(i, e);
        float* o = out + (int64_t)m * a.d + col;
        *o = a.accum ? *o + g.acc[0][i][j][e] : g.acc[0][i][j][e];
      }
  }
}

// dbg over the dense rows: per 64-row chunk partial column sums of dG, then
// a fixed-order sum of the partials (written, not accumulated).
__global__ __launch_bounds__(256) void dense_rows_dbg_part_kernel(DenseRowsArgs a) {
  const int nD = round_rows(a);
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int c = blockIdx.y;
  if (c * 64 >= nD || n >= a.F) return;
  const int r1 = min(nD, c * 64 + 64);
  float s = 0.f;
  for (int r = c * 64; r < r1; ++r) s += a.buf[(int64_t)r * 3 * a.F + n];
  a.dbg_part[(int64_t)c * a.F + n] = s;
}

__global__ __launch_bounds__(256) void dense_rows_dbg_sum_kernel(DenseRowsArgs a) {
  const int nD = round_rows(a);
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.F) return;
  if (nD == 0 && a.accum) return;
  const int nc = (nD + a.dbg_rows - 1) / a.dbg_rows;
  float s = 0.f;
  for (int c = 0; c < nc; ++c) s += a.dbg_part[(int64_t)c * a.F + n];
  a.dbg[n] = a.accum ? a.dbg[n] + s : s;
}

// Configurations.  act: 128x128 block, 4 waves, gate+up (2 B operands) then dA.
template <bool BF16IN> struct HybCfg;
template <> struct HybCfg<true> {
  using ActD2 = DmaCfg1<128, 128, 2, 4, 2>;
  using ActD1 = DmaCfg1<128, 128, 2, 4, 1>;
  using ActD2S = DmaCfg1<128, 64, 2, 2, 2>;
  using ActD1S = DmaCfg1<128, 64, 2, 2, 1>;
  using Act2 = GemmCfg<128, 128, 2, 2, OP_BF16_K, OP_BF16_K, 2>;
  using Act1 = GemmCfg<128, 128, 2, 2, OP_BF16_K, OP_BF16_K, 1>;
  using Act2S = GemmCfg<128, 64, 2, 2, OP_BF16_K, OP_BF16_K, 2>;
  using Act1S = GemmCfg<128, 64, 2, 2, OP_BF16_K, OP_BF16_K, 1>;
  using Out16 = GemmCfg<64, 64, 2, 2, OP_BF16P_K, OP_BF16_T>;
  using Wgrad16L = DmaCfg<256, 256, 2, 4, 1, false, true, true>;   // F % 256 == 0, d % 256 == 0
  using Wgrad16S = DmaCfg<64, 64, 2, 2, 1, false, true, true>;
};
template <> struct HybCfg<false> {
  using Act2 = GemmCfg<128, 128, 2, 2, OP_F32_K, OP_F32_K, 2>;
  using Act1 = GemmCfg<128, 128, 2, 2, OP_F32_K, OP_F32_K, 1>;
  using Act2S = GemmCfg<128, 64, 2, 2, OP_F32_K, OP_F32_K, 2>;
  using Act1S = GemmCfg<128, 64, 2, 2, OP_F32_K, OP_F32_K, 1>;
  using Out = GemmCfg<64, 64, 2, 2, OP_F32_K, OP_F32_T>;
  using Wgrad = GemmCfg<64, 128, 2, 2, OP_F32_T, OP_F32_T>;
  using WgradS = GemmCfg<64, 64, 2, 2, OP_F32_T, OP_F32_T>;
};

// The act kernel tiles F by 128 columns and the weight-gradient kernel tiles
// d by 128 when the shape allows; otherwise 64.
template <class Act2, class Act1, bool BF16IN, bool BWD>
static void launch_act(const DenseRowsArgs& a, hipStream_t s) {
  const int g = ((a.T + Act2::BM - 1) / Act2::BM) * (a.F / Act2::BN);
  if (g > 0) hipLaunchKernelGGL((dense_rows_act_kernel<Act2, Act1, BF16IN, BWD>), dim3(g), dim3(Act2::NTH), 0, s, a);
}

template <class Act2, class Act1, bool BWD>
static void launch_act_dma(const DenseRowsArgs& a, hipStream_t s) {
  const int g = ((a.T + Act2::BM - 1) / Act2::BM) * (a.F / Act2::BN);
  if (g > 0)
    hipLaunchKernelGGL((dense_rows_act_dma_kernel<Act2, Act1, BWD>), dim3(g), dim3(Act2::NTH), 0, s, a);
}

template <class Cfg, bool BWD>
static void launch_out(const DenseRowsArgs& a, hipStream_t s) {
  const int g = ((a.T + Cfg::BM - 1) / Cfg::BM) * (a.d / Cfg::BN);
  if (g > 0) hipLaunchKernelGGL((dense_rows_out_kernel<Cfg, BWD>), dim3(g), dim3(Cfg::NTH), 0, s, a);
}

template <class Cfg>
static void launch_wgrad(const DenseRowsArgs& a, hipStream_t s) {
  const int g = (3 * a.F / Cfg::BM) * (a.d / Cfg::BN);
  if (g > 0) hipLaunchKernelGGL((dense_rows_wgrad_kernel<Cfg>), dim3(g), dim3(Cfg::NTH), 0, s, a);
}

// The direct-to-LDS act kernels are instantiated explicitly: referenced only
// from the launchers below, the host pass emitted no launch stub for the
// backward variants.
template __global__ void dense_rows_act_dma_kernel<HybCfg<true>::ActD2, HybCfg<true>::ActD1, false>(DenseRowsArgs);
template __global__ void dense_rows_act_dma_kernel<HybCfg<true>::ActD2, HybCfg<true>::ActD1, true>(DenseRowsArgs);
template __global__ void dense_rows_act_dma_kernel<HybCfg<true>::ActD2S, HybCfg<true>::ActD1S, false>(DenseRowsArgs);
template __global__ void dense_rows_act_dma_kernel<HybCfg<true>::ActD2S, HybCfg<true>::ActD1S, true>(DenseRowsArgs);

// act GEMMs: direct-to-LDS tiles for bf16 inputs, register-staged for fp32
template <bool BF16IN, bool BWD>
struct ActLaunch {
  static void go(const DenseRowsArgs& a, hipStream_t s) {
    using C = HybCfg<false>;
    if (a.F % 128 == 0) launch_act<typename C::Act2, typename C::Act1, false, BWD>(a, s);
    else launch_act<typename C::Act2S, typename C::Act1S, false, BWD>(a, s);
  }
};
template <bool BWD>
struct ActLaunch<true, BWD> {
  static void go(const DenseRowsArgs& a, hipStream_t s) {
    using C = HybCfg<true>;
    if (a.F % 128 == 0) launch_act_dma<typename C::ActD2, typename C::ActD1, BWD>(a, s);
    else launch_act_dma<typename C::ActD2S, typename C::ActD1S, BWD>(a, s);
  }
};

template <class Cfg, bool BWD>
static void launch_out16(const DenseRowsArgs& a, hipStream_t s) {
  const int g = ((a.T + Cfg::BM - 1) / Cfg::BM) * (a.d / Cfg::BN);
  if (g > 0) hipLaunchKernelGGL((dense_rows_out16_kernel<Cfg, BWD>), dim3(g), dim3(Cfg::NTH), 0, s, a);
}

template <class Cfg>
static void launch_wgrad16(const DenseRowsArgs& a, hipStream_t s) {
  const int g = (3 * a.F / Cfg::BM) * (a.d / Cfg::BN);
  if (g > 0) hipLaunchKernelGGL((dense_rows_wgrad16_kernel<Cfg>), dim3(g), dim3(Cfg::NTH), 0, s, a);
}

// bf16 inputs: act kernel writing the bf16 planes (and, backward, the dbg
// partials of its 128-row tiles), then the plane GEMMs
template <bool BWD>
static hipError_t dense_rows_bf16(DenseRowsArgs a, hipStream_t s) {
  using C = HybCfg<true>;
  static_assert(C::ActD2::BM == C::ActD2S::BM, "one dbg partial per act row tile");
  a.dbg_rows = C::ActD2::BM;
  ActLaunch<true, BWD>::go(a, s);
  launch_out16<typename C::Out16, BWD>(a, s);
  if constexpr (BWD) {
    if (a.F % 256 == 0 && a.d % 256 == 0) launch_wgrad16<typename C::Wgrad16L>(a, s);
    else launch_wgrad16<typename C::Wgrad16S>(a, s);
    if (a.dbg) hipLaunchKernelGGL(dense_rows_dbg_sum_kernel, dim3((a.F + 255) / 256), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// fp32 inputs: the register-staged GEMMs on the fp32 intermediates
template <bool BWD>
static hipError_t dense_rows_f32(DenseRowsArgs a, hipStream_t s) {
  using C = HybCfg<false>;
  a.dbg_rows = 64;
  ActLaunch<false, BWD>::go(a, s);
  launch_out<typename C::Out, BWD>(a, s);
  if constexpr (BWD) {
    if (a.d % 128 == 0) launch_wgrad<typename C::Wgrad>(a, s);
    else launch_wgrad<typename C::WgradS>(a, s);
    if (a.dbg) {
      if (a.T > 0)
        hipLaunchKernelGGL(dense_rows_dbg_part_kernel, dim3((a.F + 255) / 256, (a.T + 63) / 64), dim3(256), 0, s, a);
      hipLaunchKernelGGL(dense_rows_dbg_sum_kernel, dim3((a.F + 255) / 256), dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

template <bool BF16IN, bool BWD>
static hipError_t dense_rows_t(const DenseRowsArgs& a, hipStream_t s) {
  if constexpr (BF16IN) return dense_rows_bf16<BWD>(a, s);
  else return dense_rows_f32<BWD>(a, s);
}

// The dense rows go in rounds of dense_row_cap(T) list entries, each through
// the whole branch with buffers of that many rows (the count is known only on
// the device: a round past it does nothing).
hipError_t launch_dense_rows_fwd(int in_dt, const void* x, const void* WgT, const void* bg, const void* WuT,
                                 const void* Wd, int T, int d, int F, const int* rows, const int* n_rows,
                                 float* actbuf, int out_dt, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cap = dense_row_cap(T);
  hipError_t e = hipSuccess;
  for (int r0 = 0; r0 < T && e == hipSuccess; r0 += cap) {
    DenseRowsArgs a{};
    a.x = x; a.WgT = WgT; a.bg = bg; a.WuT = WuT; a.Wd = Wd; a.T = cap; a.d = d; a.F = F;
    a.rows = rows + r0; a.n_rows = n_rows; a.buf = actbuf; a.y = y; a.out_bf16 = out_dt == DT_BF16;
    a.r0 = r0; a.cap = cap; a.accum = r0 > 0;
    e = in_dt == DT_BF16 ? dense_rows_t<true, false>(a, s) : dense_rows_t<false, false>(a, s);
  }
  return e;
}

hipError_t launch_dense_rows_bwd(int in_dt, const void* x, const void* WgT, const void* bg, const void* WuT,
                                 const void* Wd, const void* dY, int T, int d, int F, const int* rows,
                                 const int* n_rows, float* buf3, float* dbg_part, float* dX, float* dWgT,
                                 float* dWuT, float* dWd, float* dbg, hipStream_t s, float l1) {
  const int cap = dense_row_cap(T);
  hipError_t e = hipSuccess;
  // T == 0: one round with no rows writes zero weight gradients
  for (int r0 = 0; (r0 < T || r0 == 0) && e == hipSuccess; r0 += cap) {
    DenseRowsArgs a{};
    a.l1 = l1;
    a.x = x; a.WgT = WgT; a.bg = bg; a.WuT = WuT; a.Wd = Wd; a.dY = dY; a.T = cap; a.d = d; a.F = F;
    a.rows = rows + r0; a.n_rows = n_rows; a.buf = buf3; a.dX = dX; a.dWgT = dWgT; a.dWuT = dWuT; a.dWd = dWd;
    a.dbg_part = dbg_part; a.dbg = dbg;
    a.r0 = r0; a.cap = cap; a.accum = r0 > 0;
    e = in_dt == DT_BF16 ? dense_rows_t<true, true>(a, s) : dense_rows_t<false, true>(a, s);
    if (cap == 0) break;
  }
  return e;
}

// ------------------------------------------------------------------ sparse-branch weight gradients

constexpr int CSC_CHUNK = 256;   // tokens per count/fill chunk

// The count and fill kernels stage the masks of one chunk of CSC_CHUNK rows
// and CSC_JG column tiles in LDS (skipped rows and tiles past NT as zeros):
// consecutive threads read consecutive tiles of a row, every load of a
// thread in flight before the first LDS store.  Each wave then takes whole
// tiles, lane = neuron bit, reading each row's word as an LDS broadcast.
constexpr int CSC_JG = 4;        // column tiles per count/fill workgroup (4 measured faster than 8 and 16)

__device__ __forceinline__ void csc_stage(const uint64_t* mask, const uint8_t* skip, int T, int NT, int t0, int j0,
                                          uint64_t* sm) {
  constexpr int PER = CSC_CHUNK * CSC_JG / 256;
  uint64_t m[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = threadIdx.x + q * 256;
    const int t = t0 + i / CSC_JG, j = j0 + i % CSC_JG;
    m[q] = (t < T && j < NT && !(skip && skip[t])) ? mask[(int64_t)t * NT + j] : 0ull;
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) sm[threadIdx.x + q * 256] = m[q];
  __syncthreads();
}

// part[c][n] = number of sparse rows t in chunk c with (t, n) stored.
__global__ __launch_bounds__(256) void csc_count_kernel(const uint64_t* mask, const uint8_t* skip, int T,
                                                        int NT, int F, int* part) {
  __shared__ uint64_t sm[CSC_CHUNK * CSC_JG];
  const int c = blockIdx.y, j0 = blockIdx.x * CSC_JG;
  const int t0 = c * CSC_CHUNK, nr = min(T, t0 + CSC_CHUNK) - t0;
  csc_stage(mask, skip, T, NT, t0, j0, sm);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int jj = w; jj < CSC_JG && j0 + jj < NT; jj += 4) {
    int k = 0;
    for (int r0 = 0; r0 < nr; r0 += 8) {
      uint64_t m[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) m[q] = r0 + q < nr ? sm[(r0 + q) * CSC_JG + jj] : 0ull;
#pragma unroll
      for (int q = 0; q < 8; ++q) k += (int)((m[q] >> lane) & 1ull);
    }
    part[(int64_t)c * F + (j0 + jj) * 64 + lane] = k;
  }
}

// Per neuron n (one thread each): part[c][n] becomes the exclusive prefix of
// the chunk counts over c, and start[n] the neuron's total.  Eight chunks'
// loads are in flight at a time.
__global__ __launch_bounds__(256) void csc_chunk_scan_kernel(int* part, int nchunk, int F, int* start) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= F) return;
  int run = 0;
  for (int c0 = 0; c0 < nchunk; c0 += 8) {
    int v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = c0 + q < nchunk ? part[(int64_t)(c0 + q) * F + n] : 0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (c0 + q < nchunk) {
        part[(int64_t)(c0 + q) * F + n] = run;
        run += v[q];
      }
  }
  start[n] = run;
}

// Single workgroup: start[n] = sum of the totals of neurons < n, start[F] =
// the grand total.
__global__ __launch_bounds__(1024) void csc_total_scan_kernel(int F, int* start) {
  __shared__ int wsum[1024];
  const int tid = threadIdx.x;
  const int per = (F + 1023) / 1024;
  const int n0 = min(F, tid * per), n1 = min(F, n0 + per);
  int mine = 0;
  for (int n = n0; n < n1; ++n) mine += start[n];
  wsum[tid] = mine;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? wsum[tid - o] : 0;
    __syncthreads();
    wsum[tid] += v;
    __syncthreads();
  }
  int base = wsum[tid] - mine;
  for (int n = n0; n < n1; ++n) {
    const int tot = start[n];
    start[n] = base;
    base += tot;
  }
  if (tid == 1023) start[F] = wsum[1023];
}

// entries[pos] = flat TwELL slot offset of each stored pair of a sparse row,
// grouped by neuron, tokens ascending within a neuron; the neuron's block
// starts at start[n], chunk c's part at part[c][n] within it.
__global__ __launch_bounds__(256) void csc_fill_kernel(const uint64_t* mask, const uint8_t* skip, int T, int NT,
                                                       int F, const int* part, const int* start, uint32_t* entries,
                                                       int cap) {
  __shared__ uint64_t sm[CSC_CHUNK * CSC_JG];
  const int c = blockIdx.y, j0 = blockIdx.x * CSC_JG;
  const int t0 = c * CSC_CHUNK, nr = min(T, t0 + CSC_CHUNK) - t0;
  csc_stage(mask, skip, T, NT, t0, j0, sm);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t lower = below(lane);
  for (int jj = w; jj < CSC_JG && j0 + jj < NT; jj += 4) {
    const int j = j0 + jj;
    int pos = start[j * 64 + lane] + part[(int64_t)c * F + j * 64 + lane];
    for (int r0 = 0; r0 < nr; r0 += 8) {           // eight rows' words read before the first use
      uint64_t m[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) m[q] = r0 + q < nr ? sm[(r0 + q) * CSC_JG + jj] : 0ull;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if ((m[q] >> lane) & 1ull) {
          const int t = t0 + r0 + q;
          const uint32_t slot = (uint32_t)popc64(m[q] & lower);
          entries[pos++] = ((uint32_t)((t >> 4) * NT + j) * (uint32_t)cap + slot) * 16u + (uint32_t)(t & 15);
        }
      }
    }
  }
}

struct WgradArgs {
  const void* x;
  const void* dY;
  int T, d, F, NT;
  int cap;                 // slots per TwELL tile of the value arrays
  const int* start;
  const uint32_t* entries;
  const float* aval;
  const float* dgval;
  const float* duval;
  float* dWgT;
  float* dWuT;
  float* dWd;
  float* dbg;
};

// One workgroup per neuron n: over its entries (t ascending)
//   dWd[n] += a * dY_t,  dWgT[n] += dg * x_t,  dWuT[n] += du * x_t,  dbg[n] += dg
// Each thread owns one 16-byte column chunk of a 256-chunk column slice.
template <bool BF16IN>
__global__ __launch_bounds__(256) void wgrad_sparse_kernel(WgradArgs a) {
  constexpr int EPC = BF16IN ? 8 : 4;           // elements per 16-byte chunk
  const int n = blockIdx.x;
  const int e0 = a.start[n], e1 = a.start[n + 1];
  const int nchunk = a.d / EPC;
  float dsum = 0.f;
  for (int cb0 = 0; cb0 < nchunk; cb0 += 256) {
    const int cb = cb0 + threadIdx.x;
    const bool on = cb < nchunk;
    float accD[EPC], accG[EPC], accU[EPC];
#pragma unroll
    for (int q = 0; q < EPC; ++q) accD[q] = accG[q] = accU[q] = 0.f;
    for (int e = e0; e < e1; ++e) {
      const uint32_t off = a.entries[e];
      const int t = (int)(off / (uint32_t)(a.NT * a.cap * 16)) * 16 + (int)(off & 15u);
      const float av = a.aval[off], dg = a.dgval[off], du = a.duval[off];
      if (cb0 == 0) dsum += dg;
      if (on) {
        const uint4 xv = *(const uint4*)((const char*)a.x + ((int64_t)t * a.d + (int64_t)cb * EPC) * (BF16IN ? 2 : 4));
        const uint4 yv = *(const uint4*)((const char*)a.dY + ((int64_t)t * a.d + (int64_t)cb * EPC) * (BF16IN ? 2 : 4));
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          float xq, yq;
          if constexpr (BF16IN) {
            xq = (q & 1) ? bf16_hi(xw[q >> 1]) : bf16_lo(xw[q >> 1]);
            yq = (q & 1) ? bf16_hi(yw[q >> 1]) : bf16_lo(yw[q >> 1]);
          } else {
            xq = __uint_as_float(xw[q]);
            yq = __uint_as_float(yw[q]);
          }
          accD[q] = fmaf(av, yq, accD[q]);
          accG[q] = fmaf(dg, xq, accG[q]);
          accU[q] = fmaf(du, xq, accU[q]);
        }
      }
    }
    if (on) {
      const int64_t o = (int64_t)n * a.d + (int64_t)cb * EPC;
#pragma unroll
      for (int q = 0; q < EPC; ++q) {
        a.dWd[o + q] += accD[q];
        a.dWgT[o + q] += accG[q];
        a.dWuT[o + q] += accU[q];
      }
    }
  }
  if (a.dbg && threadIdx.x == 0) a.dbg[n] += dsum;
}

hipError_t launch_sparse_wgrad(int in_dt, const void* x, const void* dY, int T, int d, int F,
                               const TwellView& h, const uint8_t* skip, int* part, int* start,
                               uint32_t* entries, const float* aval, const float* dgval, const float* duval,
                               float* dWgT, float* dWuT, float* dWd, float* dbg, hipStream_t s) {
  const int NT = F / 64;
  const int nchunk = (T + CSC_CHUNK - 1) / CSC_CHUNK;
  if (nchunk > 0) {
    hipLaunchKernelGGL(csc_count_kernel, dim3((NT + CSC_JG - 1) / CSC_JG, nchunk), dim3(256), 0, s, h.mask, skip, T,
                       NT, F, part);
  }
  hipLaunchKernelGGL(csc_chunk_scan_kernel, dim3((F + 255) / 256), dim3(256), 0, s, part, nchunk, F, start);
  hipLaunchKernelGGL(csc_total_scan_kernel, dim3(1), dim3(1024), 0, s, F, start);
  if (nchunk > 0) {
    hipLaunchKernelGGL(csc_fill_kernel, dim3((NT + CSC_JG - 1) / CSC_JG, nchunk), dim3(256), 0, s, h.mask, skip, T,
                       NT, F, part, start, entries, h.cap);
  }
  WgradArgs a{x, dY, T, d, F, NT, h.cap, start, entries, aval, dgval, duval, dWgT, dWuT, dWd, dbg};
  if (in_dt == DT_BF16) hipLaunchKernelGGL(wgrad_sparse_kernel<true>, dim3(F), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(wgrad_sparse_kernel<false>, dim3(F), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace twell
