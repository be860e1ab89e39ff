// Forward sparse phases as GEMMs over each row block's union of active
// neurons.
//
// After the gate GEMM has packed h = ReLU(x.Wg + b) into TwELL
// (intellectnews.ru TwELL article, section "Формат TwELL вместо классической
// sparse-упаковки"), the up- and down-projections only need the neurons that
// fire (section "Слитые CUDA-ядра для инференса и гибрид для обучения").  For
// a block of 256 tokens the set of neurons that fire in ANY of them (the
// union, in ascending neuron order) is taken as the N dimension of the
// up-projection and the K dimension of the down-projection:
//
//   union lists: ulist[b][p] = p-th neuron active in block b, ucount[b] = n_b
//   up:   U[t][p] = x_t . WuT[ulist[p]]              (bf16 MFMA, fp32 accum)
//         a[t][p] = h[t, ulist[p]] * U[t][p] where (t, ulist[p]) is stored in
//         the TwELL of h, else 0; written as fp16 into adense[t][p]
//   down: y_t = sum_p a[t][p] * Wd[ulist[p]]          (fp16 MFMA, fp32 accum)
//
// Neurons that no token of the block activates are skipped whole; the
// products with the zero entries inside the union are computed and are exact
// zeros.  a is fp16 for the down GEMM (relative rounding 2^-11, within the
// 1e-3 output budget); if any |a| exceeds the fp16 range a device flag makes
// the down GEMM stand down and the TwELL-pattern kernels recompute the layer.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

namespace {

#ifndef TWELL_UNION_ROWS
#define TWELL_UNION_ROWS 256
#endif
constexpr int UB = TWELL_UNION_ROWS;   // tokens per row block
constexpr int RT = UB / 16;            // TwELL row tiles per row block

struct UnionArgs {
  const void* x;
  const void* WuT;
  const void* Wd;
  int T, d, F, NT;
  const uint64_t* mask;   // [T][NT]
  const uint8_t* skip;    // [T] or null
  const float* hval;      // TwELL values of h
  const uint8_t* hwidth;  // TwELL widths of h
  int* ulist;             // [NBLK][F]
  int* ucount;            // [NBLK]
  _Float16* adense;       // [T][F]
  int* flag;              // fp16 overflow flag
  void* y;
  int out_bf16;
};

__device__ __forceinline__ bool live(const UnionArgs& a, int t) {
  return t < a.T && !(a.skip && a.skip[t]);
}

}  // namespace

// Unions, first level: grid (64-row slabs, 64-tile chunks).  Thread (g, jj)
// ORs the masks of 16 rows for tile jj; the four row groups are combined
// through LDS into the slab's union Us[slab][j].
__global__ __launch_bounds__(256) void union_or_kernel(UnionArgs a, uint64_t* Us) {
  __shared__ uint64_t part[4][64];
  const int slab = blockIdx.x, tid = threadIdx.x;
  const int jj = tid & 63, g = tid >> 6;
  const int j = blockIdx.y * 64 + jj;
  const int t0 = slab * 64 + g * 16, t1 = min(a.T, t0 + 16);
  uint64_t u = 0;
  if (j < a.NT) {
#pragma unroll
    for (int t = t0; t < t0 + 16; ++t)
      if (t < t1 && !(a.skip && a.skip[t])) u |= a.mask[(int64_t)t * a.NT + j];
  }
  part[g][jj] = u;
  __syncthreads();
  if (g == 0 && j < a.NT) Us[(int64_t)slab * a.NT + j] = part[0][jj] | part[1][jj] | part[2][jj] | part[3][jj];
}

// Lists: one workgroup per row block; ascending positions via a scan of the
// per-tile popcounts.
__global__ __launch_bounds__(256) void union_list_kernel(UnionArgs a, const uint64_t* U) {
  __shared__ int scan[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b == 0 && tid == 0) *a.flag = 0;
  int base = 0;
  int* ul = a.ulist + (int64_t)b * a.F;
  for (int j0 = 0; j0 < a.NT; j0 += 256) {
    const int j = j0 + tid;
    uint64_t u = 0;
    if (j < a.NT) {
      const int s0 = b * (UB / 64), s1 = min((a.T + 63) / 64, s0 + UB / 64);
      for (int sl = s0; sl < s1; ++sl) u |= U[(int64_t)sl * a.NT + j];
    }
    const int c = popc64(u);
    scan[tid] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int p = base + scan[tid] - c;
    const int total = scan[255];
    __syncthreads();
    for (uint64_t m = u; m; m &= m - 1) ul[p++] = j * 64 + __ffsll((long long)m) - 1;
    base += total;
  }
  if (tid == 0) a.ucount[b] = base;
}

// Up-projection over the union.  Workgroups of one row block are consecutive
// so they share the block's x rows in L2.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void up_union_kernel(UnionArgs a) {
  static_assert(Cfg::BM == UB, "one row block per M tile");
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  const int npt = (a.F + Cfg::BN - 1) / Cfg::BN;
  const int nblk = (a.T + UB - 1) / UB;
  int b, pt;
  {
    // XCD-aware order: workgroup ids go round-robin over the 8 XCDs; XCD x
    // takes the row blocks b = x (mod 8) and sweeps them position tile by
    // position tile, so the WuT rows of neighbouring blocks' unions (largely
    // the same neurons) are reused from that XCD's L2.
    const int id = blockIdx.x;
    const int x = id & 7, k = id >> 3;
    const int nbx = (nblk - x + 7) / 8;                // row blocks on this XCD
    if (nbx == 0) return;
    pt = k / nbx;
    b = x + 8 * (k - pt * nbx);
    if (pt >= npt) return;
  }
  const int nb = a.ucount[b];
  const int p0 = pt * Cfg::BN;
  if (p0 >= nb) return;
  const int m0 = b * UB;
  const int* ul = a.ulist + (int64_t)b * a.F;

  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B{a.WuT, a.d, ul, nb};
  g.run(A, &B, m0, p0, a.d, st0, st1);

  // epilogue: a = h * u on stored pairs, else 0, stored as fp16 into
  // adense[t][p] (32 consecutive positions per half-wave store).  The masks of
  // the tile's 256 rows and the TwELL value blocks of h over the column tiles
  // its positions span are first staged in LDS (the mainloop's LDS is free
  // once it returns), so the per-element lookups stay on chip; tiles beyond
  // the staging budget fall back to global reads.  Positions in
  // [n_b, roundup64(n_b)) are written as zeros (the down GEMM reads whole
  // 64-position K tiles).  The masks take the first stage buffer, the h
  // blocks and their offsets the second.
  constexpr int SMAX = 32;                     // column tiles whose masks are staged
  static_assert(UB * SMAX * 8 <= Cfg::STAGE, "mask staging");
  constexpr int HBUDGET = (Cfg::STAGE - RT * SMAX * 4 - 64) / 4;     // floats of h
  uint64_t* sm = (uint64_t*)st0;                                    // [UB][S]
  int* hoff = (int*)st1;                                            // [RT row tiles][S]
  float* hb = (float*)(st1 + RT * SMAX * 4 + 64);                   // h blocks
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int pl = min(p0 + Cfg::BN, nb) - 1;
  const int tjf = ul[p0] >> 6, tjl = ul[pl] >> 6;
  const int S = min(tjl - tjf + 1, SMAX);
  // mask staging: four independent loads in flight per thread
  for (int q0 = tid; q0 < UB * S; q0 += 4 * Cfg::NTH) {
    uint64_t mv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * Cfg::NTH;
      const int r = q / S, sj = q - r * S;
      const int t = m0 + r;
      mv[u] = (q < UB * S && live(a, t)) ? a.mask[(int64_t)t * a.NT + tjf + sj] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q0 + u * Cfg::NTH < UB * S) sm[q0 + u * Cfg::NTH] = mv[u];
  }
  __shared__ int hmeta[1];                          // staged (row tile, column tile) pairs
  if (tid < 64) {
    // h block starts: prefix over (row tile, column tile) of width*16 floats;
    // the pairs that fit the budget form a prefix of that order
    int run = 0, nv = 0;
    for (int q0 = 0; q0 < RT * S; q0 += 64) {
      const int q = q0 + lane;
      int wdt = 0;
      if (q < RT * S) {
        const int i = q / S, sj = q - i * S;
        const int rt = (m0 >> 4) + i;
        wdt = rt * 16 < a.T ? a.hwidth[(int64_t)rt * a.NT + tjf + sj] : 0;
      }
      int incl = wdt * 16;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      const int start = run + incl - wdt * 16;
      const bool fits = q < RT * S && start + wdt * 16 <= HBUDGET;
      if (q < RT * S) hoff[q] = fits ? start : -1;
      nv += popc64(__builtin_amdgcn_ballot_w64(fits));
      run += __shfl(incl, 63);
    }
    if (lane == 0) hmeta[0] = nv;
  }
  __syncthreads();
  {
    // copy of the staged h blocks: a 16-lane group per (row tile, column
    // tile) block, 16-byte pieces (a block is width*16 contiguous floats)
    const int nv = hmeta[0];
    const int grp = tid >> 4, gl = tid & 15;
    constexpr int NG = Cfg::NTH / 16;
    for (int q0 = grp; q0 < nv; q0 += 2 * NG) {
      float4 v[2][2];
      int dst[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q = q0 + u * NG;
        int w = 0;
        const float4* src = nullptr;
        if (q < nv) {
          const int i = q / S, sj = q - i * S;
          const int rt = (m0 >> 4) + i;
          if (rt * 16 < a.T) {                    // row tiles past T hold nothing
            w = a.hwidth[(int64_t)rt * a.NT + tjf + sj];
            src = (const float4*)(a.hval + ((int64_t)rt * a.NT + tjf + sj) * 1024);
          }
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int c = gl + 16 * c2;
          dst[u][c2] = c < w * 4 ? hoff[q] / 4 + c : -1;
          v[u][c2] = c < w * 4 ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        // widths above 8 (rare): the rest of the block directly
        for (int c = gl + 32; c < w * 4; c += 16) ((float4*)hb)[hoff[q] / 4 + c] = src[c];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
          if (dst[u][c2] >= 0) ((float4*)hb)[dst[u][c2]] = v[u][c2];
    }
  }
  __syncthreads();

  bool over = false;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int p = p0 + Tile::col_of(j);
    const int n = p < nb ? ul[p] : -1;
    const int tj = n >> 6, c = n & 63, sj = tj - tjf;
    const bool wr = p < ((nb + 63) & ~63);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = Tile::row_of(i, e);
        const int t = m0 + r;
        float v = 0.f;
        if (n >= 0) {
          const uint64_t M = sj < S ? sm[r * S + sj] : (live(a, t) ? a.mask[(int64_t)t * a.NT + tj] : 0ull);
          if ((M >> c) & 1ull) {
            const int slot = popc64(M & below(c));
            const int o = sj < S ? hoff[(r >> 4) * S + sj] : -1;
            const float h = o >= 0 ? hb[o + slot * 16 + (r & 15)]
                                   : a.hval[((int64_t)(t >> 4) * a.NT + tj) * 1024 + slot * 16 + (t & 15)];
            v = h * g.acc[0][i][j][e];
            over |= !(fabsf(v) <= 65504.f);
          }
        }
        if (wr && t < a.T) a.adense[(int64_t)t * a.F + p] = (_Float16)v;
      }
  }
  if (__builtin_amdgcn_ballot_w64(over) != 0ull && lane == 0) atomicOr(a.flag, 1);
}

// Down-projection over the union: y rows of the block, one 256-column tile.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void down_union_kernel(UnionArgs a) {
  static_assert(Cfg::BM == UB, "one row block per M tile");
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS_BYTES];
  if (*a.flag) return;                              // fp16 overflow: the fallback path writes y
  const int nct = a.d / Cfg::BN;
  const int b = blockIdx.x / nct, ct = blockIdx.x - b * nct;
  const int nb = a.ucount[b];
  const int m0 = b * UB, n0 = ct * Cfg::BN;
  GemmTile<Cfg> g;
  const Operand A{a.adense, a.F, nullptr, a.T};
  const Operand B{a.Wd, a.d, a.ulist + (int64_t)b * a.F, a.F};
  g.run(A, &B, m0, n0, nb, lds);
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + GemmTile<Cfg>::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = m0 + GemmTile<Cfg>::row_of(i, e);
        if (live(a, t)) {
          const float v = g.acc[0][i][j][e];
          if (a.out_bf16) ((uint16_t*)a.y)[(int64_t)t * a.d + col] = (uint16_t)f32_to_bf16_bits(v);
          else ((float*)a.y)[(int64_t)t * a.d + col] = v;
        }
      }
  }
}

#if TWELL_UNION_ROWS == 256
using UpUnionCfg = DmaCfg<256, 256, 4, 2>;
using DownUnionCfg = GemmCfg<256, 256, 2, 4, OP_F16_K, OP_BF16_T16>;
using DownUnionCfg128 = GemmCfg<256, 128, 2, 2, OP_F16_K, OP_BF16_T16>;
using DownUnionCfg64 = GemmCfg<256, 64, 4, 1, OP_F16_K, OP_BF16_T16>;
#elif TWELL_UNION_ROWS == 128
using UpUnionCfg = DmaCfg<128, 256, 2, 4>;
using DownUnionCfg = GemmCfg<128, 256, 2, 4, OP_F16_K, OP_BF16_T16>;
using DownUnionCfg128 = GemmCfg<128, 128, 2, 2, OP_F16_K, OP_BF16_T16>;
using DownUnionCfg64 = GemmCfg<128, 64, 2, 1, OP_F16_K, OP_BF16_T16>;
#else
using UpUnionCfg = DmaCfg<64, 256, 1, 4>;
using DownUnionCfg = GemmCfg<64, 256, 1, 4, OP_F16_K, OP_BF16_T16>;
using DownUnionCfg128 = GemmCfg<64, 128, 1, 2, OP_F16_K, OP_BF16_T16>;
using DownUnionCfg64 = GemmCfg<64, 64, 1, 1, OP_F16_K, OP_BF16_T16>;
#endif

size_t union_ws_bytes(int T, int F) {
  const size_t nblk = (size_t)(T + UB - 1) / UB;
  const size_t nslab = (size_t)(T + 63) / 64;
  return nblk * F * 4 + nblk * 4 + (size_t)T * F * 2 + nslab * (F / 64) * 8 + 256 * 4;
}

hipError_t launch_union_fwd(const void* x, const void* WuT, const void* Wd, int T, int d, int F,
                            const TwellView& h, const uint8_t* skip, void* ws, void* y, int out_dt,
                            int** flag_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nblk = (T + UB - 1) / UB;
  char* w = (char*)ws;
  UnionArgs a{};
  a.x = x; a.WuT = WuT; a.Wd = Wd; a.T = T; a.d = d; a.F = F; a.NT = F / 64;
  a.mask = h.mask; a.skip = skip; a.hval = (const float*)h.val; a.hwidth = h.width;
  a.ulist = (int*)w;
  a.ucount = (int*)(w + (size_t)nblk * F * 4);
  a.adense = (_Float16*)(w + (((size_t)nblk * F * 4 + (size_t)nblk * 4 + 255) & ~(size_t)255));
  a.flag = (int*)((char*)a.adense + (((size_t)T * F * 2 + 255) & ~(size_t)255));
  uint64_t* U = (uint64_t*)((char*)a.flag + 256);
  a.y = y; a.out_bf16 = out_dt == DT_BF16;
  if (flag_out) *flag_out = a.flag;
  hipLaunchKernelGGL(union_or_kernel, dim3((T + 63) / 64, (a.NT + 63) / 64), dim3(256), 0, s, a, U);
  hipLaunchKernelGGL(union_list_kernel, dim3(nblk), dim3(256), 0, s, a, (const uint64_t*)U);
  const int npt = (F + UpUnionCfg::BN - 1) / UpUnionCfg::BN;
  const int nbx_max = (nblk + 7) / 8;
  hipLaunchKernelGGL((up_union_kernel<UpUnionCfg>), dim3(8 * nbx_max * npt), dim3(UpUnionCfg::NTH), 0, s, a);
  if (d % 256 == 0)
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg>), dim3(nblk * (d / 256)), dim3(DownUnionCfg::NTH), 0, s, a);
  else if (d % 128 == 0)
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg128>), dim3(nblk * (d / 128)), dim3(DownUnionCfg128::NTH), 0, s,
                       a);
  else
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg64>), dim3(nblk * (d / 64)), dim3(DownUnionCfg64::NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace twell
