// Sparse up- and down-projections on the TwELL pattern of the gate (generic
// kernels, used for fp32 inputs; bf16 inputs go to twell_sparse_bf16.hip).
//
// The intellectnews.ru TwELL article, section "Слитые CUDA-ядра для инференса
// и гибрид для обучения", describes the inference FFN as a few fused steps
// whose intermediates stay out of global memory, and the same page says that
// only active neurons are worth touching.  After the gate GEMM has packed
// h = ReLU(x.Wg + b) into TwELL, two kernels finish the layer:
//
//   up   (SDDMM):  a[t,n] = h[t,n] * (x_t . WuT[n])   for stored (t, n)
//   down (SpMM):   y_t    = sum over stored n of a[t,n] * Wd[n]
//
// The only intermediate that reaches memory is a, in the TwELL value slots
// (4 bytes per stored pair).
//
// Both kernels work on groups of 16 tokens (one TwELL row tile).  For a group
// the union of its rows' active neurons is gathered into a list and the
// group x union block is multiplied on the bf16 MFMA units (16x16x32): a
// neuron in the union is active in at least one of the 16 tokens, so the
// matrix cores never do less useful work than the vector ALUs would, and
// neurons shared by several tokens are loaded once.
//   * up:   each workgroup takes one slice of the neurons (f/8, one slice per
//           XCD, so each XCD keeps its slice of WuT in its own L2).
//   * down: each workgroup takes one slice of the output columns (d/8, one per
//           XCD, same reason for Wd).  a is fp32 and is fed to the MFMA as
//           bf16 hi + lo (two MFMAs), which keeps fp32-level accuracy.
#include "common.hpp"
#include "internal.hpp"

namespace twell {

struct SparseArgs {
  const void* x;          // [T][d] (up; backward: x)
  const void* W;          // WuT (up) or Wd / WgT (down), [F][d]
  const void* x2;         // backward up: dY [T][d]
  const void* W2;         // backward up: Wd; backward down: WuT
  int T, d, F, NT, NR;
  const uint64_t* mask;   // [T][NT]
  const float* hval;      // up: h values in TwELL layout
  float* aval;            // up: output a; down: input values
  float* dgval;           // backward up: output dg = da*u; backward down: input (with W)
  float* duval;           // backward up: output du = da*h; backward down: input (with W2)
  const uint8_t* skip;    // [T] or null
  void* y;                // down output [T][d]
  int out_bf16;
  int nslices;
  float l1;               // backward up: added to dg on every stored pair (activation penalty)
  int cap;                // slots per TwELL tile of the value arrays
};

constexpr int SP_WPB = 4;        // waves (token groups) per workgroup
constexpr int UP_MAXT = 32;      // column tiles per neuron slice (at most)
constexpr int UP_NBLK = 8;       // 16-neuron blocks per pass (128 neurons)
constexpr int DN_TCH = 16;       // column tiles per union chunk in the down kernel
constexpr int DN_MAXCB = 24;     // 16-column blocks per output slice

__device__ __forceinline__ bool row_live(const SparseArgs& a, int t) {
  return t < a.T && !(a.skip && a.skip[t]);
}

// Exclusive prefix sum over the wave; returns the total in *total.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* total) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  *total = __shfl(incl, 63);
  return incl - v;
}

// ------------------------------------------------------------------ up (SDDMM)

// BWD: also da = dY_t . Wd[n] on the same pattern, and the outputs become
// a = h*u, dg = da*u, du = da*h (the backward pass's per-pair quantities).
template <bool BF16IN, bool BWD>
__global__ __launch_bounds__(256) void sddmm_up_kernel(SparseArgs a) {
  __shared__ uint64_t smask[SP_WPB][16][UP_MAXT];
  __shared__ uint16_t sunion[SP_WPB][UP_MAXT * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int slice = blockIdx.x % a.nslices;
  const int grp = (blockIdx.x / a.nslices) * SP_WPB + w;
  const bool live = grp < a.NR;
  const int t0 = grp * 16;
  const int j0 = slice * a.NT / a.nslices, j1 = (slice + 1) * a.NT / a.nslices;
  const int ntl = j1 - j0;

  uint64_t U = 0;
  if (live && lane < ntl) {
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + r;
      const uint64_t m = row_live(a, t) ? a.mask[(int64_t)t * a.NT + j0 + lane] : 0ull;
      smask[w][r][lane] = m;
      U |= m;
    }
  }
  int total;
  int p = wave_excl_scan(popc64(U), lane, &total);
  for (uint64_t m = U; m; m &= m - 1) sunion[w][p++] = (uint16_t)((j0 + lane) * 64 + __ffsll((long long)m) - 1);
  __syncthreads();
  if (!live || total == 0) return;

  constexpr int KS = BF16IN ? 32 : 16;           // k per MFMA step
  constexpr int ESZ = BF16IN ? 2 : 4;
  const int64_t xoff = ((int64_t)min(t0 + (lane & 15), a.T - 1) * a.d) * ESZ;
  const char* xrow = (const char*)a.x + xoff;
  const char* yrow = BWD ? (const char*)a.x2 + xoff : nullptr;
  const int koff = (lane >> 4) * (KS / 4);       // element offset of my fragment
  const int npad = (total + 15) & ~15;
  for (int base = 0; base < npad; base += 16 * UP_NBLK) {
    const int nb = min(UP_NBLK, (npad - base) >> 4);
    int64_t wofs[UP_NBLK];
#pragma unroll
    for (int b = 0; b < UP_NBLK; ++b) {
      const int q = base + b * 16 + (lane & 15);
      const int n = sunion[w][q < total ? q : 0];
      wofs[b] = ((int64_t)n * a.d) * ESZ;
    }
    f32x4 acc[UP_NBLK], acc2[BWD ? UP_NBLK : 1];
#pragma unroll
    for (int b = 0; b < UP_NBLK; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BWD) {
#pragma unroll
      for (int b = 0; b < UP_NBLK; ++b) acc2[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int k0 = 0; k0 < a.d; k0 += KS) {
      const int64_t ko = (int64_t)(k0 + koff) * ESZ;
      const uint4 fa = *(const uint4*)(xrow + ko);
      uint4 fy;
      if constexpr (BWD) fy = *(const uint4*)(yrow + ko);
#pragma unroll
      for (int b = 0; b < UP_NBLK; ++b) {
        if (b < nb) {
          const uint4 fb = *(const uint4*)((const char*)a.W + wofs[b] + ko);
          if constexpr (BF16IN) acc[b] = mfma16(fa, fb, acc[b]);
          else acc[b] = mfma16_f32(fa, fb, acc[b]);
          if constexpr (BWD) {
            const uint4 fd = *(const uint4*)((const char*)a.W2 + wofs[b] + ko);
            if constexpr (BF16IN) acc2[b] = mfma16(fy, fd, acc2[b]);
            else acc2[b] = mfma16_f32(fy, fd, acc2[b]);
          }
        }
      }
    }
#pragma unroll
    for (int b = 0; b < UP_NBLK; ++b) {
      const int q = base + b * 16 + (lane & 15);
      if (b < nb && q < total) {
        const int n = sunion[w][q];
        const int j = n >> 6, c = n & 63;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = mfma16_row(lane, i);
          const uint64_t M = smask[w][r][j - j0];
          if ((M >> c) & 1ull) {
            const int slot = popc64(M & below(c));
            const int64_t off = ((int64_t)grp * a.NT + j) * (a.cap * 16) + slot * 16 + r;
            const float h = a.hval[off];
            a.aval[off] = h * acc[b][i];
            if constexpr (BWD) {
              a.dgval[off] = acc2[b][i] * acc[b][i] + a.l1;
              a.duval[off] = acc2[b][i] * h;
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down (SpMM)

// TWO: y_t = sum over stored n of dgval*W[n] + duval*W2[n] (the backward
// pass's dX = dG.WgT + dU.WuT on the sparse rows); otherwise aval*W[n].
template <bool BF16IN, bool TWO>
__global__ __launch_bounds__(256) void spmm_down_kernel(SparseArgs a) {
  __shared__ uint64_t smask[SP_WPB][16][DN_TCH];
  __shared__ uint16_t sunion[SP_WPB][DN_TCH * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cs = blockIdx.x % a.nslices;
  const int grp = (blockIdx.x / a.nslices) * SP_WPB + w;
  const bool live = grp < a.NR;
  const int t0 = grp * 16;
  const int ncb_all = a.d / 16;
  const int cb0 = cs * ncb_all / a.nslices;
  const int ncb = (cs + 1) * ncb_all / a.nslices - cb0;
  const int r_a = lane & 15;                 // token row of my A fragment
  constexpr int KC = BF16IN ? 32 : 16;       // neurons per MFMA step
  constexpr int EPL = KC / 4;                // neurons per lane per step

  f32x4 acc[DN_MAXCB];
#pragma unroll
  for (int cb = 0; cb < DN_MAXCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int jc = 0; jc < a.NT; jc += DN_TCH) {
    for (int q = lane; q < 16 * DN_TCH; q += 64) {
      const int r = q / DN_TCH, jj = q % DN_TCH;
      const int t = t0 + r, j = jc + jj;
      smask[w][r][jj] = (live && j < a.NT && row_live(a, t)) ? a.mask[(int64_t)t * a.NT + j] : 0ull;
    }
    __syncthreads();
    uint64_t U = 0;
    if (lane < DN_TCH) {
#pragma unroll
      for (int r = 0; r < 16; ++r) U |= smask[w][r][lane];
    }
    int total;
    int p = wave_excl_scan(popc64(U), lane, &total);
    for (uint64_t m = U; m; m &= m - 1) sunion[w][p++] = (uint16_t)((jc + lane) * 64 + __ffsll((long long)m) - 1);
    __syncthreads();

    for (int kc = 0; kc < total; kc += KC) {
      constexpr int NV = TWO ? 2 : 1;
      const float* vsrc[2] = {TWO ? a.dgval : a.aval, a.duval};
      uint32_t ahi[NV][EPL], alo[NV][EPL];
      int nid[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int q = kc + (lane >> 4) * EPL + e;
        float av[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) av[v] = 0.f;
        int n = 0;
        if (q < total) {
          n = sunion[w][q];
          const int j = n >> 6, c = n & 63;
          const uint64_t M = smask[w][r_a][j - jc];
          if ((M >> c) & 1ull) {
            const int slot = popc64(M & below(c));
            const int64_t off = ((int64_t)grp * a.NT + j) * (a.cap * 16) + slot * 16 + r_a;
#pragma unroll
            for (int v = 0; v < NV; ++v) av[v] = vsrc[v][off];
          }
        }
        nid[e] = n;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if constexpr (BF16IN) split_bf16(av[v], ahi[v][e], alo[v][e]);
          else ahi[v][e] = __float_as_uint(av[v]);
        }
      }
      uint4 Ahi[NV], Alo[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if constexpr (BF16IN) {
          Ahi[v] = make_uint4(ahi[v][0] | (ahi[v][1] << 16), ahi[v][2] | (ahi[v][3] << 16),
                              ahi[v][4] | (ahi[v][5] << 16), ahi[v][6] | (ahi[v][7] << 16));
          Alo[v] = make_uint4(alo[v][0] | (alo[v][1] << 16), alo[v][2] | (alo[v][3] << 16),
                              alo[v][4] | (alo[v][5] << 16), alo[v][6] | (alo[v][7] << 16));
        } else {
          Ahi[v] = make_uint4(ahi[v][0], ahi[v][1], ahi[v][2], ahi[v][3]);
          Alo[v] = Ahi[v];
        }
      }
#pragma unroll
      for (int cb = 0; cb < DN_MAXCB; ++cb) {
        if (cb < ncb) {
          const int col = (cb0 + cb) * 16 + (lane & 15);
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const void* Wv = v == 0 ? a.W : a.W2;
            uint4 B;
            if constexpr (BF16IN) {
              const uint16_t* W = (const uint16_t*)Wv;
              uint32_t bv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) bv[e] = W[(int64_t)nid[e] * a.d + col];
              B = make_uint4(bv[0] | (bv[1] << 16), bv[2] | (bv[3] << 16), bv[4] | (bv[5] << 16),
                             bv[6] | (bv[7] << 16));
              acc[cb] = mfma16(Ahi[v], B, acc[cb]);
              acc[cb] = mfma16(Alo[v], B, acc[cb]);
            } else {
              const uint32_t* W = (const uint32_t*)Wv;
              B = make_uint4(W[(int64_t)nid[0] * a.d + col], W[(int64_t)nid[1] * a.d + col],
                             W[(int64_t)nid[2] * a.d + col], W[(int64_t)nid[3] * a.d + col]);
              acc[cb] = mfma16_f32(Ahi[v], B, acc[cb]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  if (!live) return;
#pragma unroll
  for (int cb = 0; cb < DN_MAXCB; ++cb) {
    if (cb < ncb) {
      const int col = (cb0 + cb) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + mfma16_row(lane, i);
        if (row_live(a, t)) {
          if (a.out_bf16) ((uint16_t*)a.y)[(int64_t)t * a.d + col] = (uint16_t)f32_to_bf16_bits(acc[cb][i]);
          else ((float*)a.y)[(int64_t)t * a.d + col] = acc[cb][i];
        }
      }
    }
  }
}

static int choose_slices(int n_units, int max_per_slice) {
  int s = 8;
  while ((n_units + s - 1) / s > max_per_slice) s += 8;
  return s;
}

hipError_t launch_sddmm_up(int in_dt, const void* x, const void* WuT, int T, int d, int F,
                           const TwellView& h, float* aval, const uint8_t* skip, hipStream_t s) {
  SparseArgs a{};
  a.x = x; a.W = WuT; a.T = T; a.d = d; a.F = F; a.NT = F / 64; a.NR = (T + 15) / 16;
  a.mask = h.mask; a.hval = (const float*)h.val; a.aval = aval; a.skip = skip; a.cap = h.cap;
  if (in_dt == DT_BF16) return launch_up_bf16(x, nullptr, WuT, nullptr, T, d, F, h, aval, nullptr, nullptr, skip, s);
  a.nslices = choose_slices(a.NT, UP_MAXT);
  if (a.NR == 0) return hipSuccess;
  const int grid = ((a.NR + SP_WPB - 1) / SP_WPB) * a.nslices;
  hipLaunchKernelGGL((sddmm_up_kernel<false, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sddmm_bwd(int in_dt, const void* x, const void* dY, const void* WuT, const void* Wd, int T,
                            int d, int F, const TwellView& h, float* aval, float* dgval, float* duval,
                            const uint8_t* skip, hipStream_t s, float l1) {
  SparseArgs a{};
  a.l1 = l1;
  a.x = x; a.x2 = dY; a.W = WuT; a.W2 = Wd; a.T = T; a.d = d; a.F = F; a.NT = F / 64; a.NR = (T + 15) / 16;
  a.mask = h.mask; a.hval = (const float*)h.val; a.aval = aval; a.dgval = dgval; a.duval = duval; a.skip = skip;
  a.cap = h.cap;
  if (in_dt == DT_BF16) return launch_up_bf16(x, dY, WuT, Wd, T, d, F, h, aval, dgval, duval, skip, s, nullptr, l1);
  a.nslices = choose_slices(a.NT, UP_MAXT);
  if (a.NR == 0) return hipSuccess;
  const int grid = ((a.NR + SP_WPB - 1) / SP_WPB) * a.nslices;
  hipLaunchKernelGGL((sddmm_up_kernel<false, true>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_spmm_down(int in_dt, int out_dt, const float* aval, const void* Wd, int T, int d,
                            int F, const TwellView& pat, void* y, const uint8_t* skip, hipStream_t s) {
  SparseArgs a{};
  a.W = Wd; a.T = T; a.d = d; a.F = F; a.NT = F / 64; a.NR = (T + 15) / 16;
  a.mask = pat.mask; a.aval = (float*)aval; a.skip = skip; a.y = y; a.out_bf16 = out_dt == DT_BF16;
  a.cap = pat.cap;
  if (in_dt == DT_BF16) return launch_down_bf16(aval, nullptr, Wd, nullptr, T, d, F, pat, y, out_dt, skip, s);
  a.nslices = choose_slices(d / 16, DN_MAXCB);
  if (d / 16 < a.nslices) a.nslices = d / 16;
  if (a.NR == 0) return hipSuccess;
  const int grid = ((a.NR + SP_WPB - 1) / SP_WPB) * a.nslices;
  hipLaunchKernelGGL((spmm_down_kernel<false, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_spmm_dx(int in_dt, const float* dgval, const float* duval, const void* WgT, const void* WuT,
                          int T, int d, int F, const TwellView& pat, float* dX, const uint8_t* skip,
                          hipStream_t s) {
  SparseArgs a{};
  a.W = WgT; a.W2 = WuT; a.T = T; a.d = d; a.F = F; a.NT = F / 64; a.NR = (T + 15) / 16;
  a.mask = pat.mask; a.dgval = (float*)dgval; a.duval = (float*)duval; a.skip = skip; a.y = dX; a.out_bf16 = 0;
  a.cap = pat.cap;
  if (in_dt == DT_BF16) return launch_down_bf16(dgval, duval, WgT, WuT, T, d, F, pat, dX, DT_F32, skip, s);
  a.nslices = choose_slices(d / 16, DN_MAXCB);
  if (d / 16 < a.nslices) a.nslices = d / 16;
  if (a.NR == 0) return hipSuccess;
  const int grid = ((a.NR + SP_WPB - 1) / SP_WPB) * a.nslices;
  hipLaunchKernelGGL((spmm_down_kernel<false, true>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace twell
