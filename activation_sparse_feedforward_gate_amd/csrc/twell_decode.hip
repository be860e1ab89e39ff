// Forward for few tokens (decode-shaped batches, T <= 256, bf16 inputs,
// inference), and the dense few-token forward it is measured against.
//
// With a few dozen tokens the gate GEMM is a pass over all of WgT, and the
// up- and down-projections touch only the stored (token, neuron) pairs of
// the TwELL ([IN] "Слитые CUDA-ядра для инференса и гибрид для обучения":
// only the active neurons in the up/down phases), a few thousand of them:
//   1 gate partials   Pg[s] = x . WgT[:, Ks]^T, K split over many workgroups
//                     (64x64 output tiles of four waves on the direct-to-LDS
//                     mainloop, whose coalesced loads stream WgT at close to
//                     the rate of a plain copy)
//   2 pack + up       g = sum_s Pg[s] + b (fixed order), TwELL pack of
//                     ReLU(g) (fp32 values), then a = h * (x_t . WuT[n]) at
//                     the tile's stored pairs in fp32, kept in the TwELL
//                     layout; one workgroup of eight waves per 16x64 tile,
//                     two rows per wave, two pairs at a time
//   3 down            y_t = sum over row t's stored pairs, ascending n, of
//                     a * Wd[n], fp32: one workgroup per (row, 256 columns),
//                     each wave lists the pairs of a quarter of the row's
//                     column tiles in LDS; the four sums added in order
// All sums run in a fixed order, so results do not depend on timing.  The
// dense few-token forward keeps the split-K GEMMs throughout: gate and up
// partials in one GEMM with two B operands, act = bf16(ReLU(sum Pg + b) *
// sum Pu), then the down-projection split along K over all F neurons and a
// fixed-order reduction of its partials.
#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

// 64x64 output tiles, four waves of 32x32 each
using SplitCfg = DmaCfg<64, 64, 2, 2>;                      // K-major B
using SplitCfg2 = DmaCfg<64, 64, 2, 2, 2>;                  // two K-major B sharing A
using SplitCfgBT = DmaCfg<64, 64, 2, 2, 1, false, true>;    // [K][N] B

constexpr int KS_GATE = 4, KS_DOWN = 16;
constexpr int KS_DENSE_GU = 2;   // the dense gate/up GEMM reads twice the bytes per split: fewer splits are faster

struct DecArgs {
  const uint16_t* x;
  const uint16_t* WgT;
  const uint16_t* bg;
  const uint16_t* WuT;
  const uint16_t* Wd;
  int T, d, F, NT;
  float* aval;          // a = h * u at the stored pairs, in the TwELL layout of h
  float* pg;            // [KS_GATE][T][F]
  float* pu;            // dense path: [KS_DENSE_GU][T][F], and pg likewise
  uint16_t* ahi;        // dense path: act [T][F]
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

// 1: partial x . WgT^T over one K split.
__device__ __forceinline__ void dec_gate_split(const DecArgs& a, char* st0, char* st1) {
  const int s = blockIdx.y, n0 = blockIdx.x * 64, m0 = blockIdx.z * 64;
  int k0, kn;
  split_range(a.d, KS_GATE, s, k0, kn);
  float* P = a.pg + (int64_t)s * a.T * a.F;
  DmaTile<SplitCfg> g;
  if (kn > 0) {
    const Operand A{a.x + k0, a.d, nullptr, a.T};
    const Operand B{a.WgT + k0, a.d, nullptr, a.F};
    g.run(A, &B, m0, n0, kn, st0, st1);
  } else {
    zero_tile(g);
  }
  store_partial(g, 0, P, a.F, a.T, m0, n0);
}

__global__ __launch_bounds__(SplitCfg::NTH) void dec_gate_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfg::STAGE];
  dec_gate_split(a, st0, st1);
}

// 2: g = sum of the gate partials + bias, TwELL pack of ReLU(g), then
// a = h * (x_t . WuT[n]) at the tile's stored pairs, into aval at the pair's
// TwELL position.  One workgroup of eight waves per 16x64 tile; wave w packs
// rows 2w and 2w+1 (lane = column, every partial load in flight at once) and
// then takes those rows' pairs two at a time, in slot order, with x_t and
// both WuT rows in flight together (eight bf16 per lane per 512-element chunk
// of d, UPC chunks per pass over d); the dot products end with a fixed-order
// butterfly sum.
constexpr int PU_WAVES = 8;                              // waves per 16-row tile
constexpr int PU_RPW = 16 / PU_WAVES;                    // rows per wave (1 or 2)
static_assert(PU_RPW == 1 || PU_RPW == 2, "one or two rows per wave");

__device__ __forceinline__ float dot8(const uint4& x, const uint4& w, float acc) {
  acc += bf16_lo(x.x) * bf16_lo(w.x);
  acc += bf16_hi(x.x) * bf16_hi(w.x);
  acc += bf16_lo(x.y) * bf16_lo(w.y);
  acc += bf16_hi(x.y) * bf16_hi(w.y);
  acc += bf16_lo(x.z) * bf16_lo(w.z);
  acc += bf16_hi(x.z) * bf16_hi(w.z);
  acc += bf16_lo(x.w) * bf16_lo(w.w);
  acc += bf16_hi(x.w) * bf16_hi(w.w);
  return acc;
}

// Next stored pair of the wave's two rows: row 0's set bits first, lowest
// column first (wave-uniform).
__device__ __forceinline__ void next_pair(uint64_t& rem0, uint64_t& rem1, int& s0, int& s1, int& q, int& n,
                                          int& slot) {
  if (rem0) {
    q = 0; n = __builtin_ctzll(rem0); rem0 &= rem0 - 1; slot = s0++;
  } else {
    q = 1; n = __builtin_ctzll(rem1); rem1 &= rem1 - 1; slot = s1++;
  }
}

template <int UPC>
__global__ __launch_bounds__(64 * PU_WAVES) void dec_pack_up_kernel(DecArgs a) {
  __shared__ int wmax[PU_WAVES];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x / a.NT, j = blockIdx.x % a.NT;
  const int col = j * 64 + lane;
  const float b = a.bg ? bf16_to_f32(a.bg[col]) : 0.f;
  float v[2] = {0.f, 0.f};
  uint64_t M[2] = {0ull, 0ull};
  int wd = 0;
#pragma unroll
  for (int q = 0; q < PU_RPW; ++q) {
    const int t = i * 16 + PU_RPW * w + q;
    float g = 0.f;
    if (t < a.T) {
#pragma unroll
      for (int s = 0; s < KS_GATE; ++s) g += a.pg[((int64_t)s * a.T + t) * a.F + col];
      g += b;
    }
    v[q] = g;
    M[q] = ballot(t < a.T && g > 0.f);
    wd = max(wd, popc64(M[q]));
  }
  if (lane == 0) wmax[w] = wd;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PU_WAVES; ++k) wd = max(wd, wmax[k]);
  const int64_t tile = (int64_t)i * a.NT + j;
  if (threadIdx.x == 0) a.width[tile] = (uint8_t)wd;
  const int64_t tbase = tile * (64 * 16);
#pragma unroll
  for (int q = 0; q < PU_RPW; ++q) {
    const int r = PU_RPW * w + q, t = i * 16 + r;
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

  uint64_t rem0 = M[0], rem1 = M[1];
  int s0 = 0, s1 = 0;
  const int tr = i * 16 + PU_RPW * w;                    // the wave's first row
  while (rem0 | rem1) {
    int qa, na, sa, qb, nb, sb;
    next_pair(rem0, rem1, s0, s1, qa, na, sa);
    const bool two = (rem0 | rem1) != 0;
    qb = qa; nb = na; sb = sa;
    if (two) next_pair(rem0, rem1, s0, s1, qb, nb, sb);
    const uint16_t* xa = a.x + (int64_t)(tr + qa) * a.d;
    const uint16_t* xb = a.x + (int64_t)(tr + qb) * a.d;
    const uint16_t* wa = a.WuT + (int64_t)(j * 64 + na) * a.d;
    const uint16_t* wb = a.WuT + (int64_t)(j * 64 + nb) * a.d;
    float ua = 0.f, ub = 0.f;
    for (int k0 = 0; k0 < a.d; k0 += 512 * UPC) {
      uint4 xva[UPC], xvb[UPC], wva[UPC], wvb[UPC];
#pragma unroll
      for (int m = 0; m < UPC; ++m) {
        const int o = k0 + m * 512 + lane * 8;
        xva[m] = wva[m] = xvb[m] = wvb[m] = make_uint4(0, 0, 0, 0);
        if (o < a.d) {
          xva[m] = *(const uint4*)(xa + o);
          wva[m] = *(const uint4*)(wa + o);
          if (two) {
            xvb[m] = *(const uint4*)(xb + o);
            wvb[m] = *(const uint4*)(wb + o);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < UPC; ++m) {
        ua = dot8(xva[m], wva[m], ua);
        ub = dot8(xvb[m], wvb[m], ub);
      }
    }
    ua = wave_sum(ua);
    ub = wave_sum(ub);
    const float ha = __shfl(qa ? v[1] : v[0], na);
    const float hb = __shfl(qb ? v[1] : v[0], nb);
    if (lane == 0) {
      a.aval[tbase + sa * 16 + PU_RPW * w + qa] = ha * ua;
      if (two) a.aval[tbase + sb * 16 + PU_RPW * w + qb] = hb * ub;
    }
  }
}

// 3: y_t = sum over row t's stored pairs, in ascending neuron order, of
// a * Wd[n], fp32.  One workgroup per (256 columns of y, row t), four
// adjacent columns per lane (one 8-byte load of Wd per pair).  Wave q takes
// the q-th quarter of the row's column tiles, 64 tiles at a time: a scan of
// their counts across the lanes places each tile's pairs (neuron, a) in the
// wave's list in LDS, then the lane's Wd values of up to DPF pairs are loaded
// together before the FMAs.  The four partial sums are added in wave order.
constexpr int DPF = 16;                                  // Wd loads in flight per lane
constexpr int DL_CAP = 256;                              // list entries per wave and round
__global__ __launch_bounds__(256) void dec_down_kernel(DecArgs a) {
  __shared__ int2 list[4][DL_CAP];
  __shared__ float4 part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.y, i = t >> 4, r = t & 15;
  const int c = blockIdx.x * 256 + lane * 4;               // d % 64 == 0: c < d or all four past d
  const bool live = c < a.d;
  const uint16_t* wd = a.Wd + c;
  const int j0 = (a.NT * wave) / 4, j1 = (a.NT * (wave + 1)) / 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int jb = j0; jb < j1; jb += 64) {
    const int j = jb + lane;
    const int cj = j < j1 ? a.cnt[(int64_t)t * a.NT + j] : 0;
    int pre = cj;                                          // inclusive scan over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(pre, o);
      if (lane >= o) pre += u;
    }
    const int m = __shfl(pre, 63), ex = pre - cj;
    const int64_t tb = ((int64_t)i * a.NT + j) * 1024 + r;
    for (int e0 = 0; e0 < m; e0 += DL_CAP) {
      const int sb = max(0, e0 - ex), se = min(cj, e0 + DL_CAP - ex);
      for (int s = sb; s < se; s += 4) {
        int nn[4];
        float av[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool ok = s + u < se;
          nn[u] = ok ? a.hidx[tb + (s + u) * 16] : 0;
          av[u] = ok ? a.aval[tb + (s + u) * 16] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s + u < se) list[wave][ex + s + u - e0] = make_int2(j * 64 + nn[u], __float_as_int(av[u]));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int mm = min(DL_CAP, m - e0);
      for (int k0 = 0; k0 < mm; k0 += DPF) {
        uint2 wv[DPF];
        float aq[DPF];
#pragma unroll
        for (int q = 0; q < DPF; ++q) {
          const bool ok = k0 + q < mm;
          const int2 en = ok ? list[wave][k0 + q] : make_int2(0, 0);
          aq[q] = __int_as_float(en.y);
          wv[q] = (live && ok) ? *(const uint2*)(wd + (int64_t)en.x * a.d) : make_uint2(0, 0);
        }
#pragma unroll
        for (int q = 0; q < DPF; ++q) {
          if (k0 + q < mm) {
            acc.x += aq[q] * bf16_lo(wv[q].x);
            acc.y += aq[q] * bf16_hi(wv[q].x);
            acc.z += aq[q] * bf16_lo(wv[q].y);
            acc.w += aq[q] * bf16_hi(wv[q].y);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && live) {
    const float4 p0 = part[0][lane], p1 = part[1][lane], p2 = part[2][lane], p3 = part[3][lane];
    const float v0 = ((p0.x + p1.x) + p2.x) + p3.x, v1 = ((p0.y + p1.y) + p2.y) + p3.y;
    const float v2 = ((p0.z + p1.z) + p2.z) + p3.z, v3 = ((p0.w + p1.w) + p2.w) + p3.w;
    const int64_t e = (int64_t)t * a.d + c;
    if (a.out_bf16) {
      uint2 o;
      o.x = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
      o.y = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
      *(uint2*)((uint16_t*)a.y + e) = o;
    } else {
      *(float4*)((float*)a.y + e) = make_float4(v0, v1, v2, v3);
    }
  }
}

// Dense path, 3: y partial over one split of K = all F neurons (A = act).
__device__ __forceinline__ void dec_down(const DecArgs& a, char* st0, char* st1) {
  const int s = blockIdx.y, n0 = blockIdx.x * 64, m0 = blockIdx.z * 64;
  int k0, kn;
  split_range(a.F, KS_DOWN, s, k0, kn);
  DmaTile<SplitCfgBT> g;
  if (kn > 0) {
    const Operand B{a.Wd + (int64_t)k0 * a.d, a.d, nullptr, a.F};
    const Operand A0{a.ahi + k0, a.F, nullptr, a.T};
    g.run(A0, &B, m0, n0, kn, st0, st1);
  } else {
    zero_tile(g);
  }
  store_partial(g, 0, a.py + (int64_t)s * a.T * a.d, a.d, a.T, m0, n0);
}

__global__ __launch_bounds__(SplitCfgBT::NTH) void dense_few_down_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[SplitCfgBT::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[SplitCfgBT::STAGE];
  dec_down(a, st0, st1);
}

// Dense path, 4: y = sum of the down partials.
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

void launch_down_reduce(const DecArgs& a, hipStream_t s) {
  const dim3 grid(a.d / 64, KS_DOWN, (a.T + 63) / 64);
  hipLaunchKernelGGL(dense_few_down_kernel, grid, dim3(SplitCfgBT::NTH), 0, s, a);
  hipLaunchKernelGGL(dec_reduce_kernel, dim3((unsigned)(((int64_t)a.T * a.d + 255) / 256)), dim3(256), 0, s, a);
}

}  // namespace

size_t decode_ws_bytes(int T, int d, int F) {
  (void)d;
  return r256((size_t)KS_GATE * T * F * 4) + r256((size_t)((T + 15) / 16) * 16 * F * 4);
}

hipError_t launch_decode_fwd(const void* x, const void* WgT, const void* bg, const void* WuT, const void* Wd, int T,
                             int d, int F, const TwellView& h, void* ws, void* y, int out_dt, hipStream_t s,
                             hipEvent_t ev_gate, hipEvent_t ev_lists, hipEvent_t ev_up) {
  if (T == 0) return hipSuccess;
  DecArgs a = dec_args(x, WgT, bg, WuT, Wd, T, d, F, y, out_dt);
  char* w = (char*)ws;
  a.pg = (float*)w; w += r256((size_t)KS_GATE * T * F * 4);
  a.aval = (float*)w;
  a.cnt = h.cnt; a.width = h.width; a.hval = (float*)h.val; a.hidx = h.idx; a.hmask = h.mask;
  const int mt = (T + 63) / 64;
  hipLaunchKernelGGL(dec_gate_kernel, dim3(F / 64, KS_GATE, mt), dim3(SplitCfg::NTH), 0, s, a);
  const int NR = (T + 15) / 16;
  const unsigned ntile = (unsigned)((int64_t)NR * a.NT);
  if (ev_gate) (void)hipEventRecord(ev_gate, s);
  if (ev_lists) (void)hipEventRecord(ev_lists, s);     // no union lists on this path
  if (d <= 1024) hipLaunchKernelGGL(dec_pack_up_kernel<2>, dim3(ntile), dim3(64 * PU_WAVES), 0, s, a);
  else if (d <= 2048) hipLaunchKernelGGL(dec_pack_up_kernel<4>, dim3(ntile), dim3(64 * PU_WAVES), 0, s, a);
  else if (d <= 2560) hipLaunchKernelGGL(dec_pack_up_kernel<5>, dim3(ntile), dim3(64 * PU_WAVES), 0, s, a);
  else hipLaunchKernelGGL(dec_pack_up_kernel<8>, dim3(ntile), dim3(64 * PU_WAVES), 0, s, a);
  if (ev_up) (void)hipEventRecord(ev_up, s);
  hipLaunchKernelGGL(dec_down_kernel, dim3((unsigned)((d + 255) / 256), (unsigned)T), dim3(256), 0, s, a);
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
  launch_down_reduce(a, s);
  return hipGetLastError();
}

}  // namespace twell
