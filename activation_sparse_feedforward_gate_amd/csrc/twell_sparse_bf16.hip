// Sparse up- and down-projections for bf16 inputs, with workgroup-shared
// weight staging.
//
// Same computation as the generic kernels (intellectnews.ru TwELL article,
// section "Слитые CUDA-ядра для инференса и гибрид для обучения": after the
// gate, only active neurons are touched):
//   up   (SDDMM):  a[t,n] = h[t,n] * (x_t . WuT[n])  on the stored pairs
//                  backward: also da = dY_t . Wd[n]; a, dg = da*u, du = da*h
//   down (SpMM):   y_t = sum over stored n of a[t,n] * Wd[n]
//                  backward: dX_t = sum dg*WgT[n] + du*WuT[n]
//
// A workgroup owns 64 tokens (four 16-row TwELL row tiles, one per wave) and
// one slice of the neurons (up) or of the output columns (down).  Slices are
// assigned so that all workgroups of one slice run on one XCD (workgroup ids
// go round-robin over the 8 XCDs): the slice's weights, ~1-3 MB, stay in that
// XCD's L2 while every token group streams through it.
//
// For each 64-token group and each run of up to 16 column tiles, the union of
// the group's active neurons is laid out as "union positions": tile by tile,
// ascending column, each tile's count padded to a multiple of 8 (padding
// positions carry zero weights).  Each token's 64-bit tile mask is then
// re-expressed over the tile's union positions, so for a token and a union
// position both "is the pair stored?" and "which TwELL slot holds it?" are a
// bit test and a popcount (slots follow ascending column, as positions do).
//
// up:   the union rows of WuT (64 k at a time, one 128-byte row per position)
//       are staged in LDS and every wave multiplies its 16 tokens by them,
//       16 positions per 16x16x32 bf16 MFMA; the epilogue keeps stored pairs.
// down: the union rows of Wd (slice columns only, 32 positions at a time) are
//       staged row-major in LDS and read into the MFMA B layout with the
//       gfx950 transpose load (ds_read_b64_tr_b16); the A operand is each
//       token's a values at those positions (zero where not stored), fp32
//       split into bf16 hi + lo, fetched one step ahead.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace twell {

namespace {

constexpr int GW = 4;                 // waves (16-token row tiles) per workgroup
constexpr int GT = 16 * GW;           // tokens per workgroup
constexpr int CT = 16;                // column tiles per union chunk
constexpr int MAXPOS = CT * 64;       // padded union positions per chunk (max)
constexpr int UP_CAP = 256;           // union positions staged per pass (up)
constexpr int DN_KC = 32;             // union positions per K step (down)
constexpr int DN_MAXCB = 18;          // 16-column blocks per output slice (down)
constexpr int DN_PITCH_MAX = (DN_MAXCB * 32 + 127) / 128 * 128 + 32;   // bytes per staged row (down)
constexpr int DN_LD = (DN_KC * DN_MAXCB * 2 + 255) / 256;              // 16-byte loads per thread per K step

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

struct SpArgs {
  const uint16_t* x;    // up: x [T][d]
  const uint16_t* x2;   // up, backward: dY [T][d]
  const uint16_t* W;    // up: WuT; down: Wd (forward) or WgT (backward)
  const uint16_t* W2;   // up, backward: Wd; down, backward: WuT
  int T, d, F, NT, NR;
  const uint64_t* mask; // [T][NT]
  const uint8_t* skip;  // [T] or null
  const float* hval;    // up: h values (TwELL layout)
  float* v0;            // up: out a;   down: in a (forward) or dg (backward)
  float* v1;            // up backward: out dg;   down backward: in du
  float* v2;            // up backward: out du
  void* y;              // down: out [T][d]
  int out_bf16;
  int S;                // slices
  int ngroups;          // ceil(NR / GW)
  int nvb;              // virtual workgroups: ngroups * S (a grid may be smaller and loop over them)
  const int* gate;      // null, or a device flag: the kernel runs only if it is non-zero
  float l1;             // up backward: added to dg on every stored pair (activation penalty)
  int cap;              // slots per TwELL tile of the value arrays
};

// Virtual workgroup vb -> (token group g, slice s).  With S a multiple of 8,
// slice s runs on XCD s % 8 (ids go round-robin over the XCDs, and a grid
// that loops over the virtual workgroups has a multiple of 8 workgroups),
// phase by phase.
__device__ __forceinline__ void group_and_slice(const SpArgs& a, int vb, int& g, int& s) {
  if ((a.S & 7) == 0) {
    const int per_phase = a.ngroups * 8;
    const int phase = vb / per_phase;
    const int r = vb - phase * per_phase;
    g = r >> 3;
    s = phase * 8 + (r & 7);
  } else {
    g = vb / a.S;
    s = vb - g * a.S;
  }
}

__device__ __forceinline__ int excl_scan64(int v, int lane, int* total) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  *total = __shfl(incl, 63);
  return incl - v;
}

__device__ __forceinline__ bool live_row(const SpArgs& a, int t) {
  return t < a.T && !(a.skip && a.skip[t]);
}

// Union positions of one 64-token group over column tiles [jt0, jt0 + ntl).
struct UnionLds {
  uint64_t pm[GT][CT];       // token masks, then re-expressed over union positions
  uint64_t wu[GW][CT];       // per-wave partial unions
  uint64_t su[CT];           // group union per tile
  int base[CT + 1];          // first union position of each tile; base[CT] = total
  uint8_t gtile[MAXPOS / 8]; // tile of each group of 8 positions
  uint16_t pos_n[MAXPOS];    // neuron of each position (0xFFFF: padding)
};

__device__ void build_union(const SpArgs& a, UnionLds& L, int t0, int jt0, int ntl) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int q = tid; q < GT * CT; q += 256) {
    const int r = q / CT, jj = q % CT;
    const int t = t0 + r;
    L.pm[r][jj] = (jj < ntl && live_row(a, t)) ? a.mask[(int64_t)t * a.NT + jt0 + jj] : 0ull;
  }
  __syncthreads();
  if (lane < CT) {
    uint64_t u = 0;
#pragma unroll 4
    for (int r = 0; r < 16; ++r) u |= L.pm[w * 16 + r][lane];
    L.wu[w][lane] = u;
  }
  __syncthreads();
  if (w == 0) {
    const uint64_t U = lane < CT ? (L.wu[0][lane] | L.wu[1][lane] | L.wu[2][lane] | L.wu[3][lane]) : 0ull;
    const int pc = (popc64(U) + 7) & ~7;
    int tot;
    const int p = excl_scan64(pc, lane, &tot);
    if (lane <= CT) L.base[lane] = p;
    if (lane < CT) {
      L.su[lane] = U;
      int k = p;
      for (uint64_t m = U; m; m &= m - 1) L.pos_n[k++] = (uint16_t)((jt0 + lane) * 64 + __ffsll((long long)m) - 1);
      for (; k < p + pc; ++k) L.pos_n[k] = 0xFFFF;
      for (int g8 = p >> 3; g8 < (p + pc) >> 3; ++g8) L.gtile[g8] = (uint8_t)lane;
    }
  }
  __syncthreads();
  for (int q = tid; q < GT * CT; q += 256) {
    const int r = q / CT, jj = q % CT;
    const uint64_t M = L.pm[r][jj];
    if (M) {
      const uint64_t U = L.su[jj];
      uint64_t P = 0;
      for (uint64_t m = M; m; m &= m - 1) P |= 1ull << popc64(U & below(__ffsll((long long)m) - 1));
      L.pm[r][jj] = P;
    }
  }
  __syncthreads();
}

}  // namespace

// ------------------------------------------------------------------ up

struct UpCtx {
  const uint16_t* xr;   // my A-fragment row of x (already offset by my k-group)
  const uint16_t* yr;   // same row of dY (backward)
  int64_t rt;           // my TwELL row tile
  int j0;               // first column tile of the slice
};

// One pass over union positions [pb, pb + 16*NB): stage their WuT (and Wd)
// rows 64 k at a time, multiply, keep the stored pairs.  NB is a compile-time
// block count so the MFMA loop is branch-free.
template <int NB, int NP>
__device__ __forceinline__ void up_pass(const SpArgs& a, const UnionLds& L, char (*sw)[UP_CAP * 128],
                                        const UpCtx& c, int pb, int total) {
  constexpr int ROWS = NB * 16;
  constexpr int LDI = (ROWS * 8 + 255) / 256;   // 16-byte loads per thread per chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  uint4 pre0[LDI], pre1[NP == 2 ? LDI : 1];
  uint32_t woff[LDI];
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < LDI; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3;
    const int p = pb + row;
    const int n = (row < ROWS && p < total) ? L.pos_n[p] : 0xFFFF;
    woff[i] = n == 0xFFFF ? 0u : (uint32_t)n * (uint32_t)a.d + (uint32_t)(q & 7) * 8u;
    if (n != 0xFFFF) live |= 1u << i;
  }
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LDI; ++i) {
      pre0[i] = make_uint4(0, 0, 0, 0);
      if constexpr (NP == 2) pre1[i] = make_uint4(0, 0, 0, 0);
      if ((live >> i) & 1u) {
        pre0[i] = *(const uint4*)(a.W + woff[i] + k0);
        if constexpr (NP == 2) pre1[i] = *(const uint4*)(a.W2 + woff[i] + k0);
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < LDI; ++i) {
      const int q = tid + 256 * i;
      if (q < ROWS * 8) {
        // two 8-byte stores per chunk: fewer bank conflicts in this swizzle
        // than one 16-byte store
        const int o = swz(q >> 3, q & 7);
        *(uint2*)(sw[0] + o) = make_uint2(pre0[i].x, pre0[i].y);
        *(uint2*)(sw[0] + o + 8) = make_uint2(pre0[i].z, pre0[i].w);
        if constexpr (NP == 2) {
          *(uint2*)(sw[1] + o) = make_uint2(pre1[i].x, pre1[i].y);
          *(uint2*)(sw[1] + o + 8) = make_uint2(pre1[i].z, pre1[i].w);
        }
      }
    }
  };

  f32x4 acc[NB], acc2[NP == 2 ? NB : 1];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (NP == 2) {
#pragma unroll
    for (int b = 0; b < NB; ++b) acc2[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  load_chunk(0);
  uint4 xf[2], yf[2];
  xf[0] = *(const uint4*)(c.xr);
  xf[1] = *(const uint4*)(c.xr + 32);
  if constexpr (NP == 2) {
    yf[0] = *(const uint4*)(c.yr);
    yf[1] = *(const uint4*)(c.yr + 32);
  }
  __syncthreads();            // previous pass's readers of sw are done
  store_chunk();
  __syncthreads();
  for (int k0 = 0; k0 < a.d; k0 += 64) {
    const bool more = k0 + 64 < a.d;
    uint4 xn[2], yn[2];
    if (more) {
      load_chunk(k0 + 64);
      xn[0] = *(const uint4*)(c.xr + k0 + 64);
      xn[1] = *(const uint4*)(c.xr + k0 + 96);
      if constexpr (NP == 2) {
        yn[0] = *(const uint4*)(c.yr + k0 + 64);
        yn[1] = *(const uint4*)(c.yr + k0 + 96);
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int ch = st * 4 + (lane >> 4);
      uint4 bf[NB], bd[NP == 2 ? NB : 1];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        bf[b] = *(const uint4*)(sw[0] + swz(b * 16 + (lane & 15), ch));
        if constexpr (NP == 2) bd[b] = *(const uint4*)(sw[1] + swz(b * 16 + (lane & 15), ch));
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b] = mfma16(xf[st], bf[b], acc[b]);
        if constexpr (NP == 2) acc2[b] = mfma16(yf[st], bd[b], acc2[b]);
      }
    }
    __syncthreads();
    if (more) {
      store_chunk();
      xf[0] = xn[0];
      xf[1] = xn[1];
      if constexpr (NP == 2) {
        yf[0] = yn[0];
        yf[1] = yn[1];
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane>>4)+i at union position pb + 16b + (lane&15)
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int p = pb + b * 16 + (lane & 15);
    if (p < total && L.pos_n[p] != 0xFFFF) {
      const int jj = L.gtile[p >> 3];
      const int qp = p - L.base[jj];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mfma16_row(lane, i);
        const uint64_t P = L.pm[w * 16 + r][jj];
        if ((P >> qp) & 1ull) {
          const int slot = popc64(P & below(qp));
          const int64_t off = (c.rt * a.NT + (c.j0 + jj)) * (a.cap * 16) + slot * 16 + r;
          const float h = a.hval[off];
          const float u = acc[b][i];
          a.v0[off] = h * u;
          if constexpr (NP == 2) {
            const float da = acc2[b][i];
            a.v1[off] = da * u + a.l1;
            a.v2[off] = da * h;
          }
        }
      }
    }
  }
}

template <int NP>
__device__ __forceinline__ void up_bf16_block(const SpArgs& a, int vb, UnionLds& L,
                                              char (*sw)[UP_CAP * 128]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int g, s;
  group_and_slice(a, vb, g, s);
  const int j0 = (int)((int64_t)s * a.NT / a.S), j1 = (int)((int64_t)(s + 1) * a.NT / a.S);
  const int t0 = g * GT;
  build_union(a, L, t0, j0, j1 - j0);
  const int total = L.base[CT];
  if (total == 0) return;   // uniform over the workgroup

  // my token row for the A fragments (rows past T read row T-1; never stored)
  const int trow = min(t0 + w * 16 + (lane & 15), a.T - 1);
  UpCtx c;
  c.xr = a.x + (int64_t)trow * a.d + (lane >> 4) * 8;
  c.yr = NP == 2 ? a.x2 + (int64_t)trow * a.d + (lane >> 4) * 8 : nullptr;
  c.rt = (int64_t)g * GW + w;
  c.j0 = j0;
  // passes of 256, 128, 64, 32, 16 positions: the last one pads < 16 rows
  int pb = 0;
  while (pb < total) {
    const int rem = total - pb;
    if (rem >= 256) { up_pass<16, NP>(a, L, sw, c, pb, total); pb += 256; }
    else if (rem >= 128) { up_pass<8, NP>(a, L, sw, c, pb, total); pb += 128; }
    else if (rem >= 64) { up_pass<4, NP>(a, L, sw, c, pb, total); pb += 64; }
    else if (rem >= 32) { up_pass<2, NP>(a, L, sw, c, pb, total); pb += 32; }
    else { up_pass<1, NP>(a, L, sw, c, pb, total); pb += 16; }
  }
}

template <int NP>
__global__ __launch_bounds__(256) void up_bf16_kernel(SpArgs a) {
  __shared__ UnionLds L;
  __shared__ __attribute__((aligned(16))) char sw[NP][UP_CAP * 128];
  if (a.gate && *a.gate == 0) return;
  for (int vb = blockIdx.x; vb < a.nvb; vb += gridDim.x) {
    up_bf16_block<NP>(a, vb, L, sw);
    __syncthreads();                                 // LDS free for the next virtual workgroup
  }
}

// ------------------------------------------------------------------ down

template <int NV, int NCB>
__device__ __forceinline__ void down_bf16_block(const SpArgs& a, int vb, UnionLds& L,
                                                char (*sb)[DN_KC * DN_PITCH_MAX]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int g, s;
  group_and_slice(a, vb, g, s);
  constexpr int ncb = NCB;                       // every slice has NCB 16-column blocks
  const int c0 = s * NCB * 16, ncol = NCB * 16;
  const int pitch = (ncol * 2 + 127) / 128 * 128 + 32;   // row pitch: rows 32 bytes apart mod 128
  const int nch = ncol / 8;                              // 16-byte chunks per staged row
  const int t0 = g * GT;
  const int64_t rt = (int64_t)g * GW + w;
  const int ra = lane & 15;                              // my A-fragment token row
  const int kg = lane >> 4;                              // my 8-position group in a K step
  // transpose-load addresses (bytes) of my B fragment, column block 0
  const int tr0 = (8 * kg + (ra >> 2)) * pitch + 8 * (ra & 3);

  f32x4 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int jc = 0; jc < a.NT; jc += CT) {
    __syncthreads();                                     // previous chunk's readers are done
    build_union(a, L, t0, jc, min(CT, a.NT - jc));
    const int total = L.base[CT];
    if (total == 0) continue;                            // uniform

    uint4 pre0[DN_LD], pre1[NV == 2 ? DN_LD : 1];
    auto load_chunk = [&](int kc) {
#pragma unroll
      for (int i = 0; i < DN_LD; ++i) {
        const int q = tid + 256 * i;
        pre0[i] = make_uint4(0, 0, 0, 0);
        if constexpr (NV == 2) pre1[i] = make_uint4(0, 0, 0, 0);
        if (q < DN_KC * nch) {
          const int row = q / nch, cc = q - row * nch;
          const int p = kc + row;
          const int n = p < total ? L.pos_n[p] : 0xFFFF;
          if (n != 0xFFFF) {
            const int64_t o = (int64_t)n * a.d + c0 + cc * 8;
            pre0[i] = *(const uint4*)(a.W + o);
            if constexpr (NV == 2) pre1[i] = *(const uint4*)(a.W2 + o);
          }
        }
      }
    };
    auto store_chunk = [&]() {
#pragma unroll
      for (int i = 0; i < DN_LD; ++i) {
        const int q = tid + 256 * i;
        if (q < DN_KC * nch) {
          const int row = q / nch, cc = q - row * nch;
          *(uint4*)(sb[0] + row * pitch + cc * 16) = pre0[i];
          if constexpr (NV == 2) *(uint4*)(sb[1] + row * pitch + cc * 16) = pre1[i];
        }
      }
    };
    // a values of my token at positions kc + 8*kg + e (zero where not stored)
    float araw[NV][8];
    auto fetch_a = [&](int kc) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) araw[v][e] = 0.f;
      const int p0 = kc + 8 * kg;
      if (p0 < total) {
        const int jj = L.gtile[p0 >> 3];
        const int q0 = p0 - L.base[jj];
        const uint64_t P = L.pm[w * 16 + ra][jj];
        const uint32_t bits = (uint32_t)(P >> q0) & 0xFFu;
        if (bits) {
          const int64_t tb = (rt * a.NT + (jc + jj)) * (a.cap * 16) + ra;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if ((bits >> e) & 1u) {
              const int slot = popc64(P & below(q0 + e));
              araw[0][e] = a.v0[tb + slot * 16];
              if constexpr (NV == 2) araw[1][e] = a.v1[tb + slot * 16];
            }
          }
        }
      }
    };

    load_chunk(0);
    fetch_a(0);
    for (int kc = 0; kc < total; kc += DN_KC) {
      uint4 Ahi[NV], Alo[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split_bf16(araw[v][e], hi[e], lo[e]);
        Ahi[v] = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
        Alo[v] = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
      }
      __syncthreads();
      store_chunk();
      __syncthreads();
      if (kc + DN_KC < total) {
        load_chunk(kc + DN_KC);
        fetch_a(kc + DN_KC);
      }
      uint4 B[NV][NCB];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          lds_char* base = (lds_char*)(sb[v]) + tr0 + cb * 32;
          const v4i16 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)base);
          const v4i16 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + 4 * pitch));
          const uint2 u0 = __builtin_bit_cast(uint2, b0), u1 = __builtin_bit_cast(uint2, b1);
          B[v][cb] = make_uint4(u0.x, u0.y, u1.x, u1.y);
        }
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          acc[cb] = mfma16(Ahi[v], B[v][cb], acc[cb]);
          acc[cb] = mfma16(Alo[v], B[v][cb], acc[cb]);
        }
    }
  }

#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int col = c0 + cb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + w * 16 + mfma16_row(lane, i);
      if (live_row(a, t)) {
        if (a.out_bf16) ((uint16_t*)a.y)[(int64_t)t * a.d + col] = (uint16_t)f32_to_bf16_bits(acc[cb][i]);
        else ((float*)a.y)[(int64_t)t * a.d + col] = acc[cb][i];
      }
    }
  }
}

template <int NV, int NCB>
__global__ __launch_bounds__(256) void down_bf16_kernel(SpArgs a) {
  __shared__ UnionLds L;
  __shared__ __attribute__((aligned(16))) char sb[NV][DN_KC * DN_PITCH_MAX];
  if (a.gate && *a.gate == 0) return;
  for (int vb = blockIdx.x; vb < a.nvb; vb += gridDim.x) {
    down_bf16_block<NV, NCB>(a, vb, L, sb);
    __syncthreads();                                 // LDS free for the next virtual workgroup
  }
}

// ------------------------------------------------------------------ launchers

namespace {

// Slices: a multiple of 8 (one per XCD per phase), enough that one slice's
// weights (bytes_per_unit * units / S) stay within ~3 MB of L2, that no slice
// has more than max_units, and that small batches still fill the chip.
// Grid of a launch over nvb virtual workgroups.  A launch gated by a device
// flag (a fallback that is almost never taken) gets one workgroup per CU,
// rounded down to a multiple of 8 so that slices keep their XCD, and the
// workgroups loop over the virtual ones: when the flag is clear the launch
// costs one short wave of workgroups instead of the full grid.
int gated_grid(int nvb, const int* gate) {
  if (!gate) return nvb;
  const int g = std::max(8, device_cus() / 8 * 8);
  return std::min(nvb, g);
}

int pick_slices(int units, int max_units, double bytes_per_unit, int ngroups) {
  int S = 8;
  auto ok = [&](int s) {
    return (units + s - 1) / s <= max_units && bytes_per_unit * units / s <= 3.0 * 1024 * 1024;
  };
  while (!ok(S) && S < units) S += 8;
  while (ngroups * S < 512 && S + 8 <= units) S += 8;
  return S;
}

}  // namespace

hipError_t launch_up_bf16(const void* x, const void* dY, const void* WuT, const void* Wd, int T, int d, int F,
                          const TwellView& h, float* aval, float* dgval, float* duval, const uint8_t* skip,
                          hipStream_t s, const int* gate, float l1) {
  if ((int64_t)F * d >= ((int64_t)1 << 32)) return hipErrorInvalidValue;   // 32-bit weight offsets
  SpArgs a{};
  a.x = (const uint16_t*)x; a.x2 = (const uint16_t*)dY; a.W = (const uint16_t*)WuT; a.W2 = (const uint16_t*)Wd;
  a.T = T; a.d = d; a.F = F; a.NT = F / 64; a.NR = (T + 15) / 16;
  a.mask = h.mask; a.skip = skip; a.hval = (const float*)h.val; a.v0 = aval; a.v1 = dgval; a.v2 = duval;
  a.cap = h.cap;
  a.gate = gate;
  a.l1 = l1;
  if (a.NR == 0) return hipSuccess;
  a.ngroups = (a.NR + GW - 1) / GW;
  const int NP = dY ? 2 : 1;
  a.S = pick_slices(a.NT, CT, 64.0 * d * 2 * NP, a.ngroups);
  if ((a.NT + a.S - 1) / a.S > CT) return hipErrorInvalidValue;
  a.nvb = a.ngroups * a.S;
  const int grid = gated_grid(a.nvb, gate);
  if (NP == 2) hipLaunchKernelGGL(up_bf16_kernel<2>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(up_bf16_kernel<1>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NV>
static void launch_down_ncb(int ncb, dim3 grid, const SpArgs& a, hipStream_t s) {
  switch (ncb) {
#define TWELL_DN_CASE(K) \
    case K: hipLaunchKernelGGL((down_bf16_kernel<NV, K>), grid, dim3(256), 0, s, a); break;
    TWELL_DN_CASE(1) TWELL_DN_CASE(2) TWELL_DN_CASE(3) TWELL_DN_CASE(4) TWELL_DN_CASE(5) TWELL_DN_CASE(6)
    TWELL_DN_CASE(7) TWELL_DN_CASE(8) TWELL_DN_CASE(9) TWELL_DN_CASE(10) TWELL_DN_CASE(11) TWELL_DN_CASE(12)
    TWELL_DN_CASE(13) TWELL_DN_CASE(14) TWELL_DN_CASE(15) TWELL_DN_CASE(16) TWELL_DN_CASE(17) TWELL_DN_CASE(18)
#undef TWELL_DN_CASE
    default: break;
  }
}

hipError_t launch_down_bf16(const float* v0, const float* v1, const void* W, const void* W2, int T, int d, int F,
                            const TwellView& pat, void* y, int out_dt, const uint8_t* skip, hipStream_t s,
                            const int* gate) {
  SpArgs a{};
  a.W = (const uint16_t*)W; a.W2 = (const uint16_t*)W2;
  a.T = T; a.d = d; a.F = F; a.NT = F / 64; a.NR = (T + 15) / 16;
  a.mask = pat.mask; a.skip = skip; a.v0 = (float*)v0; a.v1 = (float*)v1; a.y = y; a.out_bf16 = out_dt == DT_BF16;
  a.cap = pat.cap;
  a.gate = gate;
  if (a.NR == 0) return hipSuccess;
  a.ngroups = (a.NR + GW - 1) / GW;
  const int NV = v1 ? 2 : 1;
  // Slices split the d/16 column blocks evenly, each at most DN_MAXCB blocks:
  // preferably S = 8P (one slice per XCD per phase) with the slice's Wd
  // columns within ~3 MB of L2 and enough workgroups to fill the chip,
  // otherwise the smallest divisor of d/16 that fits.
  const int ncb_all = d / 16;
  int S = 0;
  for (int P = 1; 8 * P <= ncb_all; ++P) {
    if (ncb_all % (8 * P)) continue;
    const int k = ncb_all / (8 * P);
    if (k > DN_MAXCB || 2.0 * F * 16 * k * NV > 3.0 * 1024 * 1024) continue;
    S = 8 * P;
    if (a.ngroups * S >= 512) break;
  }
  if (S == 0)
    for (int c = 1; c <= ncb_all && S == 0; ++c)
      if (ncb_all % c == 0 && ncb_all / c <= DN_MAXCB) S = c;
  a.S = S;
  a.nvb = a.ngroups * S;
  const dim3 grid(gated_grid(a.nvb, gate));
  if (NV == 2) launch_down_ncb<2>(ncb_all / S, grid, a, s);
  else launch_down_ncb<1>(ncb_all / S, grid, a, s);
  return hipGetLastError();
}

}  // namespace twell
