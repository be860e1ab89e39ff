// Forward sparse phases as GEMMs over each row block's union of active
// neurons.
//
// After the gate GEMM has packed h = ReLU(x.Wg + b) into TwELL
// (intellectnews.ru TwELL article, section "Формат TwELL вместо классической
// sparse-упаковки"), the up- and down-projections only need the neurons that
// fire (section "Слитые CUDA-ядра для инференса и гибрид для обучения").  For
// a block of 128 tokens the set of neurons that fire in ANY of them (the
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
// 1e-3 output budget); if any |a| (or a weight of Wd) exceeds the fp16 range a
// device flag makes the down kernel compute y per stored pair in fp32 instead.
//
// The TwELL of h may hold fewer than 64 slots per tile (hcap), and adense may
// hold fewer than F positions per row (ucap).  With block flags (bounded
// forward), a block whose tiles are wider than hcap but whose union fits
// takes h from a gate GEMM over its union (up_union_rec_kernel) instead of
// its incomplete TwELL; a block whose union is longer than ucap skips the
// GEMMs and the down kernel computes it per stored pair, with h recomputed.
#include <algorithm>

#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

namespace {

// Tokens per row block.  Smaller blocks give smaller unions (less executed
// work) but smaller GEMM tiles: 128 rows measured faster than 256 overall at
// T = 32768 with d = 2048, F = 5632 (1.5% density) and d = 2304, F = 9216
// (0.93%): union fractions 42% / 26% against 58% / 38%, tile throughput about
// 10% lower.
constexpr int UB = 128;
constexpr int RT = UB / 16;            // TwELL row tiles per row block

struct UnionArgs {
  const void* x;
  const void* WuT;
  const void* Wd;
  const _Float16* Wd16;   // fp16 copy of Wd for the down GEMM
  int T, d, F, NT;
  const uint64_t* mask;   // [T][NT]
  const uint8_t* skip;    // [T] or null
  const float* hval;      // TwELL values of h
  const uint8_t* hidx;    // TwELL column indices of h
  const uint8_t* hwidth;  // TwELL widths of h
  int* ulist;             // [NBLK][F]
  int* ucount;            // [NBLK]
  int lrows;              // rows per list block: UB, or every row (one list) for the few-token path
  _Float16* adense;       // [T][F], then spare slots
  uint32_t spare;         // element index of a spare slot (T*F)
  int* flag;              // fp16 overflow flag
  void* y;
  int out_bf16;
  // backward SDDMM over the union
  const void* dY;         // [T][d]
  float* aval;            // TwELL-shaped outputs: a = h*u, dg = da*u + l1, du = da*h
  float* dgval;
  float* duval;
  float l1;
  _Float16* dU16;         // backward: dU over the union positions (dG goes to adense)
  const _Float16* Wu16;   // backward: fp16 copy of WuT (WgT's goes to Wd16)
  // capacity-bounded forward
  int hcap;               // slots per TwELL tile of h (64: the full form)
  int ucap;               // row stride of adense: union positions a block may hold
  uint8_t* bflag;         // [NBLK] or null: 1 if block b's TwELL tiles exceed hcap (its union fits
                          // ucap), 2 if its union exceeds ucap, else 0
  const void* WgT;        // gate weights and bias, to recompute h for such blocks
  const void* bg;
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
// per-tile popcounts, then each wave writes whole tiles, one set bit per lane.
__device__ __forceinline__ void union_list_block(const UnionArgs& a, const uint64_t* U, int b, int* scan,
                                                 int* start, uint64_t* su) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int base = 0;
  bool over = false;
  int* ul = a.ulist + (int64_t)b * a.F;
  const int s0 = b * (a.lrows / 64), s1 = min((a.T + 63) / 64, s0 + a.lrows / 64);
  for (int j0 = 0; j0 < a.NT; j0 += 256) {
    const int j = j0 + tid;
    uint64_t u = 0;
    if (j < a.NT)
      for (int sl = s0; sl < s1; ++sl) u |= U[(int64_t)sl * a.NT + j];
    const int c = popc64(u);
    scan[tid] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int v = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    start[tid] = base + scan[tid] - c;
    su[tid] = u;
    if (a.bflag && j < a.NT) {
      // a tile of the block's rows wider than the TwELL capacity
      const int r0 = b * (a.lrows / 16), r1 = min((a.T + 15) / 16, r0 + a.lrows / 16);
      for (int r = r0; r < r1; ++r) over |= (int)a.hwidth[(int64_t)r * a.NT + j] > a.hcap;
    }
    const int total = scan[255];
    __syncthreads();
    const int nj = min(256, a.NT - j0);
    for (int jj = w; jj < nj; jj += 4) {
      const uint64_t m = su[jj];
      if ((m >> lane) & 1ull) ul[start[jj] + popc64(m & below(lane))] = (j0 + jj) * 64 + lane;
    }
    base += total;
    __syncthreads();                                   // scan, start and su are rewritten next
  }
  if (tid == 0) a.ucount[b] = base;
  if (a.bflag) {
    // or a union longer than adense's rows hold
    const int ov = __syncthreads_or((int)over);
    if (tid == 0) a.bflag[b] = (uint8_t)(base > a.ucap ? 2 : ov ? 1 : 0);
  }
}

__global__ __launch_bounds__(256) void union_list_kernel(UnionArgs a, const uint64_t* U) {
  __shared__ int scan[256], start[256];
  __shared__ uint64_t su[256];
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.flag = 0;
  union_list_block(a, U, blockIdx.x, scan, start, su);
}

constexpr int POSCAP = 12288;         // neuron span of a position tile covered by the LDS position map

// Up-projection over the union, one (row block b, position tile pt) tile.
// GATED = false: the non-gated ReLU FFN, a = h (no up GEMM; the tile only
// lays h out over the union positions for the down GEMM).
template <class Cfg, bool GATED>
__device__ __forceinline__ void up_union_tile(const UnionArgs& a, int b, int pt, char* st0, char* st1,
                                              int16_t* posmap, int* lcount, uint8_t* wl) {
  static_assert(Cfg::BM == UB, "one row block per M tile");
  const int nb = a.ucount[b];
  const int p0 = pt * Cfg::BN;
  if (p0 >= nb) return;
  if (a.bflag && a.bflag[b]) return;       // over capacity: up_union_rec_kernel or the down kernel
  const int m0 = b * UB;
  const int* ul = a.ulist + (int64_t)b * a.F;
  const int64_t hs = (int64_t)a.hcap * 16; // TwELL tile stride of h

  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B{a.WuT, a.d, ul, nb};

  // epilogue set-up, issued before the mainloop so that its global reads
  // (the position map, and with two stage buffers the first TwELL pieces)
  // complete under the MFMAs: see the epilogue below
  static_assert(Cfg::BN == 256 && Cfg::NW == 8 && Cfg::BM % 128 == 0 && Cfg::BM <= 256, "epilogue layout");
  static_assert(Cfg::STAGE >= 128 * 2 * Cfg::BM, "h tile: 128 positions x BM rows of fp16 per stage buffer");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int pl = min(p0 + Cfg::BN, nb) - 1;
  const int nlo = ul[p0], nhi = ul[pl];
  const bool use_map = nhi - nlo < POSCAP;
  const int tjf = nlo >> 6, S = (nhi >> 6) - tjf + 1;
  constexpr int NRT0 = Cfg::BM / 16;
  // the TwELL widths of the blocks in the span go to LDS with the position
  // map (both wait for their loads here, before the mainloop), so the scan
  // below starts without a dependent load
  const bool wpre = NRT0 * S <= Cfg::NTH;
  {
    int wv = 0;
    const int i = tid / S, sj = tid - (tid / S) * S;
    if (wpre && tid < NRT0 * S && ((m0 >> 4) + i) * 16 < a.T) wv = a.hwidth[(int64_t)((m0 >> 4) + i) * a.NT + tjf + sj];
    if (use_map)
      for (int p = p0 + tid; p <= pl; p += Cfg::NTH) posmap[ul[p] - nlo] = (int16_t)(p - p0);
    if (wpre && tid < NRT0 * S) wl[tid] = (uint8_t)wv;
  }
  constexpr int NG = Cfg::NTH / 16;        // 16-lane groups
  // blocks per group fetched ahead (none with one stage buffer: the other
  // workgroup on the CU covers the latency, and the registers are needed)
  constexpr int NPRE = Cfg::SINGLE ? 0 : 4;
  const int grp = tid >> 4, gl = tid & 15;
  // first piece (slots 0-3) of the group's first NPRE (row tile, column tile)
  // blocks, read before the width is known: only for tiles of at least 4
  // slots, so the kernels that may see a smaller TwELL capacity are the
  // single-stage ones, which read nothing ahead (checked where they launch)
  constexpr int NRT = Cfg::BM / 16;        // TwELL row tiles of the block
  struct Piece { int w; float4 v; uint32_t i; };
  Piece pre[NPRE > 0 ? NPRE : 1];
#pragma unroll
  for (int it = 0; it < NPRE; ++it) {
    const int q = grp + it * NG;
    Piece& pc = pre[it];
    pc.w = 0;
    pc.v = make_float4(0.f, 0.f, 0.f, 0.f);
    pc.i = 0;
    if (q < NRT * S) {
      const int i = q / S, sj = q - i * S;
      const int rt = (m0 >> 4) + i;
      if (rt * 16 < a.T) {
        const int64_t blk = (int64_t)rt * a.NT + tjf + sj;
        pc.w = a.hwidth[blk];
        pc.v = ((const float4*)(a.hval + blk * hs))[gl];
        pc.i = ((const uint32_t*)(a.hidx + blk * hs))[gl];
      }
    }
  }

  if constexpr (GATED) g.run(A, &B, m0, p0, a.d, st0, st1);

  // epilogue: a = h * u on stored pairs, else 0, stored as fp16 into
  // adense[t][p] (32 consecutive positions per half-wave store).  Positions in
  // [n_b, roundup64(n_b)) are written as zeros (the down GEMM reads whole
  // 64-position K tiles).  h is brought to the accumulator layout through an
  // LDS tile of fp16 (positions 0-127 in st0, 128-255 in st1; 2*BM bytes of
  // rows per position, 8-byte pieces of 4 rows XOR-swizzled by position so a
  // half-wave's 32 consecutive positions hit distinct banks): the tile is
  // zeroed, every stored TwELL pair of the block whose neuron falls in this
  // tile's positions is written at (position, row) (position from posmap,
  // the inverse of the union list over the tile's neuron span), and every
  // wave reads its h values back 4 rows at a time.  h in fp16 adds one
  // rounding (2^-11 relative) before a is itself rounded to fp16.
  const int hl = lane >> 5;
  uint32_t vbits = 0;               // largest |a| bit pattern (NaN patterns sort above every number)
  auto hoff = [](int pr, int r) {
    const int pb = pr & 127;
    return pb * (2 * Cfg::BM) + (((r >> 2) ^ (pb & 31)) << 3) + ((r & 3) << 1);
  };
  // With one stage buffer the h tile is built and consumed in two passes of
  // 128 positions (32 KB each); with two, in one pass over both buffers.
  constexpr bool SPLIT = Cfg::SINGLE;
  constexpr int NPASS = SPLIT ? 2 : 1;
  auto hbuf_of = [&](int pr) -> char* { return (SPLIT || !(pr >> 7)) ? st0 : st1; };
  // Two passes: the pairs of the second half found while scanning for the
  // first are kept in a list in the buffer's last 16 KB (h-tile offset << 16
  // | fp16 bits), so the second pass replays the list instead of scanning the
  // TwELL again; only when the list overflows does it scan again.
  constexpr int LCAP = SPLIT ? (Cfg::STAGE - 128 * 2 * Cfg::BM) / 4 : 0;
  uint32_t* plist = (uint32_t*)(st0 + 128 * 2 * Cfg::BM);
  // scatter: a 16-lane group per (row tile, column tile) block; lane piece c
  // holds slot c/4, rows 4*(c%4)..+3 of the block
  auto scatter = [&](int hp, int i, int tj, int rt, int c, const float4& v4, uint32_t i4) {
    const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rl = 4 * (c & 3) + k;                     // row in the tile
      const int n = tj * 64 + (int)((i4 >> (8 * k)) & 255u);
      if (vv[k] > 0.f && n >= nlo && n <= nhi && live(a, rt * 16 + rl)) {
        int pr;
        if (use_map) {
          pr = posmap[n - nlo];
        } else {
          int lo = p0, hi = pl;                           // n is in the union: find its position
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (ul[mid] < n) lo = mid + 1; else hi = mid;
          }
          pr = lo - p0;
        }
        if (!SPLIT || (pr >> 7) == hp) {
          *(_Float16*)(hbuf_of(pr) + hoff(pr, i * 16 + rl)) = (_Float16)vv[k];
        } else if (hp == 0) {
          const int k2 = atomicAdd(lcount, 1);
          if (k2 < LCAP)
            plist[k2] = ((uint32_t)hoff(pr, i * 16 + rl) << 16) |
                        (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)vv[k]);
        }
      }
    }
  };
  const int wrow = (wave / Cfg::WN) * (Cfg::BM / Cfg::WM);
#pragma unroll
  for (int hp = 0; hp < NPASS; ++hp) {
#pragma unroll
    for (int o = 0; o < 128 * 2 * Cfg::BM / (16 * Cfg::NTH); ++o) {
      ((float4*)st0)[o * Cfg::NTH + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (!SPLIT) ((float4*)st1)[o * Cfg::NTH + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (SPLIT && hp == 0 && tid == 0) *lcount = 0;
    __syncthreads();
    const int nl = (SPLIT && hp == 1) ? *lcount : 0;
    if (SPLIT && hp == 1 && nl <= LCAP) {
      for (int k2 = tid; k2 < nl; k2 += Cfg::NTH) {
        const uint32_t e = plist[k2];
        *(uint16_t*)(st0 + (e >> 16)) = (uint16_t)(e & 0xffffu);
      }
    } else {
#pragma unroll
    for (int it = 0; it < NPRE; ++it) {
      const int q = grp + it * NG;
      if (q >= NRT * S) break;
      const int i = q / S, sj = q - i * S;
      const int rt = (m0 >> 4) + i;
      const Piece& pc = pre[it];
      if (gl < pc.w * 4) scatter(hp, i, tjf + sj, rt, gl, pc.v, pc.i);
      const int64_t blk = (int64_t)rt * a.NT + tjf + sj;
      for (int c = gl + 16; c < pc.w * 4; c += 16)
        scatter(hp, i, tjf + sj, rt, c, ((const float4*)(a.hval + blk * hs))[c],
                ((const uint32_t*)(a.hidx + blk * hs))[c]);
    }
    // (row tile i, column tile sj) of block q, stepped without a division
    int qi = (grp + NPRE * NG) / S, qs = grp + NPRE * NG - qi * S;
    for (int q = grp + NPRE * NG; q < NRT * S; q += NG) {
      const int i = qi, sj = qs;
      qs += NG;
      while (qs >= S) { qs -= S; ++qi; }
      const int rt = (m0 >> 4) + i;
      if (rt * 16 >= a.T) continue;
      const int64_t blk = (int64_t)rt * a.NT + tjf + sj;
      const int w = wpre ? (int)wl[q] : (int)a.hwidth[blk];
      for (int c = gl; c < w * 4; c += 16)
        scatter(hp, i, tjf + sj, rt, c, ((const float4*)(a.hval + blk * hs))[c],
                ((const uint32_t*)(a.hidx + blk * hs))[c]);
    }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int pr = Tile::col_of(j);
      if (SPLIT && (pr >> 7) != hp) continue;            // wave-uniform: the wave's columns lie in one half
      const int p = p0 + pr;
      const bool wr = p < ((nb + 63) & ~63);
      const char* hbuf = hbuf_of(pr);
#pragma unroll
      for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const uint2 h2 = *(const uint2*)(hbuf + hoff(pr, wrow + i * 32 + 8 * qq + 4 * hl));
          const float hv[4] = {(float)__builtin_bit_cast(_Float16, (uint16_t)(h2.x & 0xffffu)),
                               (float)__builtin_bit_cast(_Float16, (uint16_t)(h2.x >> 16)),
                               (float)__builtin_bit_cast(_Float16, (uint16_t)(h2.y & 0xffffu)),
                               (float)__builtin_bit_cast(_Float16, (uint16_t)(h2.y >> 16))};
          const int t0 = m0 + Tile::row_of(i, 4 * qq);
          float v[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if constexpr (GATED) v[k] = hv[k] != 0.f ? hv[k] * g.acc[0][i][j][4 * qq + k] : 0.f;
            else v[k] = hv[k];
            vbits = max(vbits, __float_as_uint(v[k]) & 0x7fffffffu);
          }
          // stores of position pairs: lanes l and l^1 hold positions p and
          // p^1 of the same rows; for rows k and k+1 the even lane stores
          // (its k, the odd lane's k) at p, the odd lane (the even lane's k+1,
          // its k+1) at p-1: one 4-byte store per two elements.  Element
          // offsets stay below 2^32 (the matrix holds fewer elements); pairs
          // that are not written go to the spare slot past the matrix, so the
          // stores need no branches.
          const bool odd = lane & 1;
#pragma unroll
          for (int k = 0; k < 4; k += 2) {
            const float send = odd ? v[k] : v[k + 1];
            const float recv = __shfl_xor(send, 1);
            const int kr = odd ? k + 1 : k;                   // row this lane stores
            const _Float16 lo = (_Float16)(odd ? recv : v[k]), hi = (_Float16)(odd ? v[k + 1] : recv);
            const uint32_t pair = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            const uint32_t keep = 0u - (uint32_t)(wr && t0 + kr < a.T);
            const uint32_t o = (((uint32_t)(t0 + kr) * (uint32_t)a.ucap + (uint32_t)(p & ~1)) & keep) | (a.spare & ~keep);
            *(uint32_t*)(a.adense + o) = pair;
          }
        }
    }
    if (SPLIT && hp + 1 < NPASS) __syncthreads();         // every wave done reading before the next pass
  }
  const bool over = vbits > 0x477fe000u;   // above 65504, the largest finite fp16
  if (__builtin_amdgcn_ballot_w64(over) != 0ull && lane == 0) atomicOr(a.flag, 1);
}

// Persistent workgroups (one per CU: the LDS holds one) walk the tiles, so a
// tile's output stores drain while the next tile's first loads are in
// flight.  XCD-aware order: workgroup ids go round-robin over the 8 XCDs; the
// workgroups of XCD x take the row blocks b = x (mod 8) and sweep them
// position tile by position tile, so the WuT rows of neighbouring blocks'
// unions (largely the same neurons) are reused from that XCD's L2 (measured
// faster than keeping each block's x rows in L2 instead).
template <class Cfg, bool GATED>
__global__ __launch_bounds__(Cfg::NTH, WavesPerEU<Cfg>::value) void up_union_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_[Cfg::SINGLE ? 16 : Cfg::STAGE];
  char* st1 = Cfg::SINGLE ? st0 : st1_;
  __shared__ int16_t posmap[POSCAP];
  __shared__ uint8_t wl[Cfg::NTH];                     // TwELL widths of the tile's blocks
  __shared__ int lcount;                               // pairs in the second-pass list
  const int npt = (a.F + Cfg::BN - 1) / Cfg::BN;
  const int nblk = (a.T + UB - 1) / UB;
  const int x = blockIdx.x & 7;
  const int nbx = (nblk - x + 7) / 8;                  // row blocks on this XCD
  const int ntile = nbx * npt;
  for (int k = blockIdx.x >> 3; k < ntile; k += gridDim.x >> 3) {
    const int pt = k / nbx;
    const int b = x + 8 * (k - pt * nbx);
    up_union_tile<Cfg, GATED>(a, b, pt, st0, st1, posmap, &lcount, wl);
    __syncthreads();                                   // stage buffers and position map free again
  }
}

// Up-projection of a block whose TwELL tiles are wider than the capacity
// while its union fits (bounded forward, block flag 1): the stored slots are
// incomplete, so h comes from the gate GEMM over the block's union, computed
// beside the up GEMM on one tile with two B operands (x loaded once):
// h = x_t . WgT[n] + bg[n] where the row's mask keeps (t, n), else 0, and
// a = fp16(h) * u written to adense as in the TwELL path (zeros in the
// positions [n_b, roundup64(n_b))).  About one more GEMM over the union for
// such a block; the down kernel then treats it like any other.  GATED =
// false: the non-gated layer, a = fp16(h) from the gate GEMM alone.
template <class Cfg, bool GATED>
__device__ __forceinline__ void up_rec_tile(const UnionArgs& a, int b, int pt, char* st) {
  static_assert(Cfg::BM == UB && Cfg::NB == (GATED ? 2 : 1), "one row block per M tile, gate (and up) products");
  const int nb = a.ucount[b];
  const int p0 = pt * Cfg::BN;
  if (p0 >= nb) return;
  const int m0 = b * UB;
  const int* ul = a.ulist + (int64_t)b * a.F;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B[2] = {{a.WgT, a.d, ul, nb}, {a.WuT, a.d, ul, nb}};
  g.run(A, B, m0, p0, a.d, st, st);                  // with one B operand only the first is read
  uint32_t vbits = 0;
  const int pend = (nb + 63) & ~63;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int p = p0 + Tile::col_of(j);
    if (p >= pend) continue;
    const bool inu = p < nb;
    const int n = inu ? ul[p] : 0;
    const float bias = (inu && a.bg) ? bf16_to_f32(((const uint16_t*)a.bg)[n]) : 0.f;
    const uint64_t bit = 1ull << (n & 63);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = m0 + Tile::row_of(i, e);
        if (t >= a.T) continue;
        float v = 0.f;
        if (inu && (a.mask[(int64_t)t * a.NT + (n >> 6)] & bit)) {
          const _Float16 h16 = (_Float16)(g.acc[0][i][j][e] + bias);
          v = GATED ? (float)h16 * g.acc[GATED ? 1 : 0][i][j][e] : (float)h16;
        }
        vbits = max(vbits, __float_as_uint(v) & 0x7fffffffu);
        a.adense[(int64_t)t * a.ucap + p] = (_Float16)v;
      }
  }
  const bool over = vbits > 0x477fe000u;   // above 65504, the largest finite fp16
  if (__builtin_amdgcn_ballot_w64(over) != 0ull && (threadIdx.x & 63) == 0) atomicOr(a.flag, 1);
}

template <class Cfg, bool GATED>
__global__ __launch_bounds__(Cfg::NTH, WavesPerEU<Cfg>::value) void up_union_rec_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(1024))) char st[Cfg::STAGE];
  const int npt = (a.F + Cfg::BN - 1) / Cfg::BN;
  const int ntile = ((a.T + UB - 1) / UB) * npt;
  for (int k = blockIdx.x; k < ntile; k += gridDim.x) {
    const int b = k / npt;
    if (a.bflag[b] != 1) continue;                     // workgroup-uniform
    up_rec_tile<Cfg, GATED>(a, b, k - b * npt, st);
    __syncthreads();                                   // the stage buffer is free again
  }
}

// Backward SDDMM of the hybrid format's sparse rows over the union, one
// (row block b, position tile pt) tile: U = x.WuT[ulist]^T and
// DA = dY.Wd[ulist]^T (two bf16 MFMA GEMMs, fp32 accumulation), then for
// every stored pair (t, n) of a live row in the tile: a = h*u, dg = da*u + l1,
// du = da*h at the pair's TwELL slot.  The products at the union's other
// positions are computed and dropped: at a uniform 1% density a 128-row
// block's union holds about 72% of the neurons, and the dense MFMA GEMMs over
// it run far faster than per-pair dot products.  The pairs reach the
// accumulator layout through an LDS tile of slot numbers (256 positions x 128
// rows, one byte each, 4-row groups XOR-swizzled by position), filled like the
// up-projection's h tile.
template <class Cfg>
__device__ __forceinline__ void bwd_union_tile(const UnionArgs& a, int b, int pt, char* st0, char* st1,
                                               int16_t* posmap) {
  static_assert(Cfg::BM == UB && Cfg::BM == 128 && Cfg::BN == 256 && Cfg::NW == 8, "slot tile layout");
  static_assert(Cfg::STAGE >= 256 * 128, "slot tile: 256 positions x 128 rows of bytes");
  const int nb = a.ucount[b];
  const int p0 = pt * Cfg::BN;
  if (p0 >= nb) return;
  const int m0 = b * UB;
  const int* ul = a.ulist + (int64_t)b * a.F;
  typedef DmaTile<Cfg> Tile;
  Tile gu, gd;
  const int tid = threadIdx.x;
  const int pl = min(p0 + Cfg::BN, nb) - 1;
  const int nlo = ul[p0], nhi = ul[pl];
  const bool use_map = nhi - nlo < POSCAP;
  if (use_map)
    for (int p = p0 + tid; p <= pl; p += Cfg::NTH) posmap[ul[p] - nlo] = (int16_t)(p - p0);
  const int tjf = nlo >> 6, S = (nhi >> 6) - tjf + 1;
  {
    const Operand A{a.x, a.d, nullptr, a.T};
    const Operand B{a.WuT, a.d, ul, nb};
    gu.run(A, &B, m0, p0, a.d, st0, st1);
  }
  {
    const Operand A{a.dY, a.d, nullptr, a.T};
    const Operand B{a.Wd, a.d, ul, nb};
    gd.run(A, &B, m0, p0, a.d, st0, st1);
  }
  auto soff = [](int pr, int r) { return pr * 128 + (((r >> 2) ^ (pr & 31)) << 2) + (r & 3); };
#pragma unroll
  for (int o = 0; o < 256 * 128 / (16 * Cfg::NTH); ++o) ((uint4*)st0)[o * Cfg::NTH + tid] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  // scatter slot + 1 of every stored pair in the tile's neuron span: a 16-lane
  // group per (row tile, column tile) block, lane piece c = slot c/4, rows
  // 4*(c%4)..+3
  constexpr int NG = Cfg::NTH / 16;
  constexpr int NRT = Cfg::BM / 16;
  const int grp = tid >> 4, gl = tid & 15;
  for (int q = grp; q < NRT * S; q += NG) {
    const int i = q / S, sj = q - i * S;
    const int rt = (m0 >> 4) + i;
    if (rt * 16 >= a.T) continue;
    const int tj = tjf + sj;
    const int64_t blk = (int64_t)rt * a.NT + tj;
    const int w = a.hwidth[blk];
    for (int c = gl; c < w * 4; c += 16) {
      const float4 v4 = ((const float4*)(a.hval + blk * a.hcap * 16))[c];
      const uint32_t i4 = ((const uint32_t*)(a.hidx + blk * a.hcap * 16))[c];
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rl = 4 * (c & 3) + k;
        const int n = tj * 64 + (int)((i4 >> (8 * k)) & 255u);
        if (vv[k] > 0.f && n >= nlo && n <= nhi && live(a, rt * 16 + rl)) {
          int pr;
          if (use_map) {
            pr = posmap[n - nlo];
          } else {
            int lo = p0, hi = pl;
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if (ul[mid] < n) lo = mid + 1; else hi = mid;
            }
            pr = lo - p0;
          }
          st0[soff(pr, i * 16 + rl)] = (char)((c >> 2) + 1);
        }
      }
    }
  }
  __syncthreads();
  // per element: the stored pairs' a, dg, du at their TwELL slots, and dG, dU
  // as fp16 over the union positions (zeros elsewhere, and in the positions
  // [n_b, roundup64(n_b)) that the dX GEMM reads as whole K tiles); any value
  // beyond the fp16 range raises the flag (the per-pair dX path then runs)
  uint32_t vbits = 0;
  const int pend = (nb + 63) & ~63;
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int pr = Tile::col_of(j);
    const int p = p0 + pr;
    if (p >= pend) continue;
    const bool inu = p < nb;
    const int tj = inu ? ul[p] >> 6 : 0;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int r0 = Tile::row_of(i, 4 * qq);                   // 4 consecutive rows r0..r0+3
        const uint32_t s4 = inu ? *(const uint32_t*)(st0 + soff(pr, r0)) : 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int sl = (int)((s4 >> (8 * k)) & 255u);
          const int t = m0 + r0 + k;
          float dg = 0.f, du = 0.f;
          if (sl) {
            const int64_t off = (((int64_t)(t >> 4) * a.NT + tj) * a.hcap + (sl - 1)) * 16 + (t & 15);
            const float h = a.hval[off];
            const float u = gu.acc[0][i][j][4 * qq + k], da = gd.acc[0][i][j][4 * qq + k];
            dg = da * u + a.l1;
            du = da * h;
            a.aval[off] = h * u;
            a.dgval[off] = dg;
            a.duval[off] = du;
            vbits = max(vbits, max(__float_as_uint(dg), __float_as_uint(du)) & 0x7fffffffu);
          }
          if (t < a.T) {
            a.adense[(int64_t)t * a.F + p] = (_Float16)dg;
            a.dU16[(int64_t)t * a.F + p] = (_Float16)du;
          }
        }
      }
  }
  const bool over = vbits > 0x477fe000u;   // above 65504, the largest finite fp16
  if (__builtin_amdgcn_ballot_w64(over) != 0ull && (tid & 63) == 0) atomicOr(a.flag, 1);
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTH) void bwd_union_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[Cfg::STAGE];
  __shared__ int16_t posmap[POSCAP];
  const int npt = (a.F + Cfg::BN - 1) / Cfg::BN;
  const int nblk = (a.T + UB - 1) / UB;
  const int x = blockIdx.x & 7;
  const int nbx = (nblk - x + 7) / 8;
  const int ntile = nbx * npt;
  for (int k = blockIdx.x >> 3; k < ntile; k += gridDim.x >> 3) {
    const int pt = k / nbx;
    const int b = x + 8 * (k - pt * nbx);
    bwd_union_tile<Cfg>(a, b, pt, st0, st1, posmap);
    __syncthreads();
  }
}

// fp16 copy of Wd for the down GEMM.  A bf16 value of magnitude in
// [2^-14, 65504] is exact in fp16 (8 significant bits fit in 11); below 2^-14
// fp16 is subnormal with spacing 2^-24, so a weight under 2^-17 keeps fewer
// than 8 bits and is rounded to the nearest multiple of 2^-24 (absolute error
// at most 2^-25, far below the rounding of a = h*u to fp16).  That underflow
// raises no flag; a value beyond 65504 does, and the layer then takes the fp32
// path.
__device__ __forceinline__ void wd_to_f16_block(const uint16_t* Wd, _Float16* W16, int64_t n8, int* flag,
                                                int64_t blk) {
  const int64_t i = blk * 256 + threadIdx.x;
  bool over = false;
  if (i < n8) {
    const uint4 w = ((const uint4*)Wd)[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = bf16_lo(ws[k]), hi = bf16_hi(ws[k]);
      over |= !(fabsf(lo) <= 65504.f) || !(fabsf(hi) <= 65504.f);
      o[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    }
    ((uint4*)W16)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (__builtin_amdgcn_ballot_w64(over) != 0ull && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
}

__global__ __launch_bounds__(256) void wd_to_f16_kernel(const uint16_t* Wd, _Float16* W16, int64_t n8, int* flag) {
  wd_to_f16_block(Wd, W16, n8, flag, blockIdx.x);
}

// The row blocks' lists (workgroups [0, nlist)) and the fp16 copy of Wd (the
// rest) in one launch, when the gate GEMM has written the slab unions and
// cleared the flag.
__global__ __launch_bounds__(256) void union_list_f16_kernel(UnionArgs a, const uint64_t* U, int nlist, int64_t n8) {
  __shared__ int scan[256], start[256];
  __shared__ uint64_t su[256];
  if ((int)blockIdx.x < nlist) union_list_block(a, U, blockIdx.x, scan, start, su);
  else wd_to_f16_block((const uint16_t*)a.Wd, (_Float16*)a.Wd16, n8, a.flag, (int64_t)blockIdx.x - nlist);
}

// Down-projection over the union: y rows of the block, one column tile.  K
// runs over the block's n_b positions; A = adense holds zeros in the
// positions past n_b of the last K tile.
// TWO: the backward's dX = dG.WgT + dU.WuT over the union (A = adense with
// B = Wd16 holding WgT's fp16 copy, then A = dU16 with B = Wu16).
template <class Cfg, bool TWO>
__device__ __forceinline__ void down_union_tile(const UnionArgs& a, int b, int ct, char* st0, char* st1) {
  static_assert(Cfg::BM == UB, "one row block per M tile");
  const int nb = a.ucount[b];
  const int m0 = b * UB, n0 = ct * Cfg::BN;
  typedef DmaTile<Cfg> Tile;
  Tile g;
  const Operand A{a.adense, a.ucap, nullptr, a.T};
  const Operand B{a.Wd16, a.d, a.ulist + (int64_t)b * a.F, a.F};
  g.run(A, &B, m0, n0, nb, st0, st1);
  if constexpr (TWO) {
    const Operand A2{a.dU16, a.F, nullptr, a.T};
    const Operand B2{a.Wu16, a.d, a.ulist + (int64_t)b * a.F, a.F};
    g.run(A2, &B2, m0, n0, nb, st0, st1, false);
  }
#pragma unroll
  for (int j = 0; j < Cfg::TN; ++j) {
    const int col = n0 + Tile::col_of(j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = m0 + Tile::row_of(i, e);
        if (live(a, t)) {
          // y (a whole [T][d] output, often larger than the caches) streams
          // past them, so it does not push out the next call's x and weights
          // (about 1% on the forward loop at every size, bit-identical)
          const float v = g.acc[0][i][j][e];
          if (a.out_bf16) __builtin_nontemporal_store((uint16_t)f32_to_bf16_bits(v), (uint16_t*)a.y + (int64_t)t * a.d + col);
          else __builtin_nontemporal_store(v, (float*)a.y + (int64_t)t * a.d + col);
        }
      }
  }
}

// The same y tile per stored pair in fp32, for the forward when the overflow
// flag is set (a value of a, h or Wd beyond the fp16 range) or when the block
// is over capacity: for each live row and each stored pair (n, h) in
// ascending neuron order, a = h * (x_t . WuT[n]) (bf16 products, fp32 sums,
// one fixed-order butterfly over the wave) or a = h for the non-gated layer
// (WuT null), then y_t += a * Wd[n] over the tile's columns (CPL per lane).
// The pairs come from the TwELL slots, or, for a block over a capacity (whose
// tiles may have lost slots), from the row's mask with h = x_t . WgT[n] + bg[n]
// recomputed the same way.  Every column tile recomputes its rows' dot
// products: this path serves inputs outside the fp16 range or the capacities,
// not speed.
__device__ __forceinline__ float row_dot(const uint16_t* x, const uint16_t* w, int d, int lane) {
  float p = 0.f;
  for (int e = lane * 8; e < d; e += 512) {
    const uint4 xv = *(const uint4*)(x + e);
    const uint4 wv = *(const uint4*)(w + e);
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w}, ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p = fmaf(bf16_lo(xs[q]), bf16_lo(ws[q]), p);
      p = fmaf(bf16_hi(xs[q]), bf16_hi(ws[q]), p);
    }
  }
  return wave_sum(p);
}

template <int CPL>
__device__ void down_fallback_tile(const UnionArgs& a, int b, int n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint16_t* x = (const uint16_t*)a.x;
  const uint16_t* Wu = (const uint16_t*)a.WuT;
  const uint16_t* Wg = (const uint16_t*)a.WgT;
  const uint16_t* Wd = (const uint16_t*)a.Wd;
  const bool rec = a.bflag && a.bflag[b];
  const int64_t hs = (int64_t)a.hcap * 16;
  const int c0 = n0 + lane * CPL;
  for (int r = wave; r < UB; r += nw) {
    const int t = b * UB + r;
    if (!live(a, t)) continue;                      // wave-uniform
    const uint16_t* xt = x + (int64_t)t * a.d;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    const int64_t tile0 = (int64_t)(t >> 4) * a.NT;
    for (int j = 0; j < a.NT; ++j) {
      uint64_t m = a.mask[(int64_t)t * a.NT + j];
      const int cnt = popc64(m);
      const int64_t sb = (tile0 + j) * hs + (t & 15);     // slot s of this row: sb + 16 s
      for (int s = 0; s < cnt; ++s) {
        float hv;
        int64_t n;
        if (rec) {
          const int c = __builtin_ctzll(m);
          m &= m - 1;
          n = (int64_t)j * 64 + c;
          hv = row_dot(xt, Wg + n * a.d, a.d, lane);
          if (a.bg) hv += bf16_to_f32(((const uint16_t*)a.bg)[n]);
        } else {
          hv = a.hval[sb + 16 * s];
          n = (int64_t)j * 64 + a.hidx[sb + 16 * s];
        }
        const float av = Wu ? hv * row_dot(xt, Wu + n * a.d, a.d, lane) : hv;
        const uint16_t* wr = Wd + n * a.d + c0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(av, bf16_to_f32(wr[c]), acc[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (a.out_bf16) ((uint16_t*)a.y)[(int64_t)t * a.d + c0 + c] = (uint16_t)f32_to_bf16_bits(acc[c]);
      else ((float*)a.y)[(int64_t)t * a.d + c0 + c] = acc[c];
    }
  }
}

// Persistent workgroups walk the (row block, column tile) tiles; the
// workgroups of XCD x take the row blocks b = x (mod 8), all column tiles of
// a block together, so the block's adense rows are reused from that XCD's L2.
// In the forward, a set overflow flag sends every tile down the per-pair fp32
// path above (no separate fallback launch); the backward (TWO) stands down
// and leaves dX to its per-pair kernel.
template <class Cfg, bool TWO = false>
__global__ __launch_bounds__(Cfg::NTH, WavesPerEU<Cfg>::value) void down_union_kernel(UnionArgs a) {
  __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_[Cfg::SINGLE ? 16 : Cfg::STAGE];
  char* st1 = Cfg::SINGLE ? st0 : st1_;
  const int nct = a.d / Cfg::BN;
  const int nblk = (a.T + UB - 1) / UB;
  const int x = blockIdx.x & 7;
  const int nbx = (nblk - x + 7) / 8;
  const int ntile = nbx * nct;
  if (*a.flag) {
    if constexpr (!TWO) {
      for (int k = blockIdx.x >> 3; k < ntile; k += gridDim.x >> 3) {
        const int bi = k / nct;
        down_fallback_tile<Cfg::BN / 64>(a, x + 8 * bi, (k - bi * nct) * Cfg::BN);
      }
    }
    return;
  }
  for (int k = blockIdx.x >> 3; k < ntile; k += gridDim.x >> 3) {
    const int bi = k / nct;
    if (!TWO && a.bflag && a.bflag[x + 8 * bi] == 2) continue;   // workgroup-uniform
    down_union_tile<Cfg, TWO>(a, x + 8 * bi, k - bi * nct, st0, st1);
    __syncthreads();
  }
  if constexpr (!TWO) {
    // blocks over the union capacity (bounded forward), per pair, after the GEMM tiles
    if (a.bflag)
      for (int k = blockIdx.x >> 3; k < ntile; k += gridDim.x >> 3) {
        const int bi = k / nct;
        if (a.bflag[x + 8 * bi] == 2) down_fallback_tile<Cfg::BN / 64>(a, x + 8 * bi, (k - bi * nct) * Cfg::BN);
      }
  }
}

using UpUnionCfg = DmaCfg1<UB, 256, 2, 4>;
// gate and up products on one x tile: 128 positions, so two workgroups share a
// CU (two B operands of 256 positions took one CU each: 2b, every block
// recomputed, 2.86 against 2.52 ms for the layer)
using UpRecCfg = DmaCfg1<UB, 128, 2, 4, 2>;
using UpRecReluCfg = DmaCfg1<UB, 128, 2, 4, 1>;
using DownUnionCfg = DmaCfg1<UB, 256, 2, 4, 1, true, true>;
using DownUnionCfg128 = DmaCfg<UB, 128, 4, 2, 1, true, true>;
using DownUnionCfg64 = DmaCfg<UB, 64, 4, 2, 1, true, true>;

// Union workspace layout: lists, counts, flag and slab unions first (all the
// few-token path uses), then adense and the fp16 copy of Wd.
static size_t r256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t union_lists_ws_bytes(int T, int F) {
  const size_t nblk = (size_t)(T + UB - 1) / UB;
  const size_t nslab = (size_t)(T + 63) / 64;
  return r256(nblk * F * 4 + nblk * 4) + 256 + r256(nslab * (F / 64) * 8) + r256(nblk);
}

size_t union_ws_bytes(int T, int d, int F, int ucap) {
  if (ucap <= 0) ucap = F;
  return union_lists_ws_bytes(T, F) + r256((size_t)T * ucap * 2 + 256) + (size_t)F * d * 2;
}

namespace {

// Pointers into the union workspace (layout of union_ws_bytes).
UnionArgs union_setup(const void* x, const void* WuT, const void* Wd, int T, int d, int F, const TwellView& h,
                      const uint8_t* skip, void* ws, void* y, int out_dt, uint64_t** U, int ucap = 0) {
  const int nblk = (T + UB - 1) / UB;
  char* w = (char*)ws;
  UnionArgs a{};
  a.x = x; a.WuT = WuT; a.Wd = Wd; a.T = T; a.d = d; a.F = F; a.NT = F / 64;
  a.mask = h.mask; a.skip = skip; a.hval = (const float*)h.val; a.hidx = h.idx; a.hwidth = h.width;
  a.hcap = h.cap;
  a.ucap = ucap > 0 ? ucap : F;
  a.ulist = (int*)w;
  a.ucount = (int*)(w + (size_t)nblk * F * 4);
  w += r256((size_t)nblk * F * 4 + (size_t)nblk * 4);
  a.flag = (int*)w;
  w += 256;
  *U = (uint64_t*)w;
  w += r256((size_t)((T + 63) / 64) * a.NT * 8);
  // block flags only where a capacity can be exceeded
  if (ucap > 0) a.bflag = (uint8_t*)w;
  w += r256((size_t)nblk);
  a.adense = (_Float16*)w;                 // [T][ucap] and one spare slot
  a.spare = (uint32_t)((size_t)T * a.ucap);
  w += r256((size_t)T * a.ucap * 2 + 256);
  a.Wd16 = (const _Float16*)w;
  a.y = y; a.out_bf16 = out_dt == DT_BF16;
  a.lrows = UB;
  return a;
}

void union_lists_launch(const UnionArgs& a, const uint64_t* U, hipStream_t s) {
  const int nblk = (a.T + UB - 1) / UB;
  hipLaunchKernelGGL(union_or_kernel, dim3((a.T + 63) / 64, (a.NT + 63) / 64), dim3(256), 0, s, a, (uint64_t*)U);
  hipLaunchKernelGGL(union_list_kernel, dim3(nblk), dim3(256), 0, s, a, U);
}

}  // namespace

// Number of row blocks over capacity in the bounded forward (one workgroup).
__global__ __launch_bounds__(256) void count_flags_kernel(const uint8_t* f, int n, int* out) {
  int c = 0;
  for (int i = threadIdx.x; i < n; i += 256) c += f[i] != 0;
  __shared__ int part[256];
  part[threadIdx.x] = c;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = part[0];
}

hipError_t launch_union_over_count(int T, int F, void* ws, int ucap, int* out, hipStream_t s) {
  uint64_t* U;
  const TwellView none{};
  const UnionArgs a = union_setup(nullptr, nullptr, nullptr, T, 0, F, none, nullptr, ws, nullptr, DT_F32, &U, ucap);
  hipLaunchKernelGGL(count_flags_kernel, dim3(1), dim3(256), 0, s, (const uint8_t*)a.bflag, a.bflag ? (T + UB - 1) / UB : 0,
                     out);
  return hipGetLastError();
}

void union_slabs_and_flag(int T, int F, void* ws, uint64_t** slabs, int** flag) {
  uint64_t* U;
  const TwellView none{};
  const UnionArgs a = union_setup(nullptr, nullptr, nullptr, T, 0, F, none, nullptr, ws, nullptr, DT_F32, &U);
  *slabs = U;
  *flag = a.flag;
}

void union_lists_only(int T, int F, const TwellView& h, void* ws, int** ulist, int** ucount, uint64_t** slabs) {
  uint64_t* U;
  const UnionArgs a = union_setup(nullptr, nullptr, nullptr, T, 0, F, h, nullptr, ws, nullptr, DT_F32, &U);
  *ulist = a.ulist;
  *ucount = a.ucount;
  *slabs = U;
}

hipError_t launch_union_lists(int T, int F, const TwellView& h, void* ws, hipStream_t s, bool slabs_ready) {
  if (T == 0) return hipSuccess;
  uint64_t* U;
  UnionArgs a = union_setup(nullptr, nullptr, nullptr, T, 0, F, h, nullptr, ws, nullptr, DT_F32, &U);
  if (slabs_ready) {
    // the few-token path: one list over every row (T <= DECODE_T_MAX)
    a.lrows = (T + 63) & ~63;
    hipLaunchKernelGGL(union_list_kernel, dim3(1), dim3(256), 0, s, a, (const uint64_t*)U);
  } else {
    union_lists_launch(a, U, s);
  }
  return hipGetLastError();
}

hipError_t launch_union_fwd(const void* x, const void* WuT, const void* Wd, int T, int d, int F,
                            const TwellView& h, const uint8_t* skip, void* ws, void* y, int out_dt,
                            int** flag_out, hipStream_t s, hipEvent_t ev_lists, hipEvent_t ev_up, bool slabs_ready,
                            const void* WgT, const void* bg, int ucap) {
  if (T == 0) {
    if (ev_lists) (void)hipEventRecord(ev_lists, s);
    if (ev_up) (void)hipEventRecord(ev_up, s);
    return hipSuccess;
  }
  const int nblk = (T + UB - 1) / UB;
  uint64_t* U;
  UnionArgs a = union_setup(x, WuT, Wd, T, d, F, h, skip, ws, y, out_dt, &U, ucap);
  a.WgT = WgT;
  a.bg = bg;
  if (flag_out) *flag_out = a.flag;
  {
    const int64_t n8 = (int64_t)F * d / 8;
    const unsigned nconv = (unsigned)((n8 + 255) / 256);
    if (slabs_ready && !skip) {
      hipLaunchKernelGGL(union_list_f16_kernel, dim3((unsigned)nblk + nconv), dim3(256), 0, s, a,
                         (const uint64_t*)U, nblk, n8);
    } else {
      union_lists_launch(a, U, s);
      hipLaunchKernelGGL(wd_to_f16_kernel, dim3(nconv), dim3(256), 0, s, (const uint16_t*)Wd, (_Float16*)a.Wd16,
                         n8, a.flag);
    }
  }
  if (ev_lists) (void)hipEventRecord(ev_lists, s);
  static_assert(UpUnionCfg::SINGLE, "TwELL capacities below 4 slots need the up kernel without read-ahead");
  const int npt = (F + UpUnionCfg::BN - 1) / UpUnionCfg::BN;
  const int nbx_max = (nblk + 7) / 8;
  // persistent grids: one workgroup per CU (multiples of 8, one row of XCDs),
  // never more than the tiles of the busiest XCD need
  const int cus = device_cus();
  auto grid_for = [&](int tiles_per_xcd, int per_cu = 1) {
    return (unsigned)(8 * std::max(1, std::min(per_cu * cus / 8, tiles_per_xcd)));
  };
  if (WuT)
    hipLaunchKernelGGL((up_union_kernel<UpUnionCfg, true>), dim3(grid_for(nbx_max * npt, 2)), dim3(UpUnionCfg::NTH),
                       0, s, a);
  else   // non-gated layer: a = h
    hipLaunchKernelGGL((up_union_kernel<UpUnionCfg, false>), dim3(grid_for(nbx_max * npt, 2)), dim3(UpUnionCfg::NTH),
                       0, s, a);
  if (a.bflag) {       // blocks over the tile capacity only: h from a gate GEMM over the union
    const dim3 grid(std::max(1, std::min(2 * cus, nblk * npt * 2)));
    if (WuT) hipLaunchKernelGGL((up_union_rec_kernel<UpRecCfg, true>), grid, dim3(UpRecCfg::NTH), 0, s, a);
    else hipLaunchKernelGGL((up_union_rec_kernel<UpRecReluCfg, false>), grid, dim3(UpRecReluCfg::NTH), 0, s, a);
  }
  if (ev_up) (void)hipEventRecord(ev_up, s);
  if (d % 256 == 0)
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg>), dim3(grid_for(nbx_max * (d / 256), 2)),
                       dim3(DownUnionCfg::NTH), 0, s, a);
  else if (d % 128 == 0)
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg128>), dim3(grid_for(nbx_max * (d / 128))),
                       dim3(DownUnionCfg128::NTH), 0, s, a);
  else
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg64>), dim3(grid_for(nbx_max * (d / 64))),
                       dim3(DownUnionCfg64::NTH), 0, s, a);
  return hipGetLastError();
}

size_t union_bwd_ws_bytes(int T, int d, int F) {
  const size_t nblk = (size_t)(T + UB - 1) / UB;
  const size_t nslab = (size_t)(T + 63) / 64;
  auto r = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return r(nblk * F * 4 + nblk * 4) + r(nslab * (F / 64) * 8) + 256 + 2 * r((size_t)T * F * 2) +
         2 * r((size_t)F * d * 2);
}

hipError_t launch_union_bwd(const void* x, const void* dY, const void* WgT, const void* WuT, const void* Wd, int T,
                            int d, int F, const TwellView& h, const uint8_t* skip, void* ws, float* aval,
                            float* dgval, float* duval, float l1, float* dX, int** flag_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nblk = (T + UB - 1) / UB;
  char* w = (char*)ws;
  UnionArgs a{};
  a.x = x; a.WuT = WuT; a.Wd = Wd; a.dY = dY; a.T = T; a.d = d; a.F = F; a.NT = F / 64;
  a.mask = h.mask; a.skip = skip; a.hval = (const float*)h.val; a.hidx = h.idx; a.hwidth = h.width;
  a.hcap = h.cap;                           // slot arrays in, and out (aval, dgval, duval)
  a.ucap = F;
  auto r = [](size_t v) { return (v + 255) & ~(size_t)255; };
  a.ulist = (int*)w;
  a.ucount = (int*)(w + (size_t)nblk * F * 4);
  w += r((size_t)nblk * F * 4 + (size_t)nblk * 4);
  uint64_t* U = (uint64_t*)w;
  w += r((size_t)((T + 63) / 64) * a.NT * 8);
  a.flag = (int*)w;                         // the list kernel clears it
  w += 256;
  a.adense = (_Float16*)w;                  // dG over the union positions
  w += r((size_t)T * F * 2);
  a.dU16 = (_Float16*)w;
  w += r((size_t)T * F * 2);
  a.Wd16 = (const _Float16*)w;              // fp16 copy of WgT
  w += r((size_t)F * d * 2);
  a.Wu16 = (const _Float16*)w;              // fp16 copy of WuT
  a.lrows = UB;
  a.aval = aval; a.dgval = dgval; a.duval = duval; a.l1 = l1;
  a.y = dX; a.out_bf16 = 0;
  if (flag_out) *flag_out = a.flag;
  union_lists_launch(a, U, s);
  using BwdUnionCfg = DmaCfg<UB, 256, 2, 4>;
  const int npt = (F + BwdUnionCfg::BN - 1) / BwdUnionCfg::BN;
  const int nbx_max = (nblk + 7) / 8;
  const int cus = device_cus();
  auto grid_for = [&](int tiles_per_xcd, int per_cu = 1) {
    return (unsigned)(8 * std::max(1, std::min(per_cu * cus / 8, tiles_per_xcd)));
  };
  hipLaunchKernelGGL((bwd_union_kernel<BwdUnionCfg>), dim3(grid_for(nbx_max * npt)), dim3(BwdUnionCfg::NTH), 0, s, a);
  // fp16 copies of WgT and WuT for the dX GEMM (a value beyond the fp16 range raises the flag)
  const int64_t n8 = (int64_t)F * d / 8;
  hipLaunchKernelGGL(wd_to_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, (const uint16_t*)WgT,
                     (_Float16*)a.Wd16, n8, a.flag);
  hipLaunchKernelGGL(wd_to_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, (const uint16_t*)WuT,
                     (_Float16*)a.Wu16, n8, a.flag);
  // dX of the live rows = dG.WgT + dU.WuT over the union (stands down when the flag is set)
  if (d % 256 == 0)
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg, true>), dim3(grid_for(nbx_max * (d / 256), 2)),
                       dim3(DownUnionCfg::NTH), 0, s, a);
  else if (d % 128 == 0)
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg128, true>), dim3(grid_for(nbx_max * (d / 128))),
                       dim3(DownUnionCfg128::NTH), 0, s, a);
  else
    hipLaunchKernelGGL((down_union_kernel<DownUnionCfg64, true>), dim3(grid_for(nbx_max * (d / 64))),
                       dim3(DownUnionCfg64::NTH), 0, s, a);
  return hipGetLastError();
}

}  // namespace twell
