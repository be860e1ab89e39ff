// Gate GEMM with the TwELL pack in its epilogue, and the standalone
// pack/unpack kernels.
//
// TwELL (tile-wise ELLPACK) follows the intellectnews.ru TwELL article,
// section "Формат TwELL вместо классической sparse-упаковки", and gate.com/es
// post 20977915, paragraph 3: the gate output is cut into tiles and each tile
// is compacted where it is produced, at the end of the kernel that computes
// it, with no further launch and no second pass over the dense matrix.  Here a
// tile is 16 rows x 64 columns, the 64 columns being one wave64 ballot:
//   mask  = ballot(h > 0) per row of the tile      (bit c = column c active)
//   cnt   = popcount(mask)
//   slot  = popcount(mask & bits below my column)  (ascending column order)
//   width = max cnt over the 16 rows               (the tile's ELL width)
// Values are stored [row tile][column tile][slot][row]; slots in
// [cnt, width) hold (+0.0, index 0).
#include <type_traits>

#include "gemm_core.hpp"
#include "internal.hpp"

namespace twell {

struct GateArgs {
  const void* x;
  const void* WgT;
  const void* bg;
  int T, d, F, NT;
  uint8_t* cnt;
  uint8_t* width;
  float* val;
  uint8_t* idx;
  uint64_t* mask;
  uint64_t* slabs;   // nullable: union of each 64-row slab's masks, [ceil(T/64)][NT]
  int* flag;         // nullable: cleared by workgroup 0
  int cap;           // slots per tile in val and idx (a wider tile keeps its first cap)
};

template <bool BF16IN>
__device__ __forceinline__ float load_bias(const void* b, int n) {
  if (b == nullptr) return 0.f;
  if constexpr (BF16IN) return bf16_to_f32(((const uint16_t*)b)[n]);
  else return ((const float*)b)[n];
}

// Tile order: groups of GM row blocks sweep all column blocks, so the
// workgroups resident on one XCD share both x rows and gate weight rows in L2
// (groups of 4 measured 2% faster than 8 at T = 32768, d = 2048, F = 5632;
// 16 slower).
__device__ __forceinline__ void tile_coords(int id, int nbm, int nbn, int& bm, int& bn) {
  constexpr int GM = 4;
  const int per_group = GM * nbn;
  const int group = id / per_group;
  const int first = group * GM;
  const int gsize = min(nbm - first, GM);
  const int r = id - group * per_group;
  bm = first + r % gsize;
  bn = r / gsize;
}

template <class Cfg, bool BF16IN>
__global__ __launch_bounds__(Cfg::NTH, WavesPerEU<Cfg>::value) void gate_twell_kernel(GateArgs a) {
  static_assert((Cfg::BN / Cfg::WN) % 64 == 0 && Cfg::TN % 2 == 0, "whole 64-column TwELL tiles per wave");
  static_assert((Cfg::BM / Cfg::WM) % 64 == 0, "whole 64-row slabs per wave");
  if (a.flag && blockIdx.x == 0 && threadIdx.x == 0) *a.flag = 0;
  const int nbm = (a.T + Cfg::BM - 1) / Cfg::BM;
  const int nbn = a.F / Cfg::BN;
  int bm, bn;
  tile_coords(xcd_remap(blockIdx.x, gridDim.x), nbm, nbn, bm, bn);
  const int m0 = bm * Cfg::BM, n0 = bn * Cfg::BN;

  // the bias of this lane's columns, loaded before the mainloop so that the
  // epilogue does not start with a round trip to memory
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cl = lane & 31;
  float bias[Cfg::TN];
#pragma unroll
  for (int t = 0; t < Cfg::TN; ++t)
    bias[t] = load_bias<BF16IN>(a.bg, n0 + (wave % Cfg::WN) * (Cfg::BN / Cfg::WN) + t * 32 + cl);

  typename TileFor<Cfg>::type g;
  const Operand A{a.x, a.d, nullptr, a.T};
  const Operand B{a.WgT, a.d, nullptr, a.F};
  char* lds;
  char* lds2 = nullptr;                             // a second free region (two-stage direct-to-LDS tiles)
  if constexpr (TileFor<Cfg>::dma) {
    __shared__ __attribute__((aligned(1024))) char st0[Cfg::STAGE];
    __shared__ __attribute__((aligned(1024))) char st1_[Cfg::SINGLE ? 16 : Cfg::STAGE];
    char* st1 = Cfg::SINGLE ? st0 : st1_;
    g.run(A, &B, m0, n0, a.d, st0, st1);
    lds = st0;
    lds2 = st1_;
  } else {
    __shared__ __attribute__((aligned(16))) char buf[Cfg::LDS_BYTES];
    g.run(A, &B, m0, n0, a.d, buf);
    lds = buf;
  }

  // ---- epilogue: bias, ReLU, ballot compaction into TwELL.  Accumulator
  // blocks 2*tc and 2*tc+1 of a wave hold the 64 columns of one TwELL tile;
  // register e of a 32x32 block holds row 8*(e/4) + 4*(lane/32) + e%4, column
  // lane%32.  For each 16-row tile: (1) every lane drops its biased values into
  // a dense 16x64 LDS tile (column pairs c, c + 32 side by side), and two
  // ballots per register give the masks of two rows, which v_writelane
  // collects so that lane r (r < 16) holds row r's
  // 64-bit mask in two VGPRs (the mask bookkeeping stays on the vector unit:
  // the scalar unit is shared by the CU's waves and would serialise it);
  // (2) counts, the width (a 16-lane max) and the slab union (a 16-lane OR)
  // come from those lanes; (3) the width*16 output slots [slot][row] are
  // produced one per lane: slot s of row r is the s-th set bit of r's mask
  // (found by a branch-free binary search on popcounts), or padding (+0.0,
  // index 0) past the row's count; (4) coalesced stores of the values,
  // indices, row counts and masks.  The mainloop's LDS is free once it
  // returns.
  // Where the free LDS holds several dense tiles per wave, NH consecutive
  // 16-row tiles (four: one 64-row slab, with both stage buffers of a
  // two-stage tile; else two: one 32-row accumulator block) go through these
  // steps together, with no barrier between them, so the latencies of one
  // tile's shuffles, LDS reads and stores overlap the others' work.
  constexpr int STG = 16 * 64 * 4;                          // dense tile, per wave
  constexpr int NW = Cfg::NTH / 64;
  constexpr bool TWO_REGIONS = TileFor<Cfg>::dma && !Cfg::SINGLE && NW % 2 == 0;
  constexpr int NH = (TWO_REGIONS && Cfg::EPI_BYTES >= NW / 2 * 4 * STG) ? 4
                     : Cfg::EPI_BYTES >= NW * 2 * STG ? 2 : 1;
  static_assert(NH == 4 || Cfg::EPI_BYTES >= NW * NH * STG, "epilogue staging");
  const int wr = m0 + (wave / Cfg::WN) * (Cfg::BM / Cfg::WM);
  // NH x [16 rows][32][2]: (c, c + 32) pairs; with NH = 4 the first half of
  // the waves stage in one stage buffer, the second half in the other
  float* sdw = NH == 4 ? (float*)((wave < NW / 2 ? lds : lds2) + (wave % (NW / 2)) * NH * STG)
                       : (float*)(lds + wave * NH * STG);
  const int rsel = lane & 15;
#pragma unroll
  for (int tc = 0; tc < Cfg::TN / 2; ++tc) {
    const int wc = n0 + (wave % Cfg::WN) * (Cfg::BN / Cfg::WN) + tc * 64;
    const int j = wc >> 6;
    const float b0 = bias[2 * tc], b1 = bias[2 * tc + 1];
    uint32_t sorl = 0, sorh = 0;                    // lanes 0-15: union of their rows' masks over the slab
#pragma unroll
    for (int kb = 0; kb < 2 * Cfg::TM; kb += NH) {  // 16-row tiles kb .. kb + NH - 1 of the wave
      const int rtb = wr + kb * 16;                 // first row of the batch's first TwELL row tile
      if (rtb < a.T) {                              // wave-uniform
        const bool full = rtb + 16 * NH <= a.T;     // every row of the batch exists
        uint32_t ml[NH], mh[NH];                    // lane r < 16: row r's mask, columns 0-31 / 32-63
        // a batch with rows past T takes a copy of the loop that masks them
        // out of the ballots; every other batch takes one without that work
        auto collect = [&](auto full_c) {
          constexpr bool FULL = decltype(full_c)::value;
          auto one = [&](auto k_c, auto q_c) {
            constexpr int k = decltype(k_c)::value;
            constexpr int q = decltype(q_c)::value;
            constexpr int r0 = 8 * (q >> 2) + (q & 3);  // row of lanes 0-31; lanes 32-63 hold r0 + 4
            const float v0 = g.acc[0][(kb + k) >> 1][2 * tc][((kb + k) & 1) * 8 + q] + b0;
            const float v1 = g.acc[0][(kb + k) >> 1][2 * tc + 1][((kb + k) & 1) * 8 + q] + b1;
            uint64_t B0 = __builtin_amdgcn_ballot_w64(v0 > 0.f);
            uint64_t B1 = __builtin_amdgcn_ballot_w64(v1 > 0.f);
            if constexpr (!FULL) {
              const int rq = rtb + 16 * k + r0;
              const uint64_t rowmask =
                  (rq < a.T ? 0xffffffffull : 0ull) | (rq + 4 < a.T ? 0xffffffff00000000ull : 0ull);
              B0 &= rowmask;
              B1 &= rowmask;
            }
            *(float2*)(sdw + k * (STG / 4) + ((r0 + 4 * (lane >> 5)) * 32 + cl) * 2) = make_float2(v0, v1);
            // lane r0 (r0 + 4) of ml/mh takes row r0's (r0 + 4's) mask halves;
            // the wait states cover the ballots' scalar results
            const uint32_t b0l = (uint32_t)B0, b1l = (uint32_t)B1;
            const uint32_t b0h = (uint32_t)(B0 >> 32), b1h = (uint32_t)(B1 >> 32);
            uint32_t wl0 = ml[k], wl1 = mh[k];
            asm volatile(
                "s_nop 4\n\t"
                "v_writelane_b32 %0, %2, %6\n\t"
                "v_writelane_b32 %1, %3, %6\n\t"
                "v_writelane_b32 %0, %4, %7\n\t"
                "v_writelane_b32 %1, %5, %7"
                : "+v"(wl0), "+v"(wl1)
                : "s"(b0l), "s"(b1l), "s"(b0h), "s"(b1h), "i"(r0), "i"(r0 + 4));
            ml[k] = wl0;
            mh[k] = wl1;
          };
          auto tile = [&](auto k_c) {
            one(k_c, std::integral_constant<int, 0>{});
            one(k_c, std::integral_constant<int, 1>{});
            one(k_c, std::integral_constant<int, 2>{});
            one(k_c, std::integral_constant<int, 3>{});
            one(k_c, std::integral_constant<int, 4>{});
            one(k_c, std::integral_constant<int, 5>{});
            one(k_c, std::integral_constant<int, 6>{});
            one(k_c, std::integral_constant<int, 7>{});
          };
          tile(std::integral_constant<int, 0>{});
          if constexpr (NH >= 2) tile(std::integral_constant<int, 1>{});
          if constexpr (NH == 4) {
            tile(std::integral_constant<int, 2>{});
            tile(std::integral_constant<int, 3>{});
          }
        };
#pragma unroll
        for (int k = 0; k < NH; ++k) ml[k] = mh[k] = 0;
        if (full) collect(std::true_type{});
        else collect(std::false_type{});
        // lanes 0-15: counts; each tile's width is their maximum
        int c16[NH], width[NH];
#pragma unroll
        for (int k = 0; k < NH; ++k) c16[k] = __popc(ml[k]) + __popc(mh[k]);
#pragma unroll
        for (int k = 0; k < NH; ++k) {
          int wm = c16[k];
#pragma unroll
          for (int o = 8; o >= 1; o >>= 1) wm = max(wm, __shfl_xor(wm, o));
          width[k] = __builtin_amdgcn_readfirstlane(wm);
          sorl |= ml[k];
          sorh |= mh[k];
        }
        __builtin_amdgcn_wave_barrier();
        // output slot i (lane + 64 m) of a tile is slot i >> 4 of row rsel:
        // the (i >> 4)-th set bit of that row's mask, or padding
        uint64_t mrow[NH];
        int crow[NH];
#pragma unroll
        for (int k = 0; k < NH; ++k) {
          mrow[k] = ((uint64_t)(uint32_t)__shfl((int)mh[k], rsel) << 32) | (uint32_t)__shfl((int)ml[k], rsel);
          crow[k] = popc64(mrow[k]);
        }
        auto slot = [&](int k, int i) {
          const int sl = i >> 4;
          uint64_t m = mrow[k];
          float v = 0.f;
          int c = 0;
          if (sl < crow[k]) {
            // position of the sl-th set bit of m
            int kk = sl;
#pragma unroll
            for (int w = 32; w >= 1; w >>= 1) {
              const uint64_t lowmask = (1ull << w) - 1ull;
              const int pc = popc64(m & lowmask);
              const bool up = kk >= pc;
              kk = up ? kk - pc : kk;
              c = up ? c + w : c;
              m = up ? (m >> w) : m;
            }
            v = sdw[k * (STG / 4) + (rsel * 32 + (c & 31)) * 2 + (c >> 5)];
          }
          const int64_t tbase = ((int64_t)((rtb >> 4) + k) * a.NT + j) * (a.cap * 16);
          a.val[tbase + i] = v;
          a.idx[tbase + i] = (uint8_t)c;
        };
        // the first 64 slots of every tile of the batch, one per lane, then
        // the rest of the wider tiles (up to the capacity)
#pragma unroll
        for (int k = 0; k < NH; ++k)
          if (lane < min(width[k], a.cap) * 16) slot(k, lane);
#pragma unroll
        for (int k = 0; k < NH; ++k)
          for (int i = lane + 64; i < min(width[k], a.cap) * 16; i += 64) slot(k, i);
#pragma unroll
        for (int k = 0; k < NH; ++k) {
          const int rt0 = rtb + 16 * k;
          if (lane < 16 && rt0 + lane < a.T) {
            a.cnt[(int64_t)(rt0 + lane) * a.NT + j] = (uint8_t)c16[k];
            if (a.mask) a.mask[(int64_t)(rt0 + lane) * a.NT + j] = ((uint64_t)mh[k] << 32) | ml[k];
          }
          if (lane == 0 && rt0 < a.T) a.width[(int64_t)(rt0 >> 4) * a.NT + j] = (uint8_t)width[k];
        }
        __builtin_amdgcn_wave_barrier();
      }
      // a wave's rows start on a multiple of 64, so 16-row tiles 4s .. 4s + 3
      // are one whole 64-row slab
      if (((kb + NH) & 3) == 0) {
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) {
          sorl |= (uint32_t)__shfl_xor((int)sorl, o);
          sorh |= (uint32_t)__shfl_xor((int)sorh, o);
        }
        const int s0 = wr + (kb + NH - 4) * 16;
        if (a.slabs && s0 < a.T && lane == 0) a.slabs[(int64_t)(s0 >> 6) * a.NT + j] = ((uint64_t)sorh << 32) | sorl;
        sorl = 0;
        sorh = 0;
      }
    }
  }
}

using GateBigBf16 = DmaCfg<256, 256, 2, 4>;
// K = d <= 1024: single-stage 128x256 tiles, two workgroups per CU, so one
// workgroup's TwELL epilogue runs under the other's MFMAs (T = 16384,
// d = 1024, F = 4096: 159 -> 148 us; at d = 2048 the double-buffered 256x256
// tile is 4% faster)
using GateMidBf16 = DmaCfg1<128, 256, 2, 4>;
using GateSmallBf16 = GemmCfg<64, 64, 1, 1, OP_BF16_K, OP_BF16_K>;
using GateBigF32 = GemmCfg<256, 256, 2, 4, OP_F32_K, OP_F32_K>;
using GateSmallF32 = GemmCfg<64, 64, 1, 1, OP_F32_K, OP_F32_K>;

template <class Cfg, bool BF16IN>
static hipError_t launch_gate_cfg(const GateArgs& a, hipStream_t s) {
  const int nbm = (a.T + Cfg::BM - 1) / Cfg::BM;
  const int nbn = a.F / Cfg::BN;
  const int grid = nbm * nbn;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gate_twell_kernel<Cfg, BF16IN>), dim3(grid), dim3(Cfg::NTH), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gate_twell(int in_dt, const void* x, const void* WgT, const void* bg, int T,
                             int d, int F, const TwellView& out, hipStream_t s, uint64_t* slabs, int* flag) {
  GateArgs a{x, WgT, bg, T, d, F, F / 64, out.cnt, out.width, (float*)out.val, out.idx, out.mask,
             in_dt == DT_BF16 ? slabs : nullptr, in_dt == DT_BF16 ? flag : nullptr, out.cap};
  const bool big = T >= 512 && F % 256 == 0;
  if (in_dt == DT_BF16) {
    if (!big) return launch_gate_cfg<GateSmallBf16, true>(a, s);
    return d <= 1024 ? launch_gate_cfg<GateMidBf16, true>(a, s) : launch_gate_cfg<GateBigBf16, true>(a, s);
  }
  return big ? launch_gate_cfg<GateBigF32, false>(a, s) : launch_gate_cfg<GateSmallF32, false>(a, s);
}

// ------------------------------------------------------------------ standalone pack

template <bool BF16>
__device__ __forceinline__ float as_float(uint32_t bits) {
  if constexpr (BF16) return __uint_as_float(bits << 16);
  else return __uint_as_float(bits);
}

// One wave per (row tile, column tile); lane = column inside the tile.  The 16
// row loads are issued before any is used so that each wave keeps 16 reads in
// flight.
template <bool BF16>
__global__ __launch_bounds__(256) void pack_kernel(const void* G, int64_t ldg, int T, int F, int NT,
                                                   int NR, uint8_t* cnt, uint8_t* width, void* val,
                                                   uint8_t* idx, uint64_t* mask) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= (int64_t)NR * NT) return;
  const int i = (int)(tile / NT), j = (int)(tile % NT);
  const int col = j * 64 + lane;
  uint32_t bits[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = i * 16 + r;
    bits[r] = 0;
    if (t < T) {
      if constexpr (BF16) bits[r] = ((const uint16_t*)G)[(int64_t)t * ldg + col];
      else bits[r] = ((const uint32_t*)G)[(int64_t)t * ldg + col];
    }
  }
  uint64_t M[16];
  int w = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    M[r] = ballot(as_float<BF16>(bits[r]) > 0.f);
    w = max(w, popc64(M[r]));
  }
  if (lane == 0) width[tile] = (uint8_t)w;
  const int64_t tbase = tile * (64 * 16);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = i * 16 + r;
    const int c = popc64(M[r]);
    if (lane == 0 && t < T) {
      cnt[(int64_t)t * NT + j] = (uint8_t)c;
      if (mask) mask[(int64_t)t * NT + j] = M[r];
    }
    const int nb = popc64(M[r] & below(lane));
    const bool act = (M[r] >> lane) & 1ull;
    const int slot = act ? nb : c + (lane - nb);
    if (slot < w) {
      if constexpr (BF16) ((uint16_t*)val)[tbase + slot * 16 + r] = act ? (uint16_t)bits[r] : (uint16_t)0;
      else ((uint32_t*)val)[tbase + slot * 16 + r] = act ? bits[r] : 0u;
      idx[tbase + slot * 16 + r] = act ? (uint8_t)lane : (uint8_t)0;
    }
  }
}

hipError_t launch_pack(const void* G, int gdt, int64_t ldg, const TwellView& o, hipStream_t s) {
  const int64_t tiles = (int64_t)o.NR * o.NT;
  if (tiles == 0) return hipSuccess;
  const int grid = (int)((tiles + 3) / 4);
  if (gdt == DT_BF16)
    hipLaunchKernelGGL(pack_kernel<true>, dim3(grid), dim3(256), 0, s, G, ldg, o.T, o.F, o.NT, o.NR,
                       o.cnt, o.width, o.val, o.idx, o.mask);
  else
    hipLaunchKernelGGL(pack_kernel<false>, dim3(grid), dim3(256), 0, s, G, ldg, o.T, o.F, o.NT, o.NR,
                       o.cnt, o.width, o.val, o.idx, o.mask);
  return hipGetLastError();
}

// ------------------------------------------------------------------ unpack (test helper)

template <bool BF16>
__global__ __launch_bounds__(256) void unpack_kernel(int T, int NT, const uint8_t* cnt, const void* val,
                                                     const uint8_t* idx, void* H, int64_t ldh) {
  const int lane = threadIdx.x & 63;
  const int64_t rowtile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (t, j) pair
  if (rowtile >= (int64_t)T * NT) return;
  const int t = (int)(rowtile / NT), j = (int)(rowtile % NT);
  const int i = t >> 4, r = t & 15;
  const int64_t tbase = ((int64_t)i * NT + j) * (64 * 16);
  const int c = min((int)cnt[rowtile], 64);
  uint32_t out = 0;
  for (int s = 0; s < c; ++s) {
    if (idx[tbase + s * 16 + r] == lane) {
      if constexpr (BF16) out = ((const uint16_t*)val)[tbase + s * 16 + r];
      else out = ((const uint32_t*)val)[tbase + s * 16 + r];
    }
  }
  if constexpr (BF16) ((uint16_t*)H)[(int64_t)t * ldh + j * 64 + lane] = (uint16_t)out;
  else ((uint32_t*)H)[(int64_t)t * ldh + j * 64 + lane] = out;
}

hipError_t launch_unpack(const TwellView& in, int vdt, void* H, int64_t ldh, hipStream_t s) {
  const int64_t n = (int64_t)in.T * in.NT;
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + 3) / 4);
  if (vdt == DT_BF16)
    hipLaunchKernelGGL(unpack_kernel<true>, dim3(grid), dim3(256), 0, s, in.T, in.NT, in.cnt, in.val,
                       in.idx, H, ldh);
  else
    hipLaunchKernelGGL(unpack_kernel<false>, dim3(grid), dim3(256), 0, s, in.T, in.NT, in.cnt, in.val,
                       in.idx, H, ldh);
  return hipGetLastError();
}

}  // namespace twell
