// Tiled MFMA GEMM mainloop for gfx950: C[M,N] = sum_k A[m,k] * B[n,k].
//
// Each operand is staged through LDS in 128-byte rows (64 bf16 or 32 fp32 of
// K) with the XOR swizzle of swz().  The global -> register prefetch of tile
// k+1 overlaps the MFMAs of tile k (two LDS buffers, one barrier per K tile).
// Operand kinds:
//   OP_BF16_K  bf16, [rows][K] (K contiguous), optional row gather list
//   OP_BF16_T  bf16, [K][rows] (rows contiguous), optional K gather list;
//              copied into LDS as [k][row] and read with transpose loads
//   OP_F32S_K  fp32 [rows][K], split into bf16 hi and lo tiles
//   OP_F32S_T  fp32 [K][rows], split into bf16 hi and lo tiles
//   OP_F32_K   fp32 [rows][K] fed to fp32 MFMA (fp32 workloads)
//   OP_F32_T   fp32 [K][rows] fed to fp32 MFMA
//   OP_F16_K   fp16 [rows][K] fed to fp16 MFMA
//   OP_BF16P_K bf16 [rows][K] hi values with their lo values pair_off elements
//              further on (an fp32 quantity kept split), fed like OP_F32S_K
//   OP_BF16_T16 bf16 [K][rows], optional K gather list, converted to fp16 as
//              it is transposed into LDS (exact for |v| >= 2^-17; smaller
//              magnitudes keep fp16's subnormal resolution), fed to fp16 MFMA
// A split operand costs two MFMAs (hi and lo) per fragment; B is always exact
// in its type.  K-contiguous kinds need K % 64 == 0 (bf16) / 32 (fp32);
// transposed kinds zero-fill past K and read whole row blocks, so the caller
// launches them only on matrices whose row count is a multiple of the block.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace twell {

enum OpKind { OP_BF16_K = 0, OP_BF16_T = 1, OP_F32S_K = 2, OP_F32S_T = 3, OP_F32_K = 4, OP_F32_T = 5,
              OP_F16_K = 6, OP_BF16_T16 = 7, OP_BF16P_K = 8 };

struct Operand {
  const void* ptr;
  int64_t ld;          // elements between consecutive rows (K kinds) or K steps (T kinds)
  const int* gather;   // K kinds: row index list; T kinds: K index list; may be null
  int nrows;           // rows that exist (K kinds clamp to nrows-1)
  int64_t pair_off;    // OP_BF16P_K: elements from a hi value to its lo value
};

template <int KIND> struct KindInfo;
template <> struct KindInfo<OP_BF16_K> { static constexpr bool split = false, f32mma = false, f16 = false, trans = false; static constexpr int esz = 2; };
template <> struct KindInfo<OP_BF16_T> { static constexpr bool split = false, f32mma = false, f16 = false, trans = true;  static constexpr int esz = 2; };
template <> struct KindInfo<OP_F32S_K> { static constexpr bool split = true,  f32mma = false, f16 = false, trans = false; static constexpr int esz = 4; };
template <> struct KindInfo<OP_F32S_T> { static constexpr bool split = true,  f32mma = false, f16 = false, trans = true;  static constexpr int esz = 4; };
template <> struct KindInfo<OP_F32_K>  { static constexpr bool split = false, f32mma = true,  f16 = false, trans = false; static constexpr int esz = 4; };
template <> struct KindInfo<OP_F32_T>  { static constexpr bool split = false, f32mma = true,  f16 = false, trans = true;  static constexpr int esz = 4; };
template <> struct KindInfo<OP_F16_K>  { static constexpr bool split = false, f32mma = false, f16 = true,  trans = false; static constexpr int esz = 2; };
template <> struct KindInfo<OP_BF16_T16> { static constexpr bool split = false, f32mma = false, f16 = true, trans = true; static constexpr int esz = 2; };
template <> struct KindInfo<OP_BF16P_K> { static constexpr bool split = true, f32mma = false, f16 = false, trans = false; static constexpr int esz = 2; };

// K elements per LDS row (= per K tile).
template <int KIND> constexpr int ktile() { return KindInfo<KIND>::f32mma ? 32 : 64; }

// ------------------------------------------------------------------ loaders
// Each loader moves one K tile of a ROWS-row operand block from global memory
// into registers (load) and from registers into the swizzled LDS tile(s)
// (store).  Thread tid owns a fixed set of 16-byte chunks.

template <int KIND, int ROWS, int NTH> struct Loader;

// bf16 or fp32, K contiguous: 8 chunks of 16 bytes per row.
// Row addresses are kept as 32-bit element offsets from the operand base (the
// caller guarantees every matrix holds fewer than 2^32 elements), which keeps
// the loader's register footprint at one VGPR per 16-byte chunk.
template <int KIND, int ROWS, int NTH>
struct LoaderK {
  static constexpr int ESZ = KindInfo<KIND>::esz;
  static constexpr int CH = ROWS * 8 / NTH;
  static_assert(CH * NTH == ROWS * 8, "tile rows must divide the thread count");
  const char* base;
  uint32_t off[CH];
  uint4 r[CH];
  __device__ void init(const Operand& op, int row0, int tid) {
    base = (const char*)op.ptr;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int id = tid + q * NTH;
      int gr = min(row0 + (id >> 3), op.nrows - 1);
      if (op.gather) gr = op.gather[gr];
      off[q] = (uint32_t)gr * (uint32_t)op.ld + (uint32_t)(id & 7) * (16 / ESZ);
    }
  }
  __device__ void load(int k0, int /*K*/) {
#pragma unroll
    for (int q = 0; q < CH; ++q) r[q] = *(const uint4*)(base + ((uint64_t)off[q] + (uint32_t)k0) * ESZ);
  }
  // two 8-byte LDS stores per chunk: a 16-byte store per lane into this
  // swizzle doubles the bank conflicts (the register-staged gate GEMM runs
  // 19-29% faster with the 8-byte form)
  __device__ void store(char* lds, char* /*lds_lo*/, int tid) const {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int id = tid + q * NTH;
      const int o = swz(id >> 3, id & 7);
      *(uint2*)(lds + o) = make_uint2(r[q].x, r[q].y);
      *(uint2*)(lds + o + 8) = make_uint2(r[q].z, r[q].w);
    }
  }
};
template <int ROWS, int NTH> struct Loader<OP_BF16_K, ROWS, NTH> : LoaderK<OP_BF16_K, ROWS, NTH> {};
template <int ROWS, int NTH> struct Loader<OP_F32_K, ROWS, NTH> : LoaderK<OP_F32_K, ROWS, NTH> {};
template <int ROWS, int NTH> struct Loader<OP_F16_K, ROWS, NTH> : LoaderK<OP_F16_K, ROWS, NTH> {};

// bf16 pair, K contiguous: an fp32 quantity kept as two bf16 planes, its hi
// values at the operand's rows and its lo values pair_off elements further
// on; they go to the hi and lo tiles exactly as a split fp32 operand's do.
template <int ROWS, int NTH>
struct Loader<OP_BF16P_K, ROWS, NTH> {
  static constexpr int CH = ROWS * 8 / NTH;
  static_assert(CH * NTH == ROWS * 8, "tile rows must divide the thread count");
  const char* base;
  uint32_t lo;
  uint32_t off[CH];
  uint4 rh[CH], rl[CH];
  __device__ void init(const Operand& op, int row0, int tid) {
    base = (const char*)op.ptr;
    lo = (uint32_t)op.pair_off;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int id = tid + q * NTH;
      int gr = min(row0 + (id >> 3), op.nrows - 1);
      if (op.gather) gr = op.gather[gr];
      off[q] = (uint32_t)gr * (uint32_t)op.ld + (uint32_t)(id & 7) * 8;
    }
  }
  __device__ void load(int k0, int /*K*/) {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      rh[q] = *(const uint4*)(base + ((uint64_t)off[q] + (uint32_t)k0) * 2);
      rl[q] = *(const uint4*)(base + ((uint64_t)off[q] + lo + (uint32_t)k0) * 2);
    }
  }
  // 8-byte LDS stores, as in LoaderK: the 16-byte form measured twice the
  // bank conflicts (29% against 14%) in the same GEMM
  __device__ void store(char* lds, char* lds_lo, int tid) const {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int id = tid + q * NTH;
      const int o = swz(id >> 3, id & 7);
      *(uint2*)(lds + o) = make_uint2(rh[q].x, rh[q].y);
      *(uint2*)(lds + o + 8) = make_uint2(rh[q].z, rh[q].w);
      *(uint2*)(lds_lo + o) = make_uint2(rl[q].x, rl[q].y);
      *(uint2*)(lds_lo + o + 8) = make_uint2(rl[q].z, rl[q].w);
    }
  }
};

// 16-bit [K][rows] operands (used as B): each K tile is copied into LDS as it
// is laid out in memory, [k][row] with a padded pitch of 2*ROWS + 32 bytes
// (consecutive k rows 32 bytes apart modulo 128, so the four rows one
// transpose read touches sit in different bank groups), with 16-byte stores,
// and the MFMA fragments are read with the gfx950 transpose load
// ds_read_b64_tr_b16 (lane i of a 16-lane group receives element i of four
// consecutive k rows).  TO_F16 converts bf16 to fp16 on the way in.
template <int ROWS, int NTH, bool TO_F16>
struct LoaderTR {
  static_assert(ROWS % 64 == 0, "transposed operand block must be a multiple of 64 rows");
  static constexpr int PITCH = ROWS * 2 + 32;
  static constexpr int CPR = ROWS / 8;             // 16-byte chunks per k row
  static constexpr int CH = 64 * CPR / NTH;
  static_assert(CH * NTH == 64 * CPR, "bad thread count");
  const uint16_t* base;
  int64_t ld;
  const int* gather;
  int row0;
  uint4 r[CH];
  __device__ void init(const Operand& op, int row0_, int /*tid*/) {
    base = (const uint16_t*)op.ptr; ld = op.ld; gather = op.gather; row0 = row0_;
  }
  __device__ static uint32_t cvt2(uint32_t w) {
    const _Float16 lo = (_Float16)bf16_lo(w), hi = (_Float16)bf16_hi(w);
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  __device__ void load(int k0, int K) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int id = tid + q * NTH;
      const int k = id / CPR, cc = id - k * CPR;
      int gk = k0 + k;
      if (gk < K) {
        if (gather) gk = gather[gk];
        r[q] = *(const uint4*)(base + (int64_t)gk * ld + row0 + cc * 8);
        if constexpr (TO_F16) r[q] = make_uint4(cvt2(r[q].x), cvt2(r[q].y), cvt2(r[q].z), cvt2(r[q].w));
      } else {
        r[q] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ void store(char* lds, char* /*lds_lo*/, int tid) const {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int id = tid + q * NTH;
      const int k = id / CPR, cc = id - k * CPR;
      *(uint4*)(lds + k * PITCH + cc * 16) = r[q];
    }
  }
};
template <int ROWS, int NTH> struct Loader<OP_BF16_T, ROWS, NTH> : LoaderTR<ROWS, NTH, false> {};
template <int ROWS, int NTH> struct Loader<OP_BF16_T16, ROWS, NTH> : LoaderTR<ROWS, NTH, true> {};

typedef short trv4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) trv4i16 lds_trv4i16;
typedef __attribute__((address_space(3))) char lds_trchar;

// B fragment of a 32x32x16 MFMA from a [k][col] tile: k = 16*kk + 8*(lane/32)
// + 0..7, column col0 + lane%32.
__device__ __forceinline__ uint4 tr_frag(const char* tile, int pitch, int kk, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int krow = 16 * kk + 8 * (g >> 1) + (i >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (i & 3);
  lds_trchar* p = (lds_trchar*)tile + krow * pitch + col * 2;
  const trv4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_trv4i16*)p);
  const trv4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_trv4i16*)(p + 4 * pitch));
  const uint2 u0 = __builtin_bit_cast(uint2, v0), u1 = __builtin_bit_cast(uint2, v1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

// fp32 [rows][K] split into bf16 hi/lo tiles: 16 chunks of 4 floats per row.
template <int ROWS, int NTH>
struct Loader<OP_F32S_K, ROWS, NTH> {
  static constexpr int CH = ROWS * 16 / NTH;
  static_assert(CH * NTH == ROWS * 16, "bad thread count");
  const float* base;
  uint32_t off[CH];
  uint4 r[CH];
  __device__ void init(const Operand& op, int row0, int tid) {
    base = (const float*)op.ptr;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int id = tid + q * NTH;
      int gr = min(row0 + (id >> 4), op.nrows - 1);
      if (op.gather) gr = op.gather[gr];
      off[q] = (uint32_t)gr * (uint32_t)op.ld + (uint32_t)(id & 15) * 4u;
    }
  }
  __device__ void load(int k0, int /*K*/) {
#pragma unroll
    for (int q = 0; q < CH; ++q) r[q] = *(const uint4*)(base + (uint64_t)off[q] + (uint32_t)k0);
  }
  __device__ void store(char* lds_hi, char* lds_lo, int tid) const {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int id = tid + q * NTH;
      int row = id >> 4, c4 = id & 15;
      uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
      split_bf16(__uint_as_float(r[q].x), h0, l0);
      split_bf16(__uint_as_float(r[q].y), h1, l1);
      split_bf16(__uint_as_float(r[q].z), h2, l2);
      split_bf16(__uint_as_float(r[q].w), h3, l3);
      int off = swz(row, c4 >> 1) + (c4 & 1) * 8;
      *(uint2*)(lds_hi + off) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      *(uint2*)(lds_lo + off) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
    }
  }
};

// fp32 [K][rows] split into bf16 hi/lo tiles: a chunk is 4 rows at one k.
template <int ROWS, int NTH>
struct Loader<OP_F32S_T, ROWS, NTH> {
  static_assert(ROWS % 32 == 0, "bad rows");
  static constexpr int CH = 64 * ROWS / 4 / NTH;
  static_assert(CH * NTH == 64 * ROWS / 4, "bad thread count");
  const float* base;
  int64_t ld;
  const int* gather;
  int row0;
  uint4 r[CH];
  __device__ static void coords(int id, int& k, int& rc) {
    const int rch = ROWS / 32;
    int rest = id >> 6;
    rc = (rest % rch) * 8 + ((id >> 3) & 7);
    k = (rest / rch) * 8 + (id & 7);
  }
  __device__ void init(const Operand& op, int row0_, int /*tid*/) {
    base = (const float*)op.ptr; ld = op.ld; gather = op.gather; row0 = row0_;
  }
  __device__ void load(int k0, int K) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int k, rc;
      coords(tid + q * NTH, k, rc);
      int gk = k0 + k;
      if (gk < K) {
        if (gather) gk = gather[gk];
        r[q] = *(const uint4*)(base + (int64_t)gk * ld + row0 + rc * 4);
      } else {
        r[q] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ void store(char* lds_hi, char* lds_lo, int tid) const {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int k, rc;
      coords(tid + q * NTH, k, rc);
      const uint32_t w[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h, l;
        split_bf16(__uint_as_float(w[i]), h, l);
        int off = swz(rc * 4 + i, k >> 3) + ((k & 7) << 1);
        *(uint16_t*)(lds_hi + off) = (uint16_t)h;
        *(uint16_t*)(lds_lo + off) = (uint16_t)l;
      }
    }
  }
};

// fp32 [K][rows] for fp32 MFMA: a chunk is 4 rows at one k; K tile is 32.
template <int ROWS, int NTH>
struct Loader<OP_F32_T, ROWS, NTH> {
  static_assert(ROWS % 32 == 0, "bad rows");
  static constexpr int CH = 32 * ROWS / 4 / NTH;
  static_assert(CH * NTH == 32 * ROWS / 4, "bad thread count");
  const float* base;
  int64_t ld;
  const int* gather;
  int row0;
  uint4 r[CH];
  __device__ static void coords(int id, int& k, int& rc) {
    const int rch = ROWS / 32;
    int rest = id >> 6;
    rc = (rest % rch) * 8 + ((id >> 3) & 7);
    k = (rest / rch) * 8 + (id & 7);
  }
  __device__ void init(const Operand& op, int row0_, int /*tid*/) {
    base = (const float*)op.ptr; ld = op.ld; gather = op.gather; row0 = row0_;
  }
  __device__ void load(int k0, int K) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int k, rc;
      coords(tid + q * NTH, k, rc);
      int gk = k0 + k;
      if (gk < K) {
        if (gather) gk = gather[gk];
        r[q] = *(const uint4*)(base + (int64_t)gk * ld + row0 + rc * 4);
      } else {
        r[q] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ void store(char* lds, char* /*lds_lo*/, int tid) const {
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      int k, rc;
      coords(tid + q * NTH, k, rc);
      const uint32_t w[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(uint32_t*)(lds + swz(rc * 4 + i, k >> 2) + ((k & 3) << 2)) = w[i];
    }
  }
};

// ------------------------------------------------------------------ mainloop

template <int BM_, int BN_, int WM_, int WN_, int AKIND, int BKIND, int NB_ = 1>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NB = NB_;
  static constexpr int NTH = WM * WN * WAVE;
  static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold whole 32x32 blocks");
  static constexpr bool SINGLE = false;
  static constexpr bool ASPLIT = KindInfo<AKIND>::split;
  static constexpr bool F32MMA = KindInfo<AKIND>::f32mma;
  static constexpr bool F16MMA = KindInfo<AKIND>::f16;
  static_assert(KindInfo<BKIND>::f32mma == F32MMA, "A and B must both be fp32 or both bf16");
  static_assert(KindInfo<BKIND>::f16 == F16MMA, "A and B must both be fp16 or neither");
  static_assert(!KindInfo<BKIND>::split, "B operand is never split");
  static constexpr int KT = ktile<AKIND>();
  static constexpr bool BTR = KindInfo<BKIND>::trans && KindInfo<BKIND>::esz == 2;   // B read by transpose loads
  static constexpr int B_PITCH = BN * 2 + 32;
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BTR ? 64 * B_PITCH : BN * 128;
  static constexpr int STAGE = A_BYTES * (ASPLIT ? 2 : 1) + B_BYTES * NB;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static constexpr int EPI_BYTES = LDS_BYTES;
  static constexpr int A_KIND = AKIND, B_KIND = BKIND;
};

template <class Cfg>
struct GemmTile {
  static constexpr int TM = Cfg::TM, TN = Cfg::TN, NB = Cfg::NB, NTH = Cfg::NTH;
  f32x16 acc[NB][TM][TN];

  // Multiply the MxN block at (m0, n0) over K; LDS is Cfg::LDS_BYTES.  With
  // zero == false the products are added to the accumulators already held
  // (a second operand pair summed into the same block).
  __device__ void run(const Operand& A, const Operand* B, int m0, int n0, int K, char* lds,
                      bool zero = true) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = (wave / Cfg::WN) * (Cfg::BM / Cfg::WM);
    const int wc = (wave % Cfg::WN) * (Cfg::BN / Cfg::WN);
    if (zero) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[b][i][j][e] = 0.f;
    }

    Loader<Cfg::A_KIND, Cfg::BM, NTH> la;
    Loader<Cfg::B_KIND, Cfg::BN, NTH> lb[NB];
    la.init(A, m0, tid);
#pragma unroll
    for (int b = 0; b < NB; ++b) lb[b].init(B[b], n0, tid);

    const int nk = (K + Cfg::KT - 1) / Cfg::KT;
    auto stage_ptr = [&](int s) { return lds + s * Cfg::STAGE; };
    auto a_hi = [&](int s) { return stage_ptr(s); };
    auto a_lo = [&](int s) { return stage_ptr(s) + Cfg::A_BYTES; };
    auto b_ptr = [&](int s, int b) {
      return stage_ptr(s) + Cfg::A_BYTES * (Cfg::ASPLIT ? 2 : 1) + b * Cfg::B_BYTES;
    };

    if (nk > 0) {
      la.load(0, K);
#pragma unroll
      for (int b = 0; b < NB; ++b) lb[b].load(0, K);
      la.store(a_hi(0), a_lo(0), tid);
#pragma unroll
      for (int b = 0; b < NB; ++b) lb[b].store(b_ptr(0, b), nullptr, tid);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load((kt + 1) * Cfg::KT, K);
#pragma unroll
        for (int b = 0; b < NB; ++b) lb[b].load((kt + 1) * Cfg::KT, K);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = 2 * kk + (lane >> 5);
        uint4 fa[TM], fal[Cfg::ASPLIT ? TM : 1], fb[NB][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          fa[i] = *(const uint4*)(a_hi(cur) + swz(wr + i * 32 + (lane & 31), ch));
          if constexpr (Cfg::ASPLIT)
            fal[i] = *(const uint4*)(a_lo(cur) + swz(wr + i * 32 + (lane & 31), ch));
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (Cfg::BTR) fb[b][j] = tr_frag(b_ptr(cur, b), Cfg::B_PITCH, kk, wc + j * 32, lane);
            else fb[b][j] = *(const uint4*)(b_ptr(cur, b) + swz(wc + j * 32 + (lane & 31), ch));
          }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              if constexpr (Cfg::F32MMA) {
                acc[b][i][j] = mfma32_f32(fa[i], fb[b][j], acc[b][i][j]);
              } else if constexpr (Cfg::F16MMA) {
                acc[b][i][j] = mfma32_f16(fa[i], fb[b][j], acc[b][i][j]);
              } else {
                acc[b][i][j] = mfma32(fa[i], fb[b][j], acc[b][i][j]);
                if constexpr (Cfg::ASPLIT) acc[b][i][j] = mfma32(fal[i], fb[b][j], acc[b][i][j]);
              }
            }
      }
      if (more) {
        la.store(a_hi(cur ^ 1), a_lo(cur ^ 1), tid);
#pragma unroll
        for (int b = 0; b < NB; ++b) lb[b].store(b_ptr(cur ^ 1, b), nullptr, tid);
      }
      __syncthreads();
    }
  }

  // Row (within the block) and column of accumulator element e of block (i, j).
  __device__ static int row_of(int i, int e) {
    const int wave = threadIdx.x >> 6;
    return (wave / Cfg::WN) * (Cfg::BM / Cfg::WM) + i * 32 + mfma32_row(threadIdx.x & 63, e);
  }
  __device__ static int col_of(int j) {
    const int wave = threadIdx.x >> 6;
    return (wave % Cfg::WN) * (Cfg::BN / Cfg::WN) + j * 32 + (threadIdx.x & 31);
  }
};


// ------------------------------------------------------------------ direct-to-LDS mainloop
//
// For 16-bit K-major operands (bf16, or fp16 with F16) the K tiles move from
// global memory straight into LDS with global_load_lds_dwordx4: no staging
// registers and no LDS store instructions in the wave's stream, so the loads
// of tile k+1 run entirely under the MFMAs of tile k.  One instruction fills
// 1 KB of LDS (lane l writes bytes 16l..16l+15 of it), which is 8 consecutive
// 128-byte tile rows; the XOR swizzle is applied on the global side: the lane
// that lands on physical chunk p of row r fetches logical chunk
// p ^ (r & 7) ^ ((r >> 3) & 7) (the swizzle is its own inverse), so the
// fragment reads see the same swizzled layout as swz().  The two stage buffers
// are separate LDS arrays owned by the kernel: the compiler can then tell that
// a fragment read of one stage never overlaps the loads in flight into the
// other, and it waits for those loads only where the loop says so (a vmcnt
// wait before the barrier that hands the next stage over).
// With Cfg::BT the B operand is [K][N] (N contiguous, K optionally gathered
// through B.gather): its tile is stored as it lies in memory, 64 k-rows of
// 2*BN bytes whose 16-byte pieces are XOR-swizzled by tr_swz(k), and read
// with the gfx950 transpose load.  A 16-lane group of a transpose read takes
// 32 contiguous bytes of four consecutive k-rows and the next group the 32
// bytes after them; XOR-ing the piece index by 4*(k & 3) puts the 16 pieces
// one half-wave touches in 16 different bank groups (rows of at least 16
// pieces; narrower tiles use 2*(k & 3), distinct within each 16-lane group).  K need not be a multiple of 64 there:
// the gathered k index is clamped to K-1, so the rows read past K are real
// rows, and the caller's A must hold zeros in those K columns.
// With Cfg::AT the A operand is [K][M] in the same way (never gathered, K a
// multiple of 64), its fragments read with the same transpose load.
template <int BM_, int BN_, int WM_, int WN_, int NB_ = 1, bool F16_ = false, bool BT_ = false, bool AT_ = false>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NB = NB_;
  static constexpr bool F16MMA = F16_;
  static constexpr bool BT = BT_;                  // B given as [K][N] (see DmaTile)
  static constexpr bool AT = AT_;                  // A given as [K][M], never gathered
  static constexpr bool SINGLE = false;            // one stage buffer (DmaCfg1)
  static_assert(!BT || NB == 1, "a transposed B operand comes alone");
  static constexpr int NW = WM * WN, NTH = NW * WAVE;
  static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold whole 32x32 blocks");
  static constexpr int KT = 64;
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int EPI_BYTES = STAGE;                         // contiguous LDS free after run()
  static constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW);   // 1 KB loads per wave per operand
  static_assert(LA * 8 * NW == BM && LB * 8 * NW == BN, "block rows must split into whole 1 KB loads per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Single-stage variant: one stage buffer (a 128x256 tile needs 48 KB), so
// that two workgroups share a CU.  Inside a workgroup the loads of a K tile
// no longer run under the MFMAs of the previous one; the other workgroup's
// MFMAs fill that time, and each workgroup's output stores drain while the
// other one computes.  Kernels built on it declare __launch_bounds__(NTH,
// WPE): registers for two workgroups.
template <int BM_, int BN_, int WM_, int WN_, int NB_ = 1, bool F16_ = false, bool BT_ = false, bool AT_ = false>
struct DmaCfg1 : DmaCfg<BM_, BN_, WM_, WN_, NB_, F16_, BT_, AT_> {
  typedef DmaCfg<BM_, BN_, WM_, WN_, NB_, F16_, BT_, AT_> Base;
  static constexpr bool SINGLE = true;
  static constexpr int LDS_BYTES = Base::STAGE;
  static constexpr int WPE = 2 * Base::NW / 4;
  static_assert(2 * Base::STAGE <= 160 * 1024, "two workgroups per CU");
};

typedef __attribute__((address_space(3))) void lds_void;

// XOR applied to the 16-byte piece index of k-row k of a transposed tile
// whose rows hold `pieces` pieces.
__device__ __forceinline__ int tr_swz(int k, int pieces) { return (pieces >= 16 ? 4 : 2) * (k & 3); }

template <class Cfg>
struct DmaTile {
  static constexpr int TM = Cfg::TM, TN = Cfg::TN, NB = Cfg::NB, NW = Cfg::NW;
  f32x16 acc[NB][TM][TN];

  // Multiply the block at (m0, n0) over K (a multiple of 64 unless B is
  // transposed); st0 and st1 are the kernel's two stage arrays of Cfg::STAGE
  // bytes each.  Both are free again when run() returns.
  __device__ void run(const Operand& A, const Operand* B, int m0, int n0, int K, char* st0, char* st1,
                      bool zero = true) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = (wave / Cfg::WN) * (Cfg::BM / Cfg::WM);
    const int wc = (wave % Cfg::WN) * (Cfg::BN / Cfg::WN);
    if (zero) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[b][i][j][e] = 0.f;
    }

    // per-lane byte offsets (below 2^32: each operand is under 4 GB) of the
    // rows this lane fills; the K-tile base is wave-uniform, so each load is
    // one scalar base plus one 32-bit lane offset
    const int rsub = lane >> 3, p = lane & 7;
    uint32_t offa[Cfg::LA], offb[NB][Cfg::LB];
    constexpr int AROWB = Cfg::BM * 2, KPIA = 1024 / AROWB;  // transposed A: bytes per k-row, k-rows per load
#pragma unroll
    for (int q = 0; q < Cfg::LA; ++q) {
      if constexpr (Cfg::AT) {
        const int kr = (q * NW + wave) * KPIA + (16 * lane) / AROWB, pc = ((16 * lane) % AROWB) / 16;
        offa[q] = (uint32_t)kr * (uint32_t)A.ld * 2u + (uint32_t)(m0 * 2 + ((pc ^ tr_swz(kr, AROWB / 16)) << 4));
      } else {
        const int r = (q * NW + wave) * 8 + rsub;
        int gr = min(m0 + r, A.nrows - 1);
        if (A.gather) gr = A.gather[gr];
        offa[q] = ((uint32_t)gr * (uint32_t)A.ld + (uint32_t)(((p ^ r ^ (r >> 3)) & 7) * 8)) * 2u;
      }
    }
    constexpr int BROWB = Cfg::BN * 2, KPI = 1024 / BROWB;   // transposed B: bytes per k-row, k-rows per load
    const int* bgat = Cfg::BT ? B[0].gather : nullptr;
    const int nk = (K + 63) / 64;
    // a transposed B tile's 64 k-rows: wave w loads the KW = 64/NW k-rows
    // KW*w..KW*w+KW-1 (LB loads of KPI k-rows each), so its gathered indices
    // are KW consecutive list entries
    constexpr int KW = Cfg::LB * KPI;
    static_assert(!Cfg::BT || (KW * NW == 64 && KW % 8 == 0), "whole groups of eight k-rows per wave");
    auto bt_krow = [&](int q) { return (wave * Cfg::LB + q) * KPI + (16 * lane) / BROWB; };
    // gathered k rows of the next tile to issue, all wave-uniform: scalar
    // loads of the wave's list entries, eight at a time (constant address
    // space, into SGPRs, which keeps them out of the vector memory counter the
    // stage hand-over waits on); in the last tile, entries at or past K are
    // replaced by entry K-1 (a real row; A holds zeros in those K columns).
    // The list must hold roundup64(K) readable entries.
    typedef __attribute__((address_space(4))) const int cint;
    typedef int v8i __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(4))) const v8i cv8i;
    cint* cgat = (cint*)bgat;
    uint32_t gsc[Cfg::LB][KPI];
    auto bt_fetch = [&](int kt) {
      const int k0 = kt * 64 + wave * KW;
      const bool tail = k0 + KW > K;
      const int last = tail ? cgat[K - 1] : 0;
#pragma unroll
      for (int g8 = 0; g8 < KW / 8; ++g8) {
        v8i v = *(cv8i*)(cgat + k0 + 8 * g8);
        if (tail) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = k0 + 8 * g8 + j < K ? v[j] : last;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) gsc[(8 * g8 + j) / KPI][(8 * g8 + j) % KPI] = (uint32_t)v[j];
      }
    };
    auto gidx = [&](int q) {
      const int kl = (16 * lane) / BROWB;
      uint32_t v = gsc[q][0];
#pragma unroll
      for (int j = 1; j < KPI; ++j) v = kl == j ? gsc[q][j] : v;
      return v;
    };
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < Cfg::LB; ++q) {
        if constexpr (Cfg::BT) {
          const int kr = bt_krow(q), pc = ((16 * lane) % BROWB) / 16;
          const uint32_t col = (uint32_t)(n0 * 2 + ((pc ^ tr_swz(kr, BROWB / 16)) << 4));
          offb[b][q] = bgat ? col : (uint32_t)kr * (uint32_t)B[0].ld * 2u + col;
        } else {
          const int r = (q * NW + wave) * 8 + rsub;
          int gr = min(n0 + r, B[b].nrows - 1);
          if (B[b].gather) gr = B[b].gather[gr];
          offb[b][q] = ((uint32_t)gr * (uint32_t)B[b].ld + (uint32_t)(((p ^ r ^ (r >> 3)) & 7) * 8)) * 2u;
        }
      }
    if (Cfg::BT && bgat && nk > 0) bt_fetch(0);
    // buffer resources (base, byte range) of the operands: the loads are
    // buffer_load ... lds with a per-lane offset that stays fixed over the K
    // loop and a wave-uniform per-tile offset, so no address arithmetic is
    // repeated per tile (the range also bounds every access)
    // (a gathered operand's rows are not bounded by nrows: its range is open)
    auto rsrc = [](const Operand& op, int64_t rows) {
      const int64_t bytes = op.gather ? 0xffffffffLL : rows * op.ld * 2;
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(op.ptr), (short)0,
                                               (int)(uint32_t)(bytes < 0xffffffffLL ? bytes : 0xffffffffLL), 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t ra = rsrc(A, Cfg::AT ? (int64_t)K : (int64_t)A.nrows);
    __amdgpu_buffer_rsrc_t rb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) rb[b] = rsrc(B[b], Cfg::BT ? (int64_t)K : (int64_t)B[b].nrows);
    uint32_t bvo[Cfg::LB];            // gathered B: this tile's lane offsets, kept live through compute()

    auto issue = [&](int kt, char* st) {
      const uint32_t ka = Cfg::AT ? (uint32_t)kt * 64u * (uint32_t)A.ld * 2u : (uint32_t)kt * 128u;
#pragma unroll
      for (int q = 0; q < Cfg::LA; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (q * NW + wave) * 1024), 16, offa[q], ka, 0, 0);
      if constexpr (Cfg::BT) {
        if (bgat) {
#pragma unroll
          for (int q = 0; q < Cfg::LB; ++q) {
            bvo[q] = gidx(q) * (uint32_t)B[0].ld * 2u + offb[0][q];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[0], (lds_void*)(st + Cfg::A_BYTES + (wave * Cfg::LB + q) * 1024),
                                                     16, bvo[q], 0u, 0, 0);
          }
          if (kt + 1 < nk) bt_fetch(kt + 1);
        } else {
#pragma unroll
          for (int q = 0; q < Cfg::LB; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[0], (lds_void*)(st + Cfg::A_BYTES + (wave * Cfg::LB + q) * 1024),
                                                     16, offb[0][q], (uint32_t)kt * 64u * (uint32_t)B[0].ld * 2u, 0, 0);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int q = 0; q < Cfg::LB; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb[b],
                                                     (lds_void*)(st + Cfg::A_BYTES + b * Cfg::B_BYTES + (q * NW + wave) * 1024),
                                                     16, offb[b][q], (uint32_t)kt * 128u, 0, 0);
      }
    };
    // transposed B: this lane's byte offset inside the tile for column block
    // j (the k-tile and half offsets are added as constants).  It is passed
    // through an empty asm so that the optimizer keeps each read's address a
    // short chain from the LDS array (long chains lose the alias information
    // that lets the reads run under the loads in flight into the other stage).
    int btl[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int g = lane >> 4, i = lane & 15;
      const int krow = 8 * (g >> 1) + (i >> 2);
      const int col = wc + j * 32 + 16 * (g & 1) + 4 * (i & 3);
      btl[j] = krow * BROWB + (((col >> 3) ^ tr_swz(krow, BROWB / 16)) << 4) + (col & 7) * 2;
      if constexpr (Cfg::BT) asm volatile("" : "+v"(btl[j]));
    }
    int atl[TM];                      // the same for a transposed A, row block i
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int g = lane >> 4, ii = lane & 15;
      const int krow = 8 * (g >> 1) + (ii >> 2);
      const int row = wr + i * 32 + 16 * (g & 1) + 4 * (ii & 3);
      atl[i] = krow * AROWB + (((row >> 3) ^ tr_swz(krow, AROWB / 16)) << 4) + (row & 7) * 2;
      if constexpr (Cfg::AT) asm volatile("" : "+v"(atl[i]));
    }
    auto compute = [&](const char* st) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = 2 * kk + (lane >> 5);
        uint4 fa[TM], fb[NB][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (Cfg::AT) {
            lds_trchar* q0 = (lds_trchar*)st + atl[i] + 16 * kk * AROWB;
            const trv4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_trv4i16*)q0);
            const trv4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_trv4i16*)(q0 + 4 * AROWB));
            const uint2 u0 = __builtin_bit_cast(uint2, v0), u1 = __builtin_bit_cast(uint2, v1);
            fa[i] = make_uint4(u0.x, u0.y, u1.x, u1.y);
          } else {
            fa[i] = *(const uint4*)(st + swz(wr + i * 32 + (lane & 31), ch));
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (Cfg::BT) {
              lds_trchar* q0 = (lds_trchar*)st + btl[j] + (Cfg::A_BYTES + 16 * kk * BROWB);
              const trv4i16 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_trv4i16*)q0);
              const trv4i16 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_trv4i16*)(q0 + 4 * BROWB));
              const uint2 u0 = __builtin_bit_cast(uint2, v0), u1 = __builtin_bit_cast(uint2, v1);
              fb[b][j] = make_uint4(u0.x, u0.y, u1.x, u1.y);
            } else {
              fb[b][j] = *(const uint4*)(st + Cfg::A_BYTES + b * Cfg::B_BYTES + swz(wc + j * 32 + (lane & 31), ch));
            }
          }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              if constexpr (Cfg::F16MMA) acc[b][i][j] = mfma32_f16(fa[i], fb[b][j], acc[b][i][j]);
              else acc[b][i][j] = mfma32(fa[i], fb[b][j], acc[b][i][j]);
            }
        // scheduling hint: alternate one MFMA and one LDS read, so the reads
        // of the next step issue under this step's MFMAs
#pragma unroll
        for (int q = 0; q < NB * TM * TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    // Hand-over of a stage: this wave's loads are complete (vmcnt(0), the
    // other counters left alone), then the workgroup barrier.  The empty asm
    // statements keep the compiler from moving LDS accesses across it.
    auto stage_barrier = [] {
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // tile kt: wait for it, start loading tile kt+1 into the other stage, compute
    auto step = [&](int kt, const char* cur, char* nxt) {
      stage_barrier();
      if (kt + 1 < nk) issue(kt + 1, nxt);
      compute(cur);
      if constexpr (Cfg::BT) {
        // the loads just issued may still read their offset registers: keep
        // them from being reused by the fragment reads above
        if (bgat) {
#pragma unroll
          for (int q = 0; q < Cfg::LB; ++q) asm volatile("" ::"v"(bvo[q]));
        }
      }
    };
    if constexpr (Cfg::SINGLE) {
      // one buffer: load, hand over, compute, and let every wave finish its
      // fragment reads before the next tile's loads overwrite it
      for (int kt = 0; kt < nk; ++kt) {
        issue(kt, st0);
        stage_barrier();
        compute(st0);
        if constexpr (Cfg::BT) {
          if (bgat) {
#pragma unroll
            for (int q = 0; q < Cfg::LB; ++q) asm volatile("" ::"v"(bvo[q]));
          }
        }
        __syncthreads();
      }
    } else {
      if (nk > 0) issue(0, st0);
      int kt = 0;
      for (; kt + 1 < nk; kt += 2) {
        step(kt, st0, st1);
        step(kt + 1, st1, st0);
      }
      if (kt < nk) step(kt, st0, st1);
      __syncthreads();
    }
  }

  __device__ static int row_of(int i, int e) {
    const int wave = threadIdx.x >> 6;
    return (wave / Cfg::WN) * (Cfg::BM / Cfg::WM) + i * 32 + mfma32_row(threadIdx.x & 63, e);
  }
  __device__ static int col_of(int j) {
    const int wave = threadIdx.x >> 6;
    return (wave % Cfg::WN) * (Cfg::BN / Cfg::WN) + j * 32 + (threadIdx.x & 31);
  }
};

// Waves per SIMD a kernel on this configuration is compiled for (the second
// __launch_bounds__ argument): WPE for the single-stage configurations, else
// no constraint.
template <class C, class = void> struct WavesPerEU { static constexpr int value = 1; };
template <class C> struct WavesPerEU<C, std::void_t<decltype(C::WPE)>> { static constexpr int value = C::WPE; };

// Mainloop type of a configuration.
template <class Cfg> struct TileFor { typedef GemmTile<Cfg> type; static constexpr bool dma = false; };
template <int BM, int BN, int WM, int WN, int NB, bool F16, bool BT, bool AT>
struct TileFor<DmaCfg<BM, BN, WM, WN, NB, F16, BT, AT>> {
  typedef DmaTile<DmaCfg<BM, BN, WM, WN, NB, F16, BT, AT>> type;
  static constexpr bool dma = true;
};
template <int BM, int BN, int WM, int WN, int NB, bool F16, bool BT, bool AT>
struct TileFor<DmaCfg1<BM, BN, WM, WN, NB, F16, BT, AT>> {
  typedef DmaTile<DmaCfg1<BM, BN, WM, WN, NB, F16, BT, AT>> type;
  static constexpr bool dma = true;
};

}  // namespace twell
