// Shared device helpers for the TwELL kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;
constexpr int TILE_R = 16;   // rows per TwELL tile
constexpr int TILE_C = 64;   // columns per TwELL tile (= wave width: one ballot per row segment)

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even float -> bf16 (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Split v into hi = bf16(v) and lo = bf16(v - hi): hi + lo carries about 16
// significant bits, so an fp32 intermediate can feed a bf16 MFMA twice
// (hi and lo) and keep fp32-level accuracy.
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - __uint_as_float(hi << 16));
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// fp32 operands: a 16-byte fragment holds 4 consecutive k of one row; four
// 32x32x2 MFMAs consume it (MFMA q takes element q from every lane).
__device__ __forceinline__ f32x16 mfma32_f32(const uint4& a, const uint4& b, f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ f32x4 mfma16_f32(const uint4& a, const uint4& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

// Output layout of a 32x32 MFMA block: lane l, register i holds
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32.
__device__ __forceinline__ int mfma32_row(int lane, int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }
// Output layout of a 16x16 MFMA block: lane l, register i holds row 4*(l/16)+i, column l%16.
__device__ __forceinline__ int mfma16_row(int lane, int i) { return 4 * (lane >> 4) + i; }

// ---------------------------------------------------------------- LDS tiles
// A tile row is 128 bytes (64 bf16 or 32 fp32 of K) split in eight 16-byte
// chunks.  Chunk c of row r lives at physical chunk c ^ (r & 7) ^ ((r >> 3) & 7):
// eight consecutive rows read at the same chunk hit eight different bank
// groups (fragment reads), and the transposed 16-bit writes of eight rows
// that are eight apart land in different bank groups as well.
__device__ __forceinline__ int swz(int row, int chunk) {
  return (row << 7) + (((chunk ^ row ^ (row >> 3)) & 7) << 4);
}

// ---------------------------------------------------------------- misc

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Bits of m strictly below position c (c in 0..63).
__device__ __forceinline__ uint64_t below(int c) { return (c == 0) ? 0ull : (~0ull >> (64 - c)); }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Wave-uniform read of a value held by lane src.
__device__ __forceinline__ int readlane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Map a linear workgroup id so that the ids the hardware sends to one XCD
// (consecutive ids go round-robin over the 8 XCDs) form a contiguous range of
// the logical tile order, which keeps the tiles sharing operands in one L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  if ((n & 7) != 0) return id;
  return (id & 7) * (n >> 3) + (id >> 3);
}

}  // namespace twell
