// Shared device helpers for the gfx950 kernels of the DFlash drafter library.
//
// The one idea every matrix kernel here is built on: an MFMA 16x16 step takes,
// from each of its 64 lanes, one 16-byte fragment of the A operand and one of
// the B operand. Lane l covers row (A) / column (B) l % 16 and contributes its
// elements to the contraction; the hardware pairs A's element e of lane group
// l / 16 with B's element e of the same lane group. As long as both operands
// are loaded with the same (lane group, element) -> k assignment, any such
// assignment yields the same dot products. The kernels use that freedom to
// give each lane long contiguous runs of k (64 bytes) so global loads are
// wide and coalesced.
//
//   bf16: one 16-byte fragment = 8 elements = one v_mfma_f32_16x16x32_bf16.
//   fp32: one 16-byte fragment = 4 elements = four v_mfma_f32_16x16x4_f32.
//
// Output (C/D) layout of a 16x16 tile: lane l holds rows 4*(l/16)+i, i=0..3,
// of column l % 16.
//
// Tiled layout of the GEMM operands. Every projection weight, and every
// activation matrix a projection reads from the library's own workspace, is
// stored in the order the MFMA loop consumes it: rows in tiles of 16, k in
// chunks of KC = 16 * EPF elements (256 bytes of a row), and inside one
// (row tile, chunk) block four 1 KB fragments, fragment f holding for lane
// l = r + 16 g the EPF elements of row r at k = KC*c + 4*EPF*f + EPF*g.
// One load instruction of a wave then reads 1 KB of contiguous memory (eight
// whole 128-byte lines) instead of 64 bytes from each of 16 rows. Rows are
// padded to a multiple of 16 and k to a multiple of KC; weight padding is
// zero, activation padding is never read into a stored result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct ElemInfo;
template <> struct ElemInfo<float> {
  static constexpr int per16 = 4;  // elements per 16-byte fragment
};
template <> struct ElemInfo<bf16> {
  static constexpr int per16 = 8;
};

// Element offset of (row, k) in a tiled matrix whose rows hold nck chunks.
template <typename T>
__host__ __device__ __forceinline__ int64_t tiled_index(int row, int k, int nck) {
  constexpr int EPF = 16 / (int)sizeof(T);
  constexpr int KC = 16 * EPF;
  const int c = k / KC, kk = k % KC;
  const int f = kk / (4 * EPF), g = (kk / EPF) & 3, e = kk % EPF;
  return ((((int64_t)(row >> 4) * nck + c) * 4 + f) * 64 + g * 16 + (row & 15)) * EPF + e;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// acc += A_frag * B_frag over one 16-byte fragment per lane.
template <typename T>
__device__ __forceinline__ f32x4 mfma_frag(u32x4 a, u32x4 b, f32x4 acc);

template <>
__device__ __forceinline__ f32x4 mfma_frag<bf16>(u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mfma_frag<float>(u32x4 a, u32x4 b, f32x4 acc) {
  // Reinterpret the whole vector, then index it: bit-casting single elements
  // of an ext-vector (bit_cast<float>(a.y)) is folded to element 0 by this
  // compiler, which silently drops three quarters of the products.
  const f32x4 af = __builtin_bit_cast(f32x4, a);
  const f32x4 bf = __builtin_bit_cast(f32x4, b);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[0], bf[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[1], bf[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[2], bf[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[3], bf[3], acc, 0, 0, 0);
  return acc;
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Orderable 64-bit key: larger value wins; on equal values the lower index wins.
__device__ __forceinline__ unsigned long long argmax_key(float v, unsigned idx) {
  unsigned u = __float_as_uint(v);
  unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ unsigned argmax_index(unsigned long long key) {
  return 0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull);
}

}  // namespace dflash
