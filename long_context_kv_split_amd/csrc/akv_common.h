// Device-side constants, layout helpers and small utilities shared by the
// akv HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/akv.h"

namespace akv {

constexpr int kBlock = AKV_BLOCK_TOKENS;  // tokens per paged block
constexpr int kGroup = AKV_GROUP;         // elements per scale group
constexpr int kMaxG = 8;                  // query heads per kv head served

// 16-level Lloyd-Max quantizer for N(0,1) (minimum mean-square error levels
// of a unit Gaussian, Max 1960 / Lloyd), solved in float64 to a fixed point
// and rounded to float32.  Ascending; C[15-k] = -C[k].
__device__ __constant__ const uint32_t kLevelBits[16] = {
    0xC02EE2BFu, 0xC0046AC7u, 0xBFCF1C25u, 0xBFA0CC2Fu, 0xBF713D39u, 0xBF28215Eu,
    0xBEC6AE44u, 0xBE0379FDu, 0x3E0379FDu, 0x3EC6AE44u, 0x3F28215Eu, 0x3F713D39u,
    0x3FA0CC2Fu, 0x3FCF1C25u, 0x40046AC7u, 0x402EE2BFu};

// Decision thresholds: T[k] = largest float32 <= (C[k] + C[k+1]) / 2.  With
// code = #{k : u > T[k]} an input exactly on a midpoint goes to the lower
// index.  (Negative midpoints round down as well, so the set is not
// symmetric.)
__device__ __constant__ const uint32_t kThreshBits[15] = {
    0xC019A6C3u, 0xBFEBF8DAu, 0xBFB7F42Au, 0xBF8CB566u, 0xBF4CAF4Cu,
    0xBF05BC40u, 0xBE8435A2u, 0x00000000u, 0x3E8435A1u, 0x3F05BC40u,
    0x3F4CAF4Bu, 0x3F8CB565u, 0x3FB7F42Au, 0x3FEBF8D9u, 0x4019A6C3u};

// The 4- and 8-level Lloyd-Max quantizers for N(0,1) (code widths 2 and 3),
// solved and rounded the same way, with their round-down midpoints.
__device__ __constant__ const uint32_t kLevelBits2[4] = {0xBFC1555Du, 0xBEE7D2C9u, 0x3EE7D2C9u, 0x3FC1555Du};
__device__ __constant__ const uint32_t kThreshBits2[3] = {0xBF7B4A10u, 0x00000000u, 0x3F7B4A0Fu};
__device__ __constant__ const uint32_t kLevelBits3[8] = {
    0xC009B97Au, 0xBFAC0538u, 0xBF418990u, 0xBE7AF9F8u, 0x3E7AF9F8u, 0x3F418990u, 0x3FAC0538u, 0x4009B97Au};
__device__ __constant__ const uint32_t kThreshBits3[7] = {
    0xBFDFBC16u, 0xBF866500u, 0xBF002407u, 0x00000000u, 0x3F002407u, 0x3F866500u, 0x3FDFBC16u};

// A load of data read once per call (streamed KV): non-temporal, so it does
// not push reused lines out of the caches.
template <class T>
__device__ inline T stream_load(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// Code width of a descriptor's code_bits field (0 means 4).
__host__ __device__ inline int code_width(int code_bits) { return code_bits == 0 ? 4 : code_bits; }

// Level and threshold table of code width W.
template <int W>
__device__ inline const uint32_t* level_bits() {
  if constexpr (W == 2) return kLevelBits2;
  else if constexpr (W == 3) return kLevelBits3;
  else return kLevelBits;
}
template <int W>
__device__ inline const uint32_t* thresh_bits() {
  if constexpr (W == 2) return kThreshBits2;
  else if constexpr (W == 3) return kThreshBits3;
  else return kThreshBits;
}

// RN_32(1/sqrt(d)) for the supported head dims.
__host__ __device__ inline float inv_sqrt_d(int d) {
  return d == 64 ? 0.125f : __builtin_bit_cast(float, 0x3DB504F3u);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- layouts
// Byte offset, inside a token's K-code row, of the byte holding dims
// (32m + 8a + 2b, +1).
__host__ __device__ inline int kcode_byte(int d, int dim) {
  int m = dim >> 5, a = (dim >> 3) & 3, b = (dim >> 1) & 3;
  return (d >> 3) * a + 4 * m + b;
}
// Byte offset, inside a V-code slab, of the byte holding tokens
// (32c + 8a + 2b, +1) of dim 16t + i: per 32-token half c, 1 KB per group of
// four value tiles, and in it 16 bytes per lane 16a + i (one dword per tile).
__host__ __device__ inline int vcode_byte(int d, int tok, int dim) {
  int c = tok >> 5, a = (tok >> 3) & 3, b = (tok >> 1) & 3;
  int t = dim >> 4, i = dim & 15;
  return c * 16 * d + (t >> 2) * 1024 + (a * 16 + i) * 16 + 4 * (t & 3) + b;
}

// ---------------------------------------------------------------- vectors
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline float bf16_bits_to_float(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

__device__ inline float neg_inf() { return -__builtin_huge_valf(); }

}  // namespace akv
