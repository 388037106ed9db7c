// common.hpp -- types, constants and helpers shared by the HIP sources of the IQ4
// library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <stddef.h>

namespace iq4 {

// ---------------------------------------------------------------------------------
// Block format: 32 weights, 18 bytes (binary16 scale + 16 bytes of 4-bit indices).
constexpr int kQK = 32;
constexpr int kBlockBytes = 18;
constexpr int kNibbleBytes = 16;

// The fixed 16-level codebook of the format.
constexpr int8_t kCodebook[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                  1,    13,   25,  38,  53,  69,  89,  113};

// Register-only level lookup (no memory access): the 16 levels as int8 bytes in four
// 32-bit immediates, one byte picked with v_perm_b32.
constexpr uint32_t pack_levels(int i) {
  return (uint32_t)(uint8_t)kCodebook[i] | ((uint32_t)(uint8_t)kCodebook[i + 1] << 8) |
         ((uint32_t)(uint8_t)kCodebook[i + 2] << 16) | ((uint32_t)(uint8_t)kCodebook[i + 3] << 24);
}
constexpr uint32_t kLevels0 = pack_levels(0), kLevels1 = pack_levels(4);
constexpr uint32_t kLevels2 = pack_levels(8), kLevels3 = pack_levels(12);

__device__ __forceinline__ int level_of(uint32_t q) {
  const uint32_t sel = q & 7u;  // byte 0..3 of the second operand, 4..7 of the first
  const uint32_t b = (q < 8u) ? __builtin_amdgcn_perm(kLevels1, kLevels0, sel)
                              : __builtin_amdgcn_perm(kLevels3, kLevels2, sel);
  return (int)(int8_t)(b & 0xFFu);
}

// Packed layout: 16-row x 4-block tiles, 1 KiB of indices + 128 B of scales each.
constexpr int kTileRows = 16;
constexpr int kTileBlocks = 4;
constexpr int kTileK = kTileBlocks * kQK;  // 128
constexpr int kTileNibbleBytes = 1024;
constexpr int kTileScaleBytes = 128;

// ---------------------------------------------------------------------------------
// Matrix-core operand types (v_mfma_f32_16x16x32_{bf16,f16}).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 16x16 output, K = 32, fp32 accumulate.  Lane l (g = l / 16, c = l % 16) supplies
// A[c][8g .. 8g+7] and B[8g .. 8g+7][c]; it receives D[4g + i][c], i = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Packed pair of binary16 values: lo in bits 0-15.
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  f16x2 r = __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b);
  return __builtin_bit_cast(uint32_t, r);
}

// Non-temporal 16- and 8-byte loads (data read once: streamed past the L2).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint2 load_nt8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return uint2{v[0], v[1]};
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// bf16 bit pattern of a codebook level (exact: |c| <= 127)
__device__ __forceinline__ uint32_t bf16_of_level(int c) {
  return __float_as_uint((float)c) >> 16;
}

// hi and lo parts of two values, packed per part: hi = (bf16(v0), bf16(v1)), lo likewise
// for the residuals.  The residual v - hi is formed by a bf16 dot product whose only
// non-zero term is -1 * hi (fused with v, rounded once): exact, since v - hi is
// representable.
// The two constants (-1, 0) and (0, -1) are passed in scalar registers: as an inline
// constant, a packed bf16 operand's halves are not placed unambiguously.
__device__ __forceinline__ void split_hi_lo(float v0, float v1, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = {(__bf16)v0, (__bf16)v1};
  uint32_t k_lo = 0x0000BF80u, k_hi = 0xBF800000u;  // (-1, 0) and (0, -1) as bf16 pairs
  asm("" : "+s"(k_lo), "+s"(k_hi));                  // opaque: kept in registers
  const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, k_lo), v0, false);
  const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, k_hi), v1, false);
  const bf16x2 l = {(__bf16)r0, (__bf16)r1};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}


// Workgroup barrier that orders LDS only: it waits for no global load in flight (the
// kernels wait for their loads explicitly or through data dependences).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------------
// Host-side status handling.
int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace iq4
