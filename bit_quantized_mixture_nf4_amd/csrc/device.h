// device.h -- gfx950 device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e4b {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The 16-entry codebooks as fp32 bit patterns, code order 0..15, indexed by
// e4b_codebook. NF4: NormalFloat-4 table of the QLoRA paper
// (arXiv:2305.14314, appendix "NormalFloat 4-bit data type"). FP4: e2m1
// magnitudes {0,.5,1,1.5,2,3,4,6}/6, bit 3 = sign (code 8 = -0.0). Row 2
// (BF16) has no table. MXFP4: the unscaled E2M1 values (OCP MX v1.0).
// Usable from host and device code.
static constexpr uint32_t kCodebookBits[4][16] = {
    {0xBF800000u, 0xBF3239B1u, 0xBF066B30u, 0xBECA32A0u, 0xBE91A24Du, 0xBE3D353Fu,
     0xBDBA7871u, 0x00000000u, 0x3DA2FAFFu, 0x3E24CAE3u, 0x3E7C04DDu, 0x3EAD033Au,
     0x3EE1A4B8u, 0x3F1007ABu, 0x3F3913B3u, 0x3F800000u},
    {0x00000000u, 0x3DAAAAABu, 0x3E2AAAABu, 0x3E800000u, 0x3EAAAAABu, 0x3F000000u,
     0x3F2AAAABu, 0x3F800000u, 0x80000000u, 0xBDAAAAABu, 0xBE2AAAABu, 0xBE800000u,
     0xBEAAAAABu, 0xBF000000u, 0xBF2AAAABu, 0xBF800000u},
    {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u},
    {0x00000000u, 0x3F000000u, 0x3F800000u, 0x3FC00000u, 0x40000000u, 0x40400000u,
     0x40800000u, 0x40C00000u, 0x80000000u, 0xBF000000u, 0xBF800000u, 0xBFC00000u,
     0xC0000000u, 0xC0400000u, 0xC0800000u, 0xC0C00000u}};

__device__ __forceinline__ float codebook_value(int cb, int q) {
  return __uint_as_float(kCodebookBits[cb][q]);
}

// E8M0 scale byte -> 2^(s - 127) as fp32 (s = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  return __uint_as_float(s ? s << 23 : 0x00400000u);
}

// Two fp32 values -> packed bf16 pair (low half = `lo`), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(uint32_t(v) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return uint16_t(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

}  // namespace e4b
