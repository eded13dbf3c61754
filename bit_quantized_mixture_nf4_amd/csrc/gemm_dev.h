// gemm_dev.h -- device helpers of the grouped GEMM (gemm_wide.hip) and the LoRA kernels.
#pragma once

#include "device.h"
#include "kernels.h"

namespace e4b {

enum { A_GATHER = 0, A_DIRECT = 1 };
enum { B_NT = 0, B_NN = 1 };
enum { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_DSWIGLU = 2, EPI_ACT = 3, EPI_DACT = 4 };

constexpr int kLds = kBK + 8;  // padded row (bf16 elements): 144 bytes, conflict-free b128 access

// B_NN tile in LDS: 16-byte unit u of a row is stored at unit u ^ ((u >> 3) & 3),
// which puts the 8 threads writing one row's units on distinct banks
__device__ __forceinline__ int nn_unit(int u) { return u ^ ((u >> 3) & 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
// gfx950 LDS transpose read: within each 16-lane group, lane s supplies the
// address of 4 bf16 (row s / 4, columns 4 (s % 4) .. + 3 of a 4 x 16 block)
// and receives column s of the block (rows 0..3)
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(const_cast<uint16_t *>(p)));
}

// hardware reciprocal (about 1 ulp): the result is rounded to bf16 anyway
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace e4b
