// combine.hip -- deterministic gather-based combines (no float atomics).
//
// 0.1.0 sdist, _vendor/experts.py, Experts4bit.forward scales each expert's
// output rows by their routing weight and index_add_s them into an fp32
// accumulator. Here every token gathers its k pair rows through pos_of_pair
// and sums them in fp32 in slot order j = 0..k-1, so the result is the same
// on every run.
#include "device.h"
#include "kernels.h"

namespace e4b {

// y[t] = sum_j w[t,j] * O[pos(t,j)]   (weighted)   or   sum_j O[pos(t,j)]
// rows of H bf16; 8 elements (16 bytes) per thread and step. The unweighted
// form (the dgrad combine) also sums, when gw is given, each pair's routing-
// weight gradient over the blocks of the down dgrad: gw[t, j] = sum_i
// partial[pos(t,j)][i], one wave per pair, lane l summing blocks l, l + 64,
// ... in ascending order and the 64 lane sums added by a fixed butterfly.
template <bool WEIGHTED>
__global__ __launch_bounds__(256) void combine_rows_kernel(const uint16_t *__restrict__ O,
                                                           const int32_t *__restrict__ pos_of_pair,
                                                           const float *__restrict__ wts, int k,
                                                           int H, uint16_t *__restrict__ y,
                                                           const float *__restrict__ partial,
                                                           int n_tiles, float *__restrict__ gw) {
  const int64_t t = blockIdx.x;
  __shared__ int32_t pos[kMaxTopK];
  __shared__ float w[kMaxTopK];
  if (threadIdx.x < k) {
    pos[threadIdx.x] = pos_of_pair[t * k + threadIdx.x];
    w[threadIdx.x] = WEIGHTED ? wts[t * k + threadIdx.x] : 1.0f;
  }
  __syncthreads();
  if (!WEIGHTED && gw) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int j = wave; j < k; j += 4) {
      const float *src = partial + int64_t(pos[j]) * n_tiles;
      float sum = 0.0f;
      for (int i = lane; i < n_tiles; i += 64) sum += src[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) gw[t * k + j] = sum;
    }
  }
  for (int h = threadIdx.x * 8; h < H; h += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // up to 8 rows in flight before the first sum; the sums keep slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (j0 + jj < k) v[jj] = *reinterpret_cast<const u32x4 *>(O + int64_t(pos[j0 + jj]) * H + h);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= k) break;
        const int j = j0 + jj;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (WEIGHTED) {
            acc[2 * q] += w[j] * bf16_lo(v[jj][q]);
            acc[2 * q + 1] += w[j] * bf16_hi(v[jj][q]);
          } else {
            acc[2 * q] += bf16_lo(v[jj][q]);
            acc[2 * q + 1] += bf16_hi(v[jj][q]);
          }
        }
      }
    }
    *reinterpret_cast<u32x4 *>(y + t * H + h) =
        u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  }
}

hipError_t launch_combine_rows(const uint16_t *rows, const int32_t *pos_of_pair, const float *w,
                               int64_t T, int k, int H, uint16_t *out, hipStream_t s,
                               const e4b_kernel_events *ev) {
  if (T == 0) return hipSuccess;
  return launch_k(ev, E4B_K_COMBINE, combine_rows_kernel<true>, dim3(uint32_t(T)), dim3(256), s,
                  rows, pos_of_pair, w, k, H, out, static_cast<const float *>(nullptr), 0,
                  static_cast<float *>(nullptr));
}

hipError_t launch_combine_dgrad(const uint16_t *rows, const int32_t *pos_of_pair, int64_t T, int k,
                                int H, uint16_t *out, const float *partial, int n_tiles,
                                float *gw, hipStream_t s, const e4b_kernel_events *ev) {
  if (T == 0) return hipSuccess;
  return launch_k(ev, E4B_K_COMBINE_DGRAD, combine_rows_kernel<false>, dim3(uint32_t(T)), dim3(256),
                  s, rows, pos_of_pair, static_cast<const float *>(nullptr), k, H, out, partial,
                  n_tiles, gw);
}

}  // namespace e4b
