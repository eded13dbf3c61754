// lora.hip -- per-expert LoRA adapters over the frozen 4-bit base.
//
// The experts4bit-qlora 0.4.0 README ("Quickstart") wraps the frozen fused
// expert stack as ExpertsLoRA(base, r=8, alpha=16): trainable per-expert
// low-rank adapters, base frozen. On both projections of expert e:
//   h = W_gu x + s B_gu (A_gu x),   o = W_dn a + s B_dn (A_dn a),   s = alpha / r.
// Here the low-rank products are split into
//   * a per-pair projection onto the rank space (x A_gu^T, a A_dn^T and, in
//     the backward, grad_y B_dn and dGU B_gu): one wavefront per routed pair,
//     fp32, written as [P, 16] in sorted-pair order;
//   * one extra 16-deep MFMA slice inside the grouped GEMM that already
//     produces the projection (gemm.hip), against a bf16 pack of the scaled
//     adapter laid out by output column;
//   * the adapter gradients: per expert, a fixed-order sum over its pairs of
//     outer products (no atomics; deterministic).
#include "device.h"
#include "kernels.h"

namespace e4b {

// One thread per (expert, row n): 16 bf16 = s * M[e, n, 0..r) then zeros.
template <bool TRANS>
__global__ __launch_bounds__(256) void lora_pack_kernel(const float *__restrict__ M, int64_t EN,
                                                        int N, int r, float s,
                                                        uint16_t *__restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= EN) return;
  const int64_t e = i / N, n = i % N;
  uint32_t w[kLoraK / 2];
#pragma unroll
  for (int jj = 0; jj < kLoraK / 2; ++jj) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * jj + h;
      float m = 0.0f;
      if (j < r) m = TRANS ? M[(e * r + j) * N + n] : M[i * r + j];
      v[h] = s * m;
    }
    w[jj] = pack_bf16x2(v[0], v[1]);
  }
  u32x4 *o = reinterpret_cast<u32x4 *>(out + i * kLoraK);
  o[0] = u32x4{w[0], w[1], w[2], w[3]};
  o[1] = u32x4{w[4], w[5], w[6], w[7]};
}

__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Eight consecutive source values of row `row` at column k0 (bf16 -> fp32).
template <int SRC>
__device__ __forceinline__ void lora_src8(const uint16_t *row, int k0, int I, float (&v)[8]) {
  if (SRC == LS_GU_ACT) {
    const u32x4 gq = *reinterpret_cast<const u32x4 *>(row + k0);
    const u32x4 uq = *reinterpret_cast<const u32x4 *>(row + I + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = silu_f(bf16_lo(gq[q])) * bf16_lo(uq[q]);
      v[2 * q + 1] = silu_f(bf16_hi(gq[q])) * bf16_hi(uq[q]);
    }
  } else {
    const u32x4 q4 = *reinterpret_cast<const u32x4 *>(row + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_lo(q4[q]);
      v[2 * q + 1] = bf16_hi(q4[q]);
    }
  }
}

__device__ __forceinline__ float wave_allsum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wavefront per sorted pair s; the 64 lanes split K in runs of 8.
template <int SRC, bool MB>
__global__ __launch_bounds__(256) void lora_project_kernel(
    const uint16_t *__restrict__ src, int64_t ld, int K, int I, const int32_t *__restrict__ sorted,
    const int32_t *__restrict__ flat_idx, int topk, int64_t P, const float *__restrict__ M, int r,
    float *__restrict__ out) {
  const int64_t s = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= P) return;
  const int p = sorted[s];
  const int e = flat_idx[p];
  const uint16_t *row = SRC == LS_X_GATHER ? src + int64_t(p / topk) * ld : src + s * ld;
  float acc[kLoraK];
#pragma unroll
  for (int j = 0; j < kLoraK; ++j) acc[j] = 0.0f;
  for (int k0 = lane * 8; k0 < K; k0 += 512) {
    float xv[8];
    lora_src8<SRC>(row, k0, I, xv);
#pragma unroll
    for (int j = 0; j < kLoraK; ++j) {
      if (j < r) {
        float a = acc[j];
        if (MB) {
          const float *m = M + (int64_t(e) * K + k0) * r + j;
#pragma unroll
          for (int q = 0; q < 8; ++q) a += xv[q] * m[q * r];
        } else {
          const float4 *m = reinterpret_cast<const float4 *>(M + (int64_t(e) * r + j) * K + k0);
          const float4 m0 = m[0], m1 = m[1];
          a += xv[0] * m0.x + xv[1] * m0.y + xv[2] * m0.z + xv[3] * m0.w;
          a += xv[4] * m1.x + xv[5] * m1.y + xv[6] * m1.z + xv[7] * m1.w;
        }
        acc[j] = a;
      }
    }
  }
  float mine = 0.0f;
#pragma unroll
  for (int j = 0; j < kLoraK; ++j) {
    const float t = j < r ? wave_allsum(acc[j]) : 0.0f;
    mine = lane == j ? t : mine;
  }
  if (lane < kLoraK) out[s * kLoraK + lane] = mine;
}

// Adapter gradient: grid (column blocks of 512, expert). Thread owns two
// columns n, n + 1; the expert's pairs are visited in sorted order in
// batches of kWgBatch (their rank vectors staged in LDS, their source values
// loaded together), so every sum has one fixed order.
constexpr int kWgBatch = 32;

template <int U>
__global__ __launch_bounds__(256) void lora_wgrad_kernel(
    const uint16_t *__restrict__ src, int64_t ld, int N, int I, const int32_t *__restrict__ sorted,
    const int32_t *__restrict__ offsets, int topk, const float *__restrict__ topk_w,
    const float *__restrict__ V, bool v_weighted, int r, float sc, bool out_trans,
    float *__restrict__ out) {
  __shared__ float sv[kWgBatch][kLoraK];
  const int e = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 2;
  const int s0 = offsets[e], s1 = offsets[e + 1];
  const int nc = min(n, N - 2);  // clamped column pair (N is even); stores are guarded
  float acc[2][kLoraK];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < kLoraK; ++j) acc[c][j] = 0.0f;
  for (int b = s0; b < s1; b += kWgBatch) {
    const int nb = min(kWgBatch, s1 - b);
    __syncthreads();  // previous batch's rank vectors consumed
    for (int t = threadIdx.x; t < kWgBatch * kLoraK; t += 256) {
      const int q = t / kLoraK, j = t % kLoraK;
      float v = 0.0f;
      if (q < nb) {
        const int s = b + q;
        v = V[int64_t(s) * kLoraK + j];
        if (v_weighted) v *= topk_w[sorted[s]];
      }
      sv[q][j] = v;
    }
    __syncthreads();
    float u[kWgBatch][2];
#pragma unroll
    for (int q = 0; q < kWgBatch; ++q) {
      const int s = b + min(q, nb - 1);
      const int p = sorted[s];
      const uint16_t *row = (U == LS_X_GATHER || U == LS_WX_GATHER) ? src + int64_t(p / topk) * ld
                                                                    : src + int64_t(s) * ld;
      const uint32_t w2 = *reinterpret_cast<const uint32_t *>(row + nc);
      float u0 = bf16_lo(w2), u1 = bf16_hi(w2);
      if (U == LS_GU_ACT) {
        const uint32_t up = *reinterpret_cast<const uint32_t *>(row + I + nc);
        u0 = silu_f(u0) * bf16_lo(up);
        u1 = silu_f(u1) * bf16_hi(up);
      }
      if (U == LS_WX_GATHER) {
        const float wp = topk_w[p];
        u0 *= wp;
        u1 *= wp;
      }
      const bool live = q < nb;
      u[q][0] = live ? u0 : 0.0f;
      u[q][1] = live ? u1 : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kWgBatch; ++q)
#pragma unroll
      for (int j = 0; j < kLoraK; ++j) {
        const float v = sv[q][j];
        acc[0][j] += u[q][0] * v;
        acc[1][j] += u[q][1] * v;
      }
  }
  if (n >= N) return;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < kLoraK; ++j)
      if (j < r) {
        const int64_t o = out_trans ? (int64_t(e) * r + j) * N + n + c
                                    : (int64_t(e) * N + n + c) * r + j;
        out[o] = sc * acc[c][j];
      }
}

hipError_t launch_lora_pack(const float *M, int64_t E, int N, int r, float s, bool trans,
                            uint16_t *out, hipStream_t st) {
  const int64_t EN = E * N;
  if (EN == 0) return hipSuccess;
  const dim3 grid(uint32_t((EN + 255) / 256));
  if (trans)
    hipLaunchKernelGGL(lora_pack_kernel<true>, grid, dim3(256), 0, st, M, EN, N, r, s, out);
  else
    hipLaunchKernelGGL(lora_pack_kernel<false>, grid, dim3(256), 0, st, M, EN, N, r, s, out);
  return hipGetLastError();
}

hipError_t launch_lora_project(int src_mode, const uint16_t *src, int64_t ld, int K, int I,
                               const int32_t *sorted, const int32_t *flat_idx, int topk,
                               int64_t P, const float *M, bool m_is_b, int r, float *out,
                               hipStream_t st) {
  if (P == 0) return hipSuccess;
  const dim3 grid(uint32_t((P + 3) / 4));
#define E4B_LP(SM, MB)                                                                       \
  hipLaunchKernelGGL((lora_project_kernel<SM, MB>), grid, dim3(256), 0, st, src, ld, K, I,  \
                     sorted, flat_idx, topk, P, M, r, out)
  if (src_mode == LS_X_GATHER) {
    if (m_is_b) E4B_LP(LS_X_GATHER, true); else E4B_LP(LS_X_GATHER, false);
  } else if (src_mode == LS_ROWS) {
    if (m_is_b) E4B_LP(LS_ROWS, true); else E4B_LP(LS_ROWS, false);
  } else if (src_mode == LS_GU_ACT) {
    if (m_is_b) E4B_LP(LS_GU_ACT, true); else E4B_LP(LS_GU_ACT, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef E4B_LP
  return hipGetLastError();
}

hipError_t launch_lora_wgrad(int u_mode, const uint16_t *src, int64_t ld, int N, int I,
                             const int32_t *sorted, const int32_t *offsets, int topk,
                             const float *topk_w, int64_t E, const float *V, bool v_weighted,
                             int r, float s, bool out_trans, float *out, hipStream_t st) {
  if (E == 0 || N == 0) return hipSuccess;
  const dim3 grid(uint32_t((N / 2 + 255) / 256), uint32_t(E));
#define E4B_LW(UM)                                                                             \
  hipLaunchKernelGGL((lora_wgrad_kernel<UM>), grid, dim3(256), 0, st, src, ld, N, I, sorted,   \
                     offsets, topk, topk_w, V, v_weighted, r, s, out_trans, out)
  switch (u_mode) {
    case LS_X_GATHER: E4B_LW(LS_X_GATHER); break;
    case LS_ROWS: E4B_LW(LS_ROWS); break;
    case LS_GU_ACT: E4B_LW(LS_GU_ACT); break;
    case LS_WX_GATHER: E4B_LW(LS_WX_GATHER); break;
    default: return hipErrorInvalidValue;
  }
#undef E4B_LW
  return hipGetLastError();
}

}  // namespace e4b
