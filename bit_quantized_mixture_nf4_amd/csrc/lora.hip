// lora.hip -- per-expert LoRA adapters over the frozen 4-bit base.
//
// The experts4bit-qlora 0.4.0 README ("Quickstart") wraps the frozen fused
// expert stack as ExpertsLoRA(base, r=8, alpha=16): trainable per-expert
// low-rank adapters, base frozen. On both projections of expert e:
//   h = W_gu x + s B_gu (A_gu x),   o = W_dn a + s B_dn (A_dn a),   s = alpha / r.
// Here the low-rank products are split into
//   * a per-pair projection onto the rank space (x A_gu^T, a A_dn^T and, in
//     the backward, grad_y B_dn and dGU B_gu) on MFMA over the m-tiles of
//     the permutation, fp32, written as [P, 16] in sorted-pair order;
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

// j-major bf16 pack of an adapter for the projections: out[e, j, k] =
// bf16(M(e, k, j)) for j < r, zero for r <= j < kLoraK, with M(e, k, j) =
// A[e, j, k] (A [E, r, K]) or B[e, k, j] (B [E, K, r]). One thread per
// (e, j, run of 8 k).
template <bool MB>
__global__ __launch_bounds__(256) void lora_pack_jk_kernel(const float *__restrict__ M, int64_t E,
                                                           int K, int r, uint16_t *__restrict__ out) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_e = int64_t(kLoraK) * (K / 8);
  if (i >= E * per_e) return;
  const int64_t e = i / per_e;
  const int j = int((i % per_e) / (K / 8));
  const int k0 = int(i % (K / 8)) * 8;
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float m = 0.0f;
    if (j < r) m = MB ? M[(e * K + k0 + q) * r + j] : M[(e * r + j) * K + k0 + q];
    v[q] = m;
  }
  *reinterpret_cast<u32x4 *>(out + (e * kLoraK + j) * K + k0) =
      u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
            pack_bf16x2(v[6], v[7])};
}

// Per-pair projection as MFMA: one workgroup per m-tile (256 sorted rows of
// one expert), each wave 64 rows as four 16-row groups, K in steps of 32 with
// v_mfma_f32_16x16x32_bf16 (A = the source rows in bf16, B = the j-major
// adapter pack [E, 16, K]); out[s, j] fp32 for the tile's valid rows.
template <int SRC>
__global__ __launch_bounds__(256) void lora_project_mfma_kernel(
    const uint16_t *__restrict__ src, int64_t ld, int K, int I, const int32_t *__restrict__ sorted,
    int topk, const int4 *__restrict__ tile_map, const int32_t *__restrict__ tile_offsets, int E,
    const uint16_t *__restrict__ Mj, float *__restrict__ out) {
  const int mt = blockIdx.x;
  if (mt >= tile_offsets[E]) return;
  const int4 tm = tile_map[mt];
  const int e = tm.x, seg = tm.y, row0 = tm.z, valid = tm.w;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave * 64 >= valid) return;  // no barriers in this kernel
  const int r16 = lane & 15, kb = (lane >> 4) * 8;
  const uint16_t *rowp[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    const int srow = seg + row0 + min(wave * 64 + gi * 16 + r16, valid - 1);
    rowp[gi] = (SRC == LS_X_GATHER ? src + int64_t(sorted[srow] / topk) * ld : src + srow * ld) + kb;
  }
  const uint16_t *mp = Mj + (int64_t(e) * kLoraK + r16) * K + kb;
  f32x4 acc[4];
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) acc[gi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < K; k0 += 32) {
    const bf16x8 mb = *reinterpret_cast<const bf16x8 *>(mp + k0);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      u32x4 q;
      if (SRC == LS_GU_ACT) {
        const u32x4 gq = *reinterpret_cast<const u32x4 *>(rowp[gi] + k0);
        const u32x4 uq = *reinterpret_cast<const u32x4 *>(rowp[gi] + I + k0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          q[t] = pack_bf16x2(silu_f(bf16_lo(gq[t])) * bf16_lo(uq[t]),
                             silu_f(bf16_hi(gq[t])) * bf16_hi(uq[t]));
      } else {
        q = *reinterpret_cast<const u32x4 *>(rowp[gi] + k0);
      }
      acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, q), mb, acc[gi],
                                                        0, 0, 0);
    }
  }
  // D[row 4 * (lane / 16) + t][col lane % 16]
#pragma unroll
  for (int gi = 0; gi < 4; ++gi)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rr = wave * 64 + gi * 16 + 4 * (lane >> 4) + t;
      if (rr < valid) out[int64_t(seg + row0 + rr) * kLoraK + r16] = acc[gi][t];
    }
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
  const dim3 grid{uint32_t((EN + 255) / 256)};
  if (trans)
    hipLaunchKernelGGL(lora_pack_kernel<true>, grid, dim3(256), 0, st, M, EN, N, r, s, out);
  else
    hipLaunchKernelGGL(lora_pack_kernel<false>, grid, dim3(256), 0, st, M, EN, N, r, s, out);
  return hipGetLastError();
}

hipError_t launch_lora_pack_jk(const float *M, int64_t E, int K, int r, bool m_is_b,
                               uint16_t *out, hipStream_t st) {
  const int64_t n = E * kLoraK * (K / 8);
  if (n == 0) return hipSuccess;
  const dim3 grid{uint32_t((n + 255) / 256)};
  if (m_is_b)
    hipLaunchKernelGGL(lora_pack_jk_kernel<true>, grid, dim3(256), 0, st, M, E, K, r, out);
  else
    hipLaunchKernelGGL(lora_pack_jk_kernel<false>, grid, dim3(256), 0, st, M, E, K, r, out);
  return hipGetLastError();
}

hipError_t launch_lora_project_mfma(int src_mode, const uint16_t *src, int64_t ld, int K, int I,
                                    const int32_t *sorted, int topk, const PermView &v, int E,
                                    int64_t m_tiles_bound, const uint16_t *Mj, float *out,
                                    hipStream_t st) {
  if (m_tiles_bound == 0) return hipSuccess;
  const dim3 grid{uint32_t(m_tiles_bound)};
#define E4B_LPM(SM)                                                                          \
  hipLaunchKernelGGL((lora_project_mfma_kernel<SM>), grid, dim3(256), 0, st, src, ld, K, I,  \
                     sorted, topk, v.tile_map, v.tile_offsets, E, Mj, out)
  if (src_mode == LS_X_GATHER) E4B_LPM(LS_X_GATHER);
  else if (src_mode == LS_ROWS) E4B_LPM(LS_ROWS);
  else if (src_mode == LS_GU_ACT) E4B_LPM(LS_GU_ACT);
  else return hipErrorInvalidValue;
#undef E4B_LPM
  return hipGetLastError();
}

hipError_t launch_lora_wgrad(int u_mode, const uint16_t *src, int64_t ld, int N, int I,
                             const int32_t *sorted, const int32_t *offsets, int topk,
                             const float *topk_w, int64_t E, const float *V, bool v_weighted,
                             int r, float s, bool out_trans, float *out, hipStream_t st) {
  if (E == 0 || N == 0) return hipSuccess;
  const dim3 grid{uint32_t((N / 2 + 255) / 256), uint32_t(E)};
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
