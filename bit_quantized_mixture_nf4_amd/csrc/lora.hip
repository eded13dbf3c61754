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
//     outer products, on MFMA with the pairs as the reduction (no atomics;
//     deterministic).
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
  int rin[4];  // LS_GU_ACT: the row within the m-tile (blocked g|u)
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    rin[gi] = min(wave * 64 + gi * 16 + r16, valid - 1);
    const int srow = seg + row0 + rin[gi];
    rowp[gi] = (SRC == LS_X_GATHER ? src + int64_t(sorted[srow] / topk) * ld : src + srow * ld) + kb;
  }
  const int npb = (I + kGuBlockPairs - 1) / kGuBlockPairs;
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
        // pairs k0 + kb .. + 7: two chunks of 4 (g[4], u[4]) of the blocked g|u
        const int c = k0 + kb, pb = c / kGuBlockPairs, cc = c % kGuBlockPairs;
        const u32x4 c0 = *reinterpret_cast<const u32x4 *>(src + gu_chunk(mt, pb, npb, rin[gi], cc) * 8);
        const u32x4 c1 = *reinterpret_cast<const u32x4 *>(src + gu_chunk(mt, pb, npb, rin[gi], cc + 4) * 8);
        const u32x4 gq{c0[0], c0[1], c1[0], c1[1]};
        const u32x4 uq{c0[2], c0[3], c1[2], c1[3]};
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

// Adapter gradient on MFMA: G[n, j] = s * sum over expert e's sorted pairs p
// of U(p)[n] V(p)[j]. Grid (column blocks of 64, expert); the four waves own
// 16 columns each. The pairs are taken in chunks of 32 in sorted order: the
// chunk's U rows (64 columns, bf16) and rank vectors (bf16) are written to
// LDS transposed, so that one v_mfma_f32_16x16x32_bf16 per wave (A = U^T
// [16 n x 32 p], B = V [32 p x 16 j]) consumes the chunk; the next chunk's
// loads are in flight meanwhile. Every sum runs in one fixed order.
constexpr int kWgCols = 64;
constexpr int kWgChunk = 32;
constexpr int kWgPad = kWgChunk + 8;  // LDS row of one column / rank: 32 pairs + pad (bf16)

template <int U>
__global__ __launch_bounds__(256) void lora_wgrad_kernel(
    const uint16_t *__restrict__ src, int64_t ld, int N, int I, const int32_t *__restrict__ sorted,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tile_offsets, int topk,
    const float *__restrict__ topk_w,
    const float *__restrict__ V, bool v_weighted, int r, float sc, bool out_trans,
    float *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t su[kWgCols][kWgPad];  // U^T
  __shared__ __attribute__((aligned(16))) uint16_t sv[kLoraK][kWgPad];   // V^T
  const int e = blockIdx.y;
  const int n_base = blockIdx.x * kWgCols;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = offsets[e], s1 = offsets[e + 1];
  // staging roles: U: pair q = tid / 8 of the chunk, columns 8 * (tid % 8) ..;
  // V: threads < 128, pair tid / 4, ranks 4 * (tid % 4) ..
  const int uq = tid >> 3, un = (tid & 7) * 8;
  const int ncol = min(n_base + un, N - 8);  // clamped (N % 8 == 0); results past N are not stored
  const int vq = tid >> 2, vj = (tid & 3) * 4;
  u32x4 ureg;
  float vreg[4];
  auto load = [&](int c0) {
    const int s = min(c0 + uq, s1 - 1);
    const bool live = c0 + uq < s1;
    const int p = sorted[s];
    const uint16_t *row = (U == LS_X_GATHER || U == LS_WX_GATHER) ? src + int64_t(p / topk) * ld
                                                                  : src + int64_t(s) * ld;
    u32x4 q;
    if (U == LS_GU_ACT) {
      // pair s of expert e: row (s - s0) % 256 of m-tile tile_offsets[e] + (s - s0) / 256
      // of the blocked g|u; columns ncol .. + 7 are two chunks (g[4], u[4])
      const int rs = s - s0, mt = tile_offsets[e] + rs / kBM;
      const int npb = (I + kGuBlockPairs - 1) / kGuBlockPairs;
      const int pb = ncol / kGuBlockPairs, cc = ncol % kGuBlockPairs;
      const u32x4 c0 = *reinterpret_cast<const u32x4 *>(src + gu_chunk(mt, pb, npb, rs % kBM, cc) * 8);
      const u32x4 c1 =
          *reinterpret_cast<const u32x4 *>(src + gu_chunk(mt, pb, npb, rs % kBM, cc + 4) * 8);
      const u32x4 gq{c0[0], c0[1], c1[0], c1[1]};
      const u32x4 uu{c0[2], c0[3], c1[2], c1[3]};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        q[t] = pack_bf16x2(silu_f(bf16_lo(gq[t])) * bf16_lo(uu[t]),
                           silu_f(bf16_hi(gq[t])) * bf16_hi(uu[t]));
    } else {
      q = *reinterpret_cast<const u32x4 *>(row + ncol);
    }
    if (U == LS_WX_GATHER) {
      const float wp = topk_w[p];
#pragma unroll
      for (int t = 0; t < 4; ++t) q[t] = pack_bf16x2(wp * bf16_lo(q[t]), wp * bf16_hi(q[t]));
    }
    ureg = live ? q : u32x4{0u, 0u, 0u, 0u};
    if (tid < kWgChunk * 4) {
      const int sv_ = min(c0 + vq, s1 - 1);
      const bool vlive = c0 + vq < s1;
      const float4 v4 = *reinterpret_cast<const float4 *>(V + int64_t(sv_) * kLoraK + vj);
      const float w = v_weighted ? topk_w[sorted[sv_]] : 1.0f;
      vreg[0] = vlive ? w * v4.x : 0.0f;
      vreg[1] = vlive ? w * v4.y : 0.0f;
      vreg[2] = vlive ? w * v4.z : 0.0f;
      vreg[3] = vlive ? w * v4.w : 0.0f;
    }
  };
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (s0 < s1) load(s0);
  for (int c0 = s0; c0 < s1; c0 += kWgChunk) {
    // stage the loaded chunk transposed
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      su[un + 2 * t][uq] = uint16_t(ureg[t] & 0xFFFFu);
      su[un + 2 * t + 1][uq] = uint16_t(ureg[t] >> 16);
    }
    if (tid < kWgChunk * 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t) sv[vj + t][vq] = uint16_t(pack_bf16x2(vreg[t], 0.0f) & 0xFFFFu);
    }
    __syncthreads();
    if (c0 + kWgChunk < s1) load(c0 + kWgChunk);
    // A = U^T rows (columns n), B = V^T rows (ranks j): 8 consecutive pairs per lane
    const bf16x8 af = *reinterpret_cast<const bf16x8 *>(&su[wave * 16 + (lane & 15)][8 * (lane >> 4)]);
    const bf16x8 bf = *reinterpret_cast<const bf16x8 *>(&sv[lane & 15][8 * (lane >> 4)]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc, 0, 0, 0);
    __syncthreads();
  }
  // D[n = 4 * (lane / 16) + t][j = lane % 16] of the wave's 16 columns
  const int j = lane & 15;
  if (j >= r) return;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n_base + wave * 16 + 4 * (lane >> 4) + t;
    if (n < N) {
      const int64_t o = out_trans ? (int64_t(e) * r + j) * N + n : (int64_t(e) * N + n) * r + j;
      out[o] = sc * acc[t];
    }
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
                             const int32_t *sorted, const int32_t *offsets,
                             const int32_t *tile_offsets, int topk,
                             const float *topk_w, int64_t E, const float *V, bool v_weighted,
                             int r, float s, bool out_trans, float *out, hipStream_t st) {
  if (E == 0 || N == 0) return hipSuccess;
  const dim3 grid{uint32_t((N + kWgCols - 1) / kWgCols), uint32_t(E)};
#define E4B_LW(UM)                                                                             \
  hipLaunchKernelGGL((lora_wgrad_kernel<UM>), grid, dim3(256), 0, st, src, ld, N, I, sorted,   \
                     offsets, tile_offsets, topk, topk_w, V, v_weighted, r, s, out_trans, out)
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
