// lora.hip -- per-expert LoRA adapters over the frozen 4-bit base.
//
// The experts4bit-qlora 0.4.0 README ("Quickstart") wraps the frozen fused
// expert stack as ExpertsLoRA(base, r=8, alpha=16): trainable per-expert
// low-rank adapters, base frozen. On both projections of expert e:
//   h = W_gu x + s B_gu (A_gu x),   o = W_dn a + s B_dn (A_dn a),   s = alpha / r.
// Here the low-rank products are split into
//   * a per-pair projection onto the rank space (x A_gu^T, a A_dn^T and, in
//     the backward, grad_y B_dn and dGU B_gu) on MFMA, one wave per 16 sorted
//     rows of an m-tile (rows of a tile share one expert), fp32, written as
//     [P, 16] in sorted-pair order;
//   * one extra 16-deep MFMA slice inside the grouped GEMM that already
//     produces the projection (gemm_wide.hip), against a bf16 pack of the scaled
//     adapter laid out by output column;
//   * the four adapter gradients in one launch: per expert, a fixed-order sum
//     over its pairs of outer products, on MFMA with the pairs as the
//     reduction (no atomics; deterministic).
// All operand packs of one call are made by one launch.
#include "device.h"
#include "gemm_dev.h"
#include "kernels.h"

namespace e4b {

__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// ---- operand packs: every pack of a call in one launch ----
//   LP_COLS   : out[e, n, :] = bf16(s * B[e, n, j])   (B [E, N, r])    one thread per (e, n)
//   LP_COLS_T : out[e, n, :] = bf16(s * A[e, j, n])   (A [E, r, N])    one thread per (e, n)
//   LP_JK_A   : out[e, j, k] = bf16(A[e, j, k])       (A [E, r, K])    one thread per (e, j, 8 k)
//   LP_JK_B   : out[e, j, k] = bf16(B[e, k, j])       (B [E, K, r])    one thread per (e, 8 k)
// with zeros for r <= j < kLoraK. Item counts stay below 2^31 (checked by the
// launcher), so the index arithmetic is 32-bit.
__global__ __launch_bounds__(256) void lora_packs_kernel(LoraPackJobs jobs) {
  // the job of this block (uniform selects: no dynamic index into the arguments)
  LoraPackJob J = jobs.j[0];
  int64_t first = jobs.first_block[0];
#pragma unroll
  for (int q = 1; q < kLoraPackJobs; ++q)
    if (q < jobs.n && int64_t(blockIdx.x) >= jobs.first_block[q]) {
      J = jobs.j[q];
      first = jobs.first_block[q];
    }
  const uint32_t i = uint32_t(int64_t(blockIdx.x) - first) * 256u + threadIdx.x;
  if (i >= uint64_t(J.items)) return;
  const uint32_t r = uint32_t(jobs.r), N = uint32_t(J.N);
  if (J.type == LP_COLS || J.type == LP_COLS_T) {
    const uint32_t e = i / N, n = i - e * N;
    uint32_t w[kLoraK / 2];
#pragma unroll
    for (uint32_t jj = 0; jj < kLoraK / 2; ++jj) {
      float v[2];
#pragma unroll
      for (uint32_t h = 0; h < 2; ++h) {
        const uint32_t j = 2 * jj + h;
        float m = 0.0f;
        if (j < r) m = J.type == LP_COLS_T ? J.M[(size_t(e) * r + j) * N + n] : J.M[size_t(i) * r + j];
        v[h] = J.s * m;
      }
      w[jj] = pack_bf16x2(v[0], v[1]);
    }
    u32x4 *o = reinterpret_cast<u32x4 *>(J.out + size_t(i) * kLoraK);
    o[0] = u32x4{w[0], w[1], w[2], w[3]};
    o[1] = u32x4{w[4], w[5], w[6], w[7]};
  } else if (J.type == LP_JK_A) {
    const uint32_t K = N, kb8 = K / 8;
    const uint32_t ej = i / kb8, k0 = (i - ej * kb8) * 8;
    const uint32_t e = ej / kLoraK, j = ej - e * kLoraK;
    u32x4 o = u32x4{0u, 0u, 0u, 0u};
    if (j < r) {
      const float4 *src = reinterpret_cast<const float4 *>(J.M + (size_t(e) * r + j) * K + k0);
      const float4 a = src[0], b = src[1];
      o = u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
    }
    *reinterpret_cast<u32x4 *>(J.out + size_t(ej) * K + k0) = o;
  } else {
    const uint32_t K = N, kb8 = K / 8;
    const uint32_t e = i / kb8, k0 = (i - e * kb8) * 8;
    const float *src = J.M + (size_t(e) * K + k0) * r;  // rows k0 .. k0 + 7, r floats each
#pragma unroll
    for (uint32_t j = 0; j < kLoraK; ++j) {
      float v[8];
#pragma unroll
      for (uint32_t q = 0; q < 8; ++q) v[q] = j < r ? src[q * r + j] : 0.0f;
      *reinterpret_cast<u32x4 *>(J.out + (size_t(e) * kLoraK + j) * K + k0) =
          u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                pack_bf16x2(v[6], v[7])};
    }
  }
}

// ---- per-pair projection ----
// Grid: four workgroups per m-tile, each 64 sorted rows (four 16-row groups)
// of one expert. The four waves split K (each a contiguous quarter of the
// 32-deep steps) and run v_mfma_f32_16x16x32_bf16 (A = 16 source rows x 32 k,
// B = the j-major adapter pack [E, 16, K]; one adapter load serves the four
// row groups), four K-steps of loads in flight per batch; the quarters are
// summed through LDS in wave order.
constexpr int kProjBatch = 4;

template <int NS>
__device__ __forceinline__ void proj_steps(const uint16_t *const (&rowp)[4], const uint16_t *mp,
                                           int k0, f32x4 (&acc)[4]) {
  u32x4 a[NS][4], b[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    b[s] = *reinterpret_cast<const u32x4 *>(mp + k0 + 32 * s);
#pragma unroll
    for (int g = 0; g < 4; ++g) a[s][g] = *reinterpret_cast<const u32x4 *>(rowp[g] + k0 + 32 * s);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load of the batch issued before the first MFMA
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s][g]),
                                                       __builtin_bit_cast(bf16x8, b[s]), acc[g], 0, 0, 0);
}

template <int SRC>
__global__ __launch_bounds__(256) void lora_proj_kernel(
    const uint16_t *__restrict__ src, int64_t ld, int K, const int32_t *__restrict__ sorted,
    int topk, const int4 *__restrict__ tile_map, const int32_t *__restrict__ tile_offsets, int E,
    const uint16_t *__restrict__ Mj, float *__restrict__ out) {
  __shared__ f32x4 red[3][4][64];  // quarters 1..3: [wave - 1][row group][lane]
  const int mt = blockIdx.x >> 2;
  if (mt >= tile_offsets[E]) return;  // uniform over the workgroup
  const int4 tm = tile_map[mt];
  const int e = tm.x, base = tm.y + tm.z, valid = tm.w;
  const int r0 = (blockIdx.x & 3) * 64;
  if (r0 >= valid) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kb = (lane >> 4) * 8;
  const uint16_t *rowp[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rr = min(r0 + 16 * g + r16, valid - 1);
    rowp[g] = (SRC == LS_X_GATHER ? src + int64_t(sorted[base + rr] / topk) * ld
                                  : src + int64_t(base + rr) * ld) + kb;
  }
  const uint16_t *mp = Mj + (int64_t(e) * kLoraK + r16) * K + kb;
  const int nsteps = K / 32;
  const int st0 = wave * nsteps / 4, st1 = (wave + 1) * nsteps / 4;
  f32x4 acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int st = st0;
#pragma unroll 1
  for (; st + kProjBatch <= st1; st += kProjBatch) proj_steps<kProjBatch>(rowp, mp, 32 * st, acc);
#pragma unroll 1
  for (; st < st1; ++st) proj_steps<1>(rowp, mp, 32 * st, acc);
  if (wave > 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) red[wave - 1][g][lane] = acc[g];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 sum = ((acc[g] + red[0][g][lane]) + red[1][g][lane]) + red[2][g][lane];
    // D[row 4 * (lane / 16) + t][col lane % 16] of row group g
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = r0 + 16 * g + 4 * (lane >> 4) + t;
      if (row < valid) out[int64_t(base + row) * kLoraK + r16] = sum[t];
    }
  }
}

// ---- adapter gradients ----
// G[n, j] = s * sum over expert e's sorted pairs p of U(p)[n] V(p)[j]. Grid
// (column blocks of 64, expert, job); the four waves own 16 columns each.
// The pairs are taken in chunks of 256 in sorted order: every thread issues
// all its loads of a chunk at once (8 U pieces of 16 bytes, 4 V pieces), then
// stores them to LDS as they lie (a pair per row); the MFMA operands
// (8 consecutive pairs of one column or rank per lane) are read back with the
// LDS transpose read, and eight v_mfma_f32_16x16x32_bf16 per wave (A = U^T
// [16 n x 32 p], B = V [32 p x 16 j]) consume the chunk. The sorted-pair
// entries of the next chunk are loaded with the current chunk's data, so no
// load waits on another after the first chunk. Every sum runs in one fixed
// order.
constexpr int kWgCols = 64;
constexpr int kWgChunk = 256;
constexpr int kWgUPad = kWgCols + 8;  // LDS row of one pair's U (bf16): 144 bytes
constexpr int kWgVPad = kLoraK + 4;   // LDS row of one pair's V (bf16): 40 bytes

__global__ __launch_bounds__(256) void lora_wgrad_kernel(
    LoraWgJobs jobs, int I, const int32_t *__restrict__ sorted, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ tile_offsets, int topk, const float *__restrict__ topk_w, int r,
    float sc) {
  __shared__ __attribute__((aligned(16))) uint16_t su[kWgChunk][kWgUPad];
  __shared__ __attribute__((aligned(16))) uint16_t sv[kWgChunk][kWgVPad];
  LoraWgJob J = jobs.j[0];  // uniform selects: no dynamic index into the arguments
#pragma unroll
  for (int q = 1; q < 4; ++q)
    if (blockIdx.z == uint32_t(q)) J = jobs.j[q];
  const int N = J.N, mode = J.mode;
  const int n_base = blockIdx.x * kWgCols;
  if (n_base >= N) return;
  const int e = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = offsets[e], s1 = offsets[e + 1];
  // load roles: U: pairs tid / 8 + 32 q (q < 8), columns 8 (tid % 8) ..;
  // V: pairs tid / 4 + 64 q (q < 4), ranks 4 (tid % 4) ..
  const int upr = tid >> 3, ucg = (tid & 7) * 8;
  const int ncol = min(n_base + ucg, N - 8);  // clamped (N % 8 == 0); results past N are not stored
  const int vpr = tid >> 2, vj = (tid & 3) * 4;
  const int npb = (I + kGuBlockPairs - 1) / kGuBlockPairs;
  const bool u_sorted = mode == LS_X_GATHER || mode == LS_WX_GATHER;
  int u_idx[8], v_idx[4];  // sorted[] entries of the chunk loaded next
  u32x4 ua[8], ub[8];
  float uw[8], vw[4];
  float4 vraw[4];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    u_idx[q] = 0;
    uw[q] = 1.0f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v_idx[q] = 0;
    vw[q] = 1.0f;
  }
  auto load_idx = [&](int c0) {
    if (u_sorted) {
#pragma unroll
      for (int q = 0; q < 8; ++q) u_idx[q] = sorted[min(c0 + upr + 32 * q, s1 - 1)];
    }
    if (J.v_weighted) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v_idx[q] = sorted[min(c0 + vpr + 64 * q, s1 - 1)];
    }
  };
  auto load = [&](int c0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int s = min(c0 + upr + 32 * q, s1 - 1);
      if (mode == LS_GU_ACT) {
        // pair s of expert e: row (s - s0) % 256 of m-tile tile_offsets[e] + (s - s0) / 256
        // of the blocked g|u; columns ncol .. + 7 are two chunks (g[4], u[4])
        const int rs = s - s0, mt = tile_offsets[e] + rs / kBM;
        const int pb = ncol / kGuBlockPairs, cc = ncol % kGuBlockPairs;
        ua[q] = *reinterpret_cast<const u32x4 *>(J.src + gu_chunk(mt, pb, npb, rs % kBM, cc) * 8);
        ub[q] = *reinterpret_cast<const u32x4 *>(J.src + gu_chunk(mt, pb, npb, rs % kBM, cc + 4) * 8);
      } else {
        const int64_t row = u_sorted ? int64_t(u_idx[q] / topk) : int64_t(s);
        ua[q] = *reinterpret_cast<const u32x4 *>(J.src + row * J.ld + ncol);
        if (mode == LS_WX_GATHER) uw[q] = topk_w[u_idx[q]];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vraw[q] = *reinterpret_cast<const float4 *>(J.V + int64_t(min(c0 + vpr + 64 * q, s1 - 1)) * kLoraK + vj);
      if (J.v_weighted) vw[q] = topk_w[v_idx[q]];
    }
  };
  auto stage = [&](int c0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      u32x4 v = ua[q];
      if (mode == LS_GU_ACT) {
        const u32x4 gq{ua[q][0], ua[q][1], ub[q][0], ub[q][1]};
        const u32x4 uu{ua[q][2], ua[q][3], ub[q][2], ub[q][3]};
#pragma unroll
        for (int t = 0; t < 4; ++t)
          v[t] = pack_bf16x2(silu_f(bf16_lo(gq[t])) * bf16_lo(uu[t]),
                             silu_f(bf16_hi(gq[t])) * bf16_hi(uu[t]));
      } else if (mode == LS_WX_GATHER) {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = pack_bf16x2(uw[q] * bf16_lo(v[t]), uw[q] * bf16_hi(v[t]));
      }
      const int p = upr + 32 * q;
      *reinterpret_cast<u32x4 *>(&su[p][ucg]) = c0 + p < s1 ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = vpr + 64 * q;
      const float w = c0 + p < s1 ? vw[q] : 0.0f;
      *reinterpret_cast<u32x2 *>(&sv[p][vj]) =
          u32x2{pack_bf16x2(w * vraw[q].x, w * vraw[q].y), pack_bf16x2(w * vraw[q].z, w * vraw[q].w)};
    }
  };
  f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (s0 < s1) {
    load_idx(s0);
    load(s0);
    if (s0 + kWgChunk < s1) load_idx(s0 + kWgChunk);
  }
  // transpose-read roles: lane s of 16-lane group g supplies row 8 g + s / 4 (+ 4)
  // of a 32-pair block, columns 4 (s % 4) .. + 3 of the wave's 16
  const int ts = lane & 15, tg = lane >> 4;
  const int trow = 8 * tg + (ts >> 2), tcol = 4 * (ts & 3);
  for (int c0 = s0; c0 < s1; c0 += kWgChunk) {
    stage(c0);
    __syncthreads();
    if (c0 + kWgChunk < s1) {
      load(c0 + kWgChunk);
      if (c0 + 2 * kWgChunk < s1) load_idx(c0 + 2 * kWgChunk);
    }
    const int nk = min(kWgChunk, ((s1 - c0) + 31) & ~31) / 32;  // 32-pair blocks holding live pairs
    for (int k = 0; k < nk; ++k) {
      const uint16_t *pu = &su[32 * k + trow][wave * 16 + tcol];
      const uint16_t *pv = &sv[32 * k + trow][tcol];
      const s16x4 ulo = lds_read_tr16(pu), uhi = lds_read_tr16(pu + 4 * kWgUPad);
      const s16x4 vlo = lds_read_tr16(pv), vhi = lds_read_tr16(pv + 4 * kWgVPad);
      const bf16x8 af = __builtin_bit_cast(bf16x8, __builtin_shufflevector(ulo, uhi, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 bf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // D[n = 4 * (lane / 16) + t][j = lane % 16] of the wave's 16 columns
  const int j = lane & 15;
  if (j >= r) return;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n_base + wave * 16 + 4 * (lane >> 4) + t;
    if (n < N) {
      const int64_t o = J.out_trans ? (int64_t(e) * r + j) * N + n : (int64_t(e) * N + n) * r + j;
      J.out[o] = sc * acc[t];
    }
  }
}

hipError_t launch_lora_packs(LoraPackJobs jobs, hipStream_t st) {
  int64_t blocks = 0;
  for (int q = 0; q < jobs.n; ++q) {
    LoraPackJob &J = jobs.j[q];
    J.items = J.type == LP_JK_A ? J.E * kLoraK * (J.N / 8) : J.type == LP_JK_B ? J.E * (J.N / 8) : J.E * J.N;
    if (J.items >= (int64_t(1) << 31) || int64_t(J.E) * kLoraK * J.N >= (int64_t(1) << 31))
      return hipErrorInvalidValue;
    jobs.first_block[q] = blocks;
    blocks += (J.items + 255) / 256;
  }
  for (int q = jobs.n; q < kLoraPackJobs; ++q) jobs.first_block[q] = blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(lora_packs_kernel, dim3(uint32_t(blocks)), dim3(256), 0, st, jobs);
  return hipGetLastError();
}

hipError_t launch_lora_proj(int src_mode, const uint16_t *src, int64_t ld, int K,
                            const int32_t *sorted, int topk, const PermView &v, int E,
                            int64_t m_tiles_bound, const uint16_t *Mj, float *out, hipStream_t st) {
  if (m_tiles_bound == 0) return hipSuccess;
  const dim3 grid{uint32_t(m_tiles_bound * 4)};
  if (src_mode == LS_X_GATHER)
    hipLaunchKernelGGL((lora_proj_kernel<LS_X_GATHER>), grid, dim3(256), 0, st, src, ld, K, sorted,
                       topk, v.tile_map, v.tile_offsets, E, Mj, out);
  else if (src_mode == LS_ROWS)
    hipLaunchKernelGGL((lora_proj_kernel<LS_ROWS>), grid, dim3(256), 0, st, src, ld, K, sorted,
                       topk, v.tile_map, v.tile_offsets, E, Mj, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lora_wgrads(const LoraWgJobs &jobs, int I, const int32_t *sorted,
                              const int32_t *offsets, const int32_t *tile_offsets, int topk,
                              const float *topk_w, int64_t E, int r, float s, hipStream_t st) {
  int max_n = 0;
  for (int q = 0; q < jobs.n; ++q) max_n = jobs.j[q].N > max_n ? jobs.j[q].N : max_n;
  if (E == 0 || max_n == 0 || jobs.n == 0) return hipSuccess;
  const dim3 grid{uint32_t((max_n + kWgCols - 1) / kWgCols), uint32_t(E), uint32_t(jobs.n)};
  hipLaunchKernelGGL(lora_wgrad_kernel, grid, dim3(256), 0, st, jobs, I, sorted, offsets,
                     tile_offsets, topk, topk_w, r, s);
  return hipGetLastError();
}

}  // namespace e4b
