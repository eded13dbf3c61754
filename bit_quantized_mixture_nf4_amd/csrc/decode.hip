// decode.hip -- forward for T <= 8 tokens as bandwidth-bound dequant-GEMVs.
//
// The 0.4.0 README ("Inference" section) describes the decode fast path: a
// single-token forward skips the one-hot grouping and its per-expert host
// syncs, and single-row projections read the packed 4-bit weight directly
// instead of materializing a dequantized expert. Here, for T <= 8:
//   prep     one workgroup groups the <= 8*k routed pairs by expert (stable)
//            and lists the distinct experts in ascending order;
//   gate_up  one workgroup per (distinct expert, block of gate/up row pairs):
//            every packed byte is read once for all tokens routed to that
//            expert; a = silu(g) * u is written as bf16;
//   down     one workgroup per (distinct expert, block of rows of H);
//   combine  the shared deterministic gather-combine.
// No MFMA: each code byte is expanded through a 256-entry LDS table into two
// bf16 codebook values and contracted with bf16 activations by
// v_dot2c_f32_bf16 in fp32; the block absmax scales each lane's partial sum.
#include "device.h"
#include "kernels.h"

namespace e4b {

constexpr int kDecThreads = 256;

// Workspace layout of the decode path (inside the permutation region).
struct DecodeWs {
  int32_t *n_distinct;  // [1]
  int32_t *dexp;        // [kDecMaxPairs] expert id of distinct expert d (ascending)
  int32_t *dseg;        // [kDecMaxPairs + 1] sorted-pair offsets of distinct expert d
  int32_t *sorted;      // [P] pair id at sorted position
  int32_t *pos;         // [P] sorted position of pair id
};

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__global__ __launch_bounds__(256) void decode_prep_kernel(const int32_t *__restrict__ idx, int P,
                                                          DecodeWs w) {
  __shared__ int32_t s_e[kDecMaxPairs];
  __shared__ int32_t s_sorted[kDecMaxPairs];
  __shared__ int32_t s_first[kDecMaxPairs];
  const int p = threadIdx.x;
  if (p < P) s_e[p] = idx[p];
  __syncthreads();
  int pos = 0;
  if (p < P) {
    const int e = s_e[p];
    for (int q = 0; q < P; ++q) {
      const int eq = s_e[q];
      pos += (eq < e || (eq == e && q < p)) ? 1 : 0;
    }
    s_sorted[pos] = p;
    w.sorted[pos] = p;
    w.pos[p] = pos;
  }
  __syncthreads();
  if (p < P) s_first[p] = (p == 0 || s_e[s_sorted[p - 1]] != s_e[s_sorted[p]]) ? 1 : 0;
  __syncthreads();
  if (p < P && s_first[p]) {
    int d = 0;
    for (int q = 0; q < p; ++q) d += s_first[q];
    w.dexp[d] = s_e[s_sorted[p]];
    w.dseg[d] = p;
  }
  if (p == 0) {
    int n = 0;
    for (int q = 0; q < P; ++q) n += s_first[q];
    w.n_distinct[0] = n;
    w.dseg[n] = P;
  }
}

// One wavefront streams weight rows of one expert past a fixed slice of the
// reduction dimension: lane l owns elements [kl*EPL, kl*EPL + EPL) of every
// row (kl = l % LPR, LPR lanes per row, 64/LPR rows per pass) and keeps the
// matching slice of the input vector of each of the expert's NP tokens in
// registers (loaded once, reused for all its rows). Loads of kBatch passes are
// issued before any of them is used. Each code byte is expanded through a
// 256-entry LDS table into two bf16 codebook values and contracted with the
// inputs by v_dot2c_f32_bf16; the lane's block absmax scales its partial sum
// once; the LPR partials of a row are summed with shuffles. GATE_UP processes
// gate row u and up row I + u in the same lanes and writes a = silu(g) * up;
// otherwise row u's dot product is written.
constexpr int kBatch = 4;

template <bool GATE_UP, int NP, int EPL>
__device__ __forceinline__ void decode_rows(const uint32_t *tbl, const uint8_t *wp,
                                            const float *wa, int K_in, int n_units, int I,
                                            const uint16_t *vin, int k_route, const DecodeWs &w,
                                            int s0, uint16_t *out, int ldo, int u_first,
                                            int units_per_wave, int lane) {
  constexpr int WPL = EPL / 2;   // bf16-pair words per lane
  constexpr int NV = EPL / 32;   // 16-byte weight loads per row slice
  constexpr int NR = GATE_UP ? 2 : 1;
  const int cpr = K_in / EPL;    // lanes holding data per row
  int LPR = 1;
  while (LPR < cpr) LPR <<= 1;
  const int rpp = 64 / LPR;
  const int ru = lane / LPR, kl = lane % LPR;
  const bool kvalid = kl < cpr;
  const int kbase = kvalid ? kl * EPL : 0;
  const int row_bytes = K_in >> 1, row_blocks = K_in >> 6;
  wp += kbase >> 1;
  wa += kbase >> 6;

  // Lanes past the end of a row (kl >= cpr) read the row's first slice (always
  // in bounds) and zero their input slice, so they contribute exact zeros.
  uint32_t xr[NP][WPL];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int64_t row = GATE_UP ? int64_t(w.sorted[s0 + q] / k_route) : int64_t(s0 + q);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(vin + row * K_in + kbase);
#pragma unroll
    for (int c = 0; c < WPL / 4; ++c) {
      const u32x4 v = src[c];
#pragma unroll
      for (int t = 0; t < 4; ++t) xr[q][4 * c + t] = kvalid ? v[t] : 0u;
    }
  }

  for (int p0 = 0; p0 < units_per_wave; p0 += kBatch * rpp) {
    u32x4 wv[kBatch][NR][NV];
    float am[kBatch][NR];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int u = u_first + p0 + b * rpp + ru;
      const int uc = u < n_units ? u : 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int64_t row = r == 0 ? uc : I + uc;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(wp + row * row_bytes);
#pragma unroll
        for (int c = 0; c < NV; ++c) wv[b][r][c] = src[c];
        am[b][r] = wa[row * row_blocks];
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      float acc[NR][NP];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int q = 0; q < NP; ++q) acc[r][q] = 0.0f;
#pragma unroll
        for (int c = 0; c < NV; ++c)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t word = wv[b][r][c][t];
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              const uint32_t codes = tbl[(word >> (8 * y)) & 255u];
#pragma unroll
              for (int q = 0; q < NP; ++q)
                acc[r][q] = dot2_bf16(codes, xr[q][16 * c + 4 * t + y], acc[r][q]);
            }
          }
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          float v = acc[r][q] * am[b][r];
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1)
            if (o < LPR) v += __shfl_xor(v, o);
          acc[r][q] = v;
        }
      }
      const int u = u_first + p0 + b * rpp + ru;
      if (u < n_units && kl == 0) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const float g = acc[0][q];
          const float v = GATE_UP ? g / (1.0f + __expf(-g)) * acc[NR - 1][q] : g;
          out[int64_t(s0 + q) * ldo + u] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <bool GATE_UP, int MAXNP, int EPL>
__global__ __launch_bounds__(kDecThreads) void decode_gemv_kernel(
    const uint8_t *__restrict__ Wp, const float *__restrict__ Wa, int64_t w_e_bytes,
    int64_t w_e_blocks, int K_in, int n_units, int I, const uint16_t *__restrict__ vin,
    int k_route, DecodeWs w, int cb, uint16_t *__restrict__ out, int ldo, int units_per_wave) {
  __shared__ uint32_t tbl[256];
  const int d = blockIdx.y;
  if (d >= w.n_distinct[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // code byte -> (bf16 code of the high nibble | bf16 code of the low nibble << 16)
  tbl[tid] = pack_bf16x2(codebook_value(cb, tid >> 4), codebook_value(cb, tid & 15));
  __syncthreads();
  const int e = w.dexp[d];
  const int s0 = w.dseg[d];
  const int np = w.dseg[d + 1] - s0;  // <= T when tokens' experts are distinct
  const uint8_t *wp = Wp + int64_t(e) * w_e_bytes;
  const float *wa = Wa + int64_t(e) * w_e_blocks;
  const int u_first = (blockIdx.x * (kDecThreads / 64) + wave) * units_per_wave;
#define E4B_DEC_CASE(N)                                                                      \
  case N:                                                                                    \
    if constexpr (N <= MAXNP)                                                                \
      decode_rows<GATE_UP, N, EPL>(tbl, wp, wa, K_in, n_units, I, vin, k_route, w, s0, out, \
                                   ldo, u_first, units_per_wave, lane);                      \
    break;
  switch (np < MAXNP ? np : MAXNP) {
    E4B_DEC_CASE(1)
    E4B_DEC_CASE(2)
    E4B_DEC_CASE(3)
    E4B_DEC_CASE(4)
    E4B_DEC_CASE(5)
    E4B_DEC_CASE(6)
    E4B_DEC_CASE(7)
    E4B_DEC_CASE(8)
    default:
      break;
  }
#undef E4B_DEC_CASE
}

hipError_t launch_decode_forward(const MoePlan &p, const e4b_moe_layer *L, const uint16_t *x,
                                 const int32_t *idx, const float *wts, uint16_t *y, char *ws,
                                 hipStream_t s) {
  DecodeWs w;
  // the decode path reuses slots of the permutation region:
  // dexp <= min(E, P) entries, dseg <= min(E, P) + 1 entries
  w.n_distinct = reinterpret_cast<int32_t *>(ws + p.off_tile_offsets);
  w.dexp = reinterpret_cast<int32_t *>(ws + p.off_counts);
  w.dseg = reinterpret_cast<int32_t *>(ws + p.off_offsets);
  w.sorted = reinterpret_cast<int32_t *>(ws + p.off_sorted);
  w.pos = reinterpret_cast<int32_t *>(ws + p.off_pos);
  uint16_t *a_buf = reinterpret_cast<uint16_t *>(ws + p.off_a);
  uint16_t *o_buf = reinterpret_cast<uint16_t *>(ws + p.off_o);
  const int P = int(p.P);
  hipLaunchKernelGGL(decode_prep_kernel, dim3(1), dim3(256), 0, s, idx, P, w);

  const int ymax = int(p.P < p.E ? p.P : p.E);
  const int H = int(p.H), I = int(p.I);
  const e4b_stack &gu = L->gate_up, &dn = L->down;
  auto lanes_per_row = [](int K_in, int epl) {
    int l = 1;
    while (l < K_in / epl) l <<= 1;
    return l;
  };
  // row units per wave: kBatch passes for one token, up to 4 batches when the
  // per-wave input slices of several tokens must be amortized over more rows
  const int batches = p.T <= 1 ? 1 : (p.T <= 2 ? 2 : 4);
  auto launch_pair = [&](auto gu_kernel, auto dn_kernel, int epl) {
    // gate_up: I gate/up row pairs over K_in = H
    const int upw_g = batches * kBatch * (64 / lanes_per_row(H, epl));
    const int wg_g = (I + 4 * upw_g - 1) / (4 * upw_g);
    timer_before(E4B_K_DECODE_GATE_UP, s);
    hipLaunchKernelGGL(gu_kernel, dim3(uint32_t(wg_g), uint32_t(ymax)), dim3(kDecThreads), 0, s,
                       gu.packed, gu.absmax, gu.out * gu.in / 2, gu.out * gu.in / kBlock, H, I, I,
                       x, int(p.k), w, p.codebook, a_buf, I, upw_g);
    timer_after(E4B_K_DECODE_GATE_UP, s);
    // down: H rows over K_in = I
    const int upw_d = batches * kBatch * (64 / lanes_per_row(I, epl));
    const int wg_d = (H + 4 * upw_d - 1) / (4 * upw_d);
    timer_before(E4B_K_DECODE_DOWN, s);
    hipLaunchKernelGGL(dn_kernel, dim3(uint32_t(wg_d), uint32_t(ymax)), dim3(kDecThreads), 0, s,
                       dn.packed, dn.absmax, dn.out * dn.in / 2, dn.out * dn.in / kBlock, I, H, I,
                       a_buf, int(p.k), w, p.codebook, o_buf, H, upw_d);
    timer_after(E4B_K_DECODE_DOWN, s);
  };
  if (p.T <= 1)
    launch_pair(decode_gemv_kernel<true, 1, 64>, decode_gemv_kernel<false, 1, 64>, 64);
  else if (p.T <= 2)
    launch_pair(decode_gemv_kernel<true, 2, 64>, decode_gemv_kernel<false, 2, 64>, 64);
  else if (p.T <= 4)
    launch_pair(decode_gemv_kernel<true, 4, 32>, decode_gemv_kernel<false, 4, 32>, 32);
  else
    launch_pair(decode_gemv_kernel<true, 8, 32>, decode_gemv_kernel<false, 8, 32>, 32);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_combine_rows(o_buf, w.pos, wts, p.T, int(p.k), H, y, s);
}

}  // namespace e4b
