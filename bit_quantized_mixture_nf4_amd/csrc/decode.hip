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
// No MFMA: each 16-byte chunk of codes is expanded through a 256-entry LDS
// table (code byte -> two bf16 codebook values) and contracted with bf16
// activations by v_dot2c_f32_bf16; the block absmax is applied once per
// 64-element block to the fp32 partial sum.
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

// One workgroup: rows `row_of(r)` (r < R) of expert e's weight [*, K_in],
// contracted with the input rows of every pair of that expert.
// GATE_UP: R = 2*RJ rows (RJ gate rows j0.., then the matching up rows I+j0..);
//          output a[pos][j] = bf16(silu(g) * u).
// !GATE_UP: R rows h0.. of down; output O[pos][h] bf16.
template <bool GATE_UP>
__global__ __launch_bounds__(kDecThreads) void decode_gemv_kernel(
    const uint8_t *__restrict__ Wp, const float *__restrict__ Wa, int64_t w_e_bytes,
    int64_t w_e_blocks, int K_in, int R, int n_rows_total, int I,
    const uint16_t *__restrict__ vin, int k_route, DecodeWs w, int cb,
    uint16_t *__restrict__ out, int ldo) {
  __shared__ uint32_t tbl[256];
  __shared__ __attribute__((aligned(16))) uint32_t xs[kDecStageBytes / 4];
  __shared__ float red[kDecMaxChunks * kDecodeMaxT];
  __shared__ int32_t s_pos[kDecodeMaxT];

  const int d = blockIdx.y;
  if (d >= w.n_distinct[0]) return;
  const int e = w.dexp[d];
  const int s0 = w.dseg[d];
  // pairs of this expert: <= T <= 8 when every token's experts are distinct (a
  // documented precondition); clamped so that a violation cannot overrun LDS
  const int np_cap = min(kDecodeMaxT, kDecStageBytes / (K_in * 2));
  const int np = min(w.dseg[d + 1] - s0, np_cap);
  const int tid = threadIdx.x;

  {  // code byte -> (bf16 code of the high nibble, bf16 code of the low nibble)
    const int b = tid;
    tbl[b] = pack_bf16x2(codebook_value(cb, b >> 4), codebook_value(cb, b & 15));
  }
  if (tid < np) s_pos[tid] = s0 + tid;
  // stage input rows: gate_up -> x[token], down -> a[sorted position]
  const int kw = K_in / 2;  // uint32 words (bf16 pairs) per input row
  for (int q = 0; q < np; ++q) {
    const int spos = s0 + q;
    const int64_t src_row = GATE_UP ? int64_t(w.sorted[spos] / k_route) : int64_t(spos);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(vin + src_row * K_in);
    for (int c = tid; c < kw / 4; c += kDecThreads)
      reinterpret_cast<u32x4 *>(xs + q * kw)[c] = src[c];
  }
  __syncthreads();

  const int cpr = K_in / 32;  // 16-byte chunks per row
  const int nchunk = R * cpr;
  const uint8_t *wp = Wp + int64_t(e) * w_e_bytes;
  const float *wa = Wa + int64_t(e) * w_e_blocks;
  const int RJ = R / 2;
  for (int c = tid; c < nchunk; c += kDecThreads) {
    const int r = c / cpr, cc = c - r * cpr;
    int wrow;
    if (GATE_UP) {
      const int j = blockIdx.x * RJ + (r < RJ ? r : r - RJ);
      wrow = (r < RJ ? 0 : I) + j;
      if (j >= I) wrow = -1;
    } else {
      wrow = blockIdx.x * R + r;
      if (wrow >= n_rows_total) wrow = -1;
    }
    float part[kDecodeMaxT];
#pragma unroll
    for (int q = 0; q < kDecodeMaxT; ++q) part[q] = 0.0f;
    if (wrow >= 0) {
      const u32x4 pk =
          *reinterpret_cast<const u32x4 *>(wp + int64_t(wrow) * (K_in / 2) + cc * 16);
      const float am = wa[int64_t(wrow) * (K_in / 64) + (cc >> 1)];
      uint32_t wv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) wv[4 * i + b] = tbl[(pk[i] >> (8 * b)) & 255u];
#pragma unroll
      for (int q = 0; q < kDecodeMaxT; ++q) {
        if (q < np) {
          const u32x4 *xv = reinterpret_cast<const u32x4 *>(xs + q * kw + cc * 16);
          float s = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 xx = xv[i];
#pragma unroll
            for (int b = 0; b < 4; ++b) s = dot2_bf16(wv[4 * i + b], xx[b], s);
          }
          part[q] = s * am;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kDecodeMaxT; ++q)
      if (q < np) red[c * kDecodeMaxT + q] = part[q];
  }
  __syncthreads();

  if (GATE_UP) {
    // thread -> (gate/up row pair jj, pair q); sums over chunks in ascending order
    for (int t = tid; t < RJ * np; t += kDecThreads) {
      const int jj = t / np, q = t - jj * np;
      const int j = blockIdx.x * RJ + jj;
      if (j >= I) continue;
      float g = 0.0f, u = 0.0f;
      for (int i = 0; i < cpr; ++i) {
        g += red[(jj * cpr + i) * kDecodeMaxT + q];
        u += red[((RJ + jj) * cpr + i) * kDecodeMaxT + q];
      }
      const float a = g / (1.0f + __expf(-g)) * u;
      out[int64_t(s_pos[q]) * ldo + j] = f32_to_bf16(a);
    }
  } else {
    for (int t = tid; t < R * np; t += kDecThreads) {
      const int r = t / np, q = t - r * np;
      const int h = blockIdx.x * R + r;
      if (h >= n_rows_total) continue;
      float s = 0.0f;
      for (int i = 0; i < cpr; ++i) s += red[(r * cpr + i) * kDecodeMaxT + q];
      out[int64_t(s_pos[q]) * ldo + h] = f32_to_bf16(s);
    }
  }
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
  // gate_up: RJ gate/up row pairs per workgroup, about kDecMaxChunks chunks
  int RJ = kDecMaxChunks / (2 * (H / 32));
  if (RJ > 16) RJ = 16;
  if (RJ < 1) RJ = 1;
  const e4b_stack &gu = L->gate_up, &dn = L->down;
  timer_before(E4B_K_DECODE_GATE_UP, s);
  hipLaunchKernelGGL((decode_gemv_kernel<true>), dim3(uint32_t((I + RJ - 1) / RJ), uint32_t(ymax)),
                     dim3(kDecThreads), 0, s, gu.packed, gu.absmax, gu.out * gu.in / 2,
                     gu.out * gu.in / kBlock, H, 2 * RJ, 2 * I, I, x, int(p.k), w, p.codebook,
                     a_buf, I);
  timer_after(E4B_K_DECODE_GATE_UP, s);
  int R = kDecMaxChunks / (I / 32);
  if (R > 64) R = 64;
  if (R < 1) R = 1;
  timer_before(E4B_K_DECODE_DOWN, s);
  hipLaunchKernelGGL((decode_gemv_kernel<false>), dim3(uint32_t((H + R - 1) / R), uint32_t(ymax)),
                     dim3(kDecThreads), 0, s, dn.packed, dn.absmax, dn.out * dn.in / 2,
                     dn.out * dn.in / kBlock, I, R, H, I, a_buf, int(p.k), w, p.codebook, o_buf,
                     H);
  timer_after(E4B_K_DECODE_DOWN, s);
  return launch_combine_rows(o_buf, w.pos, wts, p.T, int(p.k), H, y, s);
}

}  // namespace e4b
